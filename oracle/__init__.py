"""CPU oracle of the speculative-decoding verify step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain fp64
C++, built from ``oracle.cpp`` by ``oracle/build.py``) and shares no code with
the GPU path.

Parity pins: every function of the oracle is pinned by the CPU tests in
``tests/test_oracle_*.py`` (closed forms, a worked example, library routines on
small inputs, brute force, and chi-square tests of the losslessness claim).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import build as _build

STOCHASTIC, GREEDY, NKL, TREE_GREEDY, BLOCK = 0, 1, 2, 3, 4

FLAG_ACCEPT_BAND = 1
FLAG_DRAW_BAND = 2
FLAG_NKL_BAND = 4
FLAG_EMPTY_RESIDUAL = 8
FLAG_INVALID = 16

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        lib.sv_oracle_verify.restype = ctypes.c_int
        lib.sv_oracle_verify.argtypes = [P, P, i32, i32, i32, P, P, P, P, P, i32, f32, P, f32, f32, P, i32, i32,
                                         i64, P, P, P, P, P, P, P, P, P, P, P, i32]
        lib.sv_oracle_sample_rows.restype = ctypes.c_int
        lib.sv_oracle_sample_rows.argtypes = [P, i32, i64, i32, P, P, P, P, i32]
        lib.sv_oracle_topk_rows.restype = ctypes.c_int
        lib.sv_oracle_topk_rows.argtypes = [P, i32, i64, i32, i32, P, i32]
        lib.sv_oracle_nkl_threshold.restype = ctypes.c_double
        lib.sv_oracle_nkl_threshold.argtypes = [f32, f32, f32, i32]
        lib.sv_oracle_consensus.restype = ctypes.c_int
        lib.sv_oracle_consensus.argtypes = [P, i32, i32, i32, i32, P, P, f32, f32, P, P, P, P, i32]
        lib.sv_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().sv_oracle_max_threads())


def sample_rows(logits: np.ndarray, dtype: str, temperature: np.ndarray, u: np.ndarray, nthreads: int = 0):
    """Draws one token per row from softmax(row / T) by the inverse CDF with the
    row's uniform.  Returns (tokens int32 [rows], margins float64 [rows])."""
    rows, V = int(logits.shape[0]), int(logits.shape[1])
    if dtype == "bf16":
        logits, dt = np.ascontiguousarray(logits, np.uint16), 1
    elif dtype == "f32":
        logits, dt = np.ascontiguousarray(logits, np.float32), 0
    else:
        raise ValueError(dtype)
    temperature = np.ascontiguousarray(temperature, np.float32)
    u = np.ascontiguousarray(u, np.float32)
    out = np.full(max(rows, 1), -7, np.int32)
    margin = np.full(max(rows, 1), np.nan)
    rc = _load().sv_oracle_sample_rows(_ptr(logits), dt, rows, V, _ptr(temperature), _ptr(u), _ptr(out),
                                       _ptr(margin), int(nthreads))
    if rc != 0:
        raise ValueError("sv_oracle_sample_rows rejected its arguments")
    return out[:rows], margin[:rows]


def topk_rows(logits: np.ndarray, dtype: str, k: int, nthreads: int = 0) -> np.ndarray:
    """The k largest logits of every row: int32 [rows, k] indices, largest
    first, the lower index first among equal logits."""
    rows, V = int(logits.shape[0]), int(logits.shape[1])
    if dtype == "bf16":
        logits, dt = np.ascontiguousarray(logits, np.uint16), 1
    elif dtype == "f32":
        logits, dt = np.ascontiguousarray(logits, np.float32), 0
    else:
        raise ValueError(dtype)
    out = np.full((max(rows, 1), k), -7, np.int32)
    if _load().sv_oracle_topk_rows(_ptr(logits), dt, rows, V, int(k), _ptr(out), int(nthreads)) != 0:
        raise ValueError("sv_oracle_topk_rows rejected its arguments")
    return out[:rows]


@dataclass
class ConsensusResult:
    nkl: np.ndarray    # float64 [positions, K, K]: KL(q_a || q_b) / ln V (NaN for invalid requests)
    state: np.ndarray  # int32 [positions]: 1 consensus, 2 divergence, 0 neither, -1 invalid request
    pair: np.ndarray   # int32 [positions]: a * K + b of the closest pair a < b (-1 invalid)
    flags: np.ndarray  # int32 [positions]: 1 / 2 near a threshold, 4 near tie of the closest pair


def consensus(drafts: np.ndarray, dtype: str, gamma: np.ndarray, K: int, temperature: np.ndarray,
              delta_c: float = 0.1, delta_d: float = 0.15, nthreads: int = 0) -> ConsensusResult:
    """Pairwise NKL of K drafts per position (rows [sum(gamma) * K, V], the K
    drafts of a position consecutive) and the consensus / divergence state."""
    gamma = np.ascontiguousarray(gamma, np.int32)
    B, V = int(gamma.shape[0]), int(drafts.shape[1])
    if dtype == "bf16":
        drafts, dt = np.ascontiguousarray(drafts, np.uint16), 1
    elif dtype == "f32":
        drafts, dt = np.ascontiguousarray(drafts, np.float32), 0
    else:
        raise ValueError(dtype)
    npos = int(gamma.astype(np.int64).sum())
    temperature = np.ascontiguousarray(temperature, np.float32)
    nkl = np.full((max(npos, 1), K, K), np.nan)
    state = np.full(max(npos, 1), -7, np.int32)
    pair = np.full(max(npos, 1), -7, np.int32)
    flags = np.zeros(max(npos, 1), np.int32)
    rc = _load().sv_oracle_consensus(_ptr(drafts), dt, B, int(K), V, _ptr(gamma), _ptr(temperature),
                                     float(delta_c), float(delta_d), _ptr(nkl), _ptr(state), _ptr(pair),
                                     _ptr(flags), int(nthreads))
    if rc != 0:
        raise ValueError("sv_oracle_consensus rejected its arguments")
    return ConsensusResult(nkl[:npos], state[:npos], pair[:npos], flags[:npos])


def nkl_threshold(delta: float, alpha: float, delta_max: float, position: int) -> float:
    """Position-adaptive NKL threshold of a draft token at 0-based position
    ``position`` of the generated sequence (float64)."""
    return float(_load().sv_oracle_nkl_threshold(float(delta), float(alpha), float(delta_max), int(position)))


@dataclass
class OracleResult:
    tokens: np.ndarray  # int32 [sum(gamma+1)]
    num_accepted: np.ndarray  # int32 [B]
    nkl: np.ndarray  # float64 [sum(gamma)] (NaN where not computed)
    p_x: np.ndarray
    q_x: np.ndarray
    alpha: np.ndarray
    resid_mass: np.ndarray  # float64 [B]
    tree_node: np.ndarray  # int32 [B]
    flags: np.ndarray  # int32 [B]
    accept_margin: np.ndarray  # float64 [B]
    draw_margin: np.ndarray  # float64 [B]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def verify(target: np.ndarray, draft: Optional[np.ndarray], dtype: str, gamma: np.ndarray,
           draft_tokens: np.ndarray, temperature: Optional[np.ndarray], u_accept: Optional[np.ndarray],
           u_resample: Optional[np.ndarray], mode: int, delta: float = 0.15,
           tree_parents: Optional[np.ndarray] = None, max_gamma: Optional[int] = None,
           total_draft_rows: Optional[int] = None, nthreads: int = 0,
           nkl_position: Optional[np.ndarray] = None, nkl_alpha: float = 0.0,
           nkl_delta_max: float = 0.0, block_min_len: int = 3) -> OracleResult:
    """Runs the oracle on host arrays (the packed layout of the C ABI).
    nkl_position (NKL mode): 0-based position of every draft token in the
    generated sequence, for the position-adaptive threshold (None: constant).
    block_min_len (block-accept mode): the shortest agreeing run that is kept."""
    lib = _load()
    gamma = np.ascontiguousarray(gamma, np.int32)
    B = int(gamma.shape[0])
    V = int(target.shape[1])
    if dtype == "bf16":
        target = np.ascontiguousarray(target, np.uint16)
        draft = None if draft is None else np.ascontiguousarray(draft, np.uint16)
        dt = 1
    elif dtype == "f32":
        target = np.ascontiguousarray(target, np.float32)
        draft = None if draft is None else np.ascontiguousarray(draft, np.float32)
        dt = 0
    else:
        raise ValueError(dtype)
    pos = gamma[gamma > 0].astype(np.int64).sum()
    R_t = int(pos + B)
    R_d = int(pos)
    if total_draft_rows is None:
        total_draft_rows = int(gamma.astype(np.int64).sum())
    if max_gamma is None:
        max_gamma = int(max(0, gamma.max()))
    c = lambda a, t: None if a is None else np.ascontiguousarray(a, t)
    draft_tokens = c(draft_tokens, np.int32)
    temperature = c(temperature, np.float32)
    u_accept = c(u_accept, np.float32)
    u_resample = c(u_resample, np.float32)
    tree_parents = c(tree_parents, np.int32)
    nkl_position = c(nkl_position, np.int32)
    out_tokens = np.full(max(R_t, 1), -7, np.int32)
    out_num = np.full(B, -7, np.int32)
    nkl = np.full(max(R_d, 1), np.nan)
    p_x = np.full(max(R_d, 1), np.nan)
    q_x = np.full(max(R_d, 1), np.nan)
    alpha = np.full(max(R_d, 1), np.nan)
    resid = np.full(B, np.nan)
    tnode = np.full(B, -1, np.int32)
    flags = np.zeros(B, np.int32)
    am = np.full(B, np.inf)
    dm = np.full(B, np.inf)
    rc = lib.sv_oracle_verify(_ptr(target), _ptr(draft), dt, B, V, _ptr(draft_tokens), _ptr(gamma),
                              _ptr(temperature), _ptr(u_accept), _ptr(u_resample), int(mode), float(delta),
                              _ptr(nkl_position), float(nkl_alpha), float(nkl_delta_max), _ptr(tree_parents),
                              int(block_min_len), int(max_gamma), int(total_draft_rows), _ptr(out_tokens),
                              _ptr(out_num), _ptr(nkl), _ptr(p_x), _ptr(q_x), _ptr(alpha), _ptr(resid),
                              _ptr(tnode), _ptr(flags), _ptr(am), _ptr(dm), int(nthreads))
    if rc != 0:
        raise ValueError("sv_oracle_verify rejected its arguments")
    return OracleResult(out_tokens[:R_t], out_num, nkl[:R_d], p_x[:R_d], q_x[:R_d], alpha[:R_d], resid,
                        tnode, flags, am, dm)


def verify_workload(w, nthreads: int = 0) -> OracleResult:
    """Convenience: runs the oracle on a ``synthetic.Workload``-like object."""
    return verify(w.target, w.draft, w.dtype, w.gamma, w.draft_tokens, w.temperature, w.u_accept,
                  w.u_resample, w.mode, w.delta, w.tree_parents, w.max_gamma, w.total_draft_rows, nthreads,
                  getattr(w, "nkl_position", None), getattr(w, "nkl_alpha", 0.0), getattr(w, "nkl_delta_max", 0.0),
                  getattr(w, "block_min_len", 3))
