"""Seeded synthetic inputs for the speculative-decoding verify step.

This module only *makes inputs*.  It holds none of the verify step's
arithmetic (no softmax, no acceptance test, no residual, no KL): both the
HIP path and the CPU oracle consume what it produces, and neither is imported
here.

Workloads follow the shapes and value distributions the source pages use for
the verify step of speculative decoding:

* target logits are ``3*N(0,1)`` per entry, plus (in the bf16 workloads) a
  ``+8`` spike at one uniformly chosen index per row;
* draft logits are the paired target row plus Gaussian noise;
* drafted tokens are *drawn from the draft softmax* (sampling drafts, as the
  losslessness argument of modified rejection sampling assumes), or taken as
  the draft row's argmax (greedy drafting, as in the argmax draft loop of the
  "投机采样" page's ``SpeculativeEngine`` listing), or the top-k children of a
  draft tree (the P-EAGLE tree of the "Parallel Drafting" page, section 2.2);
* uniforms are float32 in [0,1).

Draws of the drafter use the Gumbel-max construction: ``argmax_y(d_y/T + G_y)``
with ``G = -log(E)``, ``E ~ Exp(1)``, evaluated in float64 on the *stored*
(already rounded) draft logits.  This is an exact sampler of
``softmax(d/T)`` and computes no softmax itself.

Every random stream is a Philox4x32 counter-based generator keyed by
``(seed, workload id, purpose, row)``, so generation is deterministic and can be
split over threads without changing a single value.

bf16 storage: values are generated in float32 and rounded to bfloat16 with
round-to-nearest-even; the stored 16-bit patterns are the inputs of record for
both the oracle and the GPU path.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BASE_SEED = 20261202

# verify modes (same numbering as the C ABI)
STOCHASTIC, GREEDY, NKL, TREE_GREEDY, BLOCK = 0, 1, 2, 3, 4
MODE_NAMES = {STOCHASTIC: "stochastic", GREEDY: "greedy", NKL: "nkl", TREE_GREEDY: "tree", BLOCK: "block"}

# purposes of the random streams
_P_TARGET, _P_SPIKE, _P_DNOISE, _P_DRAW, _P_UACC, _P_URES, _P_PARAM, _P_POS = range(8)

# Trees used by the tree-draft workload.  Entry k is the parent of node k
# (node 0 is the root, whose entry is -1).  "LITERAL16": a root with 3
# children, each child with 2 children, each of those with 1 child (16 nodes,
# 15 drafted tokens).  "P_EAGLE13": the <=12-draft reading (top-3, then 2, then
# one extension per branch), 13 nodes.
TREE_LITERAL16 = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 5, 6, 7, 8, 9], np.int32)
TREE_P_EAGLE13 = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 6, 8], np.int32)


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(wid: int, purpose: int, row: int = 0, seed: int = BASE_SEED) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, wid, purpose, row])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    rounding = ((b >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One batch of verify inputs in the packed (ragged) layout.

    ``target`` has ``sum(gamma+1)`` rows, ``draft`` ``sum(gamma)`` rows (or None
    when the mode never reads draft logits).  Logit rows are stored as uint16
    bf16 patterns (``dtype == "bf16"``) or float32.
    """

    name: str
    mode: int
    batch: int
    vocab: int
    dtype: str  # "bf16" | "f32"
    gamma: np.ndarray  # int32 [B]
    target: np.ndarray  # [sum(gamma+1), V] uint16 or float32
    draft: Optional[np.ndarray]  # [sum(gamma), V] or None
    draft_tokens: np.ndarray  # int32 [sum(gamma)]
    temperature: np.ndarray  # float32 [B]
    u_accept: np.ndarray  # float32 [sum(gamma)]
    u_resample: np.ndarray  # float32 [B]
    delta: float = 0.15
    tree_parents: Optional[np.ndarray] = None  # int32 [sum(gamma)] (tree mode)
    max_gamma: int = 0
    meta: dict = field(default_factory=dict)
    # NKL mode, position-adaptive threshold: 0-based position of every draft
    # token in the generated sequence (None: the constant threshold delta)
    nkl_position: Optional[np.ndarray] = None  # int32 [sum(gamma)]
    nkl_alpha: float = 0.0
    nkl_delta_max: float = 0.0
    # block-accept mode: the shortest run of agreeing positions that is kept
    block_min_len: int = 3

    @property
    def total_draft_rows(self) -> int:
        return int(self.gamma.sum())

    @property
    def t_off(self) -> np.ndarray:
        o = np.zeros(self.batch + 1, np.int64)
        np.cumsum(self.gamma.astype(np.int64) + 1, out=o[1:])
        return o

    @property
    def d_off(self) -> np.ndarray:
        o = np.zeros(self.batch + 1, np.int64)
        np.cumsum(self.gamma.astype(np.int64), out=o[1:])
        return o

    def target_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.target) if self.dtype == "bf16" else self.target

    def draft_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.draft) if self.dtype == "bf16" else self.draft

    def logit_bytes(self) -> int:
        s = 2 if self.dtype == "bf16" else 4
        n = self.target.shape[0] + (0 if self.draft is None else self.draft.shape[0])
        return s * self.vocab * n

    def with_positions(self, start_max: int = 4096, alpha: float = 0.08, delta_max: float = 0.3,
                       seed: int = BASE_SEED, wid: int = 7) -> "Workload":
        """The same inputs with generation positions for the position-adaptive
        NKL threshold ("Chain of Draft" page, section 4.3: long generations,
        delta_base 0.15, alpha 0.08, cap 0.3).  Request b's drafts continue a
        sequence at a start position ~ U{0 .. start_max-1}; draft token i of
        request b is at start_b + i."""
        w = Workload(**{k: getattr(self, k) for k in self.__dataclass_fields__})
        g = _gen(wid, _P_POS, 0, seed)
        start = g.integers(0, start_max, self.batch, dtype=np.int64)
        d_off = self.d_off
        pos = np.empty(self.total_draft_rows, np.int32)
        for b in range(self.batch):
            pos[d_off[b]:d_off[b + 1]] = start[b] + np.arange(self.gamma[b])
        w.nkl_position, w.nkl_alpha, w.nkl_delta_max = pos, float(alpha), float(delta_max)
        w.name = self.name + "_pos"
        return w

    def with_mode(self, mode: int, delta: Optional[float] = None) -> "Workload":
        w = Workload(**{k: getattr(self, k) for k in self.__dataclass_fields__})
        w.mode = mode
        if delta is not None:
            w.delta = float(delta)
        w.name = self.name
        return w


# ----------------------------------------------------------------------------
# row generators (threaded over rows; each row has its own Philox stream)
# ----------------------------------------------------------------------------

def _par_rows(n: int, fn) -> None:
    if n == 0:
        return
    nt = _threads()
    if nt == 1 or n < 4:
        for r in range(n):
            fn(r)
        return
    with ThreadPoolExecutor(nt) as ex:
        list(ex.map(fn, range(n)))


def _target_rows(wid: int, nrows: int, V: int, scale: float, spike: float, seed: int) -> np.ndarray:
    out = np.empty((nrows, V), np.float32)

    def fn(r):
        g = _gen(wid, _P_TARGET, r, seed)
        g.standard_normal(out=out[r], dtype=np.float32)
        out[r] *= np.float32(scale)
        if spike != 0.0:
            k = int(_gen(wid, _P_SPIKE, r, seed).integers(0, V))
            out[r, k] += np.float32(spike)

    _par_rows(nrows, fn)
    return out


def _draft_rows(wid: int, tgt: np.ndarray, rows: np.ndarray, sigma: np.ndarray, seed: int) -> np.ndarray:
    """draft row k = target row rows[k] + sigma[k]*N(0,1) (float32)."""
    n, V = len(rows), tgt.shape[1]
    out = np.empty((n, V), np.float32)

    def fn(k):
        g = _gen(wid, _P_DNOISE, k, seed)
        g.standard_normal(out=out[k], dtype=np.float32)
        out[k] *= np.float32(sigma[k])
        out[k] += tgt[rows[k]]

    _par_rows(n, fn)
    return out


def _round_store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)

    def fn(r):
        out[r] = f32_to_bf16_bits(x[r])

    _par_rows(x.shape[0], fn)
    return out


def _sample_drafts(wid: int, stored_f32: np.ndarray, temps_per_row: np.ndarray, seed: int) -> np.ndarray:
    """x_k ~ softmax(d_k / T_k) by Gumbel-max in float64 on the stored values."""
    n = stored_f32.shape[0]
    out = np.empty(n, np.int32)

    def fn(k):
        g = _gen(wid, _P_DRAW, k, seed)
        e = g.standard_exponential(stored_f32.shape[1])
        z = stored_f32[k].astype(np.float64) / np.float64(np.float32(temps_per_row[k])) - np.log(e)
        out[k] = int(np.argmax(z))

    _par_rows(n, fn)
    return out


def _uniforms(wid: int, purpose: int, n: int, seed: int) -> np.ndarray:
    return _gen(wid, purpose, 0, seed).random(n, dtype=np.float32)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

def make_tiny(steps: int = 1000, gamma: int = 4, V: int = 1000, seed: int = BASE_SEED, wid: int = 0) -> Workload:
    """Tiny stochastic verify: ``steps`` independent one-request steps packed as a
    batch (B = steps), gamma=4, V=1000, fp32, T=1.  Target 3*N(0,1); draft =
    target + N(0,1); drafts sampled from the draft softmax."""
    B = steps
    gam = np.full(B, gamma, np.int32)
    t_off = np.concatenate([[0], np.cumsum(gam + 1)])
    tgt = _target_rows(wid, int(t_off[-1]), V, 3.0, 0.0, seed)
    rows = np.concatenate([np.arange(t_off[b], t_off[b] + gam[b]) for b in range(B)]).astype(np.int64)
    drf = _draft_rows(wid, tgt, rows, np.ones(len(rows), np.float32), seed)
    temps = np.ones(B, np.float32)
    trow = np.repeat(temps, gam)
    x = _sample_drafts(wid, drf, trow, seed)
    return Workload("tiny", STOCHASTIC, B, V, "f32", gam, tgt, drf, x, temps,
                    _uniforms(wid, _P_UACC, len(rows), seed), _uniforms(wid, _P_URES, B, seed),
                    max_gamma=gamma)


def make_llama3(B: int = 32, gamma: int = 5, V: int = 128256, seed: int = BASE_SEED, wid: int = 1) -> Workload:
    """Llama-3-shaped stochastic verify: B=32, gamma=5, V=128256, bf16.  Target
    3*N(0,1) + 8 spike; draft = target + N(0, 0.7^2); T in {0.6, 1.0} per
    request; drafts sampled from the draft softmax."""
    gam = np.full(B, gamma, np.int32)
    t_off = np.concatenate([[0], np.cumsum(gam + 1)])
    tgt32 = _target_rows(wid, int(t_off[-1]), V, 3.0, 8.0, seed)
    rows = np.concatenate([np.arange(t_off[b], t_off[b] + gam[b]) for b in range(B)]).astype(np.int64)
    drf32 = _draft_rows(wid, tgt32, rows, np.full(len(rows), 0.7, np.float32), seed)
    tgt, drf = _round_store(tgt32, "bf16"), _round_store(drf32, "bf16")
    del tgt32, drf32
    pg = _gen(wid, _P_PARAM, 0, seed)
    temps = np.where(pg.integers(0, 2, B) == 0, 0.6, 1.0).astype(np.float32)
    x = _sample_drafts(wid, bf16_bits_to_f32(drf), np.repeat(temps, gam), seed)
    return Workload("llama3", STOCHASTIC, B, V, "bf16", gam, tgt, drf, x, temps,
                    _uniforms(wid, _P_UACC, len(rows), seed), _uniforms(wid, _P_URES, B, seed),
                    max_gamma=gamma)


def make_long(B: int = 64, gamma: int = 16, V: int = 128256, mode: int = GREEDY, delta: float = 0.15,
              seed: int = BASE_SEED, wid: int = 2) -> Workload:
    """Long parallel drafts: B=64, gamma=16, V=128256, bf16, T=0.6.  Draft noise
    sigma_i = 0.3 + 1.2*i/(gamma-1) along the draft so acceptance decays; drafts
    are the argmax of each draft row (greedy drafting).  Runs in greedy mode or
    in NKL mode with delta=0.15."""
    gam = np.full(B, gamma, np.int32)
    t_off = np.concatenate([[0], np.cumsum(gam + 1)])
    tgt32 = _target_rows(wid, int(t_off[-1]), V, 3.0, 8.0, seed)
    rows = np.concatenate([np.arange(t_off[b], t_off[b] + gam[b]) for b in range(B)]).astype(np.int64)
    ramp = (0.3 + 1.2 * np.arange(gamma) / max(1, gamma - 1)).astype(np.float32)
    drf32 = _draft_rows(wid, tgt32, rows, np.tile(ramp, B), seed)
    tgt, drf = _round_store(tgt32, "bf16"), _round_store(drf32, "bf16")
    del tgt32, drf32
    dstored = bf16_bits_to_f32(drf)
    x = np.empty(len(rows), np.int32)

    def fn(k):
        x[k] = int(np.argmax(dstored[k]))

    _par_rows(len(rows), fn)
    temps = np.full(B, 0.6, np.float32)
    return Workload("long", mode, B, V, "bf16", gam, tgt, drf, x, temps,
                    _uniforms(wid, _P_UACC, len(rows), seed), _uniforms(wid, _P_URES, B, seed),
                    delta=delta, max_gamma=gamma)


def make_ragged(B: int = 256, gmax: int = 8, V: int = 152064, seed: int = BASE_SEED, wid: int = 3) -> Workload:
    """Large-batch ragged serving: B=256, gamma_b ~ U{1..8}, V=152064, bf16,
    packed varlen layout.  T_b ~ U[0.5,1.2], sigma_b ~ U[0.2,2.0]; drafts sampled
    from the draft softmax."""
    pg = _gen(wid, _P_PARAM, 0, seed)
    gam = pg.integers(1, gmax + 1, B).astype(np.int32)
    temps = pg.uniform(0.5, 1.2, B).astype(np.float32)
    sig = pg.uniform(0.2, 2.0, B).astype(np.float32)
    t_off = np.concatenate([[0], np.cumsum(gam + 1)])
    tgt32 = _target_rows(wid, int(t_off[-1]), V, 3.0, 8.0, seed)
    rows = np.concatenate([np.arange(t_off[b], t_off[b] + gam[b]) for b in range(B)]).astype(np.int64)
    drf32 = _draft_rows(wid, tgt32, rows, np.repeat(sig, gam), seed)
    tgt, drf = _round_store(tgt32, "bf16"), _round_store(drf32, "bf16")
    del tgt32, drf32
    x = _sample_drafts(wid, bf16_bits_to_f32(drf), np.repeat(temps, gam), seed)
    return Workload("ragged", STOCHASTIC, B, V, "bf16", gam, tgt, drf, x, temps,
                    _uniforms(wid, _P_UACC, len(rows), seed), _uniforms(wid, _P_URES, B, seed),
                    max_gamma=gmax, meta={"sigma": sig})


def _kth_largest_lowest_index(row: np.ndarray, k: int) -> int:
    # stable sort on -row puts equal values in ascending index order
    order = np.argsort(-row.astype(np.float64), kind="stable")
    return int(order[k])


def make_tree(B: int = 16, V: int = 128256, parents: np.ndarray = TREE_LITERAL16, seed: int = BASE_SEED,
              wid: int = 4, spike: float = 8.0, noise: float = 0.7, dtype: str = "bf16") -> Workload:
    """Tree draft, greedy verify: B trees given as parent arrays; one target row
    per node (3*N(0,1) + 8 spike).  The children of node n take, in id order, the
    1st, 2nd, 3rd ... largest entries of (target row n + N(0, noise^2)) (ties to
    the lowest index)."""
    parents = np.asarray(parents, np.int32)
    N = len(parents)
    gam = np.full(B, N - 1, np.int32)
    tgt32 = _target_rows(wid, B * N, V, 3.0, spike, seed)
    tgt = _round_store(tgt32, dtype)
    tstored = tgt32 if dtype == "f32" else bf16_bits_to_f32(tgt)
    del tgt32
    # draft rows: one per internal node, d_n = stored t_n + noise
    internal = sorted(set(int(p) for p in parents[1:]))
    tokens = np.zeros(B * (N - 1), np.int32)

    def fn(b):
        for n in internal:
            g = _gen(wid, _P_DNOISE, b * N + n, seed)
            d = tstored[b * N + n] + np.float32(noise) * g.standard_normal(V, dtype=np.float32)
            d = d if dtype == "f32" else bf16_bits_to_f32(f32_to_bf16_bits(d))
            kids = [c for c in range(1, N) if parents[c] == n]
            for rank, c in enumerate(kids):
                tokens[b * (N - 1) + c - 1] = _kth_largest_lowest_index(d, rank)

    _par_rows(B, fn)
    tp = np.tile(parents[1:], B).astype(np.int32)
    temps = np.ones(B, np.float32)
    return Workload(f"tree{N}", TREE_GREEDY, B, V, dtype, gam, tgt, None, tokens, temps,
                    np.zeros(B * (N - 1), np.float32), np.zeros(B, np.float32),
                    tree_parents=tp, max_gamma=N - 1)


def chains_parents(K: int, gamma: int) -> np.ndarray:
    """Parent array of K chains of gamma nodes each under one root: chain k's
    node i (0-based) has id 1 + k * gamma + i and follows the root (i = 0) or
    the chain's previous node."""
    par = np.empty(1 + K * gamma, np.int32)
    par[0] = -1
    for k in range(K):
        for i in range(gamma):
            n = 1 + k * gamma + i
            par[n] = 0 if i == 0 else n - 1
    return par


def make_multi_draft(B: int = 16, K: int = 3, gamma: int = 6, V: int = 128256, seed: int = BASE_SEED, wid: int = 6,
                     noise=(0.3, 0.7, 1.2), dtype: str = "bf16") -> Workload:
    """Several draft models per request, verified together ("keep the longest
    accepted path"): K chains of gamma drafts under a shared root, laid out as
    a tree (parent array from chains_parents).  One target row per node
    (3*N(0,1) + 8 spike: the target at the root and after each chain's
    prefix); chain k drafts greedily from its own noisy copy of the target,
    node token = argmax(target row of its parent + N(0, noise[k]^2))."""
    parents = chains_parents(K, gamma)
    N = len(parents)
    gam = np.full(B, N - 1, np.int32)
    tgt32 = _target_rows(wid, B * N, V, 3.0, 8.0, seed)
    tgt = _round_store(tgt32, dtype)
    tstored = tgt32 if dtype == "f32" else bf16_bits_to_f32(tgt)
    del tgt32
    tokens = np.zeros(B * (N - 1), np.int32)

    def fn(b):
        for n in range(1, N):
            k = (n - 1) // gamma
            g = _gen(wid, _P_DNOISE, b * N + n, seed)
            d = tstored[b * N + parents[n]] + np.float32(noise[k % len(noise)]) * g.standard_normal(V, dtype=np.float32)
            d = d if dtype == "f32" else bf16_bits_to_f32(f32_to_bf16_bits(d))
            tokens[b * (N - 1) + n - 1] = int(np.argmax(d))

    _par_rows(B, fn)
    tp = np.tile(parents[1:], B).astype(np.int32)
    return Workload(f"multi{K}x{gamma}", TREE_GREEDY, B, V, dtype, gam, tgt, None, tokens, np.ones(B, np.float32),
                    np.zeros(B * (N - 1), np.float32), np.zeros(B, np.float32), tree_parents=tp, max_gamma=N - 1,
                    meta={"K": K, "gamma": gamma})


@dataclass
class ConsensusWorkload:
    """Inputs of the consensus pass: K draft rows per position (the drafts of
    one position consecutive), one temperature per request."""
    name: str
    B: int
    K: int
    V: int
    dtype: str  # "bf16" (uint16 bit patterns) or "f32"
    gamma: np.ndarray  # int32 [B]
    drafts: np.ndarray  # [sum(gamma) * K, V] stored values
    temperature: np.ndarray  # float32 [B]
    max_gamma: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def npos(self) -> int:
        return int(self.gamma.astype(np.int64).sum())

    @property
    def logit_bytes(self) -> int:
        return int(self.drafts.nbytes)


def make_consensus(B: int = 32, K: int = 3, gamma=5, V: int = 128256, dtype: str = "bf16",
                   spread=(0.3, 2.0), temps=(0.7, 1.0, 1.3), seed: int = BASE_SEED,
                   wid: int = 7) -> ConsensusWorkload:
    """K draft models' rows at every drafted position.  Position n has a base
    row 3*N(0,1) + 8 spike (the target-like shape of the other workloads); its
    spread s_n is log-uniform in ``spread``; draft a's row is the base plus
    s_n (1 + a/4) N(0,1).  At T = 1 and the Llama-3 vocabulary the closest
    pair's NKL is about 0.09 at s = 1 and 0.23 at s = 1.5, so the default range
    gives consensus, divergence and in-between positions.  Temperatures are
    drawn per request from ``temps``; ``gamma`` is an int or an int32 [B]."""
    gam = np.full(B, int(gamma), np.int32) if np.isscalar(gamma) else np.ascontiguousarray(gamma, np.int32)
    assert gam.shape == (B,)
    npos = int(np.maximum(gam, 0).astype(np.int64).sum())
    base = _target_rows(wid, npos, V, 3.0, 8.0, seed)
    lo, hi = np.log(spread[0]), np.log(spread[1])
    s = np.array([np.exp(lo + (hi - lo) * _gen(wid, _P_PARAM, n, seed).random()) for n in range(npos)], np.float32)
    rows = np.repeat(np.arange(npos), K)
    sigma = (s[rows] * (1.0 + 0.25 * np.tile(np.arange(K), npos))).astype(np.float32)
    drafts = _round_store(_draft_rows(wid, base, rows, sigma, seed), dtype)
    del base
    tsel = _gen(wid, _P_PARAM, npos + 1, seed).integers(0, len(temps), B)
    temperature = np.asarray(temps, np.float32)[tsel]
    return ConsensusWorkload(f"consensus{K}", B, K, V, dtype, gam, drafts, temperature,
                             int(max(0, gam.max()) if B else 0), {"spread": spread})


def consensus_to_device(w: ConsensusWorkload, dev: str = "cuda:0") -> dict:
    """Uploads a consensus workload (drafts as a [positions, K, V] tensor)."""
    import torch
    if w.dtype == "bf16":
        d = torch.from_numpy(np.ascontiguousarray(w.drafts).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        d = torch.from_numpy(np.ascontiguousarray(w.drafts, np.float32)).to(dev)
    return {"drafts": d.view(w.npos, w.K, w.V),
            "gamma": torch.from_numpy(np.ascontiguousarray(w.gamma, np.int32)).to(dev),
            "temperature": torch.from_numpy(np.ascontiguousarray(w.temperature, np.float32)).to(dev)}


WORKLOADS = {
    "tiny": make_tiny,
    "llama3": make_llama3,
    "long": make_long,
    "ragged": make_ragged,
    "tree": make_tree,
}


def make(name: str, **kw) -> Workload:
    if name == "multi_draft":
        return make_multi_draft(**kw)
    if name == "tree13":
        return make_tree(parents=TREE_P_EAGLE13, wid=5, **kw)
    if name == "long_nkl":
        return make_long(mode=NKL, **kw)
    return WORKLOADS[name](**kw)


def to_device(w: Workload, dev: str = "cuda:0") -> dict:
    """Copies a workload's arrays to the GPU as torch tensors (bf16 logits keep
    their stored bit patterns).  Plain uploads, nothing else."""
    import torch
    if w.dtype == "bf16":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    return dict(
        target=conv(w.target),
        draft=None if w.draft is None else conv(w.draft),
        tokens=i32(w.draft_tokens),
        gamma=i32(w.gamma),
        temp=f32(w.temperature),
        ua=f32(w.u_accept),
        ur=f32(w.u_resample),
        parents=None if w.tree_parents is None else i32(w.tree_parents),
        nkl_position=None if w.nkl_position is None else i32(w.nkl_position),
    )


def random_workload(seed: int, mode: int, B: int, V: int, dtype: str = "bf16", gmax: int = 6,
                    gmin: int = 0, scale: float = 3.0, spike: float = 8.0, sigma: float = 0.7,
                    temp_range=(0.5, 1.2), greedy_drafts: bool = False, ties: bool = False,
                    tree: bool = False) -> Workload:
    """Small randomized workloads for edge-case parity tests (ragged gamma incl.
    zero, arbitrary V incl. values that are not a multiple of 8, optional heavy
    ties by quantising logits to a coarse grid, random parent-index trees)."""
    wid = 1000 + seed
    pg = _gen(wid, _P_PARAM, 0, seed)
    gam = pg.integers(gmin, gmax + 1, B).astype(np.int32)
    temps = pg.uniform(temp_range[0], temp_range[1], B).astype(np.float32)
    t_off = np.concatenate([[0], np.cumsum(gam + 1)])
    tgt32 = _target_rows(wid, int(t_off[-1]), V, scale, spike, seed)
    if ties:
        tgt32 = np.round(tgt32).astype(np.float32)
    rows = np.concatenate([np.arange(t_off[b], t_off[b] + gam[b]) for b in range(B)] + [np.zeros(0)]).astype(np.int64)
    drf32 = _draft_rows(wid, tgt32, rows, np.full(len(rows), sigma, np.float32), seed)
    if ties:
        drf32 = np.round(drf32).astype(np.float32)
    tgt, drf = _round_store(tgt32, dtype), _round_store(drf32, dtype)
    dstored = drf.astype(np.float32) if dtype == "f32" else bf16_bits_to_f32(drf)
    tstored = tgt.astype(np.float32) if dtype == "f32" else bf16_bits_to_f32(tgt)
    parents = None
    if tree:
        parents = np.zeros(len(rows), np.int32)
        x = np.zeros(len(rows), np.int32)
        for b in range(B):
            n_nodes = int(gam[b]) + 1
            for k in range(1, n_nodes):
                par = int(pg.integers(0, k))
                parents[int(t_off[b]) - b + k - 1] = par
                # node token: with prob 1/2 the drafter's greedy pick from a
                # lightly perturbed copy of the parent's target row (so paths
                # get accepted), else a uniformly random token
                if pg.random() < 0.5:
                    noisy = tstored[int(t_off[b]) + par] + np.float32(0.05) * pg.standard_normal(V, dtype=np.float32)
                    x[int(t_off[b]) - b + k - 1] = int(np.argmax(noisy))
                else:
                    x[int(t_off[b]) - b + k - 1] = int(pg.integers(0, V))
        mode = TREE_GREEDY
    elif greedy_drafts:
        x = np.array([int(np.argmax(dstored[k])) for k in range(len(rows))], np.int32)
    else:
        x = _sample_drafts(wid, dstored, np.repeat(temps, gam), seed)
    return Workload(f"random{seed}", mode, B, V, dtype, gam, tgt, None if tree else drf, x, temps,
                    _uniforms(wid, _P_UACC, len(rows), seed), _uniforms(wid, _P_URES, B, seed),
                    tree_parents=parents, max_gamma=max(gmax, 0))
