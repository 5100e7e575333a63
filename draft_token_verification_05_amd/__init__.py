"""Python binding of libspecverify, the gfx950 verify step of speculative /
Chain-of-Draft decoding.

The functions here only marshal arguments: every step of the verify path runs
in the HIP kernels of ``libspecverify.so`` (built by ``build.py`` from
``csrc/``).  PyTorch provides device memory and the stream.  Importing this
package loads the library and fails loudly if it is missing.

C entry points (``include/specverify.h``) and their Python counterparts:

* ``spec_verify``                -> :func:`spec_verify` (raw pointers) and :func:`verify` (tensors)
* ``spec_verify_workspace_size`` -> :func:`spec_verify_workspace_size`
* ``spec_verify_status_string``  -> :func:`spec_verify_status_string`
* ``spec_verify_version``        -> :func:`spec_verify_version`
* ``spec_verify_single_dispatch`` -> :func:`spec_verify_single_dispatch`
* ``spec_verify_noalloc``         -> :func:`spec_verify_noalloc` (raw pointers; no workspace)
* ``spec_sample_rows`` / ``spec_topk_rows`` -> :func:`sample_rows` / :func:`topk_rows` (tensors)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIB: another build of the library (default: the one in this package)
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_EINVAL, SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP = 0, -1, -2, -3, -4
SV_MODE_STOCHASTIC, SV_MODE_GREEDY, SV_MODE_NKL, SV_MODE_TREE_GREEDY, SV_MODE_BLOCK = 0, 1, 2, 3, 4
SV_DTYPE_F32, SV_DTYPE_BF16 = 0, 1
SV_MAX_GAMMA = 4096
SV_NOALLOC_SCRATCH_BYTES = 16 << 20
SV_NUM_PHASE_EVENTS = 4
MODES = {"stochastic": 0, "greedy": 1, "nkl": 2, "tree": 3, "block": 4}


class sv_config(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("max_gamma", ctypes.c_int32),
        ("wait_polls", ctypes.c_int32),
        ("total_draft_rows", ctypes.c_int64),
        ("stream", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_uint64),
        ("out_p_x", ctypes.c_void_p),
        ("out_q_x", ctypes.c_void_p),
        ("out_resid_mass", ctypes.c_void_p),
        ("out_tree_node", ctypes.c_void_p),
        ("phase_events", ctypes.c_void_p),
        ("nkl_position", ctypes.c_void_p),
        ("nkl_alpha", ctypes.c_float),
        ("nkl_delta_max", ctypes.c_float),
        ("block_min_len", ctypes.c_int32),
    ]


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"spec_verify failed: {spec_verify_status_string(status)} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    # PyTorch ships its own HIP runtime; load it first so that this library
    # binds to the same runtime (one HIP runtime per process).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libspecverify.so is not built ({LIB_PATH}); run __graft_entry__.build() "
                          "or python draft_token_verification_05_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.spec_verify.restype = ctypes.c_int
    lib.spec_verify.argtypes = [P, P, P, P, P, P, P, i32, ctypes.c_float, P, P, P, P, ctypes.POINTER(sv_config)]
    lib.spec_verify_noalloc.restype = ctypes.c_int
    lib.spec_verify_noalloc.argtypes = lib.spec_verify.argtypes
    lib.spec_verify_workspace_size.restype = ctypes.c_size_t
    lib.spec_verify_workspace_size.argtypes = [ctypes.POINTER(sv_config)]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_status_string.argtypes = [ctypes.c_int]
    lib.spec_verify_version.restype = ctypes.c_int
    lib.spec_verify_version.argtypes = []
    lib.spec_verify_single_dispatch.restype = ctypes.c_int
    lib.spec_verify_single_dispatch.argtypes = [ctypes.POINTER(sv_config), i32, i32]
    lib.spec_topk_rows.restype = ctypes.c_int
    lib.spec_topk_rows.argtypes = [P, i32, P, ctypes.POINTER(sv_config)]
    lib.spec_read_probe.restype = ctypes.c_int
    lib.spec_read_probe.argtypes = [P, ctypes.c_uint64, i32, P, P, P, P]
    lib.spec_sample_rows.restype = ctypes.c_int
    lib.spec_sample_rows.argtypes = [P, P, P, P, ctypes.POINTER(sv_config)]
    lib.spec_consensus.restype = ctypes.c_int
    lib.spec_consensus.argtypes = [P, i32, P, P, ctypes.c_float, ctypes.c_float, P, P, P, ctypes.POINTER(sv_config)]
    lib.spec_consensus_workspace_size.restype = ctypes.c_size_t
    lib.spec_consensus_workspace_size.argtypes = [ctypes.POINTER(sv_config), i32]
    return lib


_lib = _load()


def make_config(batch: int, vocab: int, dtype: int, max_gamma: int, total_draft_rows: int, stream: int = 0,
                workspace: int = 0, workspace_bytes: int = 0, out_p_x: int = 0, out_q_x: int = 0,
                out_resid_mass: int = 0, out_tree_node: int = 0, phase_events: int = 0,
                wait_polls: int = 0, nkl_position: int = 0, nkl_alpha: float = 0.0,
                nkl_delta_max: float = 0.0, block_min_len: int = 0) -> sv_config:
    return sv_config(ctypes.sizeof(sv_config), int(batch), int(vocab), int(dtype), int(max_gamma), int(wait_polls),
                     int(total_draft_rows), stream or None, workspace or None, int(workspace_bytes),
                     out_p_x or None, out_q_x or None, out_resid_mass or None, out_tree_node or None,
                     phase_events or None, nkl_position or None, float(nkl_alpha), float(nkl_delta_max),
                     int(block_min_len))


def spec_verify(target_logits: int, draft_logits: int, draft_tokens: int, gamma_per_req: int, temperature: int,
                u_accept: int, u_resample: int, mode: int, delta: float, tree_parents: int, out_tokens: int,
                out_num_accepted: int, out_nkl: int, cfg: sv_config) -> int:
    """The C entry point with raw device addresses (0 = NULL).  Returns the status."""
    return int(_lib.spec_verify(target_logits or None, draft_logits or None, draft_tokens or None,
                                gamma_per_req or None, temperature or None, u_accept or None, u_resample or None,
                                int(mode), float(delta), tree_parents or None, out_tokens or None,
                                out_num_accepted or None, out_nkl or None, ctypes.byref(cfg)))


def spec_verify_noalloc(target_logits: int, draft_logits: int, draft_tokens: int, gamma_per_req: int,
                        temperature: int, u_accept: int, u_resample: int, mode: int, delta: float, tree_parents: int,
                        out_tokens: int, out_num_accepted: int, out_nkl: int, cfg: sv_config) -> int:
    """spec_verify on the library's own fixed device scratch (cfg.workspace is
    ignored; nothing is allocated).  Returns the status."""
    return int(_lib.spec_verify_noalloc(target_logits or None, draft_logits or None, draft_tokens or None,
                                        gamma_per_req or None, temperature or None, u_accept or None,
                                        u_resample or None, int(mode), float(delta), tree_parents or None,
                                        out_tokens or None, out_num_accepted or None, out_nkl or None,
                                        ctypes.byref(cfg)))


def spec_sample_rows(logits: int, temperature: int, u: int, out_tokens: int, cfg: sv_config) -> int:
    """Raw binding of spec_sample_rows (device pointers as ints)."""
    return int(_lib.spec_sample_rows(logits or None, temperature or None, u or None, out_tokens or None,
                                     ctypes.byref(cfg)))


def spec_consensus(draft_logits: int, num_drafts: int, gamma_per_req: int, temperature: int, delta_c: float,
                   delta_d: float, out_nkl: int, out_state: int, out_pair: int, cfg: sv_config) -> int:
    """Raw binding of spec_consensus (device pointers as ints)."""
    return int(_lib.spec_consensus(draft_logits or None, int(num_drafts), gamma_per_req or None,
                                   temperature or None, float(delta_c), float(delta_d), out_nkl or None,
                                   out_state or None, out_pair or None, ctypes.byref(cfg)))


def spec_consensus_workspace_size(cfg: sv_config, num_drafts: int) -> int:
    return int(_lib.spec_consensus_workspace_size(ctypes.byref(cfg), int(num_drafts)))


def spec_topk_rows(logits: int, k: int, out_idx: int, cfg: sv_config) -> int:
    """Raw binding of spec_topk_rows (device pointers as ints)."""
    return int(_lib.spec_topk_rows(logits or None, int(k), out_idx or None, ctypes.byref(cfg)))


def spec_read_probe(buf: int, nbytes: int, wgs_per_cu: int, sink: int, stream: int = 0, ev_start: int = 0,
                    ev_stop: int = 0) -> int:
    """Measurement aid (include/specverify_probe.h): a plain read of nbytes of a
    device buffer in the row-statistics pass's pattern.  Returns the status."""
    return int(_lib.spec_read_probe(buf or None, int(nbytes), int(wgs_per_cu), sink or None, stream or None,
                                    ev_start or None, ev_stop or None))


def spec_verify_single_dispatch(cfg: sv_config, mode: int, with_nkl: bool = False) -> int:
    """1 if spec_verify runs this configuration as one kernel dispatch, else 0."""
    return int(_lib.spec_verify_single_dispatch(ctypes.byref(cfg), int(mode), int(bool(with_nkl))))


def spec_verify_workspace_size(cfg: sv_config) -> int:
    return int(_lib.spec_verify_workspace_size(ctypes.byref(cfg)))


def spec_verify_status_string(status: int) -> str:
    return _lib.spec_verify_status_string(int(status)).decode()


def spec_verify_version() -> int:
    return int(_lib.spec_verify_version())


# ----------------------------------------------------------------------------
# tensor-level convenience wrapper (PyTorch = device memory + stream only)
# ----------------------------------------------------------------------------

@dataclass
class VerifyOutput:
    tokens: "torch.Tensor"  # int32 [sum(gamma+1)]
    num_accepted: "torch.Tensor"  # int32 [B]
    nkl: Optional["torch.Tensor"] = None  # float32 [sum(gamma)]
    p_x: Optional["torch.Tensor"] = None
    q_x: Optional["torch.Tensor"] = None
    resid_mass: Optional["torch.Tensor"] = None
    tree_node: Optional["torch.Tensor"] = None


_WORKSPACES = {}
_MAX_CACHED_WORKSPACES = 64


def workspace_for(cfg: sv_config, device, stream=None, nbytes: Optional[int] = None) -> "torch.Tensor":
    """A workspace for this configuration, cached per device, stream and
    configuration (calls on different streams must not share one).  Its
    contents need no initialisation.  ``nbytes``: its size, if not
    spec_verify_workspace_size(cfg).  The tensor is recorded on ``stream`` so
    that torch's allocator does not hand its memory out again while work
    queued there may still use it, also after the cache drops it."""
    import torch
    sid = 0 if stream is None else int(stream.cuda_stream)
    nbytes = spec_verify_workspace_size(cfg) if nbytes is None else int(nbytes)
    key = (str(device), sid, cfg.batch, cfg.vocab, cfg.dtype, cfg.max_gamma, cfg.total_draft_rows, nbytes)
    ws = _WORKSPACES.pop(key, None)
    if ws is None:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        while len(_WORKSPACES) >= _MAX_CACHED_WORKSPACES:
            _WORKSPACES.pop(next(iter(_WORKSPACES)))  # the least recently used
    if stream is not None:
        ws.record_stream(stream)
    _WORKSPACES[key] = ws  # most recently used last
    return ws


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _check(t, name, dtype, numel=None, dev=None):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def verify(target_logits, draft_logits, draft_tokens, gamma_per_req, temperature=None, u_accept=None,
           u_resample=None, mode: int | str = SV_MODE_STOCHASTIC, delta: float = 0.15, tree_parents=None, *,
           max_gamma: Optional[int] = None, workspace=None, diagnostics: bool = False, out_nkl: bool = False,
           phase_events: int = 0, stream=None, wait_polls: int = 0, nkl_position=None, nkl_alpha: float = 0.0,
           nkl_delta_max: float = 0.0, block_min_len: int = 0) -> VerifyOutput:
    """Runs one verify step on device tensors (packed layout, see specverify.h).

    NKL mode: ``nkl_position`` (int32 [sum(gamma)] on the GPU, optional) gives
    every draft token's 0-based position in the generated sequence, for the
    position-adaptive threshold min(nkl_delta_max, delta * (1 + nkl_alpha *
    log2(position + 1))).  Block mode: ``block_min_len`` is the shortest run of
    agreeing positions that is kept (0: the page's 3).

    ``target_logits`` [sum(gamma+1), V] and ``draft_logits`` [sum(gamma), V] are
    torch.bfloat16 or torch.float32 on the GPU.  The call is asynchronous on
    ``stream`` (default: torch's current stream).  A ``workspace`` passed in
    needs no initialisation; calls on different streams must use different
    workspaces."""
    import torch
    if isinstance(mode, str):
        mode = MODES[mode]
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("target_logits must be a GPU tensor")
    if target_logits.dtype == torch.bfloat16:
        dt = SV_DTYPE_BF16
    elif target_logits.dtype == torch.float32:
        dt = SV_DTYPE_F32
    else:
        raise TypeError("logits must be bfloat16 or float32")
    if target_logits.dim() != 2 or not target_logits.is_contiguous():
        raise ValueError("target_logits must be a contiguous [rows, V] tensor")
    B = int(gamma_per_req.numel())
    V = int(target_logits.shape[1])
    R_d = int(draft_tokens.numel()) if draft_tokens is not None else 0
    _check(gamma_per_req, "gamma_per_req", torch.int32, B, dev)
    _check(draft_tokens, "draft_tokens", torch.int32, None, dev)
    _check(temperature, "temperature", torch.float32, B, dev)
    _check(u_accept, "u_accept", torch.float32, R_d, dev)
    _check(u_resample, "u_resample", torch.float32, B, dev)
    _check(tree_parents, "tree_parents", torch.int32, R_d, dev)
    _check(nkl_position, "nkl_position", torch.int32, R_d, dev)
    if draft_logits is not None:
        _check(draft_logits, "draft_logits", target_logits.dtype, None, dev)
        if draft_logits.dim() != 2 or draft_logits.shape[1] != V or draft_logits.shape[0] != R_d:
            raise ValueError("draft_logits must be [sum(gamma), V]")
    if target_logits.shape[0] != R_d + B:
        raise ValueError("target_logits must have sum(gamma)+B rows")
    if max_gamma is None:
        max_gamma = min(R_d, SV_MAX_GAMMA)
    out_tokens = torch.empty(max(R_d + B, 1), dtype=torch.int32, device=dev)
    out_num = torch.empty(B, dtype=torch.int32, device=dev)
    nkl = torch.empty(max(R_d, 1), dtype=torch.float32, device=dev) if (mode == SV_MODE_NKL or out_nkl) else None
    p_x = q_x = resid = tnode = None
    if diagnostics:
        p_x = torch.empty(max(R_d, 1), dtype=torch.float32, device=dev)
        q_x = torch.empty(max(R_d, 1), dtype=torch.float32, device=dev)
        resid = torch.empty(B, dtype=torch.float32, device=dev)
        tnode = torch.empty(B, dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    cfg = make_config(B, V, dt, max_gamma, R_d, stream=int(stream.cuda_stream), wait_polls=wait_polls,
                      nkl_position=_ptr(nkl_position), nkl_alpha=nkl_alpha, nkl_delta_max=nkl_delta_max,
                      block_min_len=block_min_len)
    need = spec_verify_workspace_size(cfg)
    if workspace is None:
        workspace = workspace_for(cfg, dev, stream)
    elif workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    cfg.workspace = workspace.data_ptr()
    cfg.workspace_bytes = workspace.numel()
    cfg.out_p_x, cfg.out_q_x = _ptr(p_x) or None, _ptr(q_x) or None
    cfg.out_resid_mass, cfg.out_tree_node = _ptr(resid) or None, _ptr(tnode) or None
    cfg.phase_events = phase_events or None
    st = spec_verify(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(gamma_per_req),
                     _ptr(temperature), _ptr(u_accept), _ptr(u_resample), mode, delta, _ptr(tree_parents),
                     _ptr(out_tokens), _ptr(out_num), _ptr(nkl), cfg)
    if st != SV_OK:
        raise SpecVerifyError(st)
    return VerifyOutput(out_tokens[: R_d + B], out_num, None if nkl is None else nkl[:R_d],
                        None if p_x is None else p_x[:R_d], None if q_x is None else q_x[:R_d], resid, tnode)


def sample_rows(logits, temperature, u, *, workspace=None, stream=None, phase_events: int = 0):
    """Draws one token per row of ``logits`` [rows, V] (torch.bfloat16 or
    torch.float32 on the GPU) from softmax(row / temperature[row]) with the
    uniform ``u[row]`` (see spec_sample_rows in specverify.h).  Returns an int32
    tensor [rows]; -1 marks a row with an invalid temperature or uniform."""
    import torch
    dev = logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be a GPU tensor")
    if logits.dtype == torch.bfloat16:
        dt = SV_DTYPE_BF16
    elif logits.dtype == torch.float32:
        dt = SV_DTYPE_F32
    else:
        raise TypeError("logits must be bfloat16 or float32")
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [rows, V] tensor")
    rows, V = int(logits.shape[0]), int(logits.shape[1])
    _check(temperature, "temperature", torch.float32, rows, dev)
    _check(u, "u", torch.float32, rows, dev)
    out = torch.empty(rows, dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    cfg = make_config(rows, V, dt, 0, 0, stream=int(stream.cuda_stream), phase_events=phase_events)
    if workspace is None:
        workspace = workspace_for(cfg, dev, stream)
    elif workspace.numel() < spec_verify_workspace_size(cfg):
        raise ValueError("workspace too small")
    cfg.workspace, cfg.workspace_bytes = workspace.data_ptr(), workspace.numel()
    st = spec_sample_rows(_ptr(logits), _ptr(temperature), _ptr(u), _ptr(out), cfg)
    if st != SV_OK:
        raise SpecVerifyError(st)
    return out


def topk_rows(logits, k: int, *, workspace=None, stream=None, phase_events: int = 0):
    """The k largest logits of every row of ``logits`` [rows, V] (GPU,
    bfloat16 or float32): int32 [rows, k] indices, largest first, the lower
    index first among equal logits (see spec_topk_rows in specverify.h)."""
    import torch
    dev = logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be a GPU tensor")
    dt = {torch.bfloat16: SV_DTYPE_BF16, torch.float32: SV_DTYPE_F32}.get(logits.dtype)
    if dt is None:
        raise TypeError("logits must be bfloat16 or float32")
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [rows, V] tensor")
    rows, V = int(logits.shape[0]), int(logits.shape[1])
    out = torch.empty((rows, int(k)), dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    cfg = make_config(rows, V, dt, 0, 0, stream=int(stream.cuda_stream), phase_events=phase_events)
    if workspace is None:
        workspace = workspace_for(cfg, dev, stream)
    elif workspace.numel() < spec_verify_workspace_size(cfg):
        raise ValueError("workspace too small")
    cfg.workspace, cfg.workspace_bytes = workspace.data_ptr(), workspace.numel()
    st = spec_topk_rows(_ptr(logits), int(k), _ptr(out), cfg)
    if st != SV_OK:
        raise SpecVerifyError(st)
    return out


@dataclass
class ConsensusOutput:
    state: "torch.Tensor"  # int32 [positions]: 1 consensus, 2 divergence, 0 neither, -1 invalid
    pair: "torch.Tensor"  # int32 [positions]: a * K + b of the closest pair a < b (-1 invalid)
    nkl: Optional["torch.Tensor"] = None  # float32 [positions, K, K]: KL(q_a || q_b) / ln V


def consensus(draft_logits, gamma_per_req, temperature, *, delta_c: float = 0.1, delta_d: float = 0.15,
              max_gamma: Optional[int] = None, out_nkl: bool = True, workspace=None, stream=None,
              phase_events: int = 0) -> ConsensusOutput:
    """Pairwise NKL of the K drafts of every position and the consensus state
    (see spec_consensus in specverify.h).  ``draft_logits`` is a contiguous
    [positions, K, V] GPU tensor (bfloat16 or float32), positions = sum(gamma);
    ``gamma_per_req`` int32 [B] and ``temperature`` float32 [B] on the GPU."""
    import torch
    dev = draft_logits.device
    if dev.type != "cuda":
        raise ValueError("draft_logits must be a GPU tensor")
    dt = {torch.bfloat16: SV_DTYPE_BF16, torch.float32: SV_DTYPE_F32}.get(draft_logits.dtype)
    if dt is None:
        raise TypeError("draft_logits must be bfloat16 or float32")
    if draft_logits.dim() != 3 or not draft_logits.is_contiguous():
        raise ValueError("draft_logits must be a contiguous [positions, K, V] tensor")
    npos, K, V = (int(x) for x in draft_logits.shape)
    _check(gamma_per_req, "gamma_per_req", torch.int32, None, dev)
    B = int(gamma_per_req.numel())
    _check(temperature, "temperature", torch.float32, B, dev)
    if max_gamma is None:
        max_gamma = int(gamma_per_req.max().item()) if B > 0 else 0
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    cfg = make_config(B, V, dt, max(int(max_gamma), 0), npos, stream=int(stream.cuda_stream),
                      phase_events=phase_events)
    need = spec_consensus_workspace_size(cfg, K)
    if workspace is None:
        workspace = workspace_for(cfg, dev, stream, nbytes=need)
    elif workspace.numel() < need:
        raise ValueError("workspace too small")
    cfg.workspace, cfg.workspace_bytes = workspace.data_ptr(), workspace.numel()
    state = torch.empty(max(npos, 1), dtype=torch.int32, device=dev)
    pair = torch.empty(max(npos, 1), dtype=torch.int32, device=dev)
    nkl = torch.empty((max(npos, 1), K, K), dtype=torch.float32, device=dev) if out_nkl else None
    st = spec_consensus(_ptr(draft_logits), K, _ptr(gamma_per_req), _ptr(temperature), delta_c, delta_d, _ptr(nkl),
                        _ptr(state), _ptr(pair), cfg)
    if st != SV_OK:
        raise SpecVerifyError(st)
    return ConsensusOutput(state[:npos], pair[:npos], None if nkl is None else nkl[:npos])
