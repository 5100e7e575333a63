"""Benchmark of the verify step on one MI355X.

One step = one spec_verify call over one batch of the Llama-3-shaped workload
(B = 32 requests, gamma = 5 drafted tokens each, V = 128256, bf16 logits,
stochastic mode: the whole path -- row statistics, per-request decision,
residual/bonus draw and token selection).  Inputs are resident in HBM; each
step reads a different copy of them (enough copies to cover > 1 GiB), so the
256 MB Infinity Cache cannot serve the logits of the step before.

Prints ONE JSON line with verified draft positions/s, the roofline of the
dominant kernel, per-call percentiles, a plain-read probe over the same bytes
and the CPU oracle timed on the host cores on a bounded sample of the same
workload.  The dominant kernel is the single dispatch k_fused that runs the
whole stochastic step of a short batch (the Llama-3-shaped one; its
algorithmic bytes are those of the whole step), else the row-statistics kernel
k_stats.  It is timed with HIP events that spec_verify records on the call's
stream at the dispatch's own start and end, in every --event-every'th timed
step (event records cost a few microseconds each, so they are not put into
every step); the percentiles come from those steps.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama3]

Other workloads (context lines, not the headline): tiny, tiny_greedy (1000
one-request calls, launch-bound: microseconds per call), long_greedy,
long_nkl, long_nkl_pos, long_block, ragged, tree, multi_draft, sample_llama3,
topk_llama3, consensus.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
# rocprofv3 HBM counter summaries of the dominant kernel, per workload
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "draft_token_verification_05_amd", "csrc", "kernels.hip")

WORKLOADS = {
    # name: (maker kwargs, mode, description)
    "tiny": ({}, 0, "tiny stochastic verify: 1000 independent one-request steps, B=1, gamma=4, V=1000, fp32; "
                    "one call per step"),
    "tiny_greedy": ({}, 1, "tiny greedy verify: 1000 independent one-request steps, B=1, gamma=4, V=1000, fp32; "
                           "one call per step"),
    "llama3": ({}, 0, "llama3-shaped stochastic verify: B=32, gamma=5, V=128256, bf16"),
    "long_greedy": ({"mode": 1}, 1, "long parallel drafts, greedy: B=64, gamma=16, V=128256, bf16"),
    "long_nkl": ({"mode": 2}, 2, "long parallel drafts, NKL delta=0.15, T=0.6: B=64, gamma=16, V=128256, bf16"),
    "long_nkl_pos": ({"mode": 2}, 2, "long parallel drafts, NKL with the position-adaptive threshold (delta_base=0.15, "
                                      "alpha=0.08, cap 0.3; start positions ~U{0..4095}), T=0.6: B=64, gamma=16, "
                                      "V=128256, bf16"),
    "long_block": ({"mode": 4}, 4, "long parallel drafts, block accept (runs of >= 3 agreeing tokens): B=64, "
                                     "gamma=16, V=128256, bf16"),
    "ragged": ({}, 0, "large-batch ragged stochastic: B=256, gamma~U{1..8}, V=152064, bf16"),
    "tree": ({}, 3, "tree draft greedy verify: B=16, 16-node trees, V=128256, bf16"),
    # draft-side sampling (the step before verify): one token per draft row of the llama3 batch
    "sample_llama3": ({}, -1, "draft-side sampling of the llama3-shaped batch's draft rows: 160 rows, V=128256, "
                              "bf16, per-request temperatures"),
    "topk_llama3": ({}, -1, "top-3 of each of the llama3-shaped batch's draft rows (tree-draft children): 160 rows, "
                            "V=128256, bf16"),
    # several draft models
    "multi_draft": ({}, 3, "multi-draft longest path: 3 draft chains of 6 tokens under one root per request, "
                           "verified as one tree (greedy): B=16, V=128256, bf16"),
    "consensus": ({}, -2, "consensus across 3 drafts: pairwise NKL of the drafts at every drafted position of the "
                          "llama3-shaped batch (B=32, gamma=5, 3 x 160 rows), V=128256, bf16, thresholds 0.1 / 0.15"),
}


def kernel_hash() -> str:
    """Hash of the kernel source's code: comments and whitespace do not count,
    so a profile stays valid across edits of comments only."""
    import re
    text = re.sub(r"//[^\n]*", "", open(KERNEL_SRC).read())
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary profiles/traffic_<workload>.txt, if it was taken
    on the current kernel source for that kernel (else None)."""
    path = os.path.join(PROFILE_DIR, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernels_hip_sha256_16") != kernel_hash() or kv.get("kernel") != kernel:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Hip:
    """The few HIP event calls the benchmark needs (same runtime as torch)."""

    def __init__(self):
        import torch  # noqa: F401  (loads torch's HIP runtime first)
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = ev.value
        return arr

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, arr):
        for e in arr:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))


def pct_us(ms_values):
    """p10 / median / p90 of a list of millisecond timings, in microseconds."""
    import numpy as np
    a = np.asarray(ms_values, np.float64) * 1e3
    return {"p10": round(float(np.percentile(a, 10)), 3), "p50": round(float(np.median(a)), 3),
            "p90": round(float(np.percentile(a, 90)), 3), "n": int(a.size)}


def algorithmic_bytes(w, num_accepted):
    """Bytes one step must read: every logit row the mode needs once, plus the
    terminal draw's re-read (stochastic: 2 rows after a rejection, 1 row for a
    bonus -- which the row-statistics pass never reads)."""
    import numpy as np
    s = 2 if w.dtype == "bf16" else 4
    R_d, B, V = w.total_draft_rows, w.batch, w.vocab
    if w.mode == 0:
        rowstats = 2 * R_d * V * s
        rej = int(np.sum(num_accepted < w.gamma))
        draw = (2 * rej + (B - rej)) * V * s
        return rowstats, rowstats + draw
    if w.mode == 2:
        rowstats = (2 * R_d + B) * V * s
        return rowstats, rowstats
    rowstats = (R_d + B) * V * s
    return rowstats, rowstats


def make_workload(name):
    import synthetic
    kw, mode, _ = WORKLOADS[name]
    if name in ("tiny", "tiny_greedy"):
        return synthetic.make_tiny().with_mode(mode)
    maker = {"llama3": synthetic.make_llama3, "long_greedy": synthetic.make_long, "long_nkl": synthetic.make_long,
             "long_nkl_pos": synthetic.make_long, "long_block": synthetic.make_long, "ragged": synthetic.make_ragged,
             "tree": synthetic.make_tree, "multi_draft": synthetic.make_multi_draft}[name]
    w = maker(**kw)
    return w.with_positions() if name == "long_nkl_pos" else w


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "nproc": avail}


def run_probe(nbytes, launches=64, wgs_per_cu=4, pool_bytes=1 << 30):
    """A plain read of nbytes (rounded down to 16 KB items) in the statistics
    pass's pattern, from buffers rotated through >= 1 GiB so that the Infinity
    Cache cannot serve them: per-launch times from the dispatch's own events."""
    import numpy as np
    import torch

    import draft_token_verification_05_amd as sv

    item = 16384
    nb = max(item, nbytes // item * item)
    slots = max(4, -(-pool_bytes // nb))
    pool = torch.empty(slots * nb, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    hip = Hip()
    ev = hip.events(2 * launches)
    for k in range(4):
        st = sv.spec_read_probe(pool.data_ptr() + (k % slots) * nb, nb, wgs_per_cu, sink.data_ptr(),
                                stream.cuda_stream)
        if st != 0:
            raise RuntimeError(sv.spec_verify_status_string(st))
    for k in range(launches):
        st = sv.spec_read_probe(pool.data_ptr() + (k % slots) * nb, nb, wgs_per_cu, sink.data_ptr(),
                                stream.cuda_stream, ev[2 * k], ev[2 * k + 1])
        if st != 0:
            raise RuntimeError(sv.spec_verify_status_string(st))
    torch.cuda.synchronize()
    ms = np.array([hip.elapsed_ms(ev[2 * k], ev[2 * k + 1]) for k in range(launches)])
    hip.destroy(ev)
    del pool
    med = float(np.median(ms))
    return {"bytes": int(nb), "wgs_per_cu": wgs_per_cu, "us": pct_us(ms), "GBps": round(nb / (med * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nb / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def sample_inputs(name):
    """Rows, per-row temperatures and uniforms of a sampling workload."""
    import numpy as np
    w = make_workload("llama3")
    return w, w.draft, np.repeat(w.temperature, w.gamma).astype(np.float32), w.u_accept


def run_sample_gpu(name, steps, warmup, copies_bytes=1 << 30, event_every=8):
    """Times spec_sample_rows (or spec_topk_rows, k = 3, for topk_* workloads) on
    device-resident rows (rotated copies, like run_gpu)."""
    import numpy as np
    import torch

    import draft_token_verification_05_amd as sv

    _, _, desc = WORKLOADS[name]
    w, rows_np, T_np, u_np = sample_inputs(name)
    dev = torch.device("cuda:0")
    rows, V = rows_np.shape
    base = torch.from_numpy(np.ascontiguousarray(rows_np).view(np.int16)).to(dev).view(torch.bfloat16)
    ncopies = max(2, min(64, -(-copies_bytes // (rows * V * 2))))
    copies = [base] + [base.clone() for _ in range(ncopies - 1)]
    T = torch.from_numpy(T_np).to(dev)
    u = torch.from_numpy(u_np).to(dev)
    topk = 3 if name.startswith("topk") else 0
    out = torch.empty(rows * max(1, topk), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    cfg0 = sv.make_config(rows, V, sv.SV_DTYPE_BF16, 0, 0)

    def call(k, cfg):
        if topk:
            return sv.spec_topk_rows(copies[k % ncopies].data_ptr(), topk, out.data_ptr(), cfg)
        return sv.spec_sample_rows(copies[k % ncopies].data_ptr(), T.data_ptr(), u.data_ptr(), out.data_ptr(), cfg)
    ws = torch.empty(sv.spec_verify_workspace_size(cfg0), dtype=torch.uint8, device=dev)
    hip = Hip()
    sampled = list(range(0, steps, max(1, event_every)))
    ev = hip.events(4 * len(sampled))
    ev_all = hip.events(2)
    ev_base = ctypes.addressof(ev)

    def cfg_for(k):
        e = ev_base + 4 * (k // event_every) * ctypes.sizeof(ctypes.c_void_p) if (k >= 0 and k % event_every == 0) else 0
        return sv.make_config(rows, V, sv.SV_DTYPE_BF16, 0, 0, stream.cuda_stream, ws.data_ptr(), ws.numel(),
                              phase_events=e)

    plain = cfg_for(-1)
    timed = [cfg_for(k) for k in range(steps)]
    for k in range(warmup):
        st = call(k, plain)
        if st != 0:
            raise RuntimeError(sv.spec_verify_status_string(st))
    torch.cuda.synchronize()
    hip.record(ev_all[0], stream.cuda_stream)
    for k in range(steps):
        st = call(k, timed[k])
        if st != 0:
            raise RuntimeError(sv.spec_verify_status_string(st))
    hip.record(ev_all[1], stream.cuda_stream)
    torch.cuda.synchronize()
    total_ms = hip.elapsed_ms(ev_all[0], ev_all[1])
    ks = np.array([hip.elapsed_ms(ev[4 * n + 1], ev[4 * n + 2]) for n in range(len(sampled))])
    hip.destroy(ev)
    hip.destroy(ev_all)
    # one read of every row (sampling: plus the selection's re-read of one wave-chunk, 2048 tokens)
    nbytes = rows * V * 2 + (0 if topk else rows * min(V, 2048) * 2)
    return dict(desc=desc, rows=rows, V=V, ncopies=ncopies, ms_per_step=total_ms / steps, kernel_ms=float(ks.mean()),
                kernel_pct=pct_us(ks), bytes=nbytes, sampled=len(sampled), topk=topk)


PEAK_FP32_TFLOPS = 157.3  # MI355X fp32 vector


def cons_flops_per_element(K):
    """Algorithmic fp32 operations of the consensus pass per position and
    vocabulary element: per row the exponent's fma, the exp and the sum's add
    (2 + 1 + 1); per unordered pair the difference and four fmas (t and z of
    both directions: 1 + 4 x 2)."""
    return 4 * K + 9 * K * (K - 1) // 2


def run_consensus_gpu(steps, warmup, copies_bytes=1 << 30, event_every=8):
    """Times spec_consensus on device-resident drafts (rotated copies)."""
    import numpy as np
    import torch

    import synthetic
    import draft_token_verification_05_amd as sv

    w = synthetic.make_consensus()
    d = synthetic.consensus_to_device(w)
    dev = torch.device("cuda:0")
    ncopies = max(2, min(64, -(-copies_bytes // w.logit_bytes)))
    copies = [d["drafts"]] + [d["drafts"].clone() for _ in range(ncopies - 1)]
    npos, K, V = w.npos, w.K, w.V
    out_state = torch.empty(npos, dtype=torch.int32, device=dev)
    out_pair = torch.empty(npos, dtype=torch.int32, device=dev)
    out_nkl = torch.empty(npos * K * K, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    cfg0 = sv.make_config(w.B, V, sv.SV_DTYPE_BF16, w.max_gamma, npos)
    ws = torch.empty(sv.spec_consensus_workspace_size(cfg0, K), dtype=torch.uint8, device=dev)
    hip = Hip()
    sampled = list(range(0, steps, max(1, event_every)))
    ev = hip.events(4 * len(sampled))
    ev_all = hip.events(2)
    ev_base = ctypes.addressof(ev)

    def cfg_for(k):
        e = ev_base + 4 * (k // event_every) * ctypes.sizeof(ctypes.c_void_p) if (k >= 0 and k % event_every == 0) else 0
        return sv.make_config(w.B, V, sv.SV_DTYPE_BF16, w.max_gamma, npos, stream.cuda_stream, ws.data_ptr(),
                              ws.numel(), phase_events=e)

    def call(k, cfg):
        st = sv.spec_consensus(copies[k % ncopies].data_ptr(), K, d["gamma"].data_ptr(), d["temperature"].data_ptr(),
                               0.1, 0.15, out_nkl.data_ptr(), out_state.data_ptr(), out_pair.data_ptr(), cfg)
        if st != 0:
            raise RuntimeError(sv.spec_verify_status_string(st))

    plain = cfg_for(-1)
    timed = [cfg_for(k) for k in range(steps)]
    for k in range(warmup):
        call(k, plain)
    torch.cuda.synchronize()
    hip.record(ev_all[0], stream.cuda_stream)
    for k in range(steps):
        call(k, timed[k])
    hip.record(ev_all[1], stream.cuda_stream)
    torch.cuda.synchronize()
    total_ms = hip.elapsed_ms(ev_all[0], ev_all[1])
    ks = np.array([hip.elapsed_ms(ev[4 * n + 1], ev[4 * n + 2]) for n in range(len(sampled))])
    st_ms = np.array([hip.elapsed_ms(ev[4 * n + 0], ev[4 * n + 3]) for n in range(len(sampled))])
    states = np.bincount(out_state.cpu().numpy(), minlength=3).tolist()
    hip.destroy(ev)
    hip.destroy(ev_all)
    # the pass reads every draft row once and writes per (position, chunk) a
    # 16-byte record per row and per ordered pair; one read of the drafts is
    # the step's minimum
    nch = -(-V // (256 * 16 * 8))  # chunk: 256 threads x 16 vectors x 8 bf16
    draft_bytes = npos * K * V * 2
    kbytes = draft_bytes + npos * nch * (K + K * (K - 1)) * 16
    return dict(w=w, ncopies=ncopies, ms_per_step=total_ms / steps, kernel_ms=float(ks.mean()),
                kernel_pct=pct_us(ks), step_pct=pct_us(st_ms), kernel_bytes=kbytes, step_bytes=draft_bytes,
                sampled=len(sampled), states=states, flops=npos * V * cons_flops_per_element(K))


def cpu_baseline_consensus(budget_s=8.0):
    import oracle
    import synthetic
    w = synthetic.make_consensus()
    threads = oracle.max_threads()
    run = lambda: oracle.consensus(w.drafts, w.dtype, w.gamma, w.K, w.temperature, nthreads=threads)
    run()  # warm (page-in)
    reps, t0 = 0, time.perf_counter()
    while True:
        run()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": w.npos * reps / el, "unit": "consensus positions/s", "cores": threads, "kind": "oracle",
            **cpu_info(), "sample": f"{reps} full batches of the consensus workload ({w.npos} positions x {w.K} "
                                    f"drafts each), {el:.1f} s wall on {threads} host threads"}


def _step_args(sv, w, d, mode, out_tokens, out_num, out_nkl, stream, ws, events_ptr, positions, b=None):
    """Arguments of one spec_verify call: the whole batch, or (b given) the
    one-request step b of a packed batch, by pointer offsets into it."""
    soft = mode in (0, 2)
    dt = sv.SV_DTYPE_BF16 if w.dtype == "bf16" else sv.SV_DTYPE_F32
    es = 2 if w.dtype == "bf16" else 4
    if b is None:
        B, R_d, t0, d0, b0 = w.batch, w.total_draft_rows, 0, 0, 0
    else:
        B, R_d, t0, d0, b0 = 1, int(w.gamma[b]), int(w.t_off[b]), int(w.d_off[b]), b
    V = w.vocab
    cfg = sv.make_config(B, V, dt, w.max_gamma, R_d, stream, ws.data_ptr(), ws.numel(), phase_events=events_ptr,
                         nkl_position=0 if positions is None else positions.data_ptr() + 4 * d0,
                         nkl_alpha=w.nkl_alpha, nkl_delta_max=w.nkl_delta_max)
    a = (d["target"].data_ptr() + t0 * V * es, d["draft"].data_ptr() + d0 * V * es if soft else 0,
         d["tokens"].data_ptr() + 4 * d0, d["gamma"].data_ptr() + 4 * b0,
         d["temp"].data_ptr() + 4 * b0 if soft else 0, d["ua"].data_ptr() + 4 * d0 if mode == 0 else 0,
         d["ur"].data_ptr() + 4 * b0 if mode == 0 else 0, mode, w.delta,
         d["parents"].data_ptr() + 4 * d0 if mode == 3 else 0, out_tokens.data_ptr() + 4 * t0,
         out_num.data_ptr() + 4 * b0, out_nkl.data_ptr() + 4 * d0 if mode == 2 else 0)
    return a, cfg


def run_gpu(name, steps, warmup, copies_bytes=1 << 30, event_every=8):
    import numpy as np
    import torch

    from synthetic import to_device

    import draft_token_verification_05_amd as sv

    _, mode, desc = WORKLOADS[name]
    w = make_workload(name)
    per_request = name in ("tiny", "tiny_greedy")  # one call per one-request step
    dev = torch.device("cuda:0")
    base = to_device(w)
    per_copy = w.logit_bytes()
    ncopies = 1 if per_request else max(2, min(64, -(-copies_bytes // per_copy)))
    copies = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(ncopies - 1)]
    B, V, R_d = w.batch, w.vocab, w.total_draft_rows
    stream = torch.cuda.current_stream(dev)
    dt = sv.SV_DTYPE_BF16 if w.dtype == "bf16" else sv.SV_DTYPE_F32
    cfg0 = sv.make_config(1 if per_request else B, V, dt, w.max_gamma, int(w.gamma[0]) if per_request else R_d)
    ws = torch.empty(max(sv.spec_verify_workspace_size(cfg0), 256), dtype=torch.uint8, device=dev)
    out_tokens = torch.empty(R_d + B, dtype=torch.int32, device=dev)
    out_num = torch.empty(B, dtype=torch.int32, device=dev)
    out_nkl = torch.empty(max(R_d, 1), dtype=torch.float32, device=dev)
    hip = Hip()
    sampled = list(range(0, steps, max(1, event_every)))
    ev = hip.events(4 * len(sampled))
    ev_all = hip.events(2)
    positions = None if w.nkl_position is None else torch.from_numpy(w.nkl_position).to(dev)
    ev_base = ctypes.addressof(ev)

    def args(k, events_ptr):
        d = copies[k % ncopies]
        return _step_args(sv, w, d, mode, out_tokens, out_num, out_nkl, stream.cuda_stream, ws, events_ptr, positions,
                          b=(k % B) if per_request else None)

    nplain = B if per_request else ncopies
    plain = [args(k, 0) for k in range(nplain)]
    timed = [args(k, ev_base + 4 * (k // event_every) * ctypes.sizeof(ctypes.c_void_p))
             if k % event_every == 0 else plain[k % nplain] for k in range(steps)]
    for k in range(max(warmup, B if per_request else 0)):
        a, cfg = plain[k % nplain]
        st = sv.spec_verify(*a, cfg)
        if st != 0:
            raise RuntimeError(sv.spec_verify_status_string(st))
    torch.cuda.synchronize()
    num_acc = out_num.cpu().numpy()
    t0 = time.perf_counter()
    hip.record(ev_all[0], stream.cuda_stream)
    for k in range(steps):
        a, cfg = timed[k]
        st = sv.spec_verify(*a, cfg)
        if st != 0:
            raise RuntimeError(sv.spec_verify_status_string(st))
    hip.record(ev_all[1], stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = hip.elapsed_ms(ev_all[0], ev_all[1])
    ks = np.array([hip.elapsed_ms(ev[4 * n + 1], ev[4 * n + 2]) for n in range(len(sampled))])
    st_ms = np.array([hip.elapsed_ms(ev[4 * n + 0], ev[4 * n + 3]) for n in range(len(sampled))])
    hip.destroy(ev)
    hip.destroy(ev_all)
    rowstats_bytes, step_bytes = algorithmic_bytes(w, num_acc)
    positions_total = int(w.gamma.sum())
    if per_request:  # per call: one request's share
        rowstats_bytes, step_bytes = rowstats_bytes / B, step_bytes / B
        positions_total = positions_total / B
    # events [1] and [2] bracket the single dispatch of the whole step when
    # the library runs it as one kernel, else the row-statistics kernel
    single = sv.spec_verify_single_dispatch(cfg0, mode) == 1
    return dict(w=w, desc=desc, mode=mode, steps=steps, ncopies=ncopies, total_ms=total_ms, wall_s=wall,
                ms_per_step=total_ms / steps, kernel_ms=float(ks.mean()), kernel_pct=pct_us(ks),
                step_pct=pct_us(st_ms), rowstats_bytes=rowstats_bytes, step_bytes=step_bytes,
                positions=positions_total, sampled=len(sampled), per_request=per_request,
                kernel="k_fused" if single else "k_stats", kernel_bytes=step_bytes if single else rowstats_bytes)


def cpu_baseline_sample(name, budget_s=8.0, topk=0):
    import oracle
    _, rows, T, u = sample_inputs(name)
    threads = oracle.max_threads()
    run = (lambda: oracle.topk_rows(rows, "bf16", topk, nthreads=threads)) if topk else \
        (lambda: oracle.sample_rows(rows, "bf16", T, u, nthreads=threads))
    run()  # warm (page-in)
    reps, t0 = 0, time.perf_counter()
    while True:
        run()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": rows.shape[0] * reps / el, "unit": ("top-3 draft rows/s" if topk else "sampled draft tokens/s"),
            "cores": threads, "kind": "oracle", **cpu_info(),
            "sample": f"{reps} full passes over the {rows.shape[0]} rows, {el:.1f} s wall on {threads} host threads"}


def cpu_baseline(name, budget_s=8.0):
    import oracle
    w = make_workload(name)
    threads = oracle.max_threads()
    oracle.verify_workload(w, nthreads=threads)  # warm (page-in)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.verify_workload(w, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    pos = int(w.gamma.sum()) * reps
    return {"value": pos / el, "unit": "verified draft positions/s", "cores": threads, "kind": "oracle", **cpu_info(),
            "sample": f"{reps} full batches of the {name} workload ({int(w.gamma.sum())} positions each), "
                      f"{el:.1f} s wall on {threads} host threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-probe", action="store_true", help="skip the plain-read probe")
    ap.add_argument("--event-every", type=int, default=8, metavar="N",
                    help="record the per-kernel phase events in every N-th timed step")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run 10 device-to-device copies of MIB MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.calib_copy:
        import torch
        src = torch.empty(args.calib_copy << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": args.calib_copy << 20, "launches": 10}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(requests are independent, so more GPUs would each run their own share).", file=sys.stderr)
        sys.exit(2)
    if args.workload == "consensus":
        r = run_consensus_gpu(args.steps, args.warmup, event_every=max(1, args.event_every))
        w = r["w"]
        achieved = r["kernel_bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
        tflops = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
        probe = None if args.no_probe else run_probe(int(r["step_bytes"]))
        line = {
            "metric": "consensus positions/sec (3 drafts) at V=128256 (bf16); achieved HBM GB/s vs peak",
            "value": round(w.npos / (r["ms_per_step"] * 1e-3), 1), "unit": "consensus positions/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": WORKLOADS["consensus"][2], "batch": w.B, "gamma": int(w.gamma.max()),
                       "drafts": w.K, "vocab": w.V, "logits": w.dtype, "positions_per_step": w.npos,
                       "states": r["states"], "input_copies_rotated": r["ncopies"],
                       "step_GBps": round(r["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9, 1),
                       "step_frac_of_peak": round(r["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                  4),
                       "step_us": r["step_pct"]},
            # the pass issues more vector-ALU work than its bytes take to stream
            "roofline": {"bound": "alu", "kernel": "k_cons", "achieved": round(tflops, 2),
                         "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP32_TFLOPS, 4),
                         "traffic": load_traffic("k_cons", "consensus"), "flops_per_launch": r["flops"],
                         "flops_per_element": cons_flops_per_element(w.K),
                         "hbm": {"achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": round(achieved / PEAK_HBM_GBS, 4), "bytes_per_launch": r["kernel_bytes"]},
                         "avg_launch_us": round(r["kernel_ms"] * 1e3, 3), "launch_us": r["kernel_pct"],
                         "timed_launches": r["sampled"]},
            "probe": probe,
            "cpu_baseline": None if args.no_cpu else cpu_baseline_consensus(),
        }
        if probe:
            line["roofline"]["hbm"]["frac_of_probe"] = round(achieved / probe["GBps"], 4)
        print(json.dumps(line), flush=True)
        return
    if args.workload.startswith(("sample", "topk")):
        r = run_sample_gpu(args.workload, args.steps, args.warmup, event_every=max(1, args.event_every))
        achieved = r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
        what = "top-3 draft rows" if r["topk"] else "sampled draft tokens"
        kern = "k_topk" if r["topk"] else "k_sample"
        probe = None if args.no_probe else run_probe(r["bytes"])
        line = {
            "metric": f"{what}/sec at V=128256 (bf16); achieved HBM GB/s vs peak",
            "value": round(r["rows"] / (r["ms_per_step"] * 1e-3), 1), "unit": f"{what}/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": r["desc"], "rows": r["rows"], "vocab": r["V"], "logits": "bf16",
                       "input_copies_rotated": r["ncopies"],
                       "step_GBps": round(r["bytes"] / (r["ms_per_step"] * 1e-3) / 1e9, 1),
                       "step_frac_of_peak": round(r["bytes"] / (r["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "roofline": {"bound": "hbm", "kernel": kern, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "traffic": load_traffic(kern, args.workload),
                         "bytes_per_launch": r["bytes"], "avg_launch_us": round(r["kernel_ms"] * 1e3, 3),
                         "launch_us": r["kernel_pct"], "timed_launches": r["sampled"]},
            "probe": probe,
            "cpu_baseline": None if args.no_cpu else cpu_baseline_sample(args.workload, topk=r["topk"]),
        }
        if probe:
            line["roofline"]["frac_of_probe"] = round(achieved / probe["GBps"], 4)
        print(json.dumps(line), flush=True)
        return
    r = run_gpu(args.workload, args.steps, args.warmup, event_every=max(1, args.event_every))
    w = r["w"]
    value = r["positions"] / (r["ms_per_step"] * 1e-3)
    achieved = r["kernel_bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
    traffic = load_traffic(r["kernel"], args.workload)
    probe = None if (args.no_probe or r["per_request"]) else run_probe(int(r["kernel_bytes"]))
    config = {"workload": r["desc"], "batch": 1 if r["per_request"] else w.batch, "gamma": int(w.gamma.max()),
              "vocab": w.vocab, "logits": w.dtype, "mode": ["stochastic", "greedy", "nkl", "tree", "block"][r["mode"]],
              "positions_per_step": r["positions"], "input_copies_rotated": r["ncopies"],
              "step_GBps": round(r["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9, 1),
              "step_frac_of_peak": round(r["step_bytes"] / (r["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
              "step_us": r["step_pct"]}
    if r["per_request"]:
        config["us_per_call"] = round(r["ms_per_step"] * 1e3, 3)
    line = {
        "metric": "verified draft positions/sec at V=128256 (bf16); achieved HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "verified draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": {"bound": "hbm", "kernel": r["kernel"], "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": r["kernel_bytes"],
                     "avg_launch_us": round(r["kernel_ms"] * 1e3, 3), "launch_us": r["kernel_pct"],
                     "timed_launches": r["sampled"]},
        "probe": probe,
        "cpu_baseline": None if args.no_cpu else cpu_baseline(args.workload),
    }
    if probe:
        line["roofline"]["frac_of_probe"] = round(achieved / probe["GBps"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
