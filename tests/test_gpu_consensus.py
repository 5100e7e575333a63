"""GPU parity of the consensus pass across K drafts ("Chain of Draft" page,
section 4.4, Consensus-Aware Accept) and of multi-draft longest-path
selection (tree mode over K chains), against the fp64 oracle.

Tolerance of the NKL matrix: the GPU forms every term q_a g(w) in float32
(a few float32 roundings each, at most about 1e-6 relative where the large-|w|
form cancels), sums them in float64 and stores the matrix as float32 (6e-8
relative); 2e-5 relative leaves a wide margin over both.  Zero entries are
exact on both sides (identical rows give w = 0 exactly).  States and pairs are
compared exactly wherever the oracle does not flag the position as within
1e-6 (relative) of a threshold or of a tie between pairs; there both
outcomes are correct and the GPU's is only checked to be valid."""
import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu

RTOL, ATOL = 2e-5, 1e-12


@pytest.fixture(scope="module")
def sv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import draft_token_verification_05_amd as sv  # fails loudly if the library is missing
    return sv


def run(sv, w, dc=0.1, dd=0.15, out_nkl=True, workspace=None, gamma=None):
    import torch
    d = synthetic.consensus_to_device(w)
    if gamma is not None:
        d["gamma"] = torch.from_numpy(np.ascontiguousarray(gamma, np.int32)).to("cuda:0")
    r = sv.consensus(d["drafts"], d["gamma"], d["temperature"], delta_c=dc, delta_d=dd, out_nkl=out_nkl,
                     max_gamma=max(w.max_gamma, 1), workspace=workspace)
    torch.cuda.synchronize()
    return (r.state.cpu().numpy(), r.pair.cpu().numpy(),
            None if r.nkl is None else r.nkl.cpu().numpy().astype(np.float64))


def check(sv, w, dc=0.1, dd=0.15, **kw):
    print(f"[consensus] {w.name} B={w.B} K={w.K} V={w.V} dtype={w.dtype} positions={w.npos}", flush=True)
    state, pair, nkl = run(sv, w, dc, dd, **kw)
    o = oracle.consensus(w.drafts, w.dtype, w.gamma, w.K, w.temperature, dc, dd)
    valid = o.state >= 0
    assert (state[~valid] == -1).all() and (pair[~valid] == -1).all()
    if nkl is not None:
        assert np.isnan(nkl[~valid]).all()
        on, gn = o.nkl[valid], nkl[valid]
        err = np.abs(gn - on)
        bad = err > RTOL * np.abs(on) + ATOL
        rel = err / np.maximum(np.abs(on), 1e-300)
        print(f"[consensus]   max rel err {rel[on != 0].max() if (on != 0).any() else 0:.3g}", flush=True)
        assert not bad.any(), (np.argwhere(bad)[:5], gn[bad][:5], on[bad][:5])
    exact = valid & (o.flags == 0)
    assert (state[exact] == o.state[exact]).all(), np.argwhere(state[exact] != o.state[exact])[:5]
    assert (pair[exact] == o.pair[exact]).all(), np.argwhere(pair[exact] != o.pair[exact])[:5]
    near = valid & (o.flags != 0)
    assert np.isin(state[near], [0, 1, 2]).all()
    assert all(p // w.K < p % w.K for p in pair[near])
    print(f"[consensus]   states {np.bincount(o.state[valid], minlength=3)} flagged {int(near.sum())}", flush=True)
    return state, pair, nkl, o


def test_consensus_llama3_three_drafts(sv):
    """32 requests x 5 positions x 3 drafts over the Llama-3 vocabulary."""
    w = synthetic.make_consensus()
    _, _, _, o = check(sv, w)
    assert (np.bincount(o.state, minlength=3) > 0).all()  # all three states occur


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("V,dtype", [(1000, "bf16"), (4099, "f32"), (8193, "bf16"), (20000, "f32"),
                                     (70001, "bf16")])
def test_consensus_shapes(sv, K, V, dtype):
    """Ragged gamma (zeros included), tails past the last full chunk, and the
    scalar-load path (rows whose byte length is not a multiple of 16)."""
    w = synthetic.make_consensus(B=5, K=K, gamma=np.array([3, 0, 5, 1, 2], np.int32), V=V, dtype=dtype,
                                 wid=70 + K)
    check(sv, w)


@pytest.mark.parametrize("V,dtype,spread", [(128256, "bf16", (0.002, 0.02)), (50000, "f32", (1e-3, 1e-2))])
def test_consensus_near_identical_drafts(sv, V, dtype, spread):
    """Very small KL values keep their relative accuracy (the exact form)."""
    w = synthetic.make_consensus(B=4, K=3, gamma=4, V=V, dtype=dtype, spread=spread, wid=80)
    _, _, nkl, o = check(sv, w)
    assert (o.nkl[:, 0, 1] < 1e-3).all()


def test_consensus_identical_rows_and_single_token(sv):
    w = synthetic.make_consensus(B=3, K=4, gamma=2, V=3000, wid=81)
    w.drafts = np.repeat(w.drafts[::4], 4, axis=0)  # every draft of a position the same row
    state, pair, nkl, _ = check(sv, w)
    assert (nkl == 0).all() and (state == 1).all() and (pair == 1).all()
    one = synthetic.make_consensus(B=2, K=3, gamma=2, V=1, dtype="f32", wid=82)
    state, pair, nkl, _ = check(sv, one)
    assert (nkl == 0).all() and (state == 1).all()


def test_consensus_invalid_temperatures(sv):
    w = synthetic.make_consensus(B=6, K=3, gamma=np.array([2, 3, 1, 2, 2, 1], np.int32), V=9000, wid=83)
    w.temperature = np.array([1.0, 0.0, -1.0, np.nan, np.inf, 0.8], np.float32)
    state, _, _, _ = check(sv, w)
    assert (state[2:10] == -1).all() and (state[:2] >= 0).all() and (state[10:] >= 0).all()  # requests 1..4


@pytest.mark.parametrize("gamma", [[3, 3, 3], [2, -1, 5], [3, 3, 2]])
def test_consensus_layout_errors(sv, gamma):
    """sum(gamma) != positions, or a negative gamma: -1 everywhere (the rows
    are not read)."""
    w = synthetic.make_consensus(B=3, K=2, gamma=np.array([3, 2, 2], np.int32), V=5000, wid=84)
    state, pair, nkl = run(sv, w, gamma=np.array(gamma, np.int32))
    assert (state == -1).all() and (pair == -1).all() and np.isnan(nkl).all()


@pytest.mark.parametrize("bad", [False, True])
def test_consensus_batch_above_lds_scan(sv, bad):
    """More than 1024 requests: the request map comes from the prep kernel
    instead of each workgroup's scan of gamma."""
    B = 1100
    gamma = np.zeros(B, np.int32)
    gamma[[0, 7, 513, 1024, 1099]] = [2, 1, 3, 1, 2]
    w = synthetic.make_consensus(B=B, K=2, gamma=gamma, V=3000, wid=89)
    if not bad:
        check(sv, w)
    else:
        g2 = gamma.copy()
        g2[1050] = -1
        state, pair, _ = run(sv, w, gamma=g2)
        assert (state == -1).all() and (pair == -1).all()


def test_consensus_no_positions(sv):
    w = synthetic.make_consensus(B=4, K=3, gamma=0, V=5000, wid=85)
    state, pair, nkl = run(sv, w)
    assert state.shape == (0,) and pair.shape == (0,) and nkl.shape == (0, 3, 3)


@pytest.mark.parametrize("dc,dd", [(0.05, 0.08), (0.2, 0.1), (0.0, 1e9)])
def test_consensus_thresholds(sv, dc, dd):
    w = synthetic.make_consensus(B=8, K=3, gamma=4, V=32000, wid=86)
    check(sv, w, dc, dd)


def test_consensus_repeatable_and_matrix_optional(sv):
    import torch
    w = synthetic.make_consensus(B=8, K=3, gamma=4, V=60000, wid=87)
    s1, p1, n1 = run(sv, w)
    ws = torch.full((sv.spec_consensus_workspace_size(sv.make_config(8, 60000, sv.SV_DTYPE_BF16, 4, 32), 3),),
                    255, dtype=torch.uint8, device="cuda:0")
    s2, p2, n2 = run(sv, w, workspace=ws)  # a workspace holding 0xFF bytes needs no clearing
    s3, p3, n3 = run(sv, w, out_nkl=False)
    assert n3 is None
    assert (s1 == s2).all() and (p1 == p2).all() and (n1.view(np.int64) == n2.view(np.int64)).all()
    assert (s1 == s3).all() and (p1 == p3).all()


@pytest.mark.parametrize("which", ["consensus", "divergence"])
def test_consensus_decisions_just_outside_the_flag_band(sv, which):
    """Thresholds 2e-6 (relative) above and below the closest pair's distance
    of chosen positions: outside the oracle's 1e-6 band, so the GPU must take
    the exact decision there (one-pass values that are not accurate enough
    near a threshold go through the exact pass)."""
    w = synthetic.make_consensus(B=4, K=3, gamma=4, V=128256, wid=88)
    o = oracle.consensus(w.drafts, w.dtype, w.gamma, w.K, w.temperature)
    dist = np.array([min(0.5 * (o.nkl[n, a, b] + o.nkl[n, b, a]) for a in range(3) for b in range(a + 1, 3))
                     for n in range(w.npos)])
    for n in (0, 5, 11):
        for f in (1 - 2e-6, 1 + 2e-6):
            thr = float(np.float32(dist[n] * f))
            dc, dd = (thr, 1e9) if which == "consensus" else (0.0, thr)
            ref = oracle.consensus(w.drafts, w.dtype, w.gamma, w.K, w.temperature, dc, dd)
            assert ref.flags[n] == 0, (n, f)
            state, pair, _ = run(sv, w, dc, dd)
            assert state[n] == ref.state[n] and pair[n] == ref.pair[n], (n, f, state[n], ref.state[n])


# ---------------------------------------------------------------- multi-draft longest path

@pytest.mark.parametrize("K,gamma,V,dtype", [(3, 6, 128256, "bf16"), (2, 4, 20000, "f32"), (4, 3, 8193, "bf16")])
def test_multi_draft_longest_path(K, gamma, V, dtype):
    """K drafts' chains verified in one tree-mode call: the accepted path is
    the longest accepted chain (lowest chain on ties), as in the oracle."""
    from parity import assert_parity, compare, run_gpu
    import torch
    assert torch.cuda.is_available()
    w = synthetic.make_multi_draft(B=16 if V > 100000 else 6, K=K, gamma=gamma, V=V, dtype=dtype)
    print(f"[parity] {w.name} B={w.batch} V={w.vocab} dtype={w.dtype}", flush=True)
    g = run_gpu(w)
    o = oracle.verify_workload(w)
    rep = compare(w, g, o)
    print(f"[parity]   {rep}", flush=True)
    assert_parity(rep, w.mode)
    assert (g["tree_node"] == o.tree_node).all()
