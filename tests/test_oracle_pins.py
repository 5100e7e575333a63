"""Pins of the CPU oracle to what the pages and the mathematics fix.

None of these tests re-types the oracle's formulas: each compares the oracle
with a hand-derived value, a library routine (scipy / numpy), a closed-form
law, a brute-force enumeration, or a statistical test of the losslessness
claim.  All run on the CPU.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
import synthetic
from synthetic import f32_to_bf16_bits, bf16_bits_to_f32

GOLD = os.path.join(os.path.dirname(__file__), "golden")
S, G, K, TR = oracle.STOCHASTIC, oracle.GREEDY, oracle.NKL, oracle.TREE_GREEDY


def run(target, draft, gamma, tokens, temps=None, ua=None, ur=None, mode=S, delta=0.15, parents=None,
        dtype="f32", max_gamma=None, total=None):
    gamma = np.asarray(gamma, np.int32)
    B = len(gamma)
    R_d = int(gamma[gamma > 0].sum())
    if temps is None:
        temps = np.ones(B, np.float32)
    if ua is None:
        ua = np.zeros(R_d, np.float32)
    if ur is None:
        ur = np.zeros(B, np.float32)
    return oracle.verify(np.asarray(target), None if draft is None else np.asarray(draft), dtype, gamma,
                         np.asarray(tokens, np.int32), np.asarray(temps, np.float32), np.asarray(ua, np.float32),
                         np.asarray(ur, np.float32), mode, delta, parents, max_gamma, total)


# --------------------------------------------------------------------------
# worked example (closed forms), modified rejection sampling
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1.0, 2.0, 0.5])
def test_worked_example_v4(T):
    g = json.load(open(os.path.join(GOLD, "worked_v4.json")))
    p, q, bonus = (np.array(g[k]) for k in ("p", "q", "bonus"))
    tgt = (T * np.log(np.stack([p, bonus]))).astype(np.float32)
    drf = (T * np.log(q[None, :])).astype(np.float32)
    for case in g["cases"]:
        r = run(tgt, drf, [1], [g["draft_token"]], [T], [case["u_accept"]], [case["u_resample"]])
        assert r.num_accepted[0] == case["num_accepted"], case
        assert r.tokens.tolist() == case["tokens"], case
        assert abs(r.alpha[0] - g["alpha"]) < 1e-6
        assert abs(r.p_x[0] - g["p_x"]) < 1e-6 and abs(r.q_x[0] - g["q_x"]) < 1e-6
        if case["num_accepted"] == 0:
            assert abs(r.resid_mass[0] - g["resid_mass"]) < 1e-6
        else:
            assert r.resid_mass[0] == 1.0


def test_worked_example_bf16_matches_f32():
    """bf16 inputs widen exactly: the same values given as bf16 and as fp32 give
    identical results (pins the bf16 decode)."""
    rng = np.random.default_rng(5)
    V, gam = 300, 3
    t = (3 * rng.standard_normal((gam + 1, V))).astype(np.float32)
    d = (t[:gam] + rng.standard_normal((gam, V))).astype(np.float32)
    tb, db = f32_to_bf16_bits(t), f32_to_bf16_bits(d)
    tf, df = bf16_bits_to_f32(tb), bf16_bits_to_f32(db)
    x = rng.integers(0, V, gam)
    ua = rng.random(gam).astype(np.float32)
    ur = rng.random(1).astype(np.float32)
    a = run(tb, db, [gam], x, [0.8], ua, ur, dtype="bf16")
    b = run(tf, df, [gam], x, [0.8], ua, ur, dtype="f32")
    assert a.tokens.tolist() == b.tokens.tolist()
    np.testing.assert_array_equal(a.p_x, b.p_x)
    np.testing.assert_array_equal(a.alpha, b.alpha)
    # and a decode mistake (e.g. reading the low byte) would change p_x
    ref = special.softmax(tf[0].astype(np.float64) / np.float64(np.float32(0.8)))[x[0]]
    assert abs(a.p_x[0] / ref - 1) < 1e-12


# --------------------------------------------------------------------------
# log-softmax, alpha and residual against scipy on random rows
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
def test_probabilities_match_scipy(T):
    rng = np.random.default_rng(int(T * 10))
    V, gam, B = 777, 5, 6
    t = (3 * rng.standard_normal((B * (gam + 1), V))).astype(np.float32)
    d = np.concatenate([t[b * (gam + 1): b * (gam + 1) + gam] for b in range(B)]) + \
        rng.standard_normal((B * gam, V)).astype(np.float32)
    d = d.astype(np.float32)
    x = rng.integers(0, V, B * gam)
    ua = rng.random(B * gam).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    temps = np.full(B, T, np.float32)
    r = run(t, d, [gam] * B, x, temps, ua, ur)
    Td = np.float64(np.float32(T))
    for b in range(B):
        for i in range(gam):
            P = special.softmax(t[b * (gam + 1) + i].astype(np.float64) / Td)
            Q = special.softmax(d[b * gam + i].astype(np.float64) / Td)
            k = b * gam + i
            assert abs(r.p_x[k] / P[x[k]] - 1) < 1e-11
            assert abs(r.q_x[k] / Q[x[k]] - 1) < 1e-11
            assert abs(r.alpha[k] - min(1.0, P[x[k]] / Q[x[k]])) < 1e-12
        # the decision and the terminal draw
        n = r.num_accepted[b]
        alphas = [min(1.0, r.p_x[b * gam + i] / r.q_x[b * gam + i]) for i in range(gam)]
        exp_n = next((i for i in range(gam) if not (ua[b * gam + i] <= alphas[i])), gam)
        assert n == exp_n
        assert r.tokens[b * (gam + 1): b * (gam + 1) + n].tolist() == x[b * gam: b * gam + n].tolist()
        P = special.softmax(t[b * (gam + 1) + n].astype(np.float64) / Td)
        if n < gam:
            Q = special.softmax(d[b * gam + n].astype(np.float64) / Td)
            # identity: sum max(0, p - q) = 1 - sum min(p, q)
            assert abs(r.resid_mass[b] - (1 - np.minimum(P, Q).sum())) < 1e-12
            w = np.maximum(0, P - Q)
        else:
            w = P
        cdf = np.cumsum(w) / w.sum()
        u = np.float64(ur[b])
        ystar = int(np.searchsorted(cdf, u, side="right"))
        lo = cdf[ystar - 1] if ystar > 0 else 0.0
        if min(u - lo, cdf[ystar] - u) > 1e-9:  # margin computed here, not by the oracle
            assert r.tokens[b * (gam + 1) + n] == ystar
        assert (r.tokens[b * (gam + 1) + n + 1: (b + 1) * (gam + 1)] == -1).all()


# --------------------------------------------------------------------------
# q == p: everything accepted, bonus drawn from p_gamma
# --------------------------------------------------------------------------

def test_q_equals_p_accepts_everything():
    rng = np.random.default_rng(11)
    V, gam, B = 64, 4, 4000
    rows = (3 * rng.standard_normal((gam + 1, V))).astype(np.float32)
    t = np.tile(rows, (B, 1))
    d = np.tile(rows[:gam], (B, 1))
    x = rng.integers(0, V, B * gam)  # any tokens: alpha = 1 exactly
    ua = rng.random(B * gam).astype(np.float32)
    ur = rng.random(B).astype(np.float32)
    r = run(t, d, [gam] * B, x, np.full(B, 0.9, np.float32), ua, ur)
    assert (r.num_accepted == gam).all()
    assert (r.alpha == 1.0).all()
    tok = r.tokens.reshape(B, gam + 1)
    assert (tok[:, :gam] == x.reshape(B, gam)).all()
    # bonus ~ p_gamma (chi-square)
    P = special.softmax(rows[gam].astype(np.float64) / np.float64(np.float32(0.9)))
    obs = np.bincount(tok[:, gam], minlength=V)
    keep = P * B >= 5
    exp = np.concatenate([P[keep] * B, [P[~keep].sum() * B]])
    ob = np.concatenate([obs[keep], [obs[~keep].sum()]])
    if exp[-1] == 0:
        exp, ob = exp[:-1], ob[:-1]
    assert stats.chisquare(ob, exp * ob.sum() / exp.sum()).pvalue > 1e-3


# --------------------------------------------------------------------------
# accepted-count law (closed form): P(n=k) = a^k (1-a), P(n=gamma) = a^gamma
# --------------------------------------------------------------------------

def test_accepted_count_law():
    rng = np.random.default_rng(3)
    V, gam, B = 8, 4, 200_000
    t_row = (3 * rng.standard_normal(V)).astype(np.float32)
    d_row = (t_row + rng.standard_normal(V)).astype(np.float32)
    P = special.softmax(t_row.astype(np.float64))
    Q = special.softmax(d_row.astype(np.float64))
    a = np.minimum(P, Q).sum()
    t = np.tile(t_row, (B * (gam + 1), 1))
    d = np.tile(d_row, (B * gam, 1))
    x = rng.choice(V, size=B * gam, p=Q)
    r = run(t, d, [gam] * B, x, None, rng.random(B * gam).astype(np.float32),
            rng.random(B).astype(np.float32))
    obs = np.bincount(r.num_accepted, minlength=gam + 1)
    law = np.array([a ** k * (1 - a) for k in range(gam)] + [a ** gam])
    assert abs(law.sum() - 1) < 1e-12
    assert stats.chisquare(obs, law * B).pvalue > 1e-3


# --------------------------------------------------------------------------
# losslessness at V = 8, gamma = 4, 10^6 trials; negative control
# --------------------------------------------------------------------------

def _lossless_setup(n_trials, seed=2026):
    rng = np.random.default_rng(seed)
    V, gam = 8, 4
    t_rows = (3 * rng.standard_normal((gam + 1, V))).astype(np.float32)
    d_rows = (t_rows[:gam] + rng.standard_normal((gam, V))).astype(np.float32)
    P = special.softmax(t_rows.astype(np.float64), axis=1)
    Q = special.softmax(d_rows.astype(np.float64), axis=1)
    x = np.empty((n_trials, gam), np.int32)
    for i in range(gam):
        x[:, i] = rng.choice(V, size=n_trials, p=Q[i])
    ua = rng.random(n_trials * gam).astype(np.float32)
    ur = rng.random(n_trials).astype(np.float32)
    return V, gam, t_rows, d_rows, P, Q, x, ua, ur


def _position_pvalues(tok, n_acc, P, gam):
    """p-values of 'token at slot k given the step reached k ~ p_k'."""
    pv = []
    for k in range(gam + 1):
        reached = n_acc >= k
        obs = np.bincount(tok[reached, k], minlength=P.shape[1])
        pv.append(stats.chisquare(obs, P[k] * reached.sum()).pvalue)
    return pv


def test_losslessness_chi_square():
    n = 1_000_000
    V, gam, t_rows, d_rows, P, Q, x, ua, ur = _lossless_setup(n)
    t = np.tile(t_rows, (n, 1))
    d = np.tile(d_rows, (n, 1))
    r = run(t, d, [gam] * n, x.ravel(), None, ua, ur)
    tok = r.tokens.reshape(n, gam + 1)
    pv = _position_pvalues(tok, r.num_accepted, P, gam)
    alpha = 1e-3 / len(pv)  # Bonferroni
    assert min(pv) > alpha, pv
    # first emitted token ~ p_0 unconditionally
    assert stats.chisquare(np.bincount(tok[:, 0], minlength=V), P[0] * n).pvalue > 1e-3

    # Negative control: the listing's correction (emit argmax of p_j instead of
    # redrawing from the residual) is not lossless, and the test must see it.
    bad = tok.copy()
    for k in range(gam):
        rej = r.num_accepted == k
        bad[rej, k] = int(np.argmax(P[k]))
    pv_bad = _position_pvalues(bad, r.num_accepted, P, gam)
    assert min(pv_bad) < 1e-30, pv_bad


# --------------------------------------------------------------------------
# greedy mode and ties (golden)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_greedy_golden(dtype):
    g = json.load(open(os.path.join(GOLD, "greedy_tree_small.json")))["greedy"]
    rows = np.array(g["rows"], np.float32)
    tgt = f32_to_bf16_bits(rows) if dtype == "bf16" else rows
    for case in g["cases"]:
        r = run(tgt, None, [4], case["drafts"], mode=G, dtype=dtype)
        assert r.num_accepted[0] == case["num_accepted"]
        assert r.tokens.tolist() == case["tokens"]


def test_greedy_argmax_drafts_fully_accepted_and_ties():
    rng = np.random.default_rng(8)
    V, gam, B = 513, 6, 50
    # heavy ties: integer logits on a small range
    t = rng.integers(-3, 4, size=(B * (gam + 1), V)).astype(np.float32)
    x = np.concatenate([np.argmax(t[b * (gam + 1): b * (gam + 1) + gam], axis=1) for b in range(B)])
    r = run(t, None, [gam] * B, x, mode=G)
    assert (r.num_accepted == gam).all()
    tok = r.tokens.reshape(B, gam + 1)
    assert (tok[:, :gam] == x.reshape(B, gam)).all()
    assert (tok[:, gam] == np.argmax(t[gam::gam + 1], axis=1)).all()
    # break position j of each request: emitted token is np.argmax (first max)
    j = rng.integers(0, gam, B)
    x2 = x.copy().reshape(B, gam)
    for b in range(B):
        x2[b, j[b]] = (x2[b, j[b]] + 1) % V
    r2 = run(t, None, [gam] * B, x2.ravel(), mode=G)
    assert (r2.num_accepted == j).all()
    tok2 = r2.tokens.reshape(B, gam + 1)
    for b in range(B):
        assert tok2[b, j[b]] == np.argmax(t[b * (gam + 1) + j[b]])
        assert (tok2[b, j[b] + 1:] == -1).all()


# --------------------------------------------------------------------------
# NKL
# --------------------------------------------------------------------------

def test_nkl_identical_rows_zero():
    rng = np.random.default_rng(1)
    V, gam, B = 1000, 5, 4
    t = (3 * rng.standard_normal((B * (gam + 1), V))).astype(np.float32)
    d = np.concatenate([t[b * (gam + 1): b * (gam + 1) + gam] for b in range(B)])
    r = run(t, d, [gam] * B, np.zeros(B * gam), np.full(B, 0.6, np.float32), mode=K, delta=1e-30)
    assert (r.nkl == 0.0).all()
    assert (r.num_accepted == gam).all()


@pytest.mark.parametrize("T", [0.6, 1.0])
def test_nkl_matches_scipy_entropy(T):
    rng = np.random.default_rng(4)
    V, gam, B = 4096, 4, 3
    t = (3 * rng.standard_normal((B * (gam + 1), V))).astype(np.float32)
    d = np.concatenate([t[b * (gam + 1): b * (gam + 1) + gam] for b in range(B)]) + \
        (0.5 + rng.random((B * gam, 1))).astype(np.float32) * rng.standard_normal((B * gam, V)).astype(np.float32)
    d = d.astype(np.float32)
    r = run(t, d, [gam] * B, np.zeros(B * gam), np.full(B, T, np.float32), mode=K, delta=0.15)
    Td = np.float64(np.float32(T))
    for b in range(B):
        for i in range(gam):
            P = special.softmax(t[b * (gam + 1) + i].astype(np.float64) / Td)
            Q = special.softmax(d[b * gam + i].astype(np.float64) / Td)
            ref = stats.entropy(Q, P) / np.log(V)
            assert abs(r.nkl[b * gam + i] / ref - 1) < 1e-10
        n = r.num_accepted[b]
        exp_n = next((i for i in range(gam) if not r.nkl[b * gam + i] < np.float32(0.15)), gam)
        assert n == exp_n
        assert r.tokens[b * (gam + 1) + n] == np.argmax(t[b * (gam + 1) + n])


def test_nkl_range_on_long_drafts():
    """NKL lies in [0, 1] on the long-draft workload (reduced batch), and the
    true bound 0 <= KL <= max_y (l_d - l_t) holds."""
    import synthetic
    w = synthetic.make_long(B=2, mode=K)
    r = oracle.verify_workload(w)
    assert np.isfinite(r.nkl).all()
    assert (r.nkl >= 0).all() and (r.nkl <= 1).all()
    T = np.float64(w.temperature[0])
    tf, df = w.target_f32(), w.draft_f32()
    for k in (0, 7, 15, 16, 31):
        b, i = divmod(k, 16)
        lt = special.log_softmax(tf[b * 17 + i].astype(np.float64) / T)
        ld = special.log_softmax(df[k].astype(np.float64) / T)
        assert r.nkl[k] * np.log(w.vocab) <= (ld - lt).max() + 1e-12
    # acceptance decays along the draft (noise ramps up)
    assert r.nkl.reshape(2, 16)[:, :4].mean() < r.nkl.reshape(2, 16)[:, -4:].mean()


# --------------------------------------------------------------------------
# draft-side row sampling (the drafter's draw from softmax(x/T))
# --------------------------------------------------------------------------

def test_sample_rows_cdf_steps():
    """p = (0.1, 0.2, 0.3, 0.4) at T = 1 (logits log p) has CDF steps at 0.1,
    0.3, 0.6 and 1.0; y* = min{y : C_y > u}: a uniform just below a step stays
    on the left token, just above it moves right.  The same at T = 2 with
    logits 2 log p."""
    p = np.array([0.1, 0.2, 0.3, 0.4])
    u = np.array([0.0, 0.0999, 0.1001, 0.2999, 0.3001, 0.5999, 0.6001, 0.9999], np.float32)
    want = [0, 0, 1, 1, 2, 2, 3, 3]
    for T in (1.0, 2.0):
        x = np.tile((T * np.log(p)).astype(np.float32), (len(u), 1))
        tok, margin = oracle.sample_rows(x, "f32", np.full(len(u), T, np.float32), u)
        assert tok.tolist() == want
        assert np.allclose(margin[1:], 1e-4, rtol=0.01)  # every uniform sits 1e-4 from a step


def test_sample_rows_is_the_bonus_draw():
    """A verify request with gamma = 0 draws its bonus token from target row 0
    with u_resample: the same draw as sampling that row."""
    rng = np.random.default_rng(21)
    B, V = 40, 3000
    t = (3 * rng.standard_normal((B, V))).astype(np.float32)
    T = (0.5 + rng.random(B)).astype(np.float32)
    ur = rng.random(B, dtype=np.float32)
    r = oracle.verify(t, np.zeros((0, V), np.float32), "f32", np.zeros(B, np.int32), np.zeros(0, np.int32), T,
                      np.zeros(0, np.float32), ur, S)
    tok, _ = oracle.sample_rows(t, "f32", T, ur)
    assert (r.num_accepted == 0).all() and (r.tokens == tok).all()


def test_sample_rows_chi_square():
    """200k draws from one V = 8 row: token frequencies follow scipy's softmax."""
    rng = np.random.default_rng(22)
    V, n, T = 8, 200_000, 0.7
    x = (2 * rng.standard_normal(V)).astype(np.float32)
    tok, _ = oracle.sample_rows(np.tile(x, (n, 1)), "f32", np.full(n, T, np.float32),
                                rng.random(n, dtype=np.float32))
    P = special.softmax(x.astype(np.float64) / np.float64(np.float32(T)))
    counts = np.bincount(tok, minlength=V)
    assert stats.chisquare(counts, P * n).pvalue > 1e-3


def test_sample_rows_invalid_inputs():
    x = np.zeros((5, 16), np.float32)
    T = np.array([1.0, 0.0, np.nan, 1.0, 1.0], np.float32)
    u = np.array([0.5, 0.5, 0.5, 1.0, -0.1], np.float32)
    tok, _ = oracle.sample_rows(x, "f32", T, u)
    assert tok.tolist() == [8, -1, -1, -1, -1]  # uniform 16-token row: u = 0.5 lands on token 8


def test_topk_rows_hand_cases():
    """Hand-checked rows: distinct values, ties (the lower index first), a
    tie straddling the k-th place, and k = V."""
    x = np.array([[0.5, 3.0, -1.0, 3.0, 2.0, 0.5],
                  [1.0, 1.0, 1.0, 1.0, 1.0, 1.0],
                  [-2.0, -1.0, -3.0, -1.0, -0.5, -4.0]], np.float32)
    assert oracle.topk_rows(x, "f32", 3).tolist() == [[1, 3, 4], [0, 1, 2], [4, 1, 3]]
    assert oracle.topk_rows(x, "f32", 6).tolist() == [[1, 3, 4, 0, 5, 2], [0, 1, 2, 3, 4, 5],
                                                       [4, 1, 3, 0, 2, 5]]


def test_topk_rows_first_is_the_pinned_argmax():
    """k = 1 is the greedy argmax (pinned by the greedy golden cases); every
    chosen logit is at least every other logit of its row."""
    w = synthetic.random_workload(seed=3, mode=G, B=9, V=5000, dtype="bf16", gmax=3, gmin=0, ties=True)
    top = oracle.topk_rows(w.target, "bf16", 5)
    r = oracle.verify_workload(w.with_mode(G))
    t_off = w.t_off
    xf = bf16_bits_to_f32(w.target)
    for b in range(w.batch):
        n = r.num_accepted[b]
        assert top[t_off[b] + n, 0] == r.tokens[t_off[b] + n]  # the terminal token is the row argmax
    for row in range(xf.shape[0]):
        chosen = xf[row, top[row]]
        assert (np.diff(chosen) <= 0).all()
        rest = np.delete(xf[row], top[row])
        assert chosen.min() >= rest.max()


# --------------------------------------------------------------------------
# NKL with the position-adaptive threshold ("Chain of Draft" page, section 4.3)
# --------------------------------------------------------------------------

def test_nkl_threshold_page_examples():
    g = json.load(open(os.path.join(GOLD, "nkl_threshold.json")))
    d, a, m = g["delta_base"], g["alpha"], g["delta_max"]
    for ex in g["printed_examples"] + g["cap_examples"]:
        got = oracle.nkl_threshold(d, a, m, ex["position_1based"] - 1)  # the oracle takes 0-based positions
        assert abs(got / ex["delta"] - 1) < 1e-6, ex  # float32 inputs widen to float64
    for ex in g["inconsistent_examples"]:
        got = oracle.nkl_threshold(d, a, m, ex["position_1based"] - 1)
        assert abs(got / ex["formula"] - 1) < 1e-6 and abs(got - ex["printed"]) > 0.01
    # non-decreasing along the sequence for alpha >= 0, and never above the cap
    prev = 0.0
    for pos in list(range(0, 70)) + [2 ** k - 1 for k in range(7, 31)]:
        t = oracle.nkl_threshold(d, a, m, pos)
        assert prev <= t <= np.float32(m)
        prev = t


def _nkl_rows(seed, B, gam, V, T):
    rng = np.random.default_rng(seed)
    t = (3 * rng.standard_normal((B * (gam + 1), V))).astype(np.float32)
    d = np.concatenate([t[b * (gam + 1): b * (gam + 1) + gam] for b in range(B)]) + \
        (0.3 + 1.2 * rng.random((B * gam, 1))).astype(np.float32) * rng.standard_normal((B * gam, V)).astype(np.float32)
    return t, d.astype(np.float32)


def test_nkl_adaptive_alpha_zero_is_the_constant_threshold():
    B, gam, V, T = 4, 6, 2048, 0.6
    t, d = _nkl_rows(11, B, gam, V, T)
    temps = np.full(B, T, np.float32)
    ref = oracle.verify(t, d, "f32", np.full(B, gam, np.int32), np.zeros(B * gam, np.int32), temps, None, None,
                        K, 0.15)
    pos = np.arange(B * gam, dtype=np.int32) * 977
    for dmax in (0.15, 0.5, 10.0):
        r = oracle.verify(t, d, "f32", np.full(B, gam, np.int32), np.zeros(B * gam, np.int32), temps, None, None,
                          K, 0.15, nkl_position=pos, nkl_alpha=0.0, nkl_delta_max=dmax)
        assert (r.tokens == ref.tokens).all() and (r.num_accepted == ref.num_accepted).all()
        assert np.array_equal(r.nkl, ref.nkl)


def test_nkl_adaptive_threshold_decides():
    """The decision is the first i with nkl_i >= delta_i, where nkl_i comes from
    scipy's KL and delta_i from the pinned threshold; positions near the start
    of a sequence get the base threshold, far ones a larger one."""
    B, gam, V, T = 6, 8, 4096, 0.6
    t, d = _nkl_rows(12, B, gam, V, T)
    Td = np.float64(np.float32(T))
    starts = np.array([0, 3, 60, 1023, 5000, 2 ** 21], np.int64)
    pos = np.concatenate([s + np.arange(gam) for s in starts]).astype(np.int32)
    r = oracle.verify(t, d, "f32", np.full(B, gam, np.int32), np.zeros(B * gam, np.int32), np.full(B, T, np.float32),
                      None, None, K, 0.15, nkl_position=pos, nkl_alpha=0.08, nkl_delta_max=0.3)
    nchanged = 0
    for b in range(B):
        kl = [stats.entropy(special.softmax(d[b * gam + i].astype(np.float64) / Td),
                            special.softmax(t[b * (gam + 1) + i].astype(np.float64) / Td)) / np.log(V)
              for i in range(gam)]
        thr = [oracle.nkl_threshold(0.15, 0.08, 0.3, int(pos[b * gam + i])) for i in range(gam)]
        exp_n = next((i for i in range(gam) if not kl[i] < thr[i]), gam)
        assert r.num_accepted[b] == exp_n
        assert r.tokens[b * (gam + 1) + exp_n] == np.argmax(t[b * (gam + 1) + exp_n])
        const_n = next((i for i in range(gam) if not kl[i] < np.float32(0.15)), gam)
        nchanged += exp_n != const_n
    assert nchanged > 0  # the schedule changes some decisions on these rows


def _scipy_nkl(t_row, d_row, T):
    Td = np.float64(np.float32(T))
    P = special.softmax(t_row.astype(np.float64) / Td)
    Q = special.softmax(d_row.astype(np.float64) / Td)
    return stats.entropy(Q, P) / np.log(t_row.shape[0])


@pytest.mark.parametrize("sign", [1, -1])
def test_nkl_band_flag_is_relative_to_the_threshold(sign):
    """FLAG_NKL_BAND marks a decision with |nkl_i - delta| < 1e-6 delta.  With
    delta set at a position's NKL (from scipy) times 1 +- 5e-7 the flag is set;
    at 1 +- 2e-6 and 1 +- 5e-6 it is not.  The NKL values are below 0.2, so an
    absolute band of 1e-6 would flag the 5e-6 case, and the decision at the
    position follows the side of delta."""
    B, gam, V, T = 3, 4, 4096, 0.6
    t, d = _nkl_rows(21, B, gam, V, T)
    temps = np.full(B, T, np.float32)
    for b in (1, 2):
        n = [_scipy_nkl(t[b * (gam + 1) + i], d[b * gam + i], T) for i in range(gam)]
        assert n[0] < 0.2 and all(abs(n[i] / n[0] - 1) > 1e-3 for i in range(1, gam))
        for rel, flagged in ((5e-7, True), (2e-6, False), (5e-6, False)):
            delta = float(np.float32(n[0] * (1 + sign * rel)))
            r = oracle.verify(t, d, "f32", np.full(B, gam, np.int32), np.zeros(B * gam, np.int32), temps, None,
                              None, K, delta)
            assert bool(r.flags[b] & oracle.FLAG_NKL_BAND) == flagged, (b, rel)
            assert (r.num_accepted[b] > 0) == (sign > 0), (b, rel)


@pytest.mark.parametrize("sign", [1, -1])
def test_nkl_band_flag_uses_the_position_threshold(sign):
    """With generation positions the band is taken around the position's own
    threshold delta_i = min(delta_max, delta (1 + alpha log2(pos + 1))): at
    pos = 1023 and alpha = 1/16 the threshold is 1.625 delta exactly, and delta
    is set so that delta_i is the position's NKL times 1 +- 5e-7 (flagged) or
    1 +- 5e-6 (not flagged)."""
    B, gam, V, T = 3, 4, 4096, 0.6
    t, d = _nkl_rows(21, B, gam, V, T)
    temps = np.full(B, T, np.float32)
    pos = np.zeros(B * gam, np.int32)
    for b in (1, 2):
        pos[b * gam: (b + 1) * gam] = 1023 + np.arange(gam)
    for b in (1, 2):
        n0 = _scipy_nkl(t[b * (gam + 1)], d[b * gam], T)
        for rel, flagged in ((5e-7, True), (5e-6, False)):
            delta = float(np.float32(n0 * (1 + sign * rel) / 1.625))
            r = oracle.verify(t, d, "f32", np.full(B, gam, np.int32), np.zeros(B * gam, np.int32), temps, None,
                              None, K, delta, nkl_position=pos, nkl_alpha=0.0625, nkl_delta_max=10.0)
            assert bool(r.flags[b] & oracle.FLAG_NKL_BAND) == flagged, (b, rel)
            assert (r.num_accepted[b] > 0) == (sign > 0), (b, rel)


def test_nkl_negative_position_marks_only_its_request():
    B, gam, V, T = 3, 4, 512, 1.0
    t, d = _nkl_rows(13, B, gam, V, T)
    pos = np.arange(B * gam, dtype=np.int32)
    pos[gam + 2] = -1
    r = oracle.verify(t, d, "f32", np.full(B, gam, np.int32), np.zeros(B * gam, np.int32), np.full(B, T, np.float32),
                      None, None, K, 0.15, nkl_position=pos, nkl_alpha=0.08, nkl_delta_max=0.3)
    assert r.num_accepted[1] == -1 and (r.tokens[gam + 1: 2 * (gam + 1)] == -1).all()
    assert r.num_accepted[0] >= 0 and r.num_accepted[2] >= 0


# --------------------------------------------------------------------------
# block-accept mode ("Chain of Draft" page, sections 2.2 and 3.3)
# --------------------------------------------------------------------------

BLK = oracle.BLOCK


def _onehot_rows(argmax, V, tie_at=None):
    """Target rows whose maximum is at `argmax` (and, tied, at `tie_at`)."""
    rows = np.zeros((len(argmax), V), np.float32)
    for i, a in enumerate(argmax):
        rows[i, a] = 5.0
        if tie_at is not None:
            rows[i, tie_at[i]] = 5.0
    return rows


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_accept_golden(dtype):
    g = json.load(open(os.path.join(GOLD, "block_accept.json")))
    V = g["vocab"]
    for case in g["cases"]:
        rows = _onehot_rows(case["argmax"], V, case.get("tie_at"))
        tgt = f32_to_bf16_bits(rows) if dtype == "bf16" else rows
        r = oracle.verify(tgt, None, dtype, np.array([len(case["draft"])], np.int32),
                          np.array(case["draft"], np.int32), None, None, None, BLK, block_min_len=case["min_len"])
        assert r.num_accepted[0] == case["num_accepted"], case["name"]
        assert r.tokens.tolist() == case["tokens"], case["name"]


def _runs_reference(flags, min_len):
    """End of the first longest run of 1s (regular expression over the
    flags), or 0 when it is shorter than min_len."""
    import re
    text = "".join("1" if f else "0" for f in flags)
    best = None
    for m in re.finditer("1+", text):
        if best is None or len(m.group(0)) > len(best.group(0)):
            best = m
    return best.end() if best is not None and len(best.group(0)) >= min_len else 0


@pytest.mark.parametrize("min_len", [1, 2, 3, 4])
def test_block_accept_every_agreement_pattern(min_len):
    """Every agreement pattern of gamma = 0..10 positions, packed in one call:
    the kept length equals the end of the first longest agreeing run (found by
    a regular expression), the kept tokens are the draft's and the next token
    is the target row's argmax."""
    V = 8
    gam, tgt_rows, drafts, expect = [], [], [], []
    rng = np.random.default_rng(min_len)
    for g in range(11):
        for pat in range(1 << g):
            flags = [(pat >> i) & 1 for i in range(g)]
            am = rng.integers(0, V, g + 1)
            d = [int(am[i]) if flags[i] else int((am[i] + 1 + rng.integers(0, V - 1)) % V) for i in range(g)]
            gam.append(g)
            tgt_rows.append(_onehot_rows(am, V))
            drafts += d
            e = _runs_reference(flags, min_len)
            expect.append((e, d[:e] + [int(am[e])] + [-1] * (g - e)))
    r = oracle.verify(np.concatenate(tgt_rows), None, "f32", np.array(gam, np.int32), np.array(drafts, np.int32),
                      None, None, None, BLK, block_min_len=min_len)
    t_off = np.concatenate([[0], np.cumsum(np.array(gam) + 1)])
    for b, (e, toks) in enumerate(expect):
        assert r.num_accepted[b] == e, b
        assert r.tokens[t_off[b]:t_off[b + 1]].tolist() == toks, b


def test_block_accept_equals_greedy_when_every_draft_agrees_and_rejects_bad_min_len():
    w = synthetic.random_workload(seed=51, mode=G, B=20, V=3000, dtype="bf16", gmax=7, gmin=3, greedy_drafts=True)
    tf = w.target_f32()
    w.draft_tokens = np.concatenate([np.argmax(tf[w.t_off[b]: w.t_off[b] + w.gamma[b]], axis=1)
                                     for b in range(w.batch)]).astype(np.int32)
    rg = oracle.verify_workload(w)
    rb = oracle.verify_workload(w.with_mode(BLK))
    assert (rg.num_accepted == w.gamma).all()
    assert np.array_equal(rg.tokens, rb.tokens) and np.array_equal(rg.num_accepted, rb.num_accepted)
    with pytest.raises(ValueError):
        oracle.verify(w.target, None, "bf16", w.gamma, w.draft_tokens, None, None, None, BLK, block_min_len=0)


# --------------------------------------------------------------------------
# consensus across K drafts ("Chain of Draft" page, section 4.4)
# --------------------------------------------------------------------------

def test_consensus_worked_example():
    """Two-token rows with hand-derived KL values (tests/golden/consensus_v2.json)."""
    g = json.load(open(os.path.join(GOLD, "consensus_v2.json")))
    rows = {k: np.log(np.array(v, np.float64)).astype(np.float32) for k, v in g["rows"].items()}
    for case in g["cases"]:
        names = case["drafts"]
        K = len(names)
        r = oracle.consensus(np.stack([rows[n] for n in names]), "f32", np.array([1], np.int32), K,
                             np.ones(1, np.float32))
        for a in range(K):
            assert r.nkl[0, a, a] == 0.0
            for c in range(K):
                if a != c:
                    ref = g["nkl"][names[a] + names[c]]["value"]
                    assert abs(r.nkl[0, a, c] / ref - 1) < 1e-6, (names, a, c)
        assert r.state[0] == case["state"] and r.pair[0] == case["pair"], case


@pytest.mark.parametrize("K,T", [(2, 1.0), (3, 0.6), (4, 1.3)])
def test_consensus_matches_scipy_and_rules(K, T):
    """The matrix against scipy's KL; the closest pair, the state and the flags
    follow from those scipy values."""
    rng = np.random.default_rng(K)
    V, B, gam = 2048, 3, 4
    base = 3 * rng.standard_normal((B * gam, V))
    drafts = np.concatenate([[base[n] + s * rng.standard_normal(V) for s in (0.05, 0.3, 0.6, 1.0)[:K]]
                             for n in range(B * gam)]).astype(np.float32)
    r = oracle.consensus(drafts, "f32", np.full(B, gam, np.int32), K, np.full(B, T, np.float32))
    Td = np.float64(np.float32(T))
    for n in range(B * gam):
        Q = [special.softmax(drafts[n * K + a].astype(np.float64) / Td) for a in range(K)]
        M = np.zeros((K, K))
        for a in range(K):
            for c in range(K):
                if a != c:
                    M[a, c] = stats.entropy(Q[a], Q[c]) / np.log(V)
                    assert abs(r.nkl[n, a, c] / M[a, c] - 1) < 1e-10
        pairs = [(0.5 * (M[a, c] + M[c, a]), a * K + c) for a in range(K) for c in range(a + 1, K)]
        best, pair = min(pairs)
        assert r.pair[n] == pair
        assert r.state[n] == (1 if best < np.float32(0.1) else 2 if best > np.float32(0.15) else 0)


def test_consensus_identical_drafts_and_invalid_requests():
    rng = np.random.default_rng(3)
    V, K = 5000, 3
    row = (3 * rng.standard_normal(V)).astype(np.float32)
    drafts = np.tile(row, (2 * K, 1))
    r = oracle.consensus(drafts, "f32", np.array([1, 1], np.int32), K, np.array([0.7, 0.0], np.float32))
    assert (r.nkl[0] == 0.0).all() and r.state[0] == 1 and r.pair[0] == 1  # pair (0, 1)
    assert r.state[1] == -1 and r.pair[1] == -1 and np.isnan(r.nkl[1]).all()
    one = oracle.consensus(np.ones((K, 1), np.float32), "f32", np.array([1], np.int32), K, np.ones(1, np.float32))
    assert (one.nkl[0] == 0.0).all() and one.state[0] == 1  # V = 1: one point mass, NKL 0


@pytest.mark.parametrize("thr,state_below,state_above,flag", [(0.1, 1, 0, 1), (0.15, 0, 2, 2)])
def test_consensus_threshold_crossings(thr, state_below, state_above, flag):
    """Two drafts of a one-parameter family (the second row scaled by 1 + t):
    scipy's root finder places the symmetrised distance at the threshold; just
    below and above it the state switches."""
    from scipy.optimize import brentq
    rng = np.random.default_rng(11)
    V = 1024
    x = (2 * rng.standard_normal(V)).astype(np.float64)

    def dist(t):
        P = special.softmax(x)
        Q = special.softmax(x * (1 + t))
        return 0.5 * (stats.entropy(P, Q) + stats.entropy(Q, P)) / np.log(V)

    t0 = brentq(lambda t: dist(t) - float(np.float32(thr)), 0.0, 5.0, xtol=1e-15)
    for t, state in ((t0 * (1 - 1e-4), state_below), (t0 * (1 + 1e-4), state_above)):
        drafts = np.stack([x, x * (1 + t)]).astype(np.float64)
        # exact float32 rows: the distance of the stored rows is what counts
        r = oracle.consensus(drafts.astype(np.float32), "f32", np.array([1], np.int32), 2, np.ones(1, np.float32))
        xs = drafts.astype(np.float32).astype(np.float64)
        d = 0.5 * (stats.entropy(special.softmax(xs[0]), special.softmax(xs[1])) +
                   stats.entropy(special.softmax(xs[1]), special.softmax(xs[0]))) / np.log(V)
        assert r.state[0] == state, (t, d)
        assert not (r.flags[0] & flag)


@pytest.mark.parametrize("which", ["consensus", "divergence"])
def test_consensus_flag_bands(which):
    """A threshold set at the stored rows' distance (from scipy) times
    1 +- 5e-7 is flagged (bit 1 for the consensus threshold, 2 for the
    divergence one); at 1 +- 5e-6 it is not; the state follows the side."""
    rng = np.random.default_rng(17)
    V = 3000
    x = (2 * rng.standard_normal(V)).astype(np.float32)
    y = (x + 0.8 * rng.standard_normal(V)).astype(np.float32)
    P, Q = special.softmax(x.astype(np.float64)), special.softmax(y.astype(np.float64))
    d = 0.5 * (stats.entropy(P, Q) + stats.entropy(Q, P)) / np.log(V)
    for rel, flagged in ((5e-7, True), (-5e-7, True), (5e-6, False), (-5e-6, False)):
        thr = float(np.float32(d * (1 + rel)))
        dc, dd = (thr, 10.0) if which == "consensus" else (0.0, thr)
        r = oracle.consensus(np.stack([x, y]), "f32", np.array([1], np.int32), 2, np.ones(1, np.float32), dc, dd)
        bit = 1 if which == "consensus" else 2
        assert bool(r.flags[0] & bit) == flagged, rel
        if which == "consensus":
            assert r.state[0] == (1 if rel > 0 else 0)
        else:
            assert r.state[0] == (2 if rel < 0 else 0)


def test_consensus_near_tie_flag():
    """Three identical drafts: every pair at distance 0, the first pair (0, 1)
    chosen and the near-tie flag set; well separated drafts: not set."""
    rng = np.random.default_rng(19)
    x = (3 * rng.standard_normal(4000)).astype(np.float32)
    r = oracle.consensus(np.stack([x, x, x]), "f32", np.array([1], np.int32), 3, np.ones(1, np.float32))
    assert r.pair[0] == 1 and r.flags[0] & 4
    z = np.stack([x, x + 0.1 * rng.standard_normal(4000), x + 2.0 * rng.standard_normal(4000)]).astype(np.float32)
    r = oracle.consensus(z, "f32", np.array([1], np.int32), 3, np.ones(1, np.float32))
    assert r.pair[0] == 1 and not (r.flags[0] & 4)


def test_multi_draft_longest_path_is_tree_mode_over_chains():
    """Several drafts verified together, keeping the longest accepted path
    (Gemma-4 MTP page, section 6.2), as tree mode over K chains under one root:
    the accepted length equals the longest greedy acceptance among the chains
    run one by one as separate greedy requests, the emitted tokens are that
    chain's (the lowest chain among equals) and the next token is the argmax of
    its last accepted node's row."""
    K, gam = 3, 5
    w = synthetic.make_multi_draft(B=24, K=K, gamma=gam, V=4000, noise=(0.2, 0.6, 1.0))
    rt = oracle.verify_workload(w)
    N = 1 + K * gam
    tf = w.target_f32()
    for b in range(w.batch):
        lens = []
        for k in range(K):
            rows = [b * N] + [b * N + 1 + k * gam + i for i in range(gam)]
            toks = w.draft_tokens[b * (N - 1) + k * gam: b * (N - 1) + (k + 1) * gam]
            rg = oracle.verify(tf[rows], None, "f32", np.array([gam], np.int32), toks, None, None, None, G)
            lens.append((int(rg.num_accepted[0]), k, rg.tokens))
        best = max(l for l, _, _ in lens)
        k_best = min(k for l, k, _ in lens if l == best)
        assert rt.num_accepted[b] == best, b
        ts = w.t_off[b]
        assert rt.tokens[ts: ts + best + 1].tolist() == lens[k_best][2][: best + 1].tolist(), b
        assert (rt.tokens[ts + best + 1: ts + N] == -1).all()
    assert len(set(int(n) for n in rt.num_accepted)) > 1  # the chains' acceptances differ


# --------------------------------------------------------------------------
# tree mode: golden, brute force, chain == greedy
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tree_golden(dtype):
    g = json.load(open(os.path.join(GOLD, "greedy_tree_small.json")))["tree"]
    rows = np.array(g["rows"], np.float32)
    tgt = f32_to_bf16_bits(rows) if dtype == "bf16" else rows
    par = np.array(g["parents"][1:], np.int32)
    r = run(tgt, None, [len(par)], g["node_tokens"], mode=TR, parents=par, dtype=dtype)
    assert r.num_accepted[0] == g["num_accepted"]
    assert r.tree_node[0] == g["deepest_node"]
    assert r.tokens.tolist() == g["tokens"]


def _brute_force_tree(rows, parents, toks):
    """Enumerate every root->node path; a path is accepted iff each edge's token
    equals the argmax (np.argmax: first maximum) of the edge's parent row."""
    N = len(parents) + 1
    par = [-1] + list(parents)
    best, best_path = 0, []
    for n in range(1, N):
        path, v, ok = [], n, True
        while v != 0:
            if toks[v - 1] != int(np.argmax(rows[par[v]])):
                ok = False
            path.append(v)
            v = par[v]
        if ok and len(path) > len(best_path):
            best, best_path = n, path
    return best, [toks[v - 1] for v in reversed(best_path)] + [int(np.argmax(rows[best]))]


def test_tree_brute_force_random():
    rng = np.random.default_rng(21)
    V = 12
    for trial in range(300):
        N = int(rng.integers(1, 10))
        parents = np.array([rng.integers(0, k) for k in range(1, N)], np.int32)
        rows = rng.integers(0, 4, size=(N, V)).astype(np.float32)  # ties on purpose
        toks = np.array([int(np.argmax(rows[parents[k - 1]])) if rng.random() < 0.7 else int(rng.integers(0, V))
                         for k in range(1, N)], np.int32)
        r = run(rows, None, [N - 1], toks, mode=TR, parents=parents)
        node, out = _brute_force_tree(rows, parents, list(toks))
        assert r.tree_node[0] == node
        assert r.num_accepted[0] == len(out) - 1
        assert r.tokens[: len(out)].tolist() == out
        assert (r.tokens[len(out):] == -1).all()


def test_chain_tree_equals_greedy():
    rng = np.random.default_rng(9)
    V, gam, B = 257, 7, 40
    t = rng.integers(-2, 3, size=(B * (gam + 1), V)).astype(np.float32)
    x = np.concatenate([np.argmax(t[b * (gam + 1): b * (gam + 1) + gam], axis=1) for b in range(B)])
    flip = rng.random(B * gam) < 0.15
    x[flip] = rng.integers(0, V, flip.sum())
    chain = np.tile(np.arange(gam, dtype=np.int32), B)  # parent of node k is k-1
    a = run(t, None, [gam] * B, x, mode=G)
    b = run(t, None, [gam] * B, x, mode=TR, parents=chain)
    assert a.tokens.tolist() == b.tokens.tolist()
    assert a.num_accepted.tolist() == b.num_accepted.tolist()


# --------------------------------------------------------------------------
# batching invariance and invalid data
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [S, G, K])
def test_batch_equals_single_calls(mode):
    import synthetic
    w = synthetic.random_workload(7, mode, B=9, V=300, dtype="bf16", gmax=5, gmin=0)
    full = oracle.verify_workload(w)
    t_off, d_off = w.t_off, w.d_off
    for b in range(w.batch):
        ts, te, ds, de = t_off[b], t_off[b + 1], d_off[b], d_off[b + 1]
        r = oracle.verify(w.target[ts:te], w.draft[ds:de], w.dtype, w.gamma[b:b + 1], w.draft_tokens[ds:de],
                          w.temperature[b:b + 1], w.u_accept[ds:de], w.u_resample[b:b + 1], mode, w.delta,
                          None, w.max_gamma)
        assert r.tokens.tolist() == full.tokens[ts:te].tolist()
        assert r.num_accepted[0] == full.num_accepted[b]


def test_invalid_requests_isolated():
    import synthetic
    w = synthetic.random_workload(3, S, B=6, V=200, dtype="f32", gmax=4, gmin=2)
    base = oracle.verify_workload(w)
    d_off = w.d_off
    bad = {1: "token", 2: "temp", 3: "uacc", 4: "ures"}
    w.draft_tokens = w.draft_tokens.copy()
    w.temperature = w.temperature.copy()
    w.u_accept = w.u_accept.copy()
    w.u_resample = w.u_resample.copy()
    w.draft_tokens[d_off[1]] = w.vocab
    w.temperature[2] = 0.0
    w.u_accept[d_off[3] + 1] = 1.0
    w.u_resample[4] = np.nan
    r = oracle.verify_workload(w)
    t_off = w.t_off
    for b in range(w.batch):
        seg = r.tokens[t_off[b]:t_off[b + 1]]
        if b in bad:
            assert r.num_accepted[b] == -1 and (seg == -1).all()
            assert r.flags[b] & oracle.FLAG_INVALID
        else:
            assert r.num_accepted[b] == base.num_accepted[b]
            assert seg.tolist() == base.tokens[t_off[b]:t_off[b + 1]].tolist()


def test_layout_errors_mark_everything_invalid():
    rng = np.random.default_rng(0)
    t = rng.standard_normal((8, 10)).astype(np.float32)
    d = rng.standard_normal((5, 10)).astype(np.float32)
    r = run(t, d, [3, 2], np.zeros(5), total=4)  # sum(gamma) = 5 != 4
    assert (r.num_accepted == -1).all()
    r = run(t, d, [3, -1], np.zeros(5), total=2)
    assert (r.num_accepted == -1).all()
    # gamma above max_gamma: that request only
    r = run(t, d, [3, 2], np.zeros(5), max_gamma=2)
    assert r.num_accepted[0] == -1 and r.num_accepted[1] >= 0


def test_flags_mark_boundary_decisions():
    g = json.load(open(os.path.join(GOLD, "worked_v4.json")))
    p, q = np.array(g["p"]), np.array(g["q"])
    tgt = np.log(np.stack([p, q])).astype(np.float32)
    drf = np.log(q[None, :]).astype(np.float32)
    # u within 1e-5 of alpha = 2/3: flagged; far: not flagged
    r = run(tgt, drf, [1], [2], None, [np.float32(2 / 3 + 3e-6)], [0.5])
    assert r.flags[0] & oracle.FLAG_ACCEPT_BAND
    r = run(tgt, drf, [1], [2], None, [0.9], [0.5])
    assert not (r.flags[0] & oracle.FLAG_ACCEPT_BAND) and not (r.flags[0] & oracle.FLAG_DRAW_BAND)
    # resample uniform at the residual CDF step 0.75 (= 0.3/0.4): flagged
    r = run(tgt, drf, [1], [2], None, [0.9], [np.float32(0.75 + 2e-6)])
    assert r.flags[0] & oracle.FLAG_DRAW_BAND


def test_inverse_cdf_many_draws():
    """Many terminal draws at V = 1000 against numpy's searchsorted on the
    cumulative residual (margins computed independently of the oracle)."""
    rng = np.random.default_rng(77)
    V, B = 1000, 3000
    t = (3 * rng.standard_normal((2 * B, V))).astype(np.float32)
    d = (t[0::2] + rng.standard_normal((B, V))).astype(np.float32)
    x = rng.integers(0, V, B)
    ua = np.full(B, 0.999999, np.float32)  # reject unless alpha ~ 1
    ur = rng.random(B).astype(np.float32)
    r = run(t, d, [1] * B, x, None, ua, ur)
    checked = 0
    for b in range(B):
        P = special.softmax(t[2 * b].astype(np.float64))
        n = r.num_accepted[b]
        if n == 0:
            Q = special.softmax(d[b].astype(np.float64))
            w = np.maximum(0.0, P - Q)
        else:
            w = special.softmax(t[2 * b + 1].astype(np.float64))
        cdf = np.cumsum(w) / w.sum()
        u = np.float64(ur[b])
        y = int(np.searchsorted(cdf, u, side="right"))
        lo = cdf[y - 1] if y > 0 else 0.0
        if min(u - lo, cdf[y] - u) > 1e-10:
            assert r.tokens[2 * b + n] == y, b
            checked += 1
    assert checked > 0.99 * B


def test_cdf_steps_are_strict():
    g = json.load(open(os.path.join(GOLD, "worked_v4.json")))["cdf_steps"]
    t = np.zeros((1, 4), np.float32)
    for case in g["cases"]:
        r = run(t, np.zeros((0, 4), np.float32), [0], [], None, [], [case["u_resample"]])
        assert r.num_accepted[0] == 0
        assert r.tokens.tolist() == [case["token"]], case


def test_nkl_single_token_vocabulary():
    """V = 1: KL / ln V is 0/0; both distributions are the same point mass, so
    NKL is 0 and every draft is accepted (a reading, stated in the oracle)."""
    t = np.array([[0.5], [1.0], [2.0]], np.float32)
    d = np.array([[3.0], [-1.0]], np.float32)
    r = run(t, d, [2], [0, 0], [0.7], mode=K, delta=0.15)
    assert r.nkl.tolist() == [0.0, 0.0]
    assert r.num_accepted[0] == 2 and r.tokens.tolist() == [0, 0, 0]
