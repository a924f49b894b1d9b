"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests compares the oracle with a re-typed copy of itself:
  * the target-law theorem (SpecTr-GBV page, section 2 "theoretical
    foundation" and section 3: the output keeps the target distribution),
    checked by exact black-box enumeration of the oracle's output law;
  * closed forms for E[tau]: token-level SD, GBV (P(tau >= i) = E_q[w_i]),
    recursive rejection sampling at L = 1;
  * invariants: the K-draft upper bound, monotonicity in K (SpecTr-GBV page,
    section 2 "monotonicity" and section 4 ablation on K), GBV >= token level
    (GBV is the optimal single-draft verifier, SpecTr-GBV page, section 1), GBV
    non-decreasing in L (section 4 ablation on L);
  * special cases: p = q, disjoint supports, one draft = GBV, L = 1 token = GBV,
    one-draft SpecTr = token level;
  * SpecTr's scaling factor: at L = 1 the accepted length brackets the one of
    the smallest rho that keeps the residual non-negative, found by a grid
    search over rho;
  * hand-worked examples (tests/golden/worked_examples.json);
  * planted mistakes in a copy of the oracle, each of which must fail a pin.
"""
import json
import os
import subprocess

import numpy as np
import pytest

import lawtools as lt
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
LAW_TOL = 1e-12         # fp64 rounding of the enumerated law (branch weights, reported laws)
ETAU_TOL = 1e-10        # E[tau] from exact branch probabilities (fp64)

# exhaustive grid (V, L, K): every corner of V in {2, 3, 4, 8}, L <= 3, K <= 3
# except (8, 3, 3), whose 512^3 draft realisations are covered statistically below.
GRID = [(V, L, K) for V in (2, 3, 4, 8) for L in (1, 2, 3) for K in (1, 2, 3)
        if (V, L, K) != (8, 3, 3)]


def _model(V, L, seed, **kw):
    rng = np.random.default_rng(1000 * V + 100 * L + seed)
    T = kw.pop("T", [0.7, 1.0, 1.6][seed % 3])
    zero = kw.pop("zero_frac", 0.25 if seed % 2 else 0.0)
    mode = kw.pop("draft_mode", ["noisy", "indep"][seed % 2])
    return lt.TreeModel.random(V, L, rng, T=T, zero_frac=zero, draft_mode=mode, **kw)


@pytest.mark.parametrize("V,L,K", GRID)
def test_multidraft_keeps_target_law(V, L, K):
    for seed in range(2):
        m = _model(V, L, seed)
        law, e_tau, dropped = lt.output_law(m, K, "multidraft")
        assert dropped < 1e-7
        assert abs(sum(law.values()) - 1.0) < LAW_TOL
        assert lt.extended_law_gap(m, law) < LAW_TOL
        assert e_tau <= lt.expected_tau_bound(m, K) + ETAU_TOL
        if K == 1:
            assert abs(e_tau - lt.expected_tau_gbv(m)) < ETAU_TOL
        if L == 1:
            assert abs(e_tau - lt.expected_tau_rrs_l1(m, K)) < ETAU_TOL


# SpecTr enumerates like the K-draft walk, on the same corners.
SPECTR_GRID = GRID


def draws_follow_reported_law(method, K, lib_path=None):
    """Whether the correction law the exact-law entry point reports (om/Z of the
    final draw) is the law of the token the oracle draws: bisecting the float32
    correction uniform over the draws must give the same distribution, to the
    float32 resolution of the uniform."""
    rng = np.random.default_rng(77)
    V, L, B = 8, 3, 40
    tgt = (rng.standard_normal((B, K, L + 1, V)) * 1.5).astype(np.float32)
    drf = (tgt[:, :, :L] + rng.standard_normal((B, K, L, V))).astype(np.float32)
    tok = rng.integers(0, V, (B, K, L)).astype(np.int32)
    tok[:, 1:, 0] = tok[:, :1, 0]   # shared roots, so later drafts are tested too
    T = np.full(B, 0.9, np.float32)
    ua = rng.random((B, K, L)).astype(np.float32)
    rep = oracle.verify_exact(method, tgt, drf, tok, T, ua.astype(np.float64), np.zeros(B),
                              lib_path=lib_path)

    def run(ri, u, uc):
        return oracle.verify(method, tgt[ri], drf[ri], tok[ri], T[ri], u, uc, lib_path=lib_path)

    drawn = lt.correction_law(run, np.arange(B), ua, V)
    return bool(np.abs(rep["corr_law"].sum(axis=1) - 1.0).max() < 1e-14 and
                np.abs(drawn - rep["corr_law"]).max() < V * 2.0 ** -24)


@pytest.mark.parametrize("method,K", [("multidraft", 3), ("spectr", 3), ("token", 1),
                                      ("block", 1)])
def test_reported_correction_law_matches_the_draws(method, K):
    """The exact-law pins read the correction's law from what the oracle reports;
    this pins that report to the oracle's own draws."""
    assert draws_follow_reported_law(method, K)


def spectr_l1_bracket(m, K, n_grid=4001):
    """L = 1 SpecTr, written from its definition rather than the oracle's
    search: rho* is the smallest rho in [1, K] for which K candidates tried in
    turn, each accepted with probability min(1, p/(rho q)), leave a
    non-negative residual p - P(accept with that token).  A grid over rho
    brackets rho*, and P(tau = 1) = 1 - (1 - beta(rho))^K is decreasing in rho,
    so the grid cell gives an interval for E[tau]."""
    p, q = m.p(()), m.q(())
    rhos = np.linspace(1.0, float(K), n_grid)

    def accept_and_residual(rho):
        m_ = np.minimum(q, p / rho)                       # per-try acceptance mass
        beta = m_.sum()
        tries = sum((1.0 - beta) ** i for i in range(K))  # expected tries that happen
        return 1.0 - (1.0 - beta) ** K, p - tries * m_

    ok = [accept_and_residual(r)[1].min() >= -1e-12 for r in rhos]
    g = ok.index(True)
    hi = accept_and_residual(rhos[g])[0]
    lo = hi if g == 0 else accept_and_residual(rhos[g - 1])[0]
    return hi, lo


@pytest.mark.parametrize("V,L,K", SPECTR_GRID)
def test_spectr_keeps_target_law(V, L, K):
    for seed in range(2):
        m = _model(V, L, seed)
        law, e_tau, dropped = lt.output_law(m, K, "spectr")
        assert dropped < 1e-7
        assert abs(sum(law.values()) - 1.0) < LAW_TOL
        assert lt.extended_law_gap(m, law) < LAW_TOL
        assert e_tau <= lt.expected_tau_bound(m, K) + ETAU_TOL
        if K == 1:
            assert abs(e_tau - lt.expected_tau_token(m)) < ETAU_TOL
        if L == 1:
            lo, hi = spectr_l1_bracket(m, K)
            assert lo - 1e-9 <= e_tau <= hi + 1e-9, (lo, e_tau, hi)


def test_spectr_l1_scaling_factor_is_the_smallest_feasible():
    """Larger vocabularies than the enumeration reaches: at L = 1 the oracle's
    P(tau = 1) over many realisations matches the bracket of the smallest
    feasible rho (the acceptance probability of each test is reported, so the
    expected acceptance is computed from h exactly, not sampled)."""
    rng = np.random.default_rng(31)
    for V, K in ((16, 2), (40, 4), (40, 8)):
        m = lt.TreeModel.random(V, 1, rng, T=0.9, draft_mode="noisy")
        lo, hi = spectr_l1_bracket(m, K, n_grid=20001)
        p, q = m.p(()), m.q(())
        B = 4000
        tok = rng.choice(V, size=(B, K, 1), p=q).astype(np.int32)
        tgt = np.broadcast_to(np.stack([m.tgt[()], m.tgt[()]])[None, None],
                              (B, K, 2, V)).astype(np.float32)
        drf = np.broadcast_to(m.drf[()][None, None, None], (B, K, 1, V)).astype(np.float32)
        temps = np.full(B, m.T, np.float32)
        ua = np.full((B, K, 1), 0.9999999, np.float32)   # tests reject unless h ~ 1
        uc = rng.random(B).astype(np.float32)
        o = oracle.verify("spectr", tgt, drf, tok, temps, ua, uc, diagnostics=True)
        h = o["accept_prob"][:, :, 0].astype(np.float64)
        # a draft goes untested only after a test with h ~ 1 accepted; its factor
        # in the product below is then irrelevant
        untested = np.isnan(h)
        assert (~untested[:, 0]).all()
        assert all((h[i, :np.argmax(untested[i])] > 0.9999999).any()
                   for i in np.nonzero(untested.any(axis=1))[0])
        h = np.where(untested, 0.0, h)
        # P(accept | drafts) = 1 - prod_k (1 - h_k); its mean over q^K estimates
        # 1 - (1 - beta)^K with standard error ~1e-3
        est = (1.0 - np.prod(1.0 - h, axis=1)).mean()
        se = (1.0 - np.prod(1.0 - h, axis=1)).std() / np.sqrt(B)
        assert lo - 5 * se - 1e-6 <= est <= hi + 5 * se + 1e-6, (V, K, lo, est, hi)


def _spectr_root(K, tgt_logits, drf_logits, tokens, T, u, lib_path=None):
    """One request per row of u, L = 1, the same rows in every draft."""
    B = len(u)
    V = len(tgt_logits)
    tgt = np.broadcast_to(np.array([tgt_logits, tgt_logits], np.float32)[None, None],
                          (B, K, 2, V)).copy()
    drf = np.broadcast_to(np.array([drf_logits], np.float32)[None, None], (B, K, 1, V)).copy()
    tok = np.full((B, K, 1), tokens, np.int32)
    ua = np.repeat(np.asarray(u, np.float32)[:, None, None], K, axis=1)
    return oracle.verify("spectr", tgt, drf, tok, np.full(B, T, np.float32), ua,
                         np.full(B, 0.5, np.float32), diagnostics=True, lib_path=lib_path)


def spectr_near_identical_ok(lib_path=None):
    """Rows whose total variation is ~1.2e-12 (the draft puts a little more mass
    on the last token): p > rho q nowhere once rho exceeds 1 + 1.3e-12, so
    rho* <= 1 + 1.3e-12 and the shared top token is accepted with h = 1 - 1e-12
    or more, whatever u < 1 is.  (The quotient form c <= rho cannot tell c
    from rho here: their gap rho (1 - beta)^n stays below double rounding for
    rho up to ~1.01.)"""
    o = _spectr_root(8, [0.0, -27.0, -27.0, -27.0], [0.0, -27.0, -27.0, -26.5], 0, 1.0,
                     [0.9999, 0.99999, 0.999999], lib_path)
    return bool((o["accept_len"] == 1).all() and (o["accept_prob"][:, 0, 0] >= 1 - 1e-12).all())


def spectr_near_disjoint_ok(lib_path=None):
    """Supports that share one token C with p_C = s, q_C = t: beta(rho) =
    min(t, s/rho), which is s/rho at the root, so rho* solves
    rho = sum_{i<n} (1 - s/rho)^i, a scalar equation that does not cancel.  A
    draft offering C is accepted with h = (s/t)/rho*.  (The product form
    D <= (1 - beta)^n compares two numbers within ~1e-9 of 1 here.)"""
    n, s_, t_ = 8, 3e-9, 1e-9
    tl = np.array([np.log1p(-s_), -np.inf, np.log(s_)], np.float32)
    dl = np.array([-np.inf, np.log1p(-t_), np.log(t_)], np.float32)
    p = np.exp(tl.astype(np.float64)); p /= p.sum()
    q = np.exp(dl.astype(np.float64)); q /= q.sum()
    s_, t_ = p[2], q[2]
    lo, hi = s_ / t_, float(n)                     # root lies above the breakpoint s/t
    f = lambda r: r - sum((1.0 - s_ / r) ** i for i in range(n))
    assert f(lo) < 0 <= f(hi)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        lo, hi = (mid, hi) if f(mid) < 0 else (lo, mid)
    o = _spectr_root(n, tl, dl, 2, 1.0, [0.9999], lib_path)
    want = (s_ / t_) / hi
    return abs(float(o["accept_prob"][0, 0, 0]) - want) < 1e-12 * want


def spectr_many_candidates_ok(lib_path=None):
    """K = 64 candidates, p = (0.63, 0.37), q = (0.3, 0.7): for rho >= 2.1 = the
    largest ratio no token has p > rho q, so every such rho is feasible, and
    below it D(rho) = 0.63 - 0.3 rho exceeds (1 - beta)^64 < 1e-17 until
    within ~1e-17 of 2.1: rho* = p_0/q_0 to double precision, and a draft
    offering token 1 is accepted with h = (p_1/q_1)/rho*.  (Here beta ~ 0.48 and
    rho - c ~ rho (1 - beta)^64 ~ 1e-18, below the rounding of rho.)"""
    tl = np.log(np.array([0.63, 0.37])).astype(np.float32)
    dl = np.log(np.array([0.3, 0.7])).astype(np.float32)
    p = np.exp(tl.astype(np.float64)); p /= p.sum()
    q = np.exp(dl.astype(np.float64)); q /= q.sum()
    o = _spectr_root(64, tl, dl, 1, 1.0, [0.9999], lib_path)
    want = (p[1] / q[1]) / (p[0] / q[0])
    return abs(float(o["accept_prob"][0, 0, 0]) - want) < 1e-12


def test_spectr_scaling_factor_with_many_candidates():
    assert spectr_many_candidates_ok()


def test_spectr_scaling_factor_at_nearly_identical_rows():
    assert spectr_near_identical_ok()


def test_spectr_scaling_factor_at_nearly_disjoint_rows():
    assert spectr_near_disjoint_ok()


@pytest.mark.parametrize("V,L", [(2, 1), (2, 3), (3, 2), (8, 2), (8, 3)])
def test_single_draft_rules_keep_target_law(V, L):
    for seed in range(2):
        m = _model(V, L, seed)
        law_t, et_t, _ = lt.output_law(m, 1, "token")
        law_b, et_b, _ = lt.output_law(m, 1, "block")
        assert lt.extended_law_gap(m, law_t) < LAW_TOL
        assert lt.extended_law_gap(m, law_b) < LAW_TOL
        assert abs(et_t - lt.expected_tau_token(m)) < ETAU_TOL
        assert abs(et_b - lt.expected_tau_gbv(m)) < ETAU_TOL
        assert et_b >= et_t - ETAU_TOL          # GBV is optimal among single-draft verifiers


@pytest.mark.parametrize("V,L", [(2, 2), (3, 2), (2, 3)])
def test_expected_length_monotone_in_k(V, L):
    for seed in range(3):
        m = _model(V, L, seed)
        prev = lt.expected_tau_gbv(m)
        for K in (2, 3):
            _, e_tau, _ = lt.output_law(m, K, "multidraft")
            assert e_tau >= prev - ETAU_TOL
            prev = e_tau


def test_gbv_expected_length_monotone_in_l():
    rng = np.random.default_rng(5)
    m = lt.TreeModel.random(3, 3, rng, T=0.8)
    vals = [lt.expected_tau_gbv(m, L) for L in (1, 2, 3)]
    assert vals[0] <= vals[1] <= vals[2]


def _random_batch(rng, B, K, L, V, T=0.8, same_rows=True):
    """Random tree-consistent batch: drafts with equal prefixes get equal rows."""
    tgt = rng.standard_normal((B, K, L + 1, V)).astype(np.float32) * 2
    drf = (tgt[:, :, :L] + rng.standard_normal((B, K, L, V)).astype(np.float32))
    tok = rng.integers(0, V, (B, K, L)).astype(np.int32)
    if same_rows:
        for b in range(B):
            for k in range(K):
                for j in range(L + 1):
                    for c in range(k):
                        if (tok[b, c, :j] == tok[b, k, :j]).all():
                            tgt[b, k, j] = tgt[b, c, j]
                            if j < L:
                                drf[b, k, j] = drf[b, c, j]
                            break
    temps = np.full(B, T, np.float32)
    ua = rng.random((B, K, L)).astype(np.float32)
    uc = rng.random(B).astype(np.float32)
    return tgt, drf, tok, temps, ua, uc


def test_extra_draft_never_shortens_accepted_length():
    """Pathwise monotonicity in K: the walk over drafts 0..K-1 is a prefix of the
    walk over drafts 0..K, so with the same uniforms tau can only grow."""
    rng = np.random.default_rng(11)
    for V in (3, 5, 40):
        tgt, drf, tok, temps, ua, uc = _random_batch(rng, 300, 4, 3, V)
        prev = None
        for K in (1, 2, 3, 4):
            o = oracle.verify("multidraft", tgt[:, :K], drf[:, :K], tok[:, :K], temps,
                              ua[:, :K], uc)
            if prev is not None:
                assert (o["accept_len"] >= prev).all()
            prev = o["accept_len"]


def test_one_draft_multidraft_equals_block_pathwise():
    rng = np.random.default_rng(12)
    for V in (2, 7, 64):
        tgt, drf, tok, temps, ua, uc = _random_batch(rng, 400, 1, 4, V)
        a = oracle.verify("block", tgt, drf, tok, temps, ua, uc, diagnostics=True)
        b = oracle.verify("multidraft", tgt, drf, tok, temps, ua, uc, diagnostics=True)
        for key in ("accept_len", "draft_index", "correction", "flags"):
            np.testing.assert_array_equal(a[key], b[key])
        np.testing.assert_array_equal(a["accept_prob"], b["accept_prob"])
        np.testing.assert_array_equal(a["resid_mass"], b["resid_mass"])


def test_one_draft_spectr_equals_token_pathwise():
    """With one candidate rho* = 1 and c = 1: SpecTr is token-level sampling."""
    rng = np.random.default_rng(17)
    for V in (2, 7, 64):
        tgt, drf, tok, temps, ua, uc = _random_batch(rng, 400, 1, 4, V)
        a = oracle.verify("token", tgt, drf, tok, temps, ua, uc, diagnostics=True)
        b = oracle.verify("spectr", tgt, drf, tok, temps, ua, uc, diagnostics=True)
        for key in ("accept_len", "draft_index", "correction", "flags"):
            np.testing.assert_array_equal(a[key], b[key])
        np.testing.assert_array_equal(a["accept_prob"], b["accept_prob"])
        np.testing.assert_array_equal(a["resid_mass"], b["resid_mass"])


def test_length_one_token_equals_block_pathwise():
    rng = np.random.default_rng(13)
    tgt, drf, tok, temps, ua, uc = _random_batch(rng, 500, 1, 1, 9)
    a = oracle.verify("token", tgt, drf, tok, temps, ua, uc, diagnostics=True)
    b = oracle.verify("block", tgt, drf, tok, temps, ua, uc, diagnostics=True)
    for key in ("accept_len", "draft_index", "correction"):
        np.testing.assert_array_equal(a[key], b[key])


def test_equal_distributions_accept_everything():
    """p = q at every node: every method accepts the whole block."""
    rng = np.random.default_rng(14)
    B, K, L, V = 200, 3, 4, 11
    tgt, drf, tok, temps, ua, uc = _random_batch(rng, B, K, L, V)
    drf = tgt[:, :, :L].copy()
    for method, k in (("token", 1), ("block", 1), ("multidraft", K), ("spectr", K)):
        o = oracle.verify(method, tgt[:, :k], drf[:, :k], tok[:, :k], temps, ua[:, :k], uc)
        assert (o["accept_len"] == L).all()
        assert (o["draft_index"] == 0).all()


def test_disjoint_supports_reject_and_sample_target():
    """supp(p) and supp(q) disjoint at the root: tau = 0 and the correction law is p_0."""
    V, L = 4, 2
    rng = np.random.default_rng(15)
    m = lt.TreeModel.random(V, L, rng, T=1.0)
    for pre in list(m.tgt):
        if len(pre) == 0:
            m.tgt[pre][2:] = -np.inf
        if pre in m.drf and len(pre) == 0:
            m.drf[pre][:2] = -np.inf
    for method, K in (("token", 1), ("block", 1), ("multidraft", 2), ("multidraft", 3),
                      ("spectr", 2), ("spectr", 3)):
        law, e_tau, _ = lt.output_law(m, K, method)
        assert e_tau == 0.0
        p0 = m.p(())
        for y in range(V):
            assert abs(law.get((y,), 0.0) - p0[y]) < LAW_TOL


def test_non_canonical_rows_are_never_read():
    """Rows of a draft that shares its prefix with a lower-index draft belong to
    the same node; overwriting them must not change anything."""
    rng = np.random.default_rng(16)
    tgt, drf, tok, temps, ua, uc = _random_batch(rng, 300, 4, 3, 3)
    a = {m: oracle.verify(m, tgt, drf, tok, temps, ua, uc, diagnostics=True)
         for m in ("multidraft", "spectr")}
    tgt2, drf2 = tgt.copy(), drf.copy()
    B, K, L = tok.shape
    for b in range(B):
        for k in range(1, K):
            for j in range(L + 1):
                if any((tok[b, c, :j] == tok[b, k, :j]).all() for c in range(k)):
                    tgt2[b, k, j] = np.nan
                    if j < L:
                        drf2[b, k, j] = np.nan
    for m in a:
        b2 = oracle.verify(m, tgt2, drf2, tok, temps, ua, uc, diagnostics=True)
        for key in ("accept_len", "draft_index", "correction", "flags"):
            np.testing.assert_array_equal(a[m][key], b2[key])


def test_row_lse_matches_library_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(17)
    tgt, drf, tok, temps, ua, uc = _random_batch(rng, 20, 2, 3, 50, T=0.4, same_rows=False)
    o = oracle.verify("multidraft", tgt, drf, tok, temps, ua, uc, diagnostics=True)
    B, K, L = tok.shape
    for b in range(B):
        for k in range(K):
            for j in range(L + 1):
                c = next(c for c in range(k + 1) if (tok[b, c, :j] == tok[b, k, :j]).all())
                ref = logsumexp(tgt[b, c, j].astype(np.float64) / np.float64(temps[b]))
                assert abs(o["row_lse"][b, k, j] - ref) < 1e-12 * max(1, abs(ref))
            for j in range(L):
                c = next(c for c in range(k + 1) if (tok[b, c, :j] == tok[b, k, :j]).all())
                ref = logsumexp(drf[b, c, j].astype(np.float64) / np.float64(temps[b]))
                assert abs(o["row_lse"][b, k, L + 1 + j] - ref) < 1e-12 * max(1, abs(ref))


def test_bf16_bits_are_widened_exactly():
    rng = np.random.default_rng(18)
    tgt, drf, tok, temps, ua, uc = _random_batch(rng, 50, 2, 3, 33)
    # round to bf16 (truncate the mantissa) and pass both as f32 and as bf16 bits
    t16 = (tgt.view(np.uint32) >> 16).astype(np.uint16)
    d16 = (drf.view(np.uint32) >> 16).astype(np.uint16)
    t32 = (t16.astype(np.uint32) << 16).view(np.float32)
    d32 = (d16.astype(np.uint32) << 16).view(np.float32)
    a = oracle.verify("multidraft", t32, d32, tok, temps, ua, uc, diagnostics=True)
    b = oracle.verify("multidraft", t16, d16, tok, temps, ua, uc, diagnostics=True)
    for key in ("accept_len", "draft_index", "correction", "row_lse", "resid_mass"):
        np.testing.assert_array_equal(a[key], b[key])


def test_invalid_request_data_is_flagged():
    rng = np.random.default_rng(19)
    tgt, drf, tok, temps, ua, uc = _random_batch(rng, 6, 2, 2, 10)
    tgt[0, 0, 0, 3] = np.nan                 # NaN in a node row
    tok[1, 1, 1] = 10                        # token outside [0, V)
    temps[2] = 0.0                           # T must be > 0
    ua[3, 0, 0] = 1.0                        # u must be < 1
    drf[4, 0, 1, :] = -np.inf                # a row of zero mass
    o = oracle.verify("multidraft", tgt, drf, tok, temps, ua, uc)
    assert (o["accept_len"][:5] == -1).all()
    assert (o["flags"][:5] == oracle.FLAG_INVALID).all()
    assert o["accept_len"][5] >= 0 and not o["flags"][5] & oracle.FLAG_INVALID


def test_rows_never_read_cannot_invalidate():
    """Validity is checked where a row is read: NaN in rows past the first
    token-level rejection changes nothing."""
    rng = np.random.default_rng(21)
    tgt, drf, tok, temps, ua, uc = _random_batch(rng, 20, 1, 3, 12)
    tgt[:, 0, 0, tok[:, 0, 0]] = -np.inf      # p(x) = 0: position 1 always rejects
    a = oracle.verify("token", tgt, drf, tok, temps, ua, uc)
    assert (a["accept_len"] == 0).all()
    tgt[:, 0, 1:] = np.nan
    drf[:, 0, 1:] = np.nan
    b = oracle.verify("token", tgt, drf, tok, temps, ua, uc)
    for key in ("accept_len", "draft_index", "correction", "flags"):
        np.testing.assert_array_equal(a[key], b[key])
    drf[:, 0, 0, 5] = np.nan                   # a row that is read
    c = oracle.verify("token", tgt, drf, tok, temps, ua, uc)
    assert (c["flags"] == oracle.FLAG_INVALID).all()


def _golden_examples():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)["examples"]


def _golden_inputs(e):
    K, L, V = e["K"], e["L"], e["V"]
    tgt = np.log(np.array(e["target_probs"], np.float64)).astype(np.float32)[None]
    drf = np.log(np.array(e["draft_probs"], np.float64)).astype(np.float32)[None]
    assert tgt.shape == (1, K, L + 1, V) and drf.shape == (1, K, L, V)
    return (tgt, drf, np.array(e["tokens"], np.int32)[None],
            np.array([e["T"]], np.float32), np.array(e["u_accept"], np.float32)[None],
            np.array([e["u_correct"]], np.float32))


def distinct_node_rows(tok, L):
    """Upper bound on the rows any rule may read for one request: the number of
    distinct nodes of its draft tree (prefixes of length 0..L for target rows,
    0..L-1 for draft rows), counted from the tokens alone."""
    K = tok.shape[0]
    t = sum(len({tuple(tok[k, :j]) for k in range(K)}) for j in range(L + 1))
    d = sum(len({tuple(tok[k, :j]) for k in range(K)}) for j in range(L))
    return t + d


def _shared_prefix_batch(rng, B=300, K=4, L=3, V=5, identical=False):
    """Drafts that share prefixes often (V = 5, peaked rows) and target rows close
    to the draft rows, so acceptances are frequent and later drafts are examined
    below an accepted node.  identical: every draft repeats draft 0, so the tree
    is one chain of 2L + 1 node rows."""
    tgt, drf, tok, temps, ua, uc = _random_batch(rng, B, K, L, V, T=0.5, same_rows=False)
    drf = (tgt[:, :, :L] + 0.1 * rng.standard_normal(drf.shape)).astype(np.float32)
    tok[:, 1] = tok[:, 0]                       # draft 1 repeats draft 0
    tok[:, 3, :2] = tok[:, 2, :2]               # draft 3 shares two tokens with draft 2
    if identical:
        tok[:] = tok[:, :1]
    for b in range(B):                          # rows follow the node rule
        for k in range(K):
            for j in range(L + 1):
                for c in range(k):
                    if (tok[b, c, :j] == tok[b, k, :j]).all():
                        tgt[b, k, j] = tgt[b, c, j]
                        if j < L:
                            drf[b, k, j] = drf[b, c, j]
                        break
    return tgt, drf, tok, temps, ua, uc


def test_rows_read_within_distinct_nodes():
    """The rows-read counter (the method's algorithmic bytes) never exceeds the
    number of distinct node rows of the request's draft tree."""
    rng = np.random.default_rng(31)
    for identical in (False, True):
        tgt, drf, tok, temps, ua, uc = _shared_prefix_batch(rng, identical=identical)
        bound = np.array([distinct_node_rows(tok[b], tok.shape[2]) for b in range(len(tok))])
        if identical:
            assert (bound == 2 * tok.shape[2] + 1).all()
        for method in ("multidraft", "spectr"):
            o = oracle.verify(method, tgt, drf, tok, temps, ua, uc)
            assert (o["counters"][:, 2] <= bound).all(), method
            assert (o["counters"][:, 2] >= 2).all(), method       # the root pair at least


def test_golden_worked_examples():
    ex = _golden_examples()
    for e in ex:
        tgt, drf, tok, temps, ua, uc = _golden_inputs(e)
        for method in e["methods"]:
            o = oracle.verify(method, tgt, drf, tok, temps, ua, uc, diagnostics=True)
            exp = e["expect"]
            assert o["accept_len"][0] == exp["accept_len"], (e["name"], method)
            assert o["draft_index"][0] == exp["draft_index"], (e["name"], method)
            assert o["correction"][0] == exp["correction"], (e["name"], method)
            assert abs(o["resid_mass"][0] - exp["resid_mass"]) < 1e-6, (e["name"], method)
            if "rows_read" in exp:   # distinct node rows whose logits the rules read
                assert o["counters"][0, 2] == exp["rows_read"][method], (e["name"], method)
            want = np.array([[np.nan if v is None else v for v in row]
                             for row in exp["accept_prob"]])
            got = o["accept_prob"][0]
            if method == "token":
                want = want[:1]
                got = got[:1]
            assert np.array_equal(np.isnan(got), np.isnan(want)), (e["name"], method)
            ok = ~np.isnan(want)
            assert np.allclose(got[ok], want[ok], atol=1e-6), (e["name"], method)


def test_monte_carlo_law_at_v8_l3_k3():
    """The corner (V, L, K) = (8, 3, 3) of the grid is too large to enumerate
    (8^9 draft realisations); draw drafts and uniforms instead and compare the
    law of the extended output with the target law by a chi-square test."""
    from scipy.stats import chi2
    V, L, K, n = 8, 3, 3, 60000
    rng = np.random.default_rng(20)
    m = lt.TreeModel.random(V, L, rng, T=0.9, sigma=1.0)
    nodes = {}
    tgt = np.empty((n, K, L + 1, V), np.float32)
    drf = np.empty((n, K, L, V), np.float32)
    tok = np.empty((n, K, L), np.int32)
    qcache = {}
    for i in range(n):
        for k in range(K):
            pre = ()
            for j in range(L):
                tgt[i, k, j] = m.tgt[pre]
                drf[i, k, j] = m.drf[pre]
                if pre not in qcache:
                    qcache[pre] = m.q(pre)
                x = rng.choice(V, p=qcache[pre])
                tok[i, k, j] = x
                pre = pre + (int(x),)
            tgt[i, k, L] = m.tgt[pre]
    temps = np.full(n, m.T, np.float32)
    ua = rng.random((n, K, L)).astype(np.float32)
    uc = rng.random(n).astype(np.float32)
    o = oracle.verify("multidraft", tgt, drf, tok, temps, ua, uc, threads=4)
    counts = {}
    pcache = {}
    for i in range(n):
        tau, ks, y = int(o["accept_len"][i]), int(o["draft_index"][i]), int(o["correction"][i])
        z = tuple(int(t) for t in tok[i, ks, :tau]) + (y,)
        while len(z) < L + 1:                      # extend by the target
            if z not in pcache:
                pcache[z] = m.p(z)
            z = z + (int(rng.choice(V, p=pcache[z])),)
        nodes[z] = nodes.get(z, 0) + 1
    # chi-square over the full sequence law, pooling cells with small expectation
    import itertools
    exp_, obs = [], []
    pool_e = pool_o = 0.0
    for z in itertools.product(range(V), repeat=L + 1):
        e = n * m.p_seq(z)
        c = nodes.get(z, 0)
        if e >= 8:
            exp_.append(e)
            obs.append(c)
        else:
            pool_e += e
            pool_o += c
    exp_.append(pool_e)
    obs.append(pool_o)
    exp_, obs = np.array(exp_), np.array(obs)
    stat = ((obs - exp_) ** 2 / exp_).sum()
    pval = chi2.sf(stat, len(exp_) - 1)
    assert pval > 1e-4, (stat, len(exp_), pval)


# ------------------------------------------------------------- planted mistakes

MUTANTS = {
    # the residual does not move after a rejection
    "no_beta_update": ("                H[nH++] = x;\n                beta += N;",
                       "                H[nH++] = x;\n                beta += 0.0;"),
    # R_m with the two rows transposed
    "R_transposed": ("Rm += fmax(w[m] * r->p[v] - r->q[v], 0.0);",
                     "Rm += fmax(w[m] * r->q[v] - r->p[v], 0.0);"),
    # first position not normalised by the residual mass
    "first_weight_unnormalised": ("svo_chain(1.0, r->om[x] / N, r->q[x])",
                                  "svo_chain(1.0, r->om[x], r->q[x])"),
    # GBV's h without the (1 - w) term
    "h_drops_term": ("double d = Rm + 1.0 - w[m];", "double d = Rm + 1.0;"),
    # after acceptance the residual state keeps the old weight
    "accept_state_wrong": ("alpha = w[tau];", "alpha = 1.0;"),
    # inverse CDF threshold not scaled by the mass Z
    "icdf_unscaled_threshold": ("double t = r->uc * Z;", "double t = r->uc;"),
}


SPECTR_MUTANTS = {
    # no search: rho = n is feasible but not the smallest
    "spectr_rho_is_n": ("double rho = svo_ks_rho(r, n);", "double rho = (double)n;"),
    # residual without the expected number of tries
    "spectr_residual_without_c": ("fmax(r->p[v] - c * fmin(r->q[v], r->p[v] / rho), 0.0)",
                                  "fmax(r->p[v] - fmin(r->q[v], r->p[v] / rho), 0.0)"),
    # candidates counted over all drafts, not those on the accepted prefix
    "spectr_counts_all_drafts": ("n += svo_same_prefix(r, k, own, j);", "n += 1;"),
    # acceptance ignores the scaling factor
    "spectr_accept_ignores_rho": ("svo_ratio(r->p[x], rho * r->q[x])",
                                  "svo_ratio(r->p[x], r->q[x])"),
    # per-try acceptance mass taken at rho = 1
    "spectr_beta_unscaled": ("b += fmin(r->q[v], r->p[v] / rho);",
                             "b += fmin(r->q[v], r->p[v]);"),
}

# the feasibility test evaluated in one form only
SPECTR_NUMERIC_MUTANTS = {
    "spectr_quotient_form_only": ("    if (beta <= 0x1p-10)\n        return svo_ks_c(beta, n) <= rho;",
                                  "    if (1)\n        return svo_ks_c(beta, n) <= rho;"),
    "spectr_product_form_only": ("    if (beta <= 0x1p-10)\n        return svo_ks_c(beta, n) <= rho;",
                                 "    if (0)\n        return svo_ks_c(beta, n) <= rho;"),
    "spectr_quotient_form_to_one_half": (
        "    if (beta <= 0x1p-10)\n        return svo_ks_c(beta, n) <= rho;",
        "    if (beta <= 0.5)\n        return svo_ks_c(beta, n) <= rho;"),
}


# the rows-read counter keyed by the reading draft instead of the node's owner
ROWS_MUTANTS = {
    "rows_counted_per_draft": ("r->touched[(target ? j : r->L + 1 + j) * r->K + c] = 1;",
                               "r->touched[(target ? j : r->L + 1 + j) * r->K + k] = 1;"),
}


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants")
    src = open(oracle.SRC).read()
    libs = {}
    for name, (old, new) in {**MUTANTS, **SPECTR_MUTANTS, **SPECTR_NUMERIC_MUTANTS,
                             **ROWS_MUTANTS}.items():
        assert src.count(old) == 1, name
        p = d / f"{name}.c"
        p.write_text(src.replace(old, new))
        so = d / f"{name}.so"
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC",
                               "-shared", "-o", str(so), str(p), "-lm"])
        libs[name] = str(so)
    return libs


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(mutant_libs, name):
    """Each planted mistake must break the law, a closed form, the bound on at
    least one tiny instance, or the agreement of the draws with the law the
    oracle reports for them."""
    caught = not draws_follow_reported_law("multidraft", 3, lib_path=mutant_libs[name])
    for (V, L, K) in [(2, 2, 2), (3, 2, 2), (2, 3, 1), (3, 1, 3), (2, 3, 3)]:
        if caught:
            break
        for seed in range(2):
            m = _model(V, L, seed)
            law, e_tau, _ = lt.output_law(m, K, "multidraft", lib_path=mutant_libs[name])
            gap = lt.extended_law_gap(m, law)
            bad = gap > LAW_TOL or e_tau > lt.expected_tau_bound(m, K) + ETAU_TOL
            if K == 1:
                bad |= abs(e_tau - lt.expected_tau_gbv(m)) > ETAU_TOL
            if bad:
                caught = True
                break
        if caught:
            break
    assert caught, name


@pytest.mark.parametrize("name", sorted(SPECTR_MUTANTS))
def test_planted_spectr_mistake_fails_a_pin(mutant_libs, name):
    caught = not draws_follow_reported_law("spectr", 3, lib_path=mutant_libs[name])
    for (V, L, K) in [(3, 1, 3), (2, 2, 2), (3, 2, 2), (8, 1, 3)]:
        if caught:
            break
        for seed in range(2):
            m = _model(V, L, seed)
            law, e_tau, _ = lt.output_law(m, K, "spectr", lib_path=mutant_libs[name])
            bad = lt.extended_law_gap(m, law) > LAW_TOL
            bad |= e_tau > lt.expected_tau_bound(m, K) + ETAU_TOL
            if L == 1:
                lo, hi = spectr_l1_bracket(m, K)
                bad |= not (lo - 1e-9 <= e_tau <= hi + 1e-9)
            if bad:
                caught = True
                break
        if caught:
            break
    assert caught, name


@pytest.mark.parametrize("name", sorted(SPECTR_NUMERIC_MUTANTS))
def test_planted_spectr_numeric_mistake_fails_a_pin(mutant_libs, name):
    lib = mutant_libs[name]
    assert not (spectr_near_identical_ok(lib) and spectr_near_disjoint_ok(lib)
                and spectr_many_candidates_ok(lib)), name


@pytest.mark.parametrize("name", sorted(ROWS_MUTANTS))
def test_planted_rows_read_mistake_fails_a_pin(mutant_libs, name):
    """A rows-read counter that counts the node rows of shared nodes once per
    reading draft must miss a hand-derived count or the distinct-node bound."""
    lib = mutant_libs[name]
    caught = False
    for e in _golden_examples():
        args = _golden_inputs(e)
        for method in e["methods"]:
            exp = e["expect"].get("rows_read", {})
            if method in exp:
                o = oracle.verify(method, *args, lib_path=lib)
                caught |= o["counters"][0, 2] != exp[method]
    rng = np.random.default_rng(31)
    for identical in (False, True):
        tgt, drf, tok, temps, ua, uc = _shared_prefix_batch(rng, identical=identical)
        o = oracle.verify("multidraft", tgt, drf, tok, temps, ua, uc, lib_path=lib)
        bound = np.array([distinct_node_rows(tok[b], tok.shape[2]) for b in range(len(tok))])
        caught |= bool((o["counters"][:, 2] > bound).any())
    assert caught, name
