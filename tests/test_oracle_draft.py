"""Pins of the oracle's drafting rule (svo_draft) against what the mathematics
fixes: K i.i.d. draft blocks (SpecTr-GBV page, section 2, step 1), each token
an inverse-CDF draw from the temperature softmax of its node row.

  * one draw has exactly the softmax law (its CDF boundaries, read off by
    bisection over the float32 uniform, are the softmax's partial sums);
  * with the same rows for every draft, a draw depends on its own uniform
    only, so the K blocks are independent and identically distributed;
  * drafts that meet at a node read that node's row (the lowest-index draft's)
    and never their own; drafts at different nodes read their own rows;
  * invalid data is flagged; hand-worked draws (tests/golden/draft_examples.json);
  * planted mistakes in a copy of the oracle each fail one of these.
"""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
F32_ONE_BITS = np.float32(1.0).view(np.uint32)


def _softmax(logits, T):
    l = np.asarray(logits, np.float64)
    m = l[np.isfinite(l)].max()
    e = np.where(np.isfinite(l), np.exp((l - m) / T), 0.0)
    return e / e.sum()


def draw_law(row, T, lib_path=None, dtype=np.float32):
    """Law of one draw (K = L = 1) read off by bisection over the float32 uniform:
    for each v, the smallest u whose draw is >= v."""
    V = len(row)
    logits = np.asarray(row, np.float32)
    if dtype == "bf16":
        logits = (logits.view(np.uint32) >> 16).astype(np.uint16)
    n = V - 1
    if n == 0:
        return np.ones(1)
    d = np.broadcast_to(logits[None, None, None], (n, 1, 1, V)).copy()
    temps = np.full(n, T, np.float32)
    target_v = np.arange(1, V)
    lo = np.zeros(n, np.int64)
    hi = np.full(n, int(F32_ONE_BITS), np.int64)
    run = lambda u: oracle.draft(d, temps, u.reshape(n, 1, 1), lib_path=lib_path)["tokens"][:, 0, 0]
    at_zero = run(np.zeros(n, np.float32)) >= target_v
    for _ in range(32):
        active = (hi - lo > 1) & ~at_zero
        if not active.any():
            break
        mid = (lo + hi) // 2
        up = run(mid.astype(np.uint32).view(np.float32)) >= target_v
        hi = np.where(active & up, mid, hi)
        lo = np.where(active & ~up, mid, lo)
    bnd = np.where(at_zero, 0.0, hi.astype(np.uint32).view(np.float32).astype(np.float64))
    return np.diff(np.concatenate([[0.0], bnd, [1.0]]))


@pytest.mark.parametrize("V,T", [(2, 1.0), (7, 0.25), (7, 3.0), (40, 0.7), (40, 1.6)])
def test_one_draw_has_the_softmax_law(V, T):
    rng = np.random.default_rng(100 * V + int(10 * T))
    row = rng.standard_normal(V).astype(np.float32) * 2
    row[rng.random(V) < 0.2] = -np.inf
    row[0] = 0.0
    want = _softmax(row, T)
    got = draw_law(row, T)
    assert np.abs(got - want).max() < 4e-7 * V, (got, want)


def test_one_draw_law_bf16():
    rng = np.random.default_rng(3)
    row = (rng.standard_normal(16) * 3).astype(np.float32)
    bits = (row.view(np.uint32) >> 16).astype(np.uint32) << 16
    want = _softmax(bits.view(np.float32), 0.8)
    assert np.abs(draw_law(row, 0.8, dtype="bf16") - want).max() < 1e-5


def test_single_token_vocabulary_draws_it():
    o = oracle.draft(np.zeros((3, 2, 4, 1), np.float32), np.ones(3, np.float32),
                     np.random.default_rng(0).random((3, 2, 4)).astype(np.float32))
    assert (o["tokens"] == 0).all() and (o["flags"] == 0).all()


def test_draws_use_only_their_own_uniform():
    """Rows that depend on the position only (every draft the same): a draw must
    not move when any other draw's uniform does -- independence of the K blocks
    and of their positions."""
    rng = np.random.default_rng(5)
    B, K, L, V = 64, 4, 3, 11
    rows = rng.standard_normal((L, V)).astype(np.float32) * 2
    d = np.broadcast_to(rows[None, None], (B, K, L, V)).copy()
    T = np.full(B, 0.9, np.float32)
    u = rng.random((B, K, L)).astype(np.float32)
    base = oracle.draft(d, T, u)["tokens"]
    for trial in range(6):
        u2 = rng.random((B, K, L)).astype(np.float32)
        keep = rng.random((B, K, L)) < 0.5
        u3 = np.where(keep, u, u2).astype(np.float32)
        t3 = oracle.draft(d, T, u3)["tokens"]
        assert (t3[keep] == base[keep]).all()
    # and each draw's marginal is the row's softmax (chi-square over all draws)
    from scipy.stats import chi2
    big = oracle.draft(np.broadcast_to(rows[None, None], (4000, K, L, V)).copy(),
                       np.full(4000, 0.9, np.float32),
                       rng.random((4000, K, L)).astype(np.float32))["tokens"]
    for j in range(L):
        q = _softmax(rows[j], 0.9)
        obs = np.bincount(big[:, :, j].ravel(), minlength=V)
        exp_ = q * obs.sum()
        stat = ((obs - exp_) ** 2 / exp_).sum()
        assert chi2.sf(stat, V - 1) > 1e-4


def test_drafts_meeting_at_a_node_read_its_row_only():
    """Rows of a draft whose prefix a lower-index draft shares are never read:
    filling them with NaN changes nothing."""
    rng = np.random.default_rng(7)
    B, K, L, V = 300, 4, 3, 3
    d = rng.standard_normal((B, K, L, V)).astype(np.float32)
    T = np.full(B, 1.2, np.float32)
    u = rng.random((B, K, L)).astype(np.float32)
    a = oracle.draft(d, T, u)
    tok = a["tokens"]
    d2 = d.copy()
    n_dup = 0
    for b in range(B):
        for k in range(1, K):
            for j in range(L):
                if any((tok[b, c, :j] == tok[b, k, :j]).all() for c in range(k)):
                    d2[b, k, j] = np.nan
                    n_dup += 1
    assert n_dup > 0.3 * B * (K - 1) * L
    b2 = oracle.draft(d2, T, u)
    assert (b2["tokens"] == tok).all() and (b2["flags"] == 0).all()
    assert (b2["rows"] == a["rows"]).all()


def test_drafts_at_different_nodes_read_their_own_rows():
    """Row 1 of draft 0 puts all mass on token 0, row 1 of draft 1 on token 1:
    draft 1's second token is 1 exactly when its first token differs from
    draft 0's, else 0."""
    rng = np.random.default_rng(9)
    B = 400
    d = np.zeros((B, 2, 2, 2), np.float32)
    d[:, 0, 1] = [0.0, -np.inf]
    d[:, 1, 1] = [-np.inf, 0.0]
    o = oracle.draft(d, np.ones(B, np.float32), rng.random((B, 2, 2)).astype(np.float32))
    t = o["tokens"]
    assert (t[:, 0, 1] == 0).all()
    assert (t[:, 1, 1] == (t[:, 1, 0] != t[:, 0, 0])).all()
    assert 0.3 * B < (t[:, 1, 0] != t[:, 0, 0]).sum() < 0.7 * B


def test_invalid_requests_are_flagged():
    rng = np.random.default_rng(11)
    B, K, L, V = 6, 2, 2, 4
    d = rng.standard_normal((B, K, L, V)).astype(np.float32)
    T = np.ones(B, np.float32)
    u = rng.random((B, K, L)).astype(np.float32) * 0.9
    T[0] = 0.0                       # T must be > 0
    u[1, 1, 0] = 1.0                 # u must be < 1
    d[2, 0, 0, 1] = np.nan           # the root row is always read
    d[3, 0, 1] = -np.inf             # node (x) of draft 0 at position 1: always read
    u[4, 0, 0] = 0.05                # draft 1 draws the same first token ...
    u[4, 1, 0] = 0.05
    d[4, 1, 1] = np.nan              # ... so its own row 1 is never read: valid
    o = oracle.draft(d, T, u)
    assert (o["flags"][:4] == oracle.FLAG_INVALID).all()
    assert (o["tokens"][:4] == -1).all()
    assert (o["flags"][4:] == 0).all() and (o["tokens"][4:] >= 0).all()


def test_golden_draft_examples():
    with open(os.path.join(HERE, "golden", "draft_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        u = np.array(e["u_draft"], np.float32)
        B = u.shape[0]
        probs = np.array(e["draft_probs"], np.float64)
        d = np.broadcast_to(np.log(probs).astype(np.float32)[None], (B,) + probs.shape).copy()
        o = oracle.draft(d, np.full(B, e["T"], np.float32), u)
        assert (o["tokens"] == np.array(e["expect"])).all(), (e["name"], o["tokens"])
        assert (o["margin"] > 0.01).all(), e["name"]


# ------------------------------------------------------------- planted mistakes

DRAFT_MUTANTS = {
    # every draft draws with draft 0's uniform: blocks no longer independent
    "draft_shared_uniform": ("r.uc = (double)u[k * L + j];", "r.uc = (double)u[j];"),
    # the temperature is ignored
    "draft_temperature_ignored": ("r.T = (double)temperature[b];\\n        r.q = q;",
                                  "r.T = 1.0;\\n        r.q = q;"),
    # a draft always reads its own row, also at a node a lower draft reached
    "draft_own_row": ("            if (r->X[c * r->L + i] != r->X[k * r->L + i]) { same = 0; break; }",
                      "            { same = 0; break; }"),
    # uniforms indexed position-major
    "draft_transposed_uniform": ("r.uc = (double)u[k * L + j];", "r.uc = (double)u[j * K + k];"),
}


@pytest.fixture(scope="module")
def draft_mutants(tmp_path_factory):
    d = tmp_path_factory.mktemp("draft_mutants")
    src = open(oracle.SRC).read()
    libs = {}
    for name, (old, new) in DRAFT_MUTANTS.items():
        old, new = old.replace("\\n", "\n"), new.replace("\\n", "\n")
        assert src.count(old) == 1, name
        p = d / f"{name}.c"
        p.write_text(src.replace(old, new))
        so = d / f"{name}.so"
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC",
                               "-shared", "-o", str(so), str(p), "-lm"])
        libs[name] = str(so)
    return libs


@pytest.mark.parametrize("name", sorted(DRAFT_MUTANTS))
def test_planted_draft_mistake_fails_a_pin(draft_mutants, name):
    lib = draft_mutants[name]
    failures = 0
    # the softmax law at T != 1
    row = np.array([0.0, -1.0, 0.5, -2.0, 1.0], np.float32)
    if np.abs(draw_law(row, 0.5, lib_path=lib) - _softmax(row, 0.5)).max() > 1e-5:
        failures += 1
    # independence of draws
    rng = np.random.default_rng(5)
    B, K, L, V = 64, 3, 2, 7
    rows = rng.standard_normal((L, V)).astype(np.float32)
    d = np.broadcast_to(rows[None, None], (B, K, L, V)).copy()
    T = np.ones(B, np.float32)
    u = rng.random((B, K, L)).astype(np.float32)
    base = oracle.draft(d, T, u, lib_path=lib)["tokens"]
    u2 = u.copy()
    u2[:, 1:] = rng.random((B, K - 1, L)).astype(np.float32)
    if (oracle.draft(d, T, u2, lib_path=lib)["tokens"][:, 0] != base[:, 0]).any():
        failures += 1
    # node rows: NaN in rows a lower draft's node covers must not matter
    d3 = rng.standard_normal((200, 3, 2, 2)).astype(np.float32)
    u3 = rng.random((200, 3, 2)).astype(np.float32)
    t3 = oracle.draft(d3, np.ones(200, np.float32), u3, lib_path=lib)["tokens"]
    d4 = d3.copy()
    for b in range(200):
        for k in range(1, 3):
            if any(t3[b, c, 0] == t3[b, k, 0] for c in range(k)):
                d4[b, k, 1] = np.nan
    o4 = oracle.draft(d4, np.ones(200, np.float32), u3, lib_path=lib)
    if (o4["tokens"] != t3).any() or o4["flags"].any():
        failures += 1
    # golden draws
    with open(os.path.join(HERE, "golden", "draft_examples.json")) as f:
        for e in json.load(f)["examples"]:
            uu = np.array(e["u_draft"], np.float32)
            probs = np.array(e["draft_probs"], np.float64)
            dd = np.broadcast_to(np.log(probs).astype(np.float32)[None], (uu.shape[0],) + probs.shape).copy()
            got = oracle.draft(dd, np.full(uu.shape[0], e["T"], np.float32), uu, lib_path=lib)["tokens"]
            if (got != np.array(e["expect"])).any():
                failures += 1
                break
    assert failures > 0, name
