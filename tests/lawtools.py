"""Exact-law tools for pinning the CPU oracle on tiny instances.

A tiny instance is a full *tree model*: target logits for every prefix of
length 0..L and draft logits for every prefix of length 0..L-1, over V tokens.
The tools below

  * compute the target law of sequences and the closed forms the mathematics
    gives (expected accepted length of token-level SD and of GBV, the L = 1
    recursive-rejection formula, the K-draft upper bound), directly from the
    tree model and independently of the oracle;
  * enumerate the oracle's *output law* exactly, treating the oracle as a black
    box: every draft realisation (K drafts in V^L) is weighted by its draft
    probability, every acceptance decision the oracle reports (its evaluated h)
    is branched on by feeding it the float64 uniforms 0 and h, and the
    correction token's law is the distribution the oracle reports drawing it
    from (pinned against its draws by bisecting the correction uniform).

Nothing here imports or re-implements the oracle's walk; only the model's
softmax (the definition of p and q) is computed in the test.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

import oracle

F32_ONE_BITS = np.float32(1.0).view(np.uint32)


# ------------------------------------------------------------------ models

class TreeModel:
    """Target / draft logits for every node of a depth-L tree over V tokens."""

    def __init__(self, V, L, T, tgt, drf):
        # the verifier receives T as float32; the model uses that same value
        self.V, self.L, self.T = V, L, float(np.float32(T))
        self.tgt = tgt      # dict prefix -> float32[V], prefixes of length 0..L
        self.drf = drf      # dict prefix -> float32[V], prefixes of length 0..L-1

    @staticmethod
    def random(V, L, rng, T=1.0, sigma=1.5, zero_frac=0.0, draft_mode="noisy",
               draft_sigma=1.0):
        def row(base=None):
            if base is None:
                r = (rng.standard_normal(V) * sigma).astype(np.float32)
            else:
                r = (base + rng.standard_normal(V) * draft_sigma).astype(np.float32)
            if zero_frac:
                z = rng.random(V) < zero_frac
                if z.all():
                    z[rng.integers(V)] = False
                r[z] = -np.inf
            return r
        tgt, drf = {}, {}
        for d in range(L + 1):
            for pre in itertools.product(range(V), repeat=d):
                tgt[pre] = row()
                if d < L:
                    if draft_mode == "noisy":
                        base = np.where(np.isfinite(tgt[pre]), tgt[pre], 0.0)
                        drf[pre] = row(base)
                    elif draft_mode == "equal":
                        drf[pre] = tgt[pre].copy()
                    else:
                        drf[pre] = row()
        return TreeModel(V, L, T, tgt, drf)

    # definition of the temperature softmax, in float64
    def _soft(self, logits):
        l = logits.astype(np.float64)
        m = l.max()
        e = np.exp((l - m) / self.T)
        return e / e.sum()

    def p(self, pre):
        return self._soft(self.tgt[tuple(pre)])

    def q(self, pre):
        return self._soft(self.drf[tuple(pre)])

    def p_seq(self, z):
        out = 1.0
        for i, t in enumerate(z):
            out *= self.p(z[:i])[t]
        return out

    def q_seq(self, z):
        out = 1.0
        for i, t in enumerate(z):
            out *= self.q(z[:i])[t]
        return out


# ------------------------------------------------------------- closed forms

def expected_tau_token(m: TreeModel, L=None):
    """E[tau] of standard speculative sampling: sum over i of
    E_q[prod_{j<i} min(1, p_j(x_j)/q_j(x_j))]."""
    L = m.L if L is None else L
    tot = 0.0
    for i in range(1, L + 1):
        for z in itertools.product(range(m.V), repeat=i):
            qz = m.q_seq(z)
            if qz == 0:
                continue
            a = 1.0
            for j in range(i):
                pj, qj = m.p(z[:j])[z[j]], m.q(z[:j])[z[j]]
                a *= min(1.0, pj / qj)
            tot += qz * a
    return tot


def gbv_weights(m: TreeModel, z):
    """GBV's chain w_i = min(w_{i-1} p(z_i)/q(z_i), 1) along z."""
    w = [1.0]
    for j in range(len(z)):
        pj, qj = m.p(z[:j])[z[j]], m.q(z[:j])[z[j]]
        w.append(min(w[-1] * pj / qj, 1.0))
    return w


def expected_tau_gbv(m: TreeModel, L=None):
    """E[tau] of block verification = sum_i E_q[w_i] (P(tau >= i) = E_q[w_i])."""
    L = m.L if L is None else L
    tot = 0.0
    for z in itertools.product(range(m.V), repeat=L):
        qz = m.q_seq(z)
        if qz == 0:
            continue
        tot += qz * sum(gbv_weights(m, z)[1:])
    return tot


def expected_tau_rrs_l1(m: TreeModel, K):
    """L = 1, K i.i.d. drafts, recursive rejection sampling: the chance that all K
    are rejected is prod_k TV(r_{k-1}, q) with r_0 = p and
    r_k = norm(max(r_{k-1} - q, 0))."""
    p, q = m.p(()), m.q(())
    r = p.copy()
    rej = 1.0
    for _ in range(K):
        res = np.maximum(r - q, 0.0)
        tv = res.sum()
        rej *= tv
        if tv <= 0:
            break
        r = res / tv
    return 1.0 - rej


def expected_tau_bound(m: TreeModel, K):
    """Upper bound for any K-draft verifier that keeps the target law:
    P(tau >= i, prefix = x^i) <= min(p(x^i), P(some draft starts with x^i))."""
    tot = 0.0
    for i in range(1, m.L + 1):
        for z in itertools.product(range(m.V), repeat=i):
            tot += min(m.p_seq(z), 1.0 - (1.0 - m.q_seq(z)) ** K)
    return tot


# ----------------------------------------------------------- realisations

def realisations(m: TreeModel, K):
    """All K-tuples of draft blocks with positive draft probability, with the
    rows each request carries (node rows for every draft position)."""
    seqs = [z for z in itertools.product(range(m.V), repeat=m.L) if m.q_seq(z) > 0]
    qs = {z: m.q_seq(z) for z in seqs}
    combos = list(itertools.product(seqs, repeat=K))
    R = len(combos)
    V, L = m.V, m.L
    tgt = np.empty((R, K, L + 1, V), np.float32)
    drf = np.empty((R, K, L, V), np.float32)
    tok = np.empty((R, K, L), np.int32)
    wq = np.empty(R, np.float64)
    for r, combo in enumerate(combos):
        w = 1.0
        for k, z in enumerate(combo):
            w *= qs[z]
            tok[r, k] = z
            for j in range(L + 1):
                tgt[r, k, j] = m.tgt[z[:j]]
            for j in range(L):
                drf[r, k, j] = m.drf[z[:j]]
        wq[r] = w
    return tgt, drf, tok, wq


def _f32(x):
    return np.float32(x)


def _walk_order(method, K, L):
    """Order in which the rules take their decisions: token level tests
    positions forward; SpecTr tests position by position, drafts in order;
    block walks test each draft's positions backward."""
    if method == "token":
        return [(0, j) for j in range(L)]
    if method == "spectr":
        return [(k, j) for j in range(L) for k in range(K)]
    return [(k, m - 1) for k in range(K) for m in range(L, 0, -1)]


def output_law(m: TreeModel, K, method, lib_path=None, max_paths=4000000):
    """Exact law of the oracle's output (accepted prefix + correction token),
    marginalised over draft realisations and uniforms.

    The oracle is driven through its float64-uniform entry point: every
    acceptance decision it reports (its evaluated h) is branched on with u = 0
    (accept, probability h) and u = h (reject, probability 1 - h, since a test
    accepts iff u < h), and the correction token's law at each leaf is the
    distribution the oracle reports drawing it from.  The only error is fp64
    rounding.

    Returns (law, e_tau, dropped): law maps output tuples (prefix + (y,)) to
    probabilities, e_tau is E[accept_len]; dropped (branches no uniform can
    reach) is 0 here and kept for the callers' assertions."""
    L, V = m.L, m.V
    tgt, drf, tok, wq = realisations(m, K)
    R = len(wq)
    temps = np.full(1, m.T, np.float32)
    order = _walk_order(method, K, L)
    flat_order = np.array([k * L + j for k, j in order])

    ridx = np.arange(R)
    ua = np.full((R, K, L), 0.5, np.float64)   # placeholders until a test is branched on
    fixed = np.zeros((R, K, L), bool)
    prob = np.ones(R)
    leaves = []

    def run(ri, u):
        P = len(ri)
        return oracle.verify_exact(method, tgt[ri], drf[ri], tok[ri], np.repeat(temps, P),
                                   u, np.zeros(P), lib_path=lib_path)

    while len(ridx):
        if len(ridx) > max_paths:
            raise RuntimeError("too many paths")
        out = run(ridx, ua)
        if (out["flags"] & oracle.FLAG_INVALID).any():
            raise AssertionError("oracle flagged a valid tiny instance as invalid")
        h = out["accept_prob"].reshape(len(ridx), K * L)
        pending = (~np.isnan(h) & ~fixed.reshape(len(ridx), K * L))[:, flat_order]
        has = pending.any(axis=1)
        done = ~has
        if done.any():
            leaves.append((ridx[done], prob[done], out["accept_len"][done],
                           out["draft_index"][done], out["corr_law"][done]))
        if not has.any():
            break
        sel = np.nonzero(has)[0]
        first = flat_order[np.argmax(pending[sel], axis=1)]
        hs = h[sel, first]
        k_, j_ = np.divmod(first, L)
        acc = hs > 0.0
        rej = hs < 1.0
        ua_sel, fx_sel = ua[sel], fixed[sel]
        fx_sel[np.arange(len(sel)), k_, j_] = True
        ua_a = ua_sel[acc].copy()
        ua_a[np.arange(acc.sum()), k_[acc], j_[acc]] = 0.0
        ua_r = ua_sel[rej].copy()
        ua_r[np.arange(rej.sum()), k_[rej], j_[rej]] = hs[rej]
        ridx = np.concatenate([ridx[sel][acc], ridx[sel][rej]])
        ua = np.concatenate([ua_a, ua_r])
        fixed = np.concatenate([fx_sel[acc], fx_sel[rej]])
        prob = np.concatenate([prob[sel][acc] * np.minimum(hs[acc], 1.0),
                               prob[sel][rej] * (1.0 - hs[rej])])

    lr = np.concatenate([x[0] for x in leaves])
    lp = np.concatenate([x[1] for x in leaves])
    ltau = np.concatenate([x[2] for x in leaves])
    lks = np.concatenate([x[3] for x in leaves])
    py = np.concatenate([x[4] for x in leaves])   # [leaves][V]

    law = {}
    w = wq[lr] * lp
    e_tau = float(np.dot(w, ltau))
    for n in range(len(lr)):
        tau, ks = int(ltau[n]), int(lks[n])
        pre = tuple(int(t) for t in tok[lr[n], ks, :tau]) if tau > 0 else ()
        for y in np.nonzero(py[n] > 0)[0]:
            key = pre + (int(y),)
            law[key] = law.get(key, 0.0) + w[n] * py[n, y]
    return law, e_tau, 0.0


def correction_law(run, lr, lu, V):
    """Law of the correction token at each leaf, read off by bisection over the
    float32 correction uniform (the draw is non-decreasing in u).  Used to pin
    the law the oracle reports against the draws it makes."""
    n = len(lr)
    if V == 1:
        return np.ones((n, 1))
    reps = V - 1
    rr = np.repeat(lr, reps)
    uu = np.repeat(lu, reps, axis=0)
    target_v = np.tile(np.arange(1, V), n)
    lo = np.zeros(n * reps, np.int64)                    # bits of a u with y(u) < v
    hi = np.full(n * reps, int(F32_ONE_BITS), np.int64)  # bits of a u with y(u) >= v (1.0 = none)
    y0 = run(rr, uu, np.zeros(n * reps, np.float32))["correction"]
    at_zero = y0 >= target_v
    for _ in range(32):
        active = (hi - lo > 1) & ~at_zero
        if not active.any():
            break
        mid = (lo + hi) // 2
        u = mid.astype(np.uint32).view(np.float32)
        y = run(rr, uu, u)["correction"]
        up = y >= target_v
        hi = np.where(active & up, mid, hi)
        lo = np.where(active & ~up, mid, lo)
    bnd = hi.astype(np.uint32).view(np.float32).astype(np.float64)
    bnd = np.where(at_zero, 0.0, bnd).reshape(n, reps)
    edges = np.concatenate([np.zeros((n, 1)), bnd, np.ones((n, 1))], axis=1)
    return np.diff(edges, axis=1)


def extended_law_gap(m: TreeModel, law):
    """Largest |P(output extended by the target to length L+1 = z) - p(z)| over z."""
    worst = 0.0
    for z in itertools.product(range(m.V), repeat=m.L + 1):
        lhs = 0.0
        for t in range(m.L + 1):
            pz = law.get(z[:t + 1], 0.0)
            if pz:
                ext = 1.0
                for i in range(t + 1, m.L + 1):
                    ext *= m.p(z[:i])[z[i]]
                lhs += pz * ext
        worst = max(worst, abs(lhs - m.p_seq(z)))
    return worst


def isclose(a, b, tol):
    return math.isfinite(a) and math.isfinite(b) and abs(a - b) <= tol
