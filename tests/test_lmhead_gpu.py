"""GPU parity of the fused LM head (spec_lm_head) against the oracle's float64
matrix product, and of verification fed by its statistics.

Tolerances come from the arithmetic: every bf16 x bf16 product is exact in fp32
and each of the at most d/32 + 32 fp32 additions that form a logit rounds once,
so |logit - exact| <= (d/32 + 34) 2^-24 sum_i |h_i w_i| (a bound per element,
computed here in float64).  A row's log-partition function moves by at most the
largest logit error over T, plus the fp32 exponentials (< 1e-6 relative).
"""
import numpy as np
import pytest
import torch

import oracle
import paritytools as pt
from draft_token_verification_online_amd import LmHead, Verifier

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _make(R, d, V, seed, scale=4.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    h = torch.randn((R, d), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((V, d), generator=g, device="cuda") * (scale / d ** 0.5)).to(torch.bfloat16)
    return h, w


def _bound(hb, wb):
    d = hb.shape[1]
    a = np.abs(oracle.bf16_bits_to_f64(hb)) @ np.abs(oracle.bf16_bits_to_f64(wb)).T
    return (d / 32 + 34) * 2.0 ** -24 * a


def _stats_lse(buf, rows, temps):
    raw = buf.cpu().numpy()
    shift = raw.view(np.float32).reshape(-1, 4)[:rows, 0].astype(np.float64)
    ssum = raw.view(np.float64).reshape(-1, 2)[:rows, 1]
    return shift / temps + np.log(ssum)


@pytest.mark.parametrize("R,d,V,T", [(1, 128, 1, 1.0), (130, 192, 1000, 0.7), (257, 128, 4099, 0.4),
                                     (300, 896, 8192, 1.0), (128, 3584, 2048, 0.25)])
def test_logits_and_statistics(R, d, V, T):
    print(f"[case] lm_head R={R} d={d} V={V} T={T}", flush=True)
    h, w = _make(R, d, V, 100 + R)
    temps = torch.full((R,), T, device="cuda") * (1 + 0.5 * (torch.arange(R, device="cuda") % 3))
    stats = torch.zeros(R * 16, dtype=torch.uint8, device="cuda")
    lm = LmHead(R, d, V)
    logits = lm(h, w, temps, stats=stats)
    torch.cuda.synchronize()
    hb, wb, tt = _bits(h), _bits(w), temps.cpu().numpy().astype(np.float64)
    ref, lse = oracle.lm_head(hb, wb, tt)
    bound = _bound(hb, wb)
    err = np.abs(logits.cpu().numpy().astype(np.float64) - ref)
    assert (err <= bound).all(), float((err / np.maximum(bound, 1e-300)).max())
    got = _stats_lse(stats, R, tt)
    tol = bound.max(axis=1) / tt + 1e-6 * np.maximum(1.0, np.abs(lse))
    assert (np.abs(got - lse) <= tol).all(), float(np.abs(got - lse).max())
    print(f"[parity] lm_head R={R} d={d} V={V}: max logit err {err.max():.2e} "
          f"(bound {bound.max():.2e}), max lse err {np.abs(got - lse).max():.2e}", flush=True)


@pytest.mark.parametrize("method", ["multidraft", "spectr"])
def test_lm_head_statistics_feed_verification(method):
    """Target and draft LM heads write fp32 logits and their statistics straight
    into the verifier's [B][K][2L+1] layout; verification skips its statistics
    pass.  The oracle does the same from its float64 logits (rounded to fp32).
    Decisions are compared except where a threshold lies within the logits' own
    error band of the oracle's value."""
    B, K, L, V, d = 12, 4, 4, 4096, 256
    print(f"[case] lm_head->verify {method} B={B} K={K} L={L} V={V} d={d}", flush=True)
    ht, wt = _make(B * K * (L + 1), d, V, 7)
    g = torch.Generator(device="cuda").manual_seed(8)
    hd = (ht.view(B, K, L + 1, d)[:, :, :L].float()
          + 0.5 * torch.randn((B, K, L, d), generator=g, device="cuda")).to(torch.bfloat16)
    hd = hd.reshape(B * K * L, d).contiguous()
    wd = (wt.float() + 0.3 * (4 / d ** 0.5) * torch.randn((V, d), generator=g, device="cuda")
          ).to(torch.bfloat16)
    T = (0.5 + 0.5 * (torch.arange(B, device="cuda") % 3)).float()
    Tt = T.repeat_interleave(K * (L + 1))
    Td = T.repeat_interleave(K * L)
    stats = torch.zeros(B * K * (2 * L + 1) * 16, dtype=torch.uint8, device="cuda")
    lt = LmHead(B * K * (L + 1), d, V)(ht, wt, Tt, stats=stats, group=L + 1, stride=2 * L + 1,
                                       offset=0)
    ld = LmHead(B * K * L, d, V)(hd, wd, Td, stats=stats, group=L, stride=2 * L + 1,
                                 offset=L + 1)
    torch.cuda.synchronize()

    # the oracle's own logits and tokens
    ref_t, _ = oracle.lm_head(_bits(ht), _bits(wt), Tt.cpu().numpy())
    ref_d, _ = oracle.lm_head(_bits(hd), _bits(wd), Td.cpu().numpy())
    bnd = max(_bound(_bits(ht), _bits(wt)).max(), _bound(_bits(hd), _bits(wd)).max())
    tgt32 = ref_t.astype(np.float32).reshape(B, K, L + 1, V)
    drf32 = ref_d.astype(np.float32).reshape(B, K, L, V)
    rng = np.random.default_rng(9)
    Th = T.cpu().numpy()
    tok = oracle.draft(drf32, Th, rng.random((B, K, L)).astype(np.float32))["tokens"]
    ua = rng.random((B, K, L)).astype(np.float32)
    uc = rng.random(B).astype(np.float32)
    ref = oracle.verify(method, tgt32, drf32, tok, Th, ua, uc, diagnostics=True)

    v = Verifier(method, B, K, L, V, torch.float32, diagnostics=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = v(lt.view(B, K, L + 1, V), ld.view(B, K, L, V), dev(tok), T, dev(ua), dev(uc),
            row_stats=stats)
    torch.cuda.synchronize()
    assert (out["rows_streamed"] == 0).all()
    band = 4 * bnd / float(Th.min())          # |dh| from the logit errors, in u units
    excused, bad = 0, []
    for b in range(B):
        same = all(int(out[k][b]) == int(ref[k][b]) for k in ("accept_len", "draft_index",
                                                               "correction"))
        if same:
            continue
        if ref["margin"][b] < band:
            excused += 1
        else:
            bad.append((b, float(ref["margin"][b])))
    lse_err = np.nanmax(np.abs(out["row_lse"].cpu().numpy().astype(np.float64) - ref["row_lse"]))
    print(f"[parity] lm_head->verify {method}: n={B} excused={excused} (band {band:.1e}) "
          f"lse err {lse_err:.2e}", flush=True)
    assert not bad, bad
    assert lse_err <= bnd / float(Th.min()) + 1e-5


@pytest.mark.parametrize("R,d,V,T", [(130, 192, 1000, 0.7), (257, 128, 4099, 0.4),
                                     (128, 3584, 2048, 0.25)])
def test_bf16_logits_and_their_statistics(R, d, V, T):
    """bf16 logits: each is the fp32 accumulation rounded to nearest even, so it
    lies within the accumulation bound plus half a bf16 ulp (2^-8 relative) of
    the exact product; the statistics describe the stored (rounded) values."""
    from scipy.special import logsumexp
    print(f"[case] lm_head bf16 R={R} d={d} V={V} T={T}", flush=True)
    h, w = _make(R, d, V, 300 + R)
    temps = torch.full((R,), T, device="cuda") * (1 + 0.5 * (torch.arange(R, device="cuda") % 3))
    stats = torch.zeros(R * 16, dtype=torch.uint8, device="cuda")
    lm = LmHead(R, d, V, logits_dtype=torch.bfloat16)
    logits = lm(h, w, temps, stats=stats)
    torch.cuda.synchronize()
    hb, wb, tt = _bits(h), _bits(w), temps.cpu().numpy().astype(np.float64)
    ref, _ = oracle.lm_head(hb, wb, tt)
    bound = _bound(hb, wb)
    got = oracle.bf16_bits_to_f64(_bits(logits))
    err = np.abs(got - ref)
    assert (err <= bound + (np.abs(ref) + bound) * 2.0 ** -8).all()
    lse_rounded = logsumexp(got / tt[:, None], axis=1)
    lse_gpu = _stats_lse(stats, R, tt)
    rel = np.abs(lse_gpu - lse_rounded) / np.maximum(1.0, np.abs(lse_rounded))
    assert rel.max() <= 1e-6, rel.max()
    print(f"[parity] lm_head bf16 R={R} d={d} V={V}: max logit err {err.max():.2e}, "
          f"lse of the stored values rel {rel.max():.2e}", flush=True)


@pytest.mark.parametrize("method", ["multidraft", "spectr"])
def test_bf16_lm_head_feeds_verification(method):
    """Target and draft LM heads write bf16 logits and the statistics of those
    rounded values; verification given the statistics (no statistics pass) must
    meet the parity bar against the oracle run on the same bf16 logits."""
    B, K, L, V, d = 12, 4, 4, 4096, 256
    print(f"[case] lm_head bf16->verify {method} B={B} K={K} L={L} V={V} d={d}", flush=True)
    ht, wt = _make(B * K * (L + 1), d, V, 17)
    g = torch.Generator(device="cuda").manual_seed(18)
    hd = (ht.view(B, K, L + 1, d)[:, :, :L].float()
          + 0.5 * torch.randn((B, K, L, d), generator=g, device="cuda")).to(torch.bfloat16)
    hd = hd.reshape(B * K * L, d).contiguous()
    wd = (wt.float() + 0.3 * (4 / d ** 0.5) * torch.randn((V, d), generator=g, device="cuda")
          ).to(torch.bfloat16)
    T = (0.5 + 0.5 * (torch.arange(B, device="cuda") % 3)).float()
    stats = torch.zeros(B * K * (2 * L + 1) * 16, dtype=torch.uint8, device="cuda")
    lt = LmHead(B * K * (L + 1), d, V, logits_dtype=torch.bfloat16)(
        ht, wt, T.repeat_interleave(K * (L + 1)), stats=stats, group=L + 1, stride=2 * L + 1,
        offset=0)
    ld = LmHead(B * K * L, d, V, logits_dtype=torch.bfloat16)(
        hd, wd, T.repeat_interleave(K * L), stats=stats, group=L, stride=2 * L + 1, offset=L + 1)
    torch.cuda.synchronize()
    tgt, drf = lt.view(B, K, L + 1, V), ld.view(B, K, L, V)
    rng = np.random.default_rng(19)
    Th = T.cpu().numpy()
    tok = oracle.draft(_bits(drf).reshape(B, K, L, V), Th,
                       rng.random((B, K, L)).astype(np.float32))["tokens"]
    ua = rng.random((B, K, L)).astype(np.float32)
    uc = rng.random(B).astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    batch = {"target": tgt, "draft": drf, "tokens": dev(tok), "temperature": T,
             "u_accept": dev(ua), "u_correct": dev(uc)}
    v = Verifier(method, B, K, L, V, torch.bfloat16, diagnostics=True)
    out = v(tgt, drf, batch["tokens"], T, batch["u_accept"], batch["u_correct"], row_stats=stats)
    torch.cuda.synchronize()
    assert (out["rows_streamed"] == 0).all()
    ref = pt.run_oracle(method, {"target": _bits(tgt).reshape(B, K, L + 1, V),
                                 "draft": _bits(drf).reshape(B, K, L, V), "tokens": tok,
                                 "temperature": Th, "u_accept": ua, "u_correct": uc})
    pt.check(pt.compare(method, out, ref, list(range(B)), label=f"lm_head_bf16/{method}"))


@pytest.mark.parametrize("ldt", [torch.float32, torch.bfloat16])
def test_lm_head_at_the_bench_target_shape(ldt):
    """The bench's target LM head (36 864 rows, d = 3 584, V = 151 936), in the launch
    configuration bench.py times: sampled rows (first and last of the grid, the
    last row-block, rows in the partial last column block) against the oracle's
    float64 product over the whole vocabulary, and their statistics."""
    from scipy.special import logsumexp
    R, d, V, T = 36864, 3584, 151936, 0.4
    print(f"[case] lm_head bench shape R={R} d={d} V={V} {ldt}", flush=True)
    h, w = _make(R, d, V, 7)
    temps = torch.full((R,), T, device="cuda") * (1 + 0.5 * (torch.arange(R, device="cuda") % 3))
    stats = torch.zeros(R * 16, dtype=torch.uint8, device="cuda")
    lm = LmHead(R, d, V, logits_dtype=ldt)
    logits = lm(h, w, temps, stats=stats)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 18437, R - 257, R - 1])
    hb = _bits(h[torch.as_tensor(rows, device="cuda")])
    wb = _bits(w)
    tt = temps.cpu().numpy().astype(np.float64)[rows]
    ref, lse_ref = oracle.lm_head(hb, wb, tt)
    acc_bound = _bound(hb, wb)
    bound = acc_bound
    got_t = logits[torch.as_tensor(rows, device="cuda")]
    if ldt == torch.bfloat16:
        got = oracle.bf16_bits_to_f64(_bits(got_t))
        bound = bound + (np.abs(ref) + bound) * 2.0 ** -8
        lse_want = logsumexp(got / tt[:, None], axis=1)   # statistics of the stored values
        tol = 1e-6 * np.maximum(1.0, np.abs(lse_want))
    else:
        got = got_t.cpu().numpy().astype(np.float64)
        lse_want = lse_ref
        tol = acc_bound.max(axis=1) / tt + 1e-6 * np.maximum(1.0, np.abs(lse_ref))
    err = np.abs(got - ref)
    assert (err <= bound).all(), float((err / np.maximum(bound, 1e-300)).max())
    raw = stats.view(-1, 16)[torch.as_tensor(rows, device="cuda")].reshape(-1)
    lse_gpu = _stats_lse(raw, len(rows), tt)
    assert (np.abs(lse_gpu - lse_want) <= tol).all(), float(np.abs(lse_gpu - lse_want).max())
    print(f"[parity] lm_head bench shape {ldt}: max logit err {err.max():.2e}, "
          f"max lse err {np.abs(lse_gpu - lse_want).max():.2e}", flush=True)
