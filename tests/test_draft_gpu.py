"""GPU parity of the drafting kernel (spec_draft_sample) against the CPU oracle.

Tokens must be identical, except in requests whose oracle decision log holds a
draw within 1e-6 (probability units) of a CDF boundary; those are counted.
Invalid requests must be flagged the same way, and the rows each valid request
read must agree.
"""
import numpy as np
import pytest
import torch

import oracle
import paritytools as pt
import synth
from draft_token_verification_online_amd import Drafter, Verifier

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _draft(d, temps, u):
    B, K, L, V = d.shape
    out = Drafter(B, K, L, V, d.dtype)(d, temps, u)
    torch.cuda.synchronize()
    return {k: v.clone() for k, v in out.items()}


def _host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _parity(d, temps, u, label, requests=None):
    print(f"[case] draft {label} shape={tuple(d.shape)} dtype={d.dtype}", flush=True)
    g = _draft(d, temps, u)
    B = d.shape[0]
    req = list(range(B)) if requests is None else list(requests)
    ref = oracle.draft(_host(d[req]), _host(temps[req]), _host(u[req]),
                       threads=pt.host_threads())
    gt = g["draft_tokens"].cpu().numpy()[req]
    gf = g["flags"].cpu().numpy()[req]
    gr = g["rows_streamed"].cpu().numpy()[req]
    excused, bad = 0, []
    for i in range(len(req)):
        if ref["flags"][i]:
            if not (gf[i] == ref["flags"][i] and (gt[i] == -1).all()):
                bad.append((req[i], "invalid"))
            continue
        if gf[i] != 0 or gr[i] != ref["rows"][i]:
            if ref["margin"][i] < pt.TIE_BAND:
                excused += 1
            else:
                bad.append((req[i], "flags/rows", int(gf[i]), int(gr[i]), int(ref["rows"][i])))
            continue
        if not (gt[i] == ref["tokens"][i]).all():
            if ref["margin"][i] < pt.TIE_BAND:
                excused += 1
            else:
                bad.append((req[i], "tokens", float(ref["margin"][i])))
    print(f"[parity] draft {label}: n={len(req)} excused={excused} "
          f"invalid={int((ref['flags'] != 0).sum())}", flush=True)
    assert not bad, f"{label}: {len(bad)} mismatches, first {bad[:3]}"
    return g, ref


def _inputs(w, seed):
    batch = pt.gpu_batch(w, seed)
    u = synth.draft_uniforms(w, seed, device="cuda")
    return batch["draft"], batch["temperature"], u


SMALL = [
    ("fp32_k1_l4_v32", W["tiny_fp32_b1_k1_l4_v32"], dict(B=64)),
    ("bf16_k1_v4099_scalar", W["gbv_bf16_b64_k1_l5_v32000"], dict(B=32, V=4099)),
    ("bf16_k4_v12296", W["multi_bf16_b256_k4_l4_v128256"], dict(B=48, V=12296)),
    ("bf16_k8_l8_v9000", W["multi_zipf_bf16_b512_k8_l8_v151936"], dict(B=32, V=9000)),
    ("bf16_mixedT_k4_l8_v5003", W["multi_mixedT_bf16_b1024_k4_l8_v151936"], dict(B=40, V=5003)),
    ("fp32_k3_v777", W["multi_bf16_b256_k4_l4_v128256"], dict(B=40, K=3, V=777, dtype=torch.float32)),
    # drafts close together at low T: many drafts share prefixes
    ("bf16_shared_k8_l8_v6000", W["multi_zipf_bf16_b512_k8_l8_v151936"],
     dict(B=48, V=6000, temperature=0.25)),
    # the widest one-launch draw (K = 16) with prefixes shared to deep positions
    ("bf16_shared_k16_l8_v3000", W["multi_zipf_bf16_b512_k8_l8_v151936"],
     dict(B=32, K=16, V=3000, temperature=0.1)),
]


@pytest.mark.parametrize("name,w,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(name, w, over):
    ws = synth.scaled(w, **over)
    for seed in (1, 2):
        g, ref = _parity(*_inputs(ws, seed), f"{name}/seed{seed}")
        if "shared" in name:   # the case is only worth its name if drafts do meet at nodes
            # at j = 0 every draft stands on the root, so without any sharing below
            # it a request reads 1 + K (L - 1) node rows; fewer means deeper nodes met
            assert int(g["rows_streamed"].sum()) < ws.B * (1 + ws.K * (ws.L - 1))
            # and the oracle's tokens put two drafts on one node at depth >= 2
            tok = ref["tokens"]
            deep = sum(len({tuple(tok[b, k, :j]) for k in range(ws.K)}) < ws.K
                       for b in range(ws.B) for j in range(2, ws.L))
            assert deep > 0, "no node at depth >= 2 is shared"


def test_temperatures():
    for T in (0.1, 0.4, 0.7, 1.5):
        ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=32, V=4096, temperature=T)
        _parity(*_inputs(ws, 3), f"T{T}")


def test_single_token_vocabulary():
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=8, V=1)
    g, _ = _parity(*_inputs(ws, 4), "V1")
    assert (g["draft_tokens"] == 0).all()


@pytest.mark.parametrize("K", [16, 17])
def test_draws_and_listing_in_one_launch_or_two(K):
    """K <= 16: one workgroup per request draws position j and lists the node
    rows of position j + 1; K = 17 takes a launch for each."""
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=24, K=K, L=5, V=3000,
                      temperature=0.5)
    _parity(*_inputs(ws, 6), f"K{K}")


def test_largest_k_and_l():
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=6, K=64, L=16, V=96, temperature=1.5)
    _parity(*_inputs(ws, 5), "K64_L16")


def test_invalid_requests_are_flagged():
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=8, V=1024)
    d, temps, u = _inputs(ws, 6)
    temps[0] = 0.0                          # T must be > 0
    u[1, 2, 1] = 1.0                        # u must be < 1
    d[2, 0, 0, 5] = float("nan")            # the root row is always read
    d[3, 0, 0] = float("-inf")              # a root row of zero mass
    u[4, 3, 3] = -0.5
    g, ref = _parity(d, temps, u, "invalid")
    assert (g["flags"][:5].cpu() == oracle.FLAG_INVALID).all()
    assert (g["draft_tokens"][:5] == -1).all()
    assert (g["flags"][5:].cpu() == 0).all()


def test_negative_infinity_entries():
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=24, V=4096)
    d, temps, u = _inputs(ws, 7)
    gen = torch.Generator(device="cuda").manual_seed(7)
    d.masked_fill_(torch.rand(d.shape, generator=gen, device="cuda") < 0.4, float("-inf"))
    g, _ = _parity(d, temps, u, "neg_inf_entries")
    # never a token of probability zero under the node row it was drawn from
    tok = g["draft_tokens"].cpu().numpy()
    dh = d.float().cpu().numpy()
    B, K, L, _ = d.shape
    for b in range(B):
        for k in range(K):
            for j in range(L):
                c = next(c for c in range(k + 1) if (tok[b, c, :j] == tok[b, k, :j]).all())
                assert np.isfinite(dh[b, c, j, tok[b, k, j]]), (b, k, j)


def test_rows_of_shared_nodes_are_never_read():
    ws = synth.scaled(W["multi_zipf_bf16_b512_k8_l8_v151936"], B=16, V=2048, temperature=0.3)
    d, temps, u = _inputs(ws, 8)
    a = _draft(d, temps, u)
    tok = a["draft_tokens"].cpu().numpy()
    B, K, L, _ = d.shape
    n = 0
    for b in range(B):
        for k in range(1, K):
            for j in range(L):
                if any((tok[b, c, :j] == tok[b, k, :j]).all() for c in range(k)):
                    d[b, k, j] = float("nan")
                    n += 1
    assert n > 0
    b2 = _draft(d, temps, u)
    for key in ("draft_tokens", "flags", "rows_streamed"):
        assert torch.equal(a[key], b2[key]), key


def test_misaligned_rows_take_the_scalar_path():
    ws = synth.scaled(W["gbv_bf16_b64_k1_l5_v32000"], B=16, V=2048)
    d, temps, u = _inputs(ws, 9)
    buf = torch.empty(d.numel() + 1, dtype=d.dtype, device="cuda")
    view = buf[1:].view(d.shape)
    view.copy_(d)
    _parity(view, temps, u, "misaligned")


def test_draft_then_verify_end_to_end():
    """Drafts drawn on the GPU and verified on the GPU, against the oracle drawing
    and verifying its own drafts from the same logits and uniforms; compared on
    the requests whose draws agree (all but ties)."""
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=32, V=8192)
    batch = pt.gpu_batch(ws, 10)
    u = synth.draft_uniforms(ws, 10, device="cuda")
    g = _draft(batch["draft"], batch["temperature"], u)
    ref = oracle.draft(_host(batch["draft"]), _host(batch["temperature"]), _host(u))
    gt = g["draft_tokens"].cpu().numpy()
    ok = (ref["margin"] >= pt.TIE_BAND) & (gt == ref["tokens"]).all(axis=(1, 2))
    assert (ok | (ref["margin"] < pt.TIE_BAND)).all()
    req = [b for b in range(ws.B) if ok[b]]
    host = synth.to_host(batch, req)
    host["tokens"] = ref["tokens"][req]          # the oracle verifies its own draws
    batch["tokens"] = g["draft_tokens"].contiguous()
    for method in ("multidraft", "spectr"):
        B, K, L1, V = batch["target"].shape
        v = Verifier(method, B, K, L1 - 1, V, batch["target"].dtype, diagnostics=True)
        out = v(batch["target"], batch["draft"], batch["tokens"], batch["temperature"],
                batch["u_accept"], batch["u_correct"])
        torch.cuda.synchronize()
        r = pt.run_oracle(method, host)
        pt.check(pt.compare(method, out, r, req, label=f"draft+{method}"))


FULL = ["multi_bf16_b256_k4_l4_v128256", "multi_zipf_bf16_b512_k8_l8_v151936",
        "multi_mixedT_bf16_b1024_k4_l8_v151936"]


@pytest.mark.parametrize("seed,n", [(1234, 24), (4321, 64)], ids=["seed1234", "seed4321"])
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name, seed, n):
    w = W[name]
    d, temps, u = _inputs(w, seed)
    rng = np.random.default_rng(seed + 1)
    req = sorted(rng.choice(w.B, size=min(w.B, n), replace=False).tolist())
    _parity(d, temps, u, f"full/{name}/seed{seed}", requests=req)
    del d
    torch.cuda.empty_cache()
