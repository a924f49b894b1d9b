"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Integer outputs (accept_len, draft_index, correction) must be bit-identical,
except for requests whose oracle decision log holds a decision within 1e-6 of
its threshold (or a degenerate residual); those are counted and reported.
Diagnostics: row ln-partition functions within 1e-5 relative, acceptance
probabilities within 1e-5 absolute, correction mass within 1e-5 relative.
"""
import numpy as np
import pytest
import torch

import oracle
import paritytools as pt
import synth
from draft_token_verification_online_amd import Verifier

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _verify(method, batch, diagnostics=True):
    t = batch["target"]
    B, K, L1, V = t.shape
    v = Verifier(method, B, K, L1 - 1, V, t.dtype, diagnostics=diagnostics)
    # the workspace's contents need not be initialised: every byte starts as NaN
    # bits, so a value read before this call wrote it shows in the outputs
    v.workspace.fill_(0xFF)
    out = v(batch["target"], batch["draft"], batch["tokens"], batch["temperature"],
            batch["u_accept"], batch["u_correct"])
    torch.cuda.synchronize()
    return out


def _parity(method, batch, label, requests=None, diagnostics=True):
    print(f"[case] {label} method={method} shape={tuple(batch['target'].shape)} "
          f"dtype={batch['target'].dtype}", flush=True)
    out = _verify(method, batch, diagnostics=diagnostics)
    B = batch["target"].shape[0]
    req = list(range(B)) if requests is None else list(requests)
    host = synth.to_host(batch, req)
    ref = pt.run_oracle(method, host, diagnostics=diagnostics)
    rep = pt.compare(method, out, ref, req, diagnostics=diagnostics, label=label)
    pt.check(rep)
    return rep, out, ref


# ---------------------------------------------------------------- small sizes
# Several tiles of the walk (512 threads x 8 elements), ragged tails, the
# scalar path (V not a multiple of 8), every temperature the pages study.

SMALL = [
    # name, workload, overrides
    ("tiny_fp32", W["tiny_fp32_b1_k1_l4_v32"], dict(B=64)),
    ("gbv_bf16_v8200", W["gbv_bf16_b64_k1_l5_v32000"], dict(B=48, V=8200)),
    ("gbv_bf16_v4099_scalar", W["gbv_bf16_b64_k1_l5_v32000"], dict(B=32, V=4099)),
    ("multi_k4_v12296", W["multi_bf16_b256_k4_l4_v128256"], dict(B=48, V=12296)),
    ("multi_zipf_k8_l8_v9000", W["multi_zipf_bf16_b512_k8_l8_v151936"], dict(B=32, V=9000)),
    ("multi_mixedT_k4_l8_v5003", W["multi_mixedT_bf16_b1024_k4_l8_v151936"], dict(B=40, V=5003)),
    ("multi_fp32_k3_v777", W["multi_bf16_b256_k4_l4_v128256"],
     dict(B=40, K=3, V=777, dtype=torch.float32)),
    # drafts close to the target at low T: long accepted prefixes, many drafts
    # sharing them, so the walk computes statistics of rows below accepted nodes
    ("multi_highaccept_k8_l8_v6000", W["multi_zipf_bf16_b512_k8_l8_v151936"],
     dict(B=48, V=6000, sigma_draft=0.3, temperature=0.25)),
]


# Row lengths at the edges of the streaming loops: the statistics kernel (256
# threads) consumes a first tile of 256 chunks and then groups of 8 x 256 bf16
# chunks (4 x 256 fp32); the walk's sweeps (512 threads) groups of 2 x 512 bf16
# chunks; the inverse CDF groups of 4 tiles of 512 chunks.  V = 8 * chunks.
STREAM_EDGES = [
    ("v8184", 8184, torch.bfloat16),     # 1023 chunks: one short of a sweep group
    ("v8192", 8192, torch.bfloat16),     # exactly one sweep group
    ("v16384", 16384, torch.bfloat16),   # two sweep groups, one inverse-CDF group
    ("v16392", 16392, torch.bfloat16),   # and one chunk more
    ("v18424", 18424, torch.bfloat16),   # statistics: first tile + group minus one chunk
    ("v18432", 18432, torch.bfloat16),   # first tile + exactly one group
    ("v18440", 18440, torch.bfloat16),   # and one chunk more
    ("v34816", 34816, torch.bfloat16),   # first tile + two groups
    ("v10240_fp32", 10240, torch.float32),   # first tile + one fp32 group
    ("v10248_fp32", 10248, torch.float32),
]


@pytest.mark.parametrize("name,V,dtype", STREAM_EDGES, ids=[s[0] for s in STREAM_EDGES])
def test_streaming_group_edges(name, V, dtype):
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=16, V=V, dtype=dtype)
    batch = pt.gpu_batch(ws, 3)
    for method in ("multidraft", "spectr"):
        _parity(method, batch, f"edges_{name}")


@pytest.mark.parametrize("name,w,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(name, w, over):
    ws = synth.scaled(w, **over)
    methods = (("token", "block", "spectr") if ws.K == 1
               else ("multidraft", "spectr", "spectr_bisect"))
    for seed in (1, 2):
        batch = pt.gpu_batch(ws, seed)
        for method in methods:
            _parity(method, batch, f"{name}/seed{seed}")


def test_block_equals_multidraft_with_one_draft():
    ws = synth.scaled(W["gbv_bf16_b64_k1_l5_v32000"], B=64, V=3000)
    batch = pt.gpu_batch(ws, 3)
    a = _verify("block", batch)
    b = _verify("multidraft", batch)
    for k in ("accept_len", "draft_index", "correction", "flags"):
        assert torch.equal(a[k], b[k]), k


def test_spectr_equals_token_with_one_draft():
    """One candidate per position: rho* = 1, c = 1, SpecTr is token-level sampling."""
    ws = synth.scaled(W["gbv_bf16_b64_k1_l5_v32000"], B=64, V=3000)
    batch = pt.gpu_batch(ws, 3)
    a = _verify("token", batch)
    b = _verify("spectr", batch)
    for k in ("accept_len", "draft_index", "correction", "flags", "resid_mass"):
        assert torch.equal(a[k].nan_to_num(-7.0), b[k].nan_to_num(-7.0)), k


def test_temperatures_of_the_ablation():
    """T in {0.1, 0.4, 0.7} (SpecTr-GBV page, section 4, ablations)."""
    for T in (0.1, 0.4, 0.7):
        ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=32, V=4096, temperature=T)
        batch = pt.gpu_batch(ws, 4)
        for method in ("multidraft", "spectr"):
            _parity(method, batch, f"multi_T{T}")


# ---------------------------------------------------------------- edge cases

def test_empty_batch_is_a_noop():
    v = Verifier("multidraft", 0, 2, 3, 64, torch.bfloat16)
    z = torch.empty(0, device="cuda")
    out = v(torch.empty((0, 2, 4, 64), dtype=torch.bfloat16, device="cuda"),
            torch.empty((0, 2, 3, 64), dtype=torch.bfloat16, device="cuda"),
            torch.empty((0, 2, 3), dtype=torch.int32, device="cuda"), z,
            torch.empty((0, 2, 3), device="cuda"), z)
    torch.cuda.synchronize()
    assert out["accept_len"].numel() == 0


def test_invalid_requests_are_flagged():
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=8, V=1024)
    batch = pt.gpu_batch(ws, 5)
    batch["target"][0, 0, 0, 7] = float("nan")          # NaN in a node row
    batch["tokens"][1, 2, 1] = 1024                     # token outside [0, V)
    batch["temperature"][2] = 0.0                       # T must be > 0
    batch["u_accept"][3, 0, 0] = 1.0                    # u must be < 1
    batch["draft"][4, 0, 2] = float("-inf")             # a row of zero mass
    batch["u_correct"][5] = -0.25                       # u must be >= 0
    for method in ("multidraft", "spectr"):
        rep, out, ref = _parity(method, batch, "invalid")
        al = out["accept_len"].cpu().numpy()
        # the zero-mass row sits below the root: the K-draft walk reads it on this
        # batch, SpecTr only if its accepted path passes that node (parity above
        # already checks that the GPU flags exactly what the oracle flags)
        bad = [0, 1, 2, 3, 4, 5] if method == "multidraft" else [0, 1, 2, 3, 5]
        assert (al[bad] == -1).all()
        assert (out["flags"].cpu().numpy()[bad] & oracle.FLAG_INVALID).all()
        assert (al[6:] >= 0).all()


def test_equal_rows_accept_whole_block():
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=16, V=2048)
    batch = pt.gpu_batch(ws, 6)
    batch["draft"].copy_(batch["target"][:, :, :ws.L])
    for method in ("multidraft", "spectr"):
        rep, out, _ = _parity(method, batch, "p_equals_q")
        assert (out["accept_len"] == ws.L).all()


def test_single_token_vocabulary():
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=8, V=1)
    batch = pt.gpu_batch(ws, 7)
    for method in ("multidraft", "spectr"):
        rep, out, _ = _parity(method, batch, "V1")
        assert (out["accept_len"] == ws.L).all() and (out["correction"] == 0).all()


def test_largest_k_and_l():
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=6, K=64, L=16, V=96,
                      temperature=1.5)
    batch = pt.gpu_batch(ws, 8)
    for method in ("multidraft", "spectr"):
        _parity(method, batch, "K64_L16")


@pytest.mark.parametrize("method", ["multidraft", "spectr"])
def test_duplicate_rows_are_never_read(method):
    ws = synth.scaled(W["multi_zipf_bf16_b512_k8_l8_v151936"], B=16, V=2048)
    batch = pt.gpu_batch(ws, 9)
    ref = _verify(method, batch)
    ref = {k: v.clone() for k, v in ref.items()}
    tok = batch["tokens"].cpu().numpy()
    B, K, L = tok.shape
    for b in range(B):
        for k in range(1, K):
            for j in range(L + 1):
                if any((tok[b, c, :j] == tok[b, k, :j]).all() for c in range(k)):
                    batch["target"][b, k, j] = float("nan")
                    if j < L:
                        batch["draft"][b, k, j] = float("nan")
    out = _verify(method, batch)
    for k in ("accept_len", "draft_index", "correction", "flags", "row_lse", "resid_mass"):
        assert torch.equal(out[k].nan_to_num(-7.0), ref[k].nan_to_num(-7.0)), k


def test_negative_infinity_entries():
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=24, V=4096)
    batch = pt.gpu_batch(ws, 10)
    g = torch.Generator(device="cuda").manual_seed(10)
    for key in ("target", "draft"):
        mask = torch.rand(batch[key].shape, generator=g, device="cuda") < 0.3
        batch[key].masked_fill_(mask, float("-inf"))
    # redraw nothing: tokens may now sit on zero-probability entries of q
    for method in ("multidraft", "spectr"):
        _parity(method, batch, "neg_inf_entries")


def _root_rejections(flat, seed, V=65536, B=16):
    """K = 8 drafts whose first tokens (three distinct ones) have p ~ e^-100 and
    a large q at the root, so every draft is rejected there and each rejection but the last
    is followed by a residual-mass sweep of the root pair (duplicates included).
    The root's target row is -100 at the tokens the walk samples to judge
    whether a node list fits (every 128th token at V = 65536), so the row
    samples as sparse either way.  flat: every other logit ~ N(0, 0.5^2) at
    T = 1, so about half the tokens keep residual weight and every wave's list
    overflows (the walk falls back to full sweeps); otherwise logits ~ N(0, 5^2)
    at T = 0.4 and the lists are used.  Rows of more than 64 tiles of 4096 tokens
    (V = 300 000) keep the lists for the mass sweeps, but the correction draw
    takes the full sweep."""
    K, L = 8, 2
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    sig, T = (0.5, 1.0) if flat else (5.0, 0.4)
    tgt = torch.randn((B, K, L + 1, V), generator=g, device="cuda") * sig
    tgt[..., ::128] = -100.0
    drf = tgt[:, :, :L] + torch.randn((B, K, L, V), generator=g, device="cuda")
    drf[..., ::128] = 5.0 if flat else 30.0     # q(x) >> p(x) at the drafted first tokens
    firsts = 128 * torch.randint(0, V // 128, (B, 3), generator=g, device="cuda")
    pick = torch.randint(0, 3, (B, K), generator=g, device="cuda")
    tokens = torch.randint(0, V, (B, K, L), generator=g, device="cuda", dtype=torch.int32)
    tokens[:, :, 0] = torch.gather(firsts, 1, pick).to(torch.int32)
    return {"target": tgt.to(torch.bfloat16).contiguous(),
            "draft": drf.to(torch.bfloat16).contiguous(), "tokens": tokens.contiguous(),
            "temperature": torch.full((B,), T, device="cuda"),
            "u_accept": torch.rand((B, K, L), generator=g, device="cuda"),
            "u_correct": torch.rand((B,), generator=g, device="cuda")}


@pytest.mark.parametrize("flat,V,B", [(False, 65536, 16), (True, 65536, 16), (False, 300000, 8)],
                         ids=["lists_used", "lists_overflow", "lists_used_long_rows"])
def test_repeated_root_rejections(flat, V, B):
    batch = _root_rejections(flat, 11, V, B)
    rep, out, ref = _parity("multidraft", batch, f"root_rejections_flat{int(flat)}_v{V}")
    assert (out["accept_len"] == 0).all(), "every draft is rejected at the root"


NEAR_TIE_CASES = [
    # name, workload overrides, method
    ("k4_generic", dict(B=64), "multidraft"),
    # drafts within noise 0.05 of the target at T = 0.25: weights near 1, the GBV
    # tests below the last position ill-conditioned (h = R / (R + 1 - w))
    ("k4_illcond", dict(B=192, sigma_draft=0.05, temperature=0.25), "multidraft"),
    ("k1_block_illcond", dict(B=192, K=1, L=5, sigma_draft=0.05, temperature=0.25), "block"),
    ("k1_token", dict(B=64, K=1, L=5), "token"),
    ("k4_spectr", dict(B=48), "spectr"),
    ("k4_spectr_bisect", dict(B=48), "spectr_bisect"),
]


@pytest.mark.parametrize("name,over,method", NEAR_TIE_CASES, ids=[c[0] for c in NEAR_TIE_CASES])
def test_near_ties_are_taken_again_in_fp64(name, over, method):
    """Uniforms placed 1.5e-6 to 6e-6 (and 2e-7) from the oracle's threshold of
    draft 0's first decision -- the test at the last position (h = w_L), or, where
    that rejects, the one below it (h = R / (R + 1 - w), ill-conditioned when w is
    near 1) -- make decisions that fp32 exponentials cannot take reliably.  The
    library must take every such request again in fp64: every request whose
    oracle margin is at least 1e-6 matches the oracle bit for bit (the parity
    bar), and every request with an oracle decision within 5e-6 is marked."""
    from draft_token_verification_online_amd import SV_FLAG_NEAR_TIE, SV_FLAG_REDONE
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], V=4096, **over)
    batch = pt.gpu_batch(ws, 12)
    L = ws.L
    ua = batch["u_accept"].clone()
    if "illcond" in name:
        # make draft 0's test at position L reject (unless w_L is exactly 1), so the
        # ill-conditioned test at position L - 1 is the one taken next
        ua[:, 0, L - 1] = float(np.float32(1.0) - np.float32(2.0 ** -24))
    ref0 = pt.run_oracle(method, synth.to_host(dict(batch, u_accept=ua.contiguous())))
    deltas = [3e-6, -3e-6, 1.5e-6, -1.5e-6, 2e-7, -2e-7, 6e-6, -6e-6]
    placed = 0
    for b in range(ws.B):
        hp = ref0["accept_prob"][b, 0]
        # the first decision the rule takes for draft 0 (token level and SpecTr
        # test position 1 first; the block walk tests position L first, or L - 1)
        cands = ([0] if method in ("token", "spectr", "spectr_bisect") else
                 [L - 2] if "illcond" in name else [L - 1])
        for j in cands:
            if j >= 0 and not np.isnan(hp[j]) and 0.01 < hp[j] < 0.99:
                ua[b, 0, j] = float(np.float32(hp[j] + deltas[(b + j) % len(deltas)]))
                placed += 1
                break
    assert placed >= 16, placed
    batch2 = dict(batch, u_accept=ua.contiguous())
    rep, out, ref = _parity(method, batch2, f"near_tie/{name}")
    fl = out["flags"].cpu().numpy()
    marked = (fl & (SV_FLAG_NEAR_TIE | SV_FLAG_REDONE)) != 0
    print(f"[near-tie] {name}: placed={placed} redone={int(((fl & SV_FLAG_REDONE) != 0).sum())} "
          f"oracle<5e-6={int((ref['margin'] < 5e-6).sum())} excused={rep['excused']}", flush=True)
    assert marked[ref["margin"] < 5e-6].all()
    # fp64 margins: a request taken again carries the near-tie bit exactly when the
    # oracle's margin is well inside the band
    redone = (fl & SV_FLAG_REDONE) != 0
    assert ((fl[redone] & SV_FLAG_NEAR_TIE) != 0)[ref["margin"][redone] < 9e-6].all()
    assert ((fl[redone] & SV_FLAG_NEAR_TIE) == 0)[ref["margin"][redone] > 1.1e-5].all()
    # A request taken again in fp64 takes exact arithmetic's decisions, also where
    # they differ from the fast walk's and lead to drafts it never tested: it
    # equals the oracle wherever the oracle's margin is far above double rounding
    # (the parity bar above excuses every request within 1e-6).
    g = {k: out[k].cpu().numpy() for k in ("accept_len", "draft_index", "correction")}
    strict = np.nonzero(redone & (ref["margin"] > 1e-9))[0]
    off = [int(b) for b in strict if any(int(g[k][b]) != int(ref[k][b]) for k in g)]
    print(f"[near-tie] {name}: redone with margin > 1e-9: {len(strict)}, differing: {off[:8]}",
          flush=True)
    assert not off, (name, off[:8])




@pytest.mark.parametrize("diagnostics", [False, True], ids=["plain", "diagnostics"])
def test_fp64_walk_reaches_drafts_the_fast_walk_never_tested(diagnostics):
    """Two drafts of two tokens.  Draft 0's first token is less likely under the
    target than under the draft (w_1 < 1), its test at position 1 rejects
    (u = 1 - 2^-24 > h_1), and its test at the last position gets u = the float32
    rounding of the exact w_2 (margins ~1e-8 of either sign), so every such
    request is taken again in fp64 and about half of them reject draft 0 and go
    on to draft 1.  Where the fast walk took the other side of such a test, the
    fp64 walk reaches draft 1's node rows at position 1, which the fast walk
    never needed and the fp64 statistics launch leaves out: the re-walk must
    compute them rather than read the workspace (filled with NaN bits).  Every
    request taken again equals the oracle exactly (its margins are far above
    double rounding)."""
    B, K, L, V = 96, 2, 2, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    tgt = torch.randn((B, K, L + 1, V), generator=g, device="cuda") * 2.0
    drf = tgt[:, :, :L] + torch.randn((B, K, L, V), generator=g, device="cuda") * 0.5
    tokens = torch.randint(0, V, (B, K, L), generator=g, device="cuda", dtype=torch.int32)
    tokens[:, 1, 0] = (tokens[:, 0, 0] + 1 + torch.randint(0, V - 1, (B,), generator=g,
                                                           device="cuda", dtype=torch.int32)) % V
    # the root is one node: both drafts read the same row pair there
    tgt[:, 1, 0] = tgt[:, 0, 0]
    drf[:, 1, 0] = drf[:, 0, 0]
    a = tokens[:, 0, 0].long()
    idx = torch.arange(B, device="cuda")
    drf[idx, 0, 0, a] = tgt[idx, 0, 0, a] + 1.0
    drf[idx, 1, 0, a] = drf[idx, 0, 0, a]
    ua = torch.rand((B, K, L), generator=g, device="cuda")
    ua[:, 0, 0] = float(np.float32(1.0) - np.float32(2.0 ** -24))
    batch = {"target": tgt.to(torch.bfloat16).contiguous(),
             "draft": drf.to(torch.bfloat16).contiguous(), "tokens": tokens.contiguous(),
             "temperature": torch.ones((B,), device="cuda"),
             "u_accept": ua.contiguous(),
             "u_correct": torch.rand((B,), generator=g, device="cuda")}
    w2 = pt.run_oracle("multidraft", synth.to_host(batch), diagnostics=True)["accept_prob"][:, 0, L - 1]
    placed, rejects = 0, 0
    for b in range(B):
        if 0.05 < w2[b] < 0.95:
            ua[b, 0, L - 1] = float(np.float32(w2[b]))
            placed += 1
            rejects += float(np.float32(w2[b])) > w2[b]   # exact arithmetic rejects draft 0 there
    assert placed >= 48 and rejects >= 16, (placed, rejects)
    batch["u_accept"] = ua.contiguous()
    rep, out, ref = _parity("multidraft", batch, f"fp64_reaches_untested/{diagnostics}",
                            diagnostics=diagnostics)
    from draft_token_verification_online_amd import SV_FLAG_REDONE
    fl = out["flags"].cpu().numpy()
    redone = (fl & SV_FLAG_REDONE) != 0
    got = {k: out[k].cpu().numpy() for k in ("accept_len", "draft_index", "correction")}
    strict = np.nonzero(redone & (ref["margin"] > 1e-10))[0]
    off = [int(b) for b in strict if any(int(got[k][b]) != int(ref[k][b]) for k in got)]
    print(f"[fp64-untested] placed={placed} exact rejects={rejects} redone={int(redone.sum())} "
          f"strict={len(strict)} differing: {off[:8]}", flush=True)
    assert len(strict) >= 16, len(strict)
    assert not off, off[:8]

@pytest.mark.parametrize("method", ["multidraft", "spectr"])
def test_team_members_that_never_answer(method, monkeypatch):
    """The fp64 re-walk's teams: with SV_TEAM_WAIT_TICKS=0 the first workgroup
    of every team stops waiting for its members at once and sums their ranges
    itself (the fallback for members that cannot start), for the rest of the
    request.  Partial sums are added in member order either way, so every
    output, diagnostics included, equals the normal run's bit for bit, and the
    oracle's to the parity bar.  Uniforms at the oracle's threshold of draft 0's
    first decision list about 50 of 64 requests (teams of five)."""
    ws = synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], V=4096, B=64)
    batch = pt.gpu_batch(ws, 12)
    L = ws.L
    ref0 = pt.run_oracle(method, synth.to_host(batch))
    ua = batch["u_accept"].clone()
    deltas = [3e-6, -3e-6, 1.5e-6, -1.5e-6, 2e-7, -2e-7]
    j = 0 if method == "spectr" else L - 1
    for b in range(ws.B):
        h = ref0["accept_prob"][b, 0, j]
        if not np.isnan(h) and 0.01 < h < 0.99:
            ua[b, 0, j] = float(np.float32(h + deltas[b % len(deltas)]))
    batch = dict(batch, u_accept=ua.contiguous())
    normal = _verify(method, batch)
    monkeypatch.setenv("SV_TEAM_WAIT_TICKS", "0")
    rep, alone, ref = _parity(method, batch, f"team_fallback/{method}")
    from draft_token_verification_online_amd import SV_FLAG_REDONE
    redone = int(((alone["flags"] & SV_FLAG_REDONE) != 0).sum())
    print(f"[team-fallback] {method}: redone {redone}", flush=True)
    assert redone >= 16, redone
    for k in normal:
        a, b = normal[k], alone[k]
        if a.dtype.is_floating_point:
            assert torch.equal(torch.isnan(a), torch.isnan(b)), k
            a, b = torch.nan_to_num(a), torch.nan_to_num(b)
        assert torch.equal(a, b), k

# ------------------------------------------------------- one draft, split-V
# With K = 1 every call runs the single-draft kernels: slices of 1024 chunks
# (8192 tokens) per workgroup, residual sums per (position, slice), the draw's
# crossing found over slices and rescanned in one.

SINGLE_EDGES = [("v8192_one_slice", 8192, torch.bfloat16), ("v8200_one_chunk_over", 8200,
                 torch.bfloat16), ("v16384_two_slices", 16384, torch.bfloat16),
                ("v24577_scalar_ragged", 24577, torch.bfloat16),
                ("v9000_fp32", 9000, torch.float32), ("v151936_19_slices", 151936, torch.bfloat16)]


@pytest.mark.parametrize("name,V,dtype", SINGLE_EDGES, ids=[e[0] for e in SINGLE_EDGES])
def test_single_draft_slices(name, V, dtype):
    for T, sig in ((0.7, 1.5), (0.1, 0.3), (1.0, 0.05)):   # the last accepts whole blocks often
        ws = synth.scaled(W["gbv_bf16_b64_k1_l5_v32000"], B=24, V=V, dtype=dtype, temperature=T,
                          sigma_draft=sig)
        batch = pt.gpu_batch(ws, 21)
        for method in ("token", "block", "multidraft", "spectr"):
            _parity(method, batch, f"single_{name}_T{T}")


def test_single_draft_invalid_only_where_read():
    """Rows the single-draft rules never read cannot make a request invalid:
    the token rule stops at its first rejection, GBV reads every row below the
    bonus row and the bonus row only at tau = L."""
    ws = synth.scaled(W["gbv_bf16_b64_k1_l5_v32000"], B=12, V=9000)
    batch = pt.gpu_batch(ws, 22)
    L = ws.L
    x0 = batch["tokens"][:, 0, 0].long()
    # requests 0-3: the first token has p = 0, so token level rejects at position 1
    for b in range(4):
        batch["target"][b, 0, 0, x0[b]] = float("-inf")
    batch["target"][0, 0, 3, 11] = float("nan")        # read by GBV only
    batch["draft"][1, 0, 2, 5] = float("inf")          # read by GBV only
    batch["target"][2, 0, L].fill_(float("-inf"))      # the bonus row: never reached
    batch["temperature"][4] = float("nan")             # invalid for every rule
    batch["u_correct"][5] = 1.0
    batch["tokens"][6, 0, 3] = ws.V                    # out of range
    batch["draft"][7, 0, 0, 17] = float("nan")         # the root pair is always read
    for method in ("token", "block"):
        rep, out, ref = _parity(method, batch, f"single_invalid_{method}")
        al = out["accept_len"].cpu().numpy()
        assert (al[[4, 5, 6, 7]] == -1).all()
        if method == "token":
            assert (al[[0, 1, 2, 3]] == 0).all()
        else:
            assert (al[[0, 1]] == -1).all()


def test_misaligned_rows_take_the_scalar_path():
    ws = synth.scaled(W["gbv_bf16_b64_k1_l5_v32000"], B=16, V=2048)
    batch = pt.gpu_batch(ws, 11)
    for key in ("target", "draft"):
        t = batch[key]
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        view = buf[1:].view(t.shape)             # 2-byte offset: not 16-byte aligned
        view.copy_(t)
        batch[key] = view
    for method in ("block", "spectr"):
        _parity(method, batch, "misaligned")


# ---------------------------------------------------------------- full sizes
# The five workloads at their full shapes, in the launch configuration the
# benchmark times (no diagnostics).  Every request of the batch is checked
# against the oracle, which runs over host copies of 64 requests at a time.

FULL = list(W)
FULL_CASES = [(n, m) for n in FULL
              for m in W[n].methods + (("spectr", "spectr_bisect") if W[n].K > 1 else ())]


@pytest.mark.parametrize("name,method", FULL_CASES, ids=[f"{n}-{m}" for n, m in FULL_CASES])
def test_full_size_full_batch_parity(name, method):
    """The whole batch at its full size on the GPU and every request of it
    through the oracle."""
    w = W[name]
    batch = pt.gpu_batch(w, 1234)
    print(f"[case] full/{name} method={method} shape={tuple(batch['target'].shape)}", flush=True)
    out = _verify(method, batch, diagnostics=False)
    ref = pt.oracle_on_device_batch(method, batch)
    rep = pt.compare(method, out, ref, list(range(w.B)), diagnostics=False,
                     label=f"full/{name}/{method}")
    pt.check(rep)
    assert rep["n"] == w.B
    del batch
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity_second_seed(name):
    """A second full-size batch, 64 requests of it sampled for the oracle."""
    w = W[name]
    seed = 4321
    batch = pt.gpu_batch(w, seed)
    rng = np.random.default_rng(seed + 1)
    req = sorted(rng.choice(w.B, size=min(w.B, 64), replace=False).tolist())
    for method in w.methods + (("spectr",) if w.K > 1 else ()):
        _parity(method, batch, f"full/{name}/seed{seed}", requests=req, diagnostics=False)
    del batch
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", FULL[2:])
def test_full_size_diagnostics(name):
    w = W[name]
    batch = pt.gpu_batch(w, 99)
    req = [0, 1, w.B // 2, w.B - 1]
    for method in w.methods + (("spectr",) if w.K > 1 else ()):
        _parity(method, batch, f"full_diag/{name}", requests=req, diagnostics=True)
    del batch
    torch.cuda.empty_cache()
