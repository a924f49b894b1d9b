"""Seeded synthetic inputs for batched draft-token verification.

This module is shared by the tests, the smoke check and the benchmark.  It
holds none of the verification arithmetic: it draws logits, samples draft
tokens with the Gumbel-max trick (exact sampling from softmax(row / T), a
published method) and draws the uniforms that the verifier consumes.

Layout produced (row-major, on `device`):
  target [B][K][L+1][V], draft [B][K][L][V]  (float32 or bfloat16)
  tokens int32 [B][K][L], temperature float32 [B],
  u_accept float32 [B][K][L] in [0, 1), u_correct float32 [B] in [0, 1).

Tree consistency: the row of draft k at position j describes the node reached
by the prefix tokens[b][k][0..j-1].  Drafts that share a prefix get bit-equal
rows (copied from the lowest-index draft with that prefix); the K drafts are
i.i.d. because each one draws its own Gumbel noise at every position.

The workloads below follow the shapes, value distributions and temperatures of
the five synthetic configurations that stand in for the pages' datasets, which
are not available: the SpecTr-GBV page evaluates on real models and datasets
(section 4) and studies T in {0.1, 0.4, 0.7} (section 4, ablations).
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    L: int
    V: int
    dtype: torch.dtype
    sigma_target: float          # target logits ~ N(0, sigma_target^2)
    sigma_draft: float           # draft row = target row + N(0, sigma_draft^2)
    temperature: float           # T for every request (see mixed_temps)
    methods: tuple               # verification methods this workload exercises
    peak_frac: float = 0.0       # fraction of target entries raised by peak_add
    peak_add: float = 0.0
    zipf: float = 0.0            # target += -zipf * ln(rank), rank = v + 1
    mixed_temps: tuple = ()      # (T_even, T_odd): per-request temperature by parity
    sigma_draft_range: tuple = ()  # (lo, hi): per-request draft noise ~ U[lo, hi]


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_b1_k1_l4_v32", 1, 1, 4, 32, torch.float32, 3.0, 1.0, 1.0,
                 ("token", "block")),
        Workload("gbv_bf16_b64_k1_l5_v32000", 64, 1, 5, 32000, torch.bfloat16, 4.0, 1.5, 0.7,
                 ("block",), peak_frac=0.01, peak_add=8.0),
        Workload("multi_bf16_b256_k4_l4_v128256", 256, 4, 4, 128256, torch.bfloat16, 4.0, 1.0,
                 0.7, ("multidraft",)),
        Workload("multi_zipf_bf16_b512_k8_l8_v151936", 512, 8, 8, 151936, torch.bfloat16, 5.0,
                 2.0, 0.4, ("multidraft",), zipf=1.1),
        Workload("multi_mixedT_bf16_b1024_k4_l8_v151936", 1024, 4, 8, 151936, torch.bfloat16,
                 4.0, 1.0, 0.7, ("multidraft",), mixed_temps=(0.1, 0.7),
                 sigma_draft_range=(0.5, 3.0)),
    ]
}

# the workload the benchmark reports by default: the largest multi-draft case
BENCH_DEFAULT = "multi_zipf_bf16_b512_k8_l8_v151936"


def scaled(w: Workload, **over) -> Workload:
    """A copy of a workload with some fields replaced (smaller B or V for tests)."""
    return dataclasses.replace(w, **over)


def _gumbel(shape, gen, device):
    u = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    u = u.clamp_(min=1e-20)
    return -torch.log(-torch.log(u))


def generate(w: Workload, seed: int, device="cpu") -> dict:
    """Draw one batch of inputs for workload `w` from `seed` (deterministic per device)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    B, K, L, V = w.B, w.K, w.L, w.V

    if w.mixed_temps:
        t_even, t_odd = w.mixed_temps
        temps = torch.where(torch.arange(B, device=device) % 2 == 0,
                            torch.tensor(t_even, device=device),
                            torch.tensor(t_odd, device=device)).float()
    else:
        temps = torch.full((B,), float(w.temperature), device=device)
    if w.sigma_draft_range:
        lo, hi = w.sigma_draft_range
        sig_d = lo + (hi - lo) * torch.rand((B,), generator=gen, device=device)
    else:
        sig_d = torch.full((B,), float(w.sigma_draft), device=device)

    bias = None
    if w.zipf:
        bias = -w.zipf * torch.log(torch.arange(1, V + 1, device=device, dtype=torch.float32))

    target = torch.empty((B, K, L + 1, V), dtype=w.dtype, device=device)
    draft = torch.empty((B, K, L, V), dtype=w.dtype, device=device)
    tokens = torch.empty((B, K, L), dtype=torch.int32, device=device)
    kk = torch.arange(K, device=device)
    # same[b, k, k'] : drafts k and k' share the prefix built so far
    same = torch.ones((B, K, K), dtype=torch.bool, device=device)
    for j in range(L + 1):
        # canonical draft of each node: lowest index with the same prefix
        canon = torch.where(same, kk.view(1, 1, K), K).amin(dim=2)          # [B, K]
        idx = canon.view(B, K, 1).expand(B, K, V)
        rows = torch.randn((B, K, V), generator=gen, device=device) * w.sigma_target
        if w.peak_frac:
            mask = torch.rand((B, K, V), generator=gen, device=device) < w.peak_frac
            rows = rows + w.peak_add * mask.float()
        if bias is not None:
            rows = rows + bias.view(1, 1, V)
        rows = torch.gather(rows.to(w.dtype), 1, idx)
        target[:, :, j] = rows
        if j == L:
            break
        noise = torch.randn((B, K, V), generator=gen, device=device) * sig_d.view(B, 1, 1)
        drows = torch.gather((rows.float() + noise).to(w.dtype), 1, idx)
        draft[:, :, j] = drows
        g = _gumbel((B, K, V), gen, device)
        x = torch.argmax(drows.float() / temps.view(B, 1, 1) + g, dim=2).to(torch.int32)
        tokens[:, :, j] = x
        same = same & (x.view(B, K, 1) == x.view(B, 1, K))
        del rows, noise, drows, g

    u_accept = torch.rand((B, K, L), generator=gen, device=device, dtype=torch.float32)
    u_correct = torch.rand((B,), generator=gen, device=device, dtype=torch.float32)
    return {
        "target": target, "draft": draft, "tokens": tokens, "temperature": temps.float(),
        "u_accept": u_accept, "u_correct": u_correct,
    }


def to_host(batch: dict, requests=None) -> dict:
    """Copy a batch (or a subset of its requests) to host numpy arrays for the oracle.
    bfloat16 logits become their uint16 bit patterns."""
    out = {}
    for k, t in batch.items():
        if requests is not None:
            t = t[torch.as_tensor(requests, device=t.device, dtype=torch.long)]
        t = t.detach().to("cpu")
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
            out[k] = t.numpy().view("uint16")
        else:
            out[k] = t.numpy()
    return out


def dense_bytes(w: Workload) -> int:
    """Logit bytes of one batch: B*K*(2L+1)*V*sizeof(dtype)."""
    es = torch.empty((), dtype=w.dtype).element_size()
    return w.B * w.K * (2 * w.L + 1) * w.V * es


def tokens_per_step(w: Workload) -> int:
    """Verified draft tokens of one batch: B*K*L."""
    return w.B * w.K * w.L


def draft_uniforms(w: Workload, seed: int, device="cpu") -> torch.Tensor:
    """Uniforms in [0, 1) for drafting [B][K][L], from a stream of their own
    (independent of the verification uniforms of generate())."""
    gen = torch.Generator(device=device)
    gen.manual_seed(0x5EED0000 + 7919 * seed + 17)
    return torch.rand((w.B, w.K, w.L), generator=gen, device=device, dtype=torch.float32)
