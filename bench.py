#!/usr/bin/env python3
"""Benchmark: verified draft tokens per second of batched verification on one MI355X.

One step = one call of the verification entry point over one batch of
synthetic inputs already resident in HBM (both kernels: row statistics and
the per-request walk).  Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--method M]

M is a verification method (token, block, multidraft -- the default for
multi-draft workloads --, spectr, spectr_bisect), "draft" to time the drafting kernel
instead (drafted tokens per second), or "lmhead" to time the fused LM heads
(synthetic target and draft projections, --d-target and --d-draft) feeding
verification, against the same with the statistics left to the verifier.  --pipeline times the one-GPU emulation
of MineDraft's two-batch schedule: each step verifies one batch on one HIP
stream while the other batch is drafted on a second stream, roles alternating.

The roofline object describes the row-statistics kernel (the one that streams
the logits), timed with HIP events recorded on the launch stream around its
launches in a second pass over the same steps (the timed pass records no events).
achieved = the method's algorithmic bytes per
step -- the node rows the method itself reads (the oracle's count over the
whole batch, each row once, V * sizeof(logit) bytes) -- over that kernel's
time per step; roofline.sustained holds the bytes it actually streamed (its
speculative over-read included) over the same time.  The cpu_baseline object
times the CPU oracle (unmodified, single-threaded per request) on a bounded
sample of the same batch across the host's cores; the oracle then runs over the
rest of the batch untimed, and the parity object counts the requests of the
timed batch whose integer outputs or flag bits differ from it (mismatches),
apart from those the oracle puts within 1e-6 of a threshold (excused).
Batches smaller than 1 GiB are rotated through enough copies (8 to 64, 1 GiB in
all where that fits) that every step reads its logits from HBM, not from the
memory-side cache.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores, published
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# sources of each profiled kernel family (besides the shared device helpers, the
# launch code and the C header): a summary stays valid while these are unchanged
KERNEL_SOURCES = {"rowstats": ("sv_rowstats.hpp", "sv_walk.hpp", "sv_spectr.hpp", "sv_single.hpp",
                               "sv_redo.hpp"),
                  "draft": ("sv_draft.hpp",),
                  "lmhead": ("sv_lmhead.hpp",)}


def kernel_source_hash(kernel: str = "rowstats") -> str:
    from draft_token_verification_online_amd import build as svbuild
    own = KERNEL_SOURCES[kernel] + ("sv_device.hpp", "spec_verify.hip", "spec_verify.h")
    h = hashlib.sha256()
    for p in sorted(svbuild.DEPS):
        if os.path.basename(p) in own:
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles through the HIP runtime already loaded by torch."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.made.append(ev.value)
        return ev.value

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)
        self.made = []


def read_traffic(workload: str, method: str):
    """HBM bytes per step of the streaming kernel (the row-statistics kernel, or
    the drafting kernel for method "draft"; its launches in one step) from the
    committed rocprofv3 PMC summary (FETCH_SIZE and WRITE_SIZE runs, scaled by a
    copy-kernel calibration), or None when absent or taken on other sources."""
    kernel = {"draft": "draft", "lmhead": "lmhead"}.get(method, "rowstats")
    path = os.path.join(PROFILES, f"{kernel}_{method}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash(kernel):
        return None
    return float(d["bytes_per_step"])


def host_threads():
    """Oracle worker threads: the host cores this process may run on, at most 16
    (the host share of one GPU on the benchmark machines)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(method, batch, w, out, target_cpu_s: float, chunk: int = 64):
    """The CPU oracle on the benchmark's own batch: timed on a bounded sample (the
    first requests, about target_cpu_s of CPU work), then run untimed over the
    rest of the batch, so that every request of the timed batch is checked
    against the GPU's outputs `out` and the rows the method reads (A_visit)
    are counted over the whole batch."""
    import numpy as np
    import oracle
    import synth
    threads = host_threads()
    method = {"spectr_bisect": "spectr"}.get(method, method)   # the rule it implements
    host1 = synth.to_host(batch, [0])
    t = time.perf_counter()
    oracle.verify(method, host1["target"], host1["draft"], host1["tokens"],
                  host1["temperature"], host1["u_accept"], host1["u_correct"])
    t_one = max(time.perf_counter() - t, 1e-4)
    m = int(np.clip(round(target_cpu_s / t_one), min(threads, w.B), w.B))

    wall = 0.0

    def run(reqs, timed):
        nonlocal wall
        host = synth.to_host(batch, reqs)          # the host copy is not timed
        t = time.perf_counter()
        r = oracle.verify(method, host["target"], host["draft"], host["tokens"],
                          host["temperature"], host["u_accept"], host["u_correct"],
                          threads=threads)
        if timed:
            wall += time.perf_counter() - t
        return r

    parts = []
    for i in range(0, w.B, chunk):
        reqs = list(range(i, min(i + chunk, w.B)))
        head = [r for r in reqs if r < m]
        if head:
            parts.append(run(head, True))
        if len(head) < len(reqs):
            parts.append(run(reqs[len(head):], False))
        if (i // chunk) % 4 == 3:
            log(f"[bench] oracle: {min(i + chunk, w.B)} of {w.B} requests")
    ref = {k: np.concatenate([p[k] for p in parts], axis=0) for k in parts[0]}
    cpu = {
        "value": m * w.K * w.L / wall,
        "unit": "verified draft tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {m} of {w.B} requests of the timed batch ({m * w.K * w.L} draft "
                  f"tokens), fp64 C oracle, one request per thread on {threads} threads "
                  f"(host reports {os.cpu_count()} cores), {wall:.2f} s wall",
    }
    # the timed batch against the oracle: integers and flag bits bit-exact, except
    # requests the oracle itself puts within 1e-6 of a threshold (or degenerate)
    g = {k: out[k].cpu().numpy() for k in ("accept_len", "draft_index", "correction", "flags")}
    mism = excused = ties = 0
    for b in range(w.B):
        of = int(ref["flags"][b])
        tie = not (of & 2) and (ref["margin"][b] < 1e-6 or bool(of & 1))
        ties += int(tie)
        same = all(int(g[k][b]) == int(ref[k][b]) for k in ("accept_len", "draft_index",
                                                              "correction"))
        same &= (int(g["flags"][b]) & 3) == (of & 3)
        if not same:
            if tie:
                excused += 1
            else:
                mism += 1
    parity = {"n": w.B, "mismatches": mism, "excused": excused, "oracle_ties": ties,
              "oracle_within_1e-5": int(((ref["margin"] < 1e-5) & ((ref["flags"] & 2) == 0)).sum()),
              "near_tie_flagged_by_gpu": int(((g["flags"] & 4) != 0).sum()),
              "redone_in_fp64": int(((g["flags"] & 8) != 0).sum())}
    visit = {"requests": w.B, "oracle_rows_per_request": float(ref["counters"][:, 2].mean()),
             "oracle_rows": int(ref["counters"][:, 2].sum())}
    return cpu, parity, visit


def cpu_baseline_draft(batch, u, w, target_cpu_s: float):
    import numpy as np
    import oracle
    import synth
    threads = host_threads()
    host = lambda reqs: (synth.to_host(batch, reqs)["draft"],
                         batch["temperature"][reqs].cpu().numpy(), u[reqs].cpu().numpy())
    t = time.perf_counter()
    oracle.draft(*host([0]))
    t_one = max(time.perf_counter() - t, 1e-4)
    m = int(np.clip(round(target_cpu_s / t_one), threads, w.B))
    args = host(list(range(m)))
    t = time.perf_counter()
    oracle.draft(*args, threads=threads)
    wall = time.perf_counter() - t
    return {
        "value": m * w.K * w.L / wall,
        "unit": "drafted tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {m} of {w.B} requests of the same batch ({m * w.K * w.L} draws), "
                  f"fp64 C oracle, one request per thread, {wall:.2f} s wall",
    }


def copy_calibration(torch, mib):
    if not mib:
        return
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 3 copies of {n} bytes")


def run_draft(args, w, name):
    """Time spec_draft_sample: B*K*L draws per step from the workload's draft logits."""
    import torch
    import synth
    import draft_token_verification_online_amd as sv
    log(f"[bench] generating {name} on cuda:0 (seed {args.seed})")
    batch = synth.generate(w, args.seed, device="cuda")
    u = synth.draft_uniforms(w, args.seed, device="cuda")
    torch.cuda.synchronize()
    es = 2 if w.dtype == torch.bfloat16 else 4
    dr = sv.Drafter(w.B, w.K, w.L, w.V, w.dtype)
    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(args.warmup):
        dr(batch["draft"], batch["temperature"], u, stream=stream)
    torch.cuda.synchronize()
    evs = [[hip.create(), hip.create()] + [None] * (sv.N_PHASE_EVENTS - 2)
           for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps of draft sampling on {name}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        dr(batch["draft"], batch["temperature"], u, stream=stream, events=evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = [hip.elapsed_ms(e[0], e[1]) for e in evs]
    hip.close()
    ms_per_step = wall * 1e3 / args.steps
    k_mean = sum(kern) / len(kern)
    rows = int(dr.out["rows_streamed"].sum())
    byts = rows * w.V * es
    achieved = byts / (k_mean * 1e-3) / 1e9
    value = synth.tokens_per_step(w) / (ms_per_step * 1e-3)
    log(f"[bench] {ms_per_step:.3f} ms/step, kernels {k_mean:.3f} ms, {achieved:.0f} GB/s, "
        f"{value / 1e6:.2f} M drafted tokens/s")
    copy_calibration(torch, args.copy_calibration_mib)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        cpu = cpu_baseline_draft(batch, u, w, args.cpu_seconds)
        log(f"[bench] cpu baseline {cpu['value']:.0f} tokens/s on {cpu['cores']} threads")
    return {
        "metric": "drafted tokens/s (B*K*L) + achieved HBM GB/s of the drafting kernel",
        "value": value,
        "unit": "drafted tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "method": "draft", "B": w.B, "K": w.K, "L": w.L,
                   "V": w.V, "logits": "bf16" if es == 2 else "fp32", "seed": args.seed},
        "roofline": {"bound": "hbm", "kernel": "draft_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": read_traffic(name, "draft")},
        "cpu_baseline": cpu,
        "detail": {"kernels_ms": k_mean, "rows_streamed_per_step": rows,
                   "rows_streamed_bytes": byts,
                   "invalid_requests": int((dr.out["flags"] != 0).sum())},
    }


def run_pipeline(args, w, name, method):
    """MineDraft's two-batch schedule on one GPU (TwoBatchPipeline): step i
    verifies batch i%2 on one stream while batch (i+1)%2 is drafted on another.
    Verification of a batch waits for its drafting in the previous step, and
    drafting waits for that batch's verification in the previous step."""
    import torch
    import synth
    from draft_token_verification_online_amd.pipeline import TwoBatchPipeline
    log(f"[bench] generating two batches of {name} on cuda:0")
    batches = [synth.generate(w, args.seed + i, device="cuda") for i in range(2)]
    # a pool of uniforms made before timing, cycled through by step
    pool = [[(synth.draft_uniforms(w, args.seed + 10 * j + b, device="cuda"),
              synth.generate(synth.scaled(w, V=8), args.seed + 10 * j + b,
                             device="cuda")["u_accept"],
              synth.generate(synth.scaled(w, V=8), args.seed + 10 * j + b,
                             device="cuda")["u_correct"]) for b in range(2)] for j in range(4)]
    torch.cuda.synchronize()
    pipe = TwoBatchPipeline(method, batches, lambda i, b: pool[i % 4][b])
    s = pipe.s_verify

    def draft(b):
        bt = batches[b]
        pipe.drafters[b](bt["draft"], bt["temperature"], pool[0][b][0], stream=s.cuda_stream)

    def verify(b):
        bt = batches[b]
        pipe.verifiers[b](bt["target"], bt["draft"], pipe.drafters[b].out["draft_tokens"],
                          bt["temperature"], pool[0][b][1], pool[0][b][2], stream=s.cuda_stream)

    def timed(fn, n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / n

    # each piece alone, on one stream
    for b in range(2):
        draft(b)
    for _ in range(args.warmup):
        verify(0)
    t_verify = timed(lambda: verify(0), args.steps)
    t_draft = timed(lambda: draft(1), args.steps)
    # serial schedule: verify A, then draft B, on one stream
    t_serial = timed(lambda: (verify(0), draft(1)), args.steps)
    # overlapped: the two-batch schedule on two streams
    pipe.prime()
    for _ in range(args.warmup):
        pipe.step()
    t_over = timed(pipe.step, args.steps)
    tokens = synth.tokens_per_step(w)
    log(f"[bench] pipeline: verify {t_verify:.3f} ms, draft {t_draft:.3f} ms, serial "
        f"{t_serial:.3f} ms/step, overlapped {t_over:.3f} ms/step "
        f"({t_serial / t_over:.2f}x)")
    return {
        "metric": "verified draft tokens/s with drafting of the other batch overlapped "
                  "(two-batch schedule, two HIP streams)",
        "value": tokens / (t_over * 1e-3),
        "unit": "verified draft tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_over, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "method": method, "pipeline": "verify A | draft B",
                   "B": w.B, "K": w.K, "L": w.L, "V": w.V, "seed": args.seed},
        "roofline": None,
        "cpu_baseline": None,
        "detail": {"verify_ms": t_verify, "draft_ms": t_draft, "serial_ms": t_serial,
                   "overlapped_ms": t_over, "overlap_speedup": t_serial / t_over,
                   "ideal_ms": max(t_verify, t_draft)},
    }


def run_lmhead(args, w, name):
    """Target and draft LM heads (logits + statistics) feeding a verification call
    that skips its statistics pass, against the unfused sequence."""
    import torch
    import synth
    import draft_token_verification_online_amd as sv
    B, K, L, V = w.B, w.K, w.L, w.V
    dt, dd = args.d_target, args.d_draft
    Rt, Rd = B * K * (L + 1), B * K * L
    method = "multidraft" if w.K > 1 else "block"
    log(f"[bench] synthetic LM heads d={dt}/{dd} for {name} ({Rt}+{Rd} rows, V={V})")
    g = torch.Generator(device="cuda").manual_seed(args.seed)
    ht = torch.randn((Rt, dt), generator=g, device="cuda").to(torch.bfloat16)
    wt = (torch.randn((V, dt), generator=g, device="cuda") * (4 / dt ** 0.5)).to(torch.bfloat16)
    hd = torch.randn((Rd, dd), generator=g, device="cuda").to(torch.bfloat16)
    wd = (torch.randn((V, dd), generator=g, device="cuda") * (4 / dd ** 0.5)).to(torch.bfloat16)
    base = synth.generate(synth.scaled(w, V=8), args.seed, device="cuda")   # temperatures, uniforms
    T = base["temperature"]
    Tt, Td = T.repeat_interleave(K * (L + 1)), T.repeat_interleave(K * L)
    ldt = torch.bfloat16 if args.lm_logits == "bf16" else torch.float32
    lt, ld = sv.LmHead(Rt, dt, V, logits_dtype=ldt), sv.LmHead(Rd, dd, V, logits_dtype=ldt)
    stats = torch.empty(B * K * (2 * L + 1) * 16, dtype=torch.uint8, device="cuda")
    ver = sv.Verifier(method, B, K, L, V, ldt)
    ld(hd, wd, Td)
    drafter = sv.Drafter(B, K, L, V, ldt)
    tok = drafter(ld.logits.view(B, K, L, V), T,
                  synth.draft_uniforms(w, args.seed, device="cuda"))["draft_tokens"].clone()
    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream

    def fused(ev=None):
        lt(ht, wt, Tt, stats=stats, group=L + 1, stride=2 * L + 1, offset=0, stream=stream,
           events=ev)
        ld(hd, wd, Td, stats=stats, group=L, stride=2 * L + 1, offset=L + 1, stream=stream)
        ver(lt.logits.view(B, K, L + 1, V), ld.logits.view(B, K, L, V), tok, T,
            base["u_accept"], base["u_correct"], stream=stream, row_stats=stats)

    def unfused():
        lt(ht, wt, Tt, stream=stream)
        ld(hd, wd, Td, stream=stream)
        ver(lt.logits.view(B, K, L + 1, V), ld.logits.view(B, K, L, V), tok, T,
            base["u_accept"], base["u_correct"], stream=stream)

    def timed(fn, n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / n

    for _ in range(args.warmup):
        fused()
        unfused()
    evs = [[hip.create(), hip.create()] + [None] * (sv.N_PHASE_EVENTS - 2)
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fused(evs[i])
    torch.cuda.synchronize()
    t_fused = (time.perf_counter() - t0) * 1e3 / args.steps
    t_lm = sum(hip.elapsed_ms(e[0], e[1]) for e in evs) / args.steps   # target LM head
    hip.close()
    t_unfused = timed(unfused, args.steps)
    t_lmd = timed(lambda: ld(hd, wd, Td, stream=stream), args.steps)
    t_ver_given = timed(lambda: ver(lt.logits.view(B, K, L + 1, V), ld.logits.view(B, K, L, V),
                                    tok, T, base["u_accept"], base["u_correct"], stream=stream,
                                    row_stats=stats), args.steps)
    t_ver_own = timed(lambda: ver(lt.logits.view(B, K, L + 1, V), ld.logits.view(B, K, L, V),
                                  tok, T, base["u_accept"], base["u_correct"], stream=stream),
                      args.steps)
    copy_calibration(torch, args.copy_calibration_mib)
    flops = 2.0 * Rt * V * dt
    tflops = flops / (t_lm * 1e-3) / 1e12
    log(f"[bench] target LM head {t_lm:.3f} ms ({tflops:.0f} TFLOP/s), draft LM head "
        f"{t_lmd:.3f} ms; verify given stats {t_ver_given:.3f} ms, own stats {t_ver_own:.3f} ms; "
        f"fused step {t_fused:.3f} ms, unfused {t_unfused:.3f} ms")
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        from threadpoolctl import threadpool_info
        n = 32
        hb = lambda x: x[:n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        wbt = wt.view(torch.int16).cpu().numpy().view(np.uint16)
        wbd = wd.view(torch.int16).cpu().numpy().view(np.uint16)
        t = time.perf_counter()
        oracle.lm_head(hb(ht), wbt, Tt[:n].cpu().numpy())
        ct = (time.perf_counter() - t) / n
        t = time.perf_counter()
        oracle.lm_head(hb(hd), wbd, Td[:n].cpu().numpy())
        cd = (time.perf_counter() - t) / n
        step_s = Rt * ct + Rd * cd
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        cpu = {"value": B * K * L / step_s, "unit": "verified draft tokens/s", "cores": threads,
               "kind": "oracle",
               "sample": f"oracle LM heads (float64 BLAS product) on {n} target and {n} draft rows, "
                         f"scaled to the {Rt}+{Rd} rows of a step; verification not included"}
    return {
        "metric": "verified draft tokens/s through fused LM heads + verification",
        "value": B * K * L / (t_fused * 1e-3),
        "unit": "verified draft tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": t_fused, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "method": "lmhead+" + method, "B": B, "K": K, "L": L,
                   "V": V, "d_target": dt, "d_draft": dd, "logits": args.lm_logits,
                   "seed": args.seed},
        "roofline": {"bound": "mfma", "kernel": "lm_head_kernel (target)", "achieved": tflops,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": read_traffic(name, "lmhead")},
        "cpu_baseline": cpu,
        "detail": {"lm_target_ms": t_lm, "lm_draft_ms": t_lmd, "verify_given_stats_ms": t_ver_given,
                   "verify_own_stats_ms": t_ver_own, "fused_ms": t_fused, "unfused_ms": t_unfused,
                   "target_gemm_tflop": flops / 1e12},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--method", default=None)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU work (summed over cores) spent on the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--d-target", type=int, default=3584, help="hidden size of the target LM head")
    ap.add_argument("--d-draft", type=int, default=896, help="hidden size of the draft LM head")
    ap.add_argument("--lm-logits", choices=("f32", "bf16"), default="f32",
                    help="element type of the logits the LM heads write (--method lmhead)")
    ap.add_argument("--pipeline", action="store_true",
                    help="time the two-batch verify/draft overlap on two streams")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies to cycle through (0: enough for 1 GiB, at least 8, "
                         "when one batch is smaller than 1 GiB)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run plain device copies of this many MiB (a "
                         "reference kernel of known traffic for rocprofv3 PMC runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build verifies each request on one "
              f"device and has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import draft_token_verification_online_amd as sv
    from draft_token_verification_online_amd import build as svbuild

    if not os.path.exists(svbuild.LIB):
        log("library not built; building")
        svbuild.build()
    if not torch.cuda.is_available():
        log("no HIP device visible")
        sys.exit(1)

    name = args.workload or synth.BENCH_DEFAULT
    w = synth.WORKLOADS[name]
    method = args.method or w.methods[-1]
    torch.cuda.set_device(0)
    if method == "draft":
        print(json.dumps(run_draft(args, w, name)), flush=True)
        return
    if method == "lmhead":
        print(json.dumps(run_lmhead(args, w, name)), flush=True)
        return
    if args.pipeline:
        print(json.dumps(run_pipeline(args, w, name, method)), flush=True)
        return
    log(f"[bench] generating {name} on cuda:0 (seed {args.seed})")
    batch = synth.generate(w, args.seed, device="cuda")
    torch.cuda.synchronize()
    es = 2 if w.dtype == torch.bfloat16 else 4
    dense = synth.dense_bytes(w)
    # Inputs smaller than the memory-side cache would be served from it on every
    # step after the first: rotate through copies at different addresses, at
    # least 8 and 1 GiB of logits in all, so each step reads from HBM (at most 64:
    # a batch of a few KB is bound by launch latency, not by where it is read from).
    copies = args.rotate if args.rotate else (1 if dense >= (1 << 30)
                                              else min(64, max(8, -(-(1 << 30) // dense))))
    inputs = [batch] + [{k: v.clone() for k, v in batch.items()} for _ in range(copies - 1)]
    torch.cuda.synchronize()
    if copies > 1:
        log(f"[bench] rotating {copies} input copies ({copies * dense / 2**30:.2f} GiB of logits)")

    ver = sv.Verifier(method, w.B, w.K, w.L, w.V, w.dtype)

    def args_of(i):
        bt = inputs[i % copies]
        return (bt["target"], bt["draft"], bt["tokens"], bt["temperature"], bt["u_accept"],
                bt["u_correct"])

    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup):
        ver(*args_of(i), stream=stream)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps of {method} on {name}")
    # the timed steps carry no events (an event record costs microseconds of GPU
    # time, comparable to a whole step of the small workloads)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ver(*args_of(i), stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same steps again with events around the launches, for the kernel times
    evs = [[hip.create() for _ in range(sv.N_PHASE_EVENTS)] for _ in range(args.steps)]
    for i in range(args.steps):
        ver(*args_of(i), stream=stream, events=evs[i])
    torch.cuda.synchronize()

    # events: [0] stats launch 1 [1] walk round 1 [2] stats launch 2 [3] walk round 2 [4]
    phase = [[hip.elapsed_ms(e[i], e[i + 1]) for i in range(4)] for e in evs]
    stats_ms = [p[0] + p[2] for p in phase]
    walk_ms = [p[1] + p[3] for p in phase]
    phase_mean = [sum(p[i] for p in phase) / len(phase) for i in range(4)]
    hip.close()
    rows = int(ver.out["rows_streamed"].sum())          # rows the statistics kernel streamed
    stats_bytes = rows * w.V * es
    ms_per_step = wall * 1e3 / args.steps
    tokens = synth.tokens_per_step(w)
    value = tokens / (ms_per_step * 1e-3)
    st_mean = sum(stats_ms) / len(stats_ms)
    wk_mean = sum(walk_ms) / len(walk_ms)
    streamed_gbps = stats_bytes / (st_mean * 1e-3) / 1e9
    flags = ver.out["flags"].cpu()
    log(f"[bench] {ms_per_step:.3f} ms/step, stats {st_mean:.3f} ms, walk {wk_mean:.3f} ms, "
        f"{streamed_gbps:.0f} GB/s node-row stream, {value / 1e6:.2f} M tokens/s")

    copy_calibration(torch, args.copy_calibration_mib)

    traffic = read_traffic(name, method)
    cpu = parity = None
    roofline = {"bound": "hbm", "kernel": "rowstats_kernel", "achieved": None,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": None, "traffic": traffic}
    a_visit = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline and parity of the timed batch (oracle) ...")
        cpu, parity, visit = cpu_baseline(method, batch, w, ver.out, args.cpu_seconds)
        log(f"[bench] cpu baseline {cpu['value']:.0f} tokens/s on {cpu['cores']} threads; "
            f"parity {parity}")
        # algorithmic bytes: the rows the method itself reads (oracle count over the
        # whole batch), each once
        a_bytes = visit["oracle_rows"] * w.V * es
        achieved = a_bytes / (st_mean * 1e-3) / 1e9
        roofline.update(achieved=achieved, frac=achieved / HBM_PEAK_GBPS)
        a_visit = {"requests": visit["requests"],
                   "oracle_rows_per_request": visit["oracle_rows_per_request"],
                   "gpu_rows_streamed_per_request": rows / w.B,
                   "bytes_per_step": a_bytes,
                   "step_GBps": a_bytes / (ms_per_step * 1e-3) / 1e9,
                   "step_frac_of_peak": a_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    # what the statistics kernel streamed (its speculative over-read included)
    roofline["sustained"] = {"achieved": streamed_gbps, "frac": streamed_gbps / HBM_PEAK_GBPS,
                             "bytes_per_step": stats_bytes}

    line = {
        "metric": "verified draft tokens/s (B*K*L) + achieved HBM GB/s of verify kernel",
        "value": value,
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "method": method, "B": w.B, "K": w.K, "L": w.L,
                   "V": w.V, "logits": "bf16" if es == 2 else "fp32",
                   "seed": args.seed, "input_copies": copies},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "detail": {
            "rowstats_ms": st_mean,
            "walk_ms": wk_mean,
            "phase_ms": {"rowstats_first_visit": phase_mean[0], "walk_round1": phase_mean[1],
                         "rowstats_after_accept": phase_mean[2], "walk_round2": phase_mean[3]},
            "rows_streamed_per_step": rows,
            "rows_streamed_bytes": stats_bytes,
            "dense_logit_bytes": dense,
            "dense_equiv_GBps_per_step": dense / (ms_per_step * 1e-3) / 1e9,
            "mean_accept_len": float(ver.out["accept_len"].float().mean()),
            "invalid_requests": int(((flags & 2) != 0).sum()),
            "a_visit": a_visit,
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
