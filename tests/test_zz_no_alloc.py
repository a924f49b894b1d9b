"""spec_verify_multidraft_noalloc: the multi-draft call with its workspace in
scratch memory the library holds (for callers that cannot allocate), checked
against spec_verify_multidraft with a caller workspace on the same inputs.

Two calls in a row on one device, the second with a smaller input, so the
second runs on scratch that still holds the first call's contents."""
import ctypes

import numpy as np
import pytest
import torch

import paritytools as pt
import synth
import draft_token_verification_online_amd as sv
from draft_token_verification_online_amd import Verifier

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
KEYS = ("accept_len", "draft_index", "correction", "flags", "rows_streamed")


def _both(batch, diagnostics=False):
    t = batch["target"]
    B, K, L1, V = t.shape
    args = (batch["target"], batch["draft"], batch["tokens"], batch["temperature"],
            batch["u_accept"], batch["u_correct"])
    a = Verifier("multidraft", B, K, L1 - 1, V, t.dtype, diagnostics=diagnostics,
                 noalloc=True)
    b = Verifier("multidraft", B, K, L1 - 1, V, t.dtype, diagnostics=diagnostics)
    b.workspace.fill_(0xA5)                      # the caller's workspace needs no clearing
    ga = {k: v.clone() for k, v in a(*args).items()}
    torch.cuda.synchronize()
    gb = {k: v.clone() for k, v in b(*args).items()}
    torch.cuda.synchronize()
    return ga, gb


def test_noalloc_equals_the_workspace_call_on_two_calls():
    cases = [
        ("first", synth.scaled(W["multi_bf16_b256_k4_l4_v128256"], B=48, V=12296), 1),
        # smaller: fewer requests, the scalar path (V not a multiple of 8), K = 3
        ("second_smaller", synth.scaled(W["multi_zipf_bf16_b512_k8_l8_v151936"], B=20, K=3,
                                        L=5, V=4099), 2),
    ]
    for label, w, seed in cases:
        print(f"[case] noalloc {label} B={w.B} K={w.K} L={w.L} V={w.V}", flush=True)
        batch = pt.gpu_batch(w, seed)
        ga, gb = _both(batch)
        for k in KEYS:
            assert torch.equal(ga[k], gb[k]), (label, k)
        # and both to the parity bar against the oracle
        ref = pt.run_oracle("multidraft", synth.to_host(batch), diagnostics=False)
        rep = pt.compare("multidraft", ga, ref, list(range(w.B)), diagnostics=False,
                         label=f"noalloc/{label}")
        pt.check(rep)


def test_noalloc_diagnostics_and_high_acceptance():
    """Diagnostics (one round, every node row streamed) and a batch whose walks
    stop after acceptances (two rounds through the scratch's row list)."""
    w = synth.scaled(W["multi_zipf_bf16_b512_k8_l8_v151936"], B=24, V=6000, sigma_draft=0.3,
                     temperature=0.25)
    batch = pt.gpu_batch(w, 3)
    for diag in (True, False):
        ga, gb = _both(batch, diagnostics=diag)
        for k in ga:
            assert torch.equal(ga[k].nan_to_num(-7.0), gb[k].nan_to_num(-7.0)), (diag, k)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = sv.load_library()
    B, K, L, V = 1024, 4, 8, 151936
    assert sv.workspace_size(B, K, L, V, sv.SV_BF16) > sv.SV_NOALLOC_SCRATCH_BYTES
    base = 1 << 20      # never dereferenced: the size check comes first
    ins = sv.SvInputs(B, K, L, V, sv.SV_BF16, base, base, base, base, base, base, None)
    outs = sv.SvOutputs(base, base, base, None, None, None, None, None)
    rc = lib.spec_verify_multidraft_noalloc(ctypes.byref(ins), ctypes.byref(outs), None)
    assert rc == sv.SV_EUNSUPPORTED
    assert sv.workspace_size(512, 8, 8, V, sv.SV_BF16) <= sv.SV_NOALLOC_SCRATCH_BYTES
