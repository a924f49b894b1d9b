"""Helpers for comparing the HIP path with the CPU oracle on the same inputs.

The parity bar: integer outputs (accept_len, draft_index, correction) and the
degenerate and invalid flag bits are identical to the oracle's, except for
requests whose ORACLE decision log holds a decision within TIE_BAND of its
threshold, or that the ORACLE found degenerate; those are counted ("excused").
Nothing the GPU reports about itself can excuse a request.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
import synth

TIE_BAND = 1e-6          # decisions this close to their threshold are excused (counted)
LSE_RTOL = 1e-5          # ln-partition functions of the rows, relative
H_ATOL = 1e-5            # acceptance probabilities h in [0, 1], absolute
Z_RTOL = 1e-5            # residual mass of the correction distribution, relative
Z_ATOL = 1e-7
NEAR_TIE_FLAG = 4        # SV_FLAG_NEAR_TIE


def host_threads():
    """Oracle worker threads: the host cores this process may run on, at most 16
    (the host share of one GPU on the test machines)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# the oracle method that states the rule each library method implements
ORACLE_METHOD = {"spectr_bisect": "spectr"}


def run_oracle(method, host, diagnostics=True, requests=None):
    return oracle.verify(ORACLE_METHOD.get(method, method), host["target"], host["draft"], host["tokens"],
                         host["temperature"], host["u_accept"], host["u_correct"],
                         diagnostics=diagnostics, threads=host_threads(), requests=requests)


def oracle_on_device_batch(method, batch, requests=None, *, diagnostics=False, chunk=64):
    """Run the oracle on requests of a batch that lives in device memory, copying
    `chunk` requests at a time to the host (so a full-size batch never sits in
    host memory whole).  Returns the oracle's outputs indexed by position in
    `requests` (all requests when None)."""
    B = batch["target"].shape[0]
    req = list(range(B)) if requests is None else list(requests)
    parts = []
    for i in range(0, len(req), chunk):
        sub = req[i:i + chunk]
        host = synth.to_host(batch, sub)
        parts.append(run_oracle(method, host, diagnostics=diagnostics))
        del host
    if not parts:
        return run_oracle(method, synth.to_host(batch, []), diagnostics=diagnostics)
    return {k: np.concatenate([p[k] for p in parts], axis=0) for k in parts[0]}


def compare(method, gpu_out, ref, requests, *, diagnostics=True, label=""):
    """Compare GPU outputs (dict of tensors over the whole batch) with oracle
    outputs (dict of arrays indexed by position in `requests`).  Returns a report;
    check() raises on any unexcused mismatch or diagnostic outside tolerance."""
    g = {k: v.detach().cpu().numpy() for k, v in gpu_out.items()}
    req = np.asarray(requests)
    rep = {"label": label, "n": len(req), "excused": 0, "oracle_ties": 0, "mismatch": [],
           "max_lse_rel": 0.0, "max_h_abs": 0.0, "max_z_rel": 0.0, "invalid": 0,
           "degenerate": 0, "unflagged_ties": []}
    for i, b in enumerate(req):
        oflags = int(ref["flags"][i])
        gflags = int(g["flags"][b]) if "flags" in g else None
        o_inv = bool(oflags & oracle.FLAG_INVALID)
        o_deg = bool(oflags & oracle.FLAG_DEGENERATE)
        rep["invalid"] += o_inv
        rep["degenerate"] += o_deg
        # the oracle alone decides which requests sit in the tie band
        o_tie = (not o_inv) and (ref["margin"][i] < TIE_BAND or o_deg)
        rep["oracle_ties"] += o_tie
        # the library flags every decision within 1e-5 of its threshold
        if gflags is not None and not o_inv and ref["margin"][i] < TIE_BAND \
                and not gflags & NEAR_TIE_FLAG:
            rep["unflagged_ties"].append(int(b))
        same = all(int(g[k][b]) == int(ref[k][i])
                   for k in ("accept_len", "draft_index", "correction"))
        if gflags is not None:
            same &= bool(gflags & oracle.FLAG_INVALID) == o_inv
            same &= bool(gflags & oracle.FLAG_DEGENERATE) == o_deg
        if not same:
            if o_tie:
                rep["excused"] += 1
            else:
                rep["mismatch"].append(
                    (int(b), {k: (int(g[k][b]), int(ref[k][i]))
                              for k in ("accept_len", "draft_index", "correction")},
                     float(ref["margin"][i]), gflags, oflags))
            continue
        if not diagnostics or o_inv:
            continue
        # softmax: ln-partition function of every row
        lg, lo = g["row_lse"][b].astype(np.float64), ref["row_lse"][i]
        rel = np.abs(lg - lo) / np.maximum(1.0, np.abs(lo))
        rep["max_lse_rel"] = max(rep["max_lse_rel"], float(np.nanmax(rel)))
        # acceptance probabilities where the GPU evaluated h
        hg, ho = g["accept_prob"][b].astype(np.float64), ref["accept_prob"][i]
        m = ~np.isnan(hg)
        assert not np.isnan(ho[m]).any(), (label, b, "GPU evaluated a test the oracle did not")
        if m.any():
            rep["max_h_abs"] = max(rep["max_h_abs"], float(np.abs(hg[m] - ho[m]).max()))
        # residual mass of the correction distribution
        zg, zo = float(g["resid_mass"][b]), float(ref["resid_mass"][i])
        zerr = abs(zg - zo) / max(abs(zo), Z_ATOL / Z_RTOL)
        rep["max_z_rel"] = max(rep["max_z_rel"], zerr)
    return rep


def check(rep):
    assert not rep["mismatch"], f"{rep['label']}: {len(rep['mismatch'])} unexcused mismatches, " \
                                f"first {rep['mismatch'][:3]}"
    assert not rep["unflagged_ties"], \
        f"{rep['label']}: oracle near ties the library did not flag: {rep['unflagged_ties'][:8]}"
    assert rep["excused"] <= rep["oracle_ties"], rep
    assert rep["max_lse_rel"] <= LSE_RTOL, rep
    assert rep["max_h_abs"] <= H_ATOL, rep
    assert rep["max_z_rel"] <= Z_RTOL, rep
    print(f"[parity] {rep['label']}: n={rep['n']} excused={rep['excused']} "
          f"oracle_ties={rep['oracle_ties']} invalid={rep['invalid']} "
          f"degenerate={rep['degenerate']} lse_rel={rep['max_lse_rel']:.2e} "
          f"h_abs={rep['max_h_abs']:.2e} z_rel={rep['max_z_rel']:.2e}", flush=True)


def gpu_batch(w: synth.Workload, seed: int):
    return synth.generate(w, seed, device="cuda")
