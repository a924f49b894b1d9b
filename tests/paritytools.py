"""Helpers for comparing the HIP path with the CPU oracle on the same inputs."""
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


def host_threads():
    return max(1, min(16, os.cpu_count() or 1))


def run_oracle(method, host, diagnostics=True, requests=None):
    return oracle.verify(method, host["target"], host["draft"], host["tokens"],
                         host["temperature"], host["u_accept"], host["u_correct"],
                         diagnostics=diagnostics, threads=host_threads(), requests=requests)


def compare(method, gpu_out, ref, requests, *, diagnostics=True, label=""):
    """Compare GPU outputs (dict of tensors over the whole batch) with oracle
    outputs (dict of arrays indexed by position in `requests`).  Returns a report;
    raises AssertionError on any unexcused mismatch or diagnostic outside tolerance."""
    g = {k: v.detach().cpu().numpy() for k, v in gpu_out.items()}
    req = np.asarray(requests)
    rep = {"label": label, "n": len(req), "excused": 0, "mismatch": [], "max_lse_rel": 0.0,
           "max_h_abs": 0.0, "max_z_rel": 0.0, "invalid": 0, "degenerate": 0}
    for i, b in enumerate(req):
        same = all(int(g[k][b]) == int(ref[k][i]) for k in ("accept_len", "draft_index",
                                                            "correction"))
        oflags = int(ref["flags"][i])
        gflags = int(g["flags"][b]) if "flags" in g else 0
        rep["invalid"] += bool(oflags & oracle.FLAG_INVALID)
        rep["degenerate"] += bool((oflags | gflags) & oracle.FLAG_DEGENERATE)
        near_tie = ref["margin"][i] < TIE_BAND or ((oflags | gflags) & oracle.FLAG_DEGENERATE)
        # the library flags every decision within 1e-5 of its threshold (SV_FLAG_NEAR_TIE = 4)
        if ref["margin"][i] < TIE_BAND and "flags" in g and not (oflags & oracle.FLAG_INVALID):
            assert gflags & 4, (label, int(b), "a near tie the library did not flag")
        if not same or (gflags & oracle.FLAG_INVALID) != (oflags & oracle.FLAG_INVALID):
            if near_tie and not ((gflags ^ oflags) & oracle.FLAG_INVALID):
                rep["excused"] += 1
            else:
                rep["mismatch"].append(
                    (int(b), {k: (int(g[k][b]), int(ref[k][i]))
                              for k in ("accept_len", "draft_index", "correction")},
                     float(ref["margin"][i]), gflags, oflags))
            continue
        if not diagnostics or oflags & oracle.FLAG_INVALID:
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
    assert rep["max_lse_rel"] <= LSE_RTOL, rep
    assert rep["max_h_abs"] <= H_ATOL, rep
    assert rep["max_z_rel"] <= Z_RTOL, rep
    print(f"[parity] {rep['label']}: n={rep['n']} excused={rep['excused']} "
          f"invalid={rep['invalid']} degenerate={rep['degenerate']} "
          f"lse_rel={rep['max_lse_rel']:.2e} h_abs={rep['max_h_abs']:.2e} "
          f"z_rel={rep['max_z_rel']:.2e}", flush=True)


def gpu_batch(w: synth.Workload, seed: int):
    return synth.generate(w, seed, device="cuda")
