"""CPU oracle for batched draft-token verification (ctypes wrapper of spec_oracle.c).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never uses it and
shares no code with it; the product path fails loudly instead of falling back
here.

The C file states the rules it implements and the passages of the pages they
follow.  This wrapper only marshals numpy arrays and splits a batch across
host threads (each request is verified by the unmodified single-threaded
code; the C call releases the GIL).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "spec_oracle.c")
LIB = os.path.join(_HERE, "libsvoracle.so")

TOKEN, BLOCK, MULTI, SPECTR = 0, 1, 2, 3
F32, BF16 = 0, 1
FLAG_DEGENERATE, FLAG_INVALID = 1, 2
METHODS = {"token": TOKEN, "block": BLOCK, "multidraft": MULTI, "spectr": SPECTR}

_lock = threading.Lock()
_libs = {}


def build() -> str:
    """Compile spec_oracle.c with gcc (plain C99, no fast-math, no contraction)."""
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-o", LIB, SRC, "-lm"]
    subprocess.check_call(cmd)
    return LIB


def _load(path=None):
    """Load the oracle library (or, for tests that plant a mistake in a copy of
    the oracle, the library at `path`)."""
    with _lock:
        key = path or LIB
        if key in _libs:
            return _libs[key]
        if path is None and (not os.path.exists(LIB) or
                             os.path.getmtime(LIB) < os.path.getmtime(SRC)):
            build()
        lib = ctypes.CDLL(key)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.svo_draft.restype = ctypes.c_int
        lib.svo_draft.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, i32, i32,
                                  vp, vp, vp, vp]
        lib.svo_verify.restype = ctypes.c_int
        lib.svo_verify.argtypes = [i32, i32, i32, i32, i32, i32,
                                   vp, vp, vp, vp, vp, vp,
                                   i32, i32,
                                   vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.svo_verify_exact.restype = ctypes.c_int
        lib.svo_verify_exact.argtypes = [i32, i32, i32, i32, i32, i32,
                                         vp, vp, vp, vp, vp, vp,
                                         i32, i32,
                                         vp, vp, vp, vp, vp, vp, vp]
        _libs[key] = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_logits(a):
    """float32 array, or bf16 bit patterns as uint16; returns (contiguous array, dtype code)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"logits must be float32 or bf16 bits as uint16, got {a.dtype}")


def verify(method, target, draft, tokens, temperature, u_accept, u_correct, *,
           diagnostics: bool = False, threads: int = 1, requests=None,
           lib_path=None) -> dict:
    """Run the oracle on a batch held in host memory.

    target [B][K][L+1][V], draft [B][K][L][V]: float32, or bf16 as uint16 bits.
    tokens int32 [B][K][L]; temperature float32 [B]; u_accept float32 [B][K][L];
    u_correct float32 [B].  `requests` optionally restricts the work to a
    sorted list of request indices (the other outputs stay at their fill value).
    Returns a dict of numpy arrays: accept_len, draft_index, correction, flags,
    margin, counters [B][3] and, with diagnostics, row_lse, accept_prob, resid_mass.
    """
    lib = _load(lib_path)
    m = METHODS[method] if isinstance(method, str) else int(method)
    target, dt = _as_logits(target)
    draft, dt2 = _as_logits(draft)
    if dt != dt2:
        raise TypeError("target and draft logits must share a dtype")
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    u_accept = np.ascontiguousarray(u_accept, dtype=np.float32)
    u_correct = np.ascontiguousarray(u_correct, dtype=np.float32)
    B, K, L1, V = target.shape
    L = L1 - 1
    if draft.shape != (B, K, L, V) or tokens.shape != (B, K, L) or \
            u_accept.shape != (B, K, L) or temperature.shape != (B,) or u_correct.shape != (B,):
        raise ValueError("inconsistent shapes")

    out = {
        "accept_len": np.full(B, -2, np.int32),
        "draft_index": np.full(B, -2, np.int32),
        "correction": np.full(B, -2, np.int32),
        "flags": np.zeros(B, np.int32),
        "margin": np.full(B, np.nan, np.float64),
        "counters": np.zeros((B, 3), np.int64),
    }
    if diagnostics:
        out["row_lse"] = np.full((B, K, 2 * L + 1), np.nan, np.float64)
        out["accept_prob"] = np.full((B, K, L), np.nan, np.float64)
        out["resid_mass"] = np.full(B, np.nan, np.float64)

    def run(b0, b1):
        rc = lib.svo_verify(m, B, K, L, V, dt, _ptr(target), _ptr(draft), _ptr(tokens),
                            _ptr(temperature), _ptr(u_accept), _ptr(u_correct), b0, b1,
                            _ptr(out["accept_len"]), _ptr(out["draft_index"]),
                            _ptr(out["correction"]), _ptr(out["flags"]),
                            _ptr(out.get("row_lse")), _ptr(out.get("accept_prob")),
                            _ptr(out.get("resid_mass")), _ptr(out["margin"]),
                            _ptr(out["counters"]))
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (rc={rc})")

    if requests is None and threads <= 1:
        run(0, B)
        return out
    reqs = list(range(B)) if requests is None else sorted(int(b) for b in requests)
    if threads <= 1 or len(reqs) <= 1:
        for b in reqs:
            run(b, b + 1)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda b: run(b, b + 1), reqs))
    return out


def verify_exact(method, target, draft, tokens, temperature, u_accept, u_correct, *,
                 lib_path=None) -> dict:
    """svo_verify_exact: the oracle with float64 uniforms, returning accept_len,
    draft_index, correction, flags, accept_prob [B][K][L] and resid_mass [B]
    like verify(..., diagnostics=True), plus corr_law [B][V]: the distribution
    the correction token is drawn from.  For enumerating the output law exactly:
    u = 0 takes the accepting branch of a test with h > 0, u = h the rejecting
    one, and the correction's law is read off corr_law."""
    lib = _load(lib_path)
    m = METHODS[method] if isinstance(method, str) else int(method)
    target, dt = _as_logits(target)
    draft, dt2 = _as_logits(draft)
    if dt != dt2:
        raise TypeError("target and draft logits must share a dtype")
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    u_accept = np.ascontiguousarray(u_accept, dtype=np.float64)
    u_correct = np.ascontiguousarray(u_correct, dtype=np.float64)
    B, K, L1, V = target.shape
    L = L1 - 1
    if draft.shape != (B, K, L, V) or tokens.shape != (B, K, L) or \
            u_accept.shape != (B, K, L) or temperature.shape != (B,) or u_correct.shape != (B,):
        raise ValueError("inconsistent shapes")
    out = {
        "accept_len": np.full(B, -2, np.int32),
        "draft_index": np.full(B, -2, np.int32),
        "correction": np.full(B, -2, np.int32),
        "flags": np.zeros(B, np.int32),
        "accept_prob": np.full((B, K, L), np.nan, np.float64),
        "resid_mass": np.full(B, np.nan, np.float64),
        "corr_law": np.full((B, V), np.nan, np.float64),
    }
    rc = lib.svo_verify_exact(m, B, K, L, V, dt, _ptr(target), _ptr(draft), _ptr(tokens),
                              _ptr(temperature), _ptr(u_accept), _ptr(u_correct), 0, B,
                              _ptr(out["accept_len"]), _ptr(out["draft_index"]),
                              _ptr(out["correction"]), _ptr(out["flags"]),
                              _ptr(out["accept_prob"]), _ptr(out["resid_mass"]),
                              _ptr(out["corr_law"]))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return out


def draft(draft_logits, temperature, u_draft, *, threads: int = 1, requests=None,
          lib_path=None) -> dict:
    """Sample K i.i.d. draft blocks (svo_draft) on a batch held in host memory.

    draft_logits [B][K][L][V]: float32, or bf16 as uint16 bits; temperature
    float32 [B]; u_draft float32 [B][K][L].  Returns tokens [B][K][L], flags,
    margin and rows (node rows read) per request; requests outside `requests`
    keep tokens -2."""
    lib = _load(lib_path)
    d, dt = _as_logits(draft_logits)
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    u_draft = np.ascontiguousarray(u_draft, dtype=np.float32)
    B, K, L, V = d.shape
    if temperature.shape != (B,) or u_draft.shape != (B, K, L):
        raise ValueError("inconsistent shapes")
    out = {"tokens": np.full((B, K, L), -2, np.int32), "flags": np.zeros(B, np.int32),
           "margin": np.full(B, np.nan, np.float64), "rows": np.zeros(B, np.int32)}

    def run(b0, b1):
        rc = lib.svo_draft(B, K, L, V, dt, _ptr(d), _ptr(temperature), _ptr(u_draft), b0, b1,
                           _ptr(out["tokens"]), _ptr(out["flags"]), _ptr(out["margin"]),
                           _ptr(out["rows"]))
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (rc={rc})")

    reqs = list(range(B)) if requests is None else sorted(int(b) for b in requests)
    if requests is None and threads <= 1:
        run(0, B)
    elif threads <= 1 or len(reqs) <= 1:
        for b in reqs:
            run(b, b + 1)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda b: run(b, b + 1), reqs))
    return out


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) widened exactly to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def lm_head(hidden_bits, weight_bits, temperature):
    """Logits and their row statistics, the step that produces the verifier's
    inputs: logits[r][v] = sum_i h[r][i] w[v][i] over the bf16 hidden states
    [R][d] and the bf16 LM-head weight [V][d] (bit patterns, widened exactly),
    in float64 by a library matrix product; lse[r] = ln sum_v exp(l_rv / T_r),
    the natural-log partition function of the temperature softmax of each row
    (written out as max/T + ln sum exp((l - max)/T)).  Returns (logits, lse)."""
    h = bf16_bits_to_f64(hidden_bits)
    w = bf16_bits_to_f64(weight_bits)
    logits = h @ w.T
    T = np.asarray(temperature, np.float64).reshape(-1, 1)
    m = logits.max(axis=1, keepdims=True)
    lse = (m / T + np.log(np.exp((logits - m) / T).sum(axis=1, keepdims=True)))[:, 0]
    return logits, lse
