"""Batched draft-token verification on AMD MI355X -- Python binding.

Thin ctypes layer over libspec_verify.so (C ABI in include/spec_verify.h).
It only marshals arguments: every step of the verification runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.
There is no CPU fallback: if the library is missing or the tensors are not on
a HIP device, the calls raise.

    from draft_token_verification_online_amd import spec_verify_multidraft
    out = spec_verify_multidraft(target, draft, tokens, temperature, u_accept, u_correct)
    out["accept_len"], out["draft_index"], out["correction"]
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspec_verify.so")

SV_OK, SV_EINVAL, SV_EUNSUPPORTED, SV_EHIP, SV_EWORKSPACE = range(5)
SV_F32, SV_BF16 = 0, 1
SV_FLAG_DEGENERATE, SV_FLAG_INVALID, SV_FLAG_NEAR_TIE, SV_FLAG_REDONE = 1, 2, 4, 8
SV_NEAR_TIE = 1e-5
SV_MAX_K, SV_MAX_L, SV_MAX_V = 64, 16, 1 << 22
SV_NOALLOC_SCRATCH_BYTES = 128 << 20

_vp = ctypes.c_void_p


class SvInputs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("K", ctypes.c_int32), ("L", ctypes.c_int32),
                ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("target_logits", _vp), ("draft_logits", _vp), ("draft_tokens", _vp),
                ("temperature", _vp), ("u_accept", _vp), ("u_correct", _vp),
                ("row_stats", _vp)]


class SvOutputs(ctypes.Structure):
    _fields_ = [("accept_len", _vp), ("draft_index", _vp), ("correction", _vp),
                ("flags", _vp), ("row_lse", _vp), ("accept_prob", _vp), ("resid_mass", _vp),
                ("rows_streamed", _vp)]


N_PHASE_EVENTS = 5


class SvLaunch(ctypes.Structure):
    _fields_ = [("stream", _vp), ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("phase_events", _vp * N_PHASE_EVENTS)]


class SvDraftInputs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("K", ctypes.c_int32), ("L", ctypes.c_int32),
                ("V", ctypes.c_int32), ("dtype", ctypes.c_int32), ("draft_logits", _vp),
                ("temperature", _vp), ("u_draft", _vp)]


class SvDraftOutputs(ctypes.Structure):
    _fields_ = [("draft_tokens", _vp), ("flags", _vp), ("rows_streamed", _vp)]


class SvLmInputs(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("d", ctypes.c_int32), ("V", ctypes.c_int32),
                ("hidden", _vp), ("weight", _vp), ("temperature", _vp)]


class SvLmOutputs(ctypes.Structure):
    _fields_ = [("logits", _vp), ("row_stats", _vp), ("stats_group", ctypes.c_int32),
                ("stats_stride", ctypes.c_int32), ("stats_offset", ctypes.c_int32),
                ("logits_dtype", ctypes.c_int32)]


class SpecVerifyError(RuntimeError):
    pass


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the C ABI library (built by draft_token_verification_online_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise SpecVerifyError(
            f"{path} is missing: build it with `python -m draft_token_verification_online_amd.build`"
            " (there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    lib.sv_workspace_size.restype = ctypes.c_size_t
    lib.sv_workspace_size.argtypes = [ctypes.c_int32] * 5
    for name in ("spec_verify_token", "spec_verify_block", "spec_verify_multidraft",
                 "spec_verify_spectr", "spec_verify_spectr_bisect"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(SvInputs), ctypes.POINTER(SvOutputs),
                      ctypes.POINTER(SvLaunch)]
    lib.spec_verify_multidraft_noalloc.restype = ctypes.c_int
    lib.spec_verify_multidraft_noalloc.argtypes = [ctypes.POINTER(SvInputs),
                                                   ctypes.POINTER(SvOutputs), _vp]
    lib.sv_draft_workspace_size.restype = ctypes.c_size_t
    lib.sv_draft_workspace_size.argtypes = [ctypes.c_int32] * 5
    lib.spec_draft_sample.restype = ctypes.c_int
    lib.spec_draft_sample.argtypes = [ctypes.POINTER(SvDraftInputs), ctypes.POINTER(SvDraftOutputs),
                                      ctypes.POINTER(SvLaunch)]
    lib.sv_lm_workspace_size.restype = ctypes.c_size_t
    lib.sv_lm_workspace_size.argtypes = [ctypes.c_int32] * 3
    lib.spec_lm_head.restype = ctypes.c_int
    lib.spec_lm_head.argtypes = [ctypes.POINTER(SvLmInputs), ctypes.POINTER(SvLmOutputs),
                                 ctypes.POINTER(SvLaunch)]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_status_string.argtypes = [ctypes.c_int]
    lib.sv_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def workspace_size(B, K, L, V, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (SV_BF16 if dtype == torch.bfloat16 else SV_F32)
    return int(load_library().sv_workspace_size(B, K, L, V, code))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_bytes(t, nbytes: int, what: str):
    """A raw device buffer argument: a contiguous uint8 tensor in GPU memory of
    at least `nbytes` bytes (the library writes or reads that many)."""
    if t.dtype != torch.uint8 or not t.is_contiguous() or t.dim() != 1:
        raise ValueError(f"{what} must be a contiguous 1-D uint8 tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must live in GPU memory")
    if t.numel() < nbytes:
        raise ValueError(f"{what} holds {t.numel()} bytes, {nbytes} needed")


class Verifier:
    """Holds outputs and workspace for repeated calls on inputs of one shape.

    method: "token", "block", "multidraft", "spectr" or "spectr_bisect" (SpecTr with its
    scaling factor found by plain bisection).  diagnostics=True also returns
    row_lse [B][K][2L+1], accept_prob [B][K][L] and resid_mass [B].  noalloc=True
    (multidraft only) calls spec_verify_multidraft_noalloc, which takes its
    workspace from scratch memory the library holds, so no workspace tensor is
    made here."""

    _ENTRY = {"token": "spec_verify_token", "block": "spec_verify_block",
              "multidraft": "spec_verify_multidraft", "spectr": "spec_verify_spectr",
              "spectr_bisect": "spec_verify_spectr_bisect"}

    def __init__(self, method, B, K, L, V, dtype, device="cuda", diagnostics=False,
                 with_flags=True, noalloc=False):
        lib = load_library()
        if method not in self._ENTRY:
            raise ValueError(f"unknown method {method!r}")
        if noalloc and method != "multidraft":
            raise ValueError("noalloc is a variant of spec_verify_multidraft only")
        self.method, self.shape = method, (B, K, L, V)
        self.dtype = dtype
        self.noalloc = noalloc
        self._fn = getattr(lib, "spec_verify_multidraft_noalloc" if noalloc
                           else self._ENTRY[method])
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.out = {"accept_len": torch.empty(B, **i32),
                    "draft_index": torch.empty(B, **i32),
                    "correction": torch.empty(B, **i32)}
        if with_flags or diagnostics:
            self.out["flags"] = torch.empty(B, **i32)
            self.out["rows_streamed"] = torch.empty(B, **i32)
        if diagnostics:
            f32 = dict(dtype=torch.float32, device=dev)
            self.out["row_lse"] = torch.empty((B, K, 2 * L + 1), **f32)
            self.out["accept_prob"] = torch.empty((B, K, L), **f32)
            self.out["resid_mass"] = torch.empty(B, **f32)
        nbytes = workspace_size(B, K, L, V, _dtype_code(torch.empty((), dtype=dtype)))
        if nbytes == 0:
            raise ValueError(f"sizes out of range: B={B} K={K} L={L} V={V}")
        self.workspace = None if noalloc else torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self._outs = SvOutputs(*[_ptr(self.out.get(k)) for k in
                                 ("accept_len", "draft_index", "correction", "flags",
                                  "row_lse", "accept_prob", "resid_mass", "rows_streamed")])

    def __call__(self, target, draft, tokens, temperature, u_accept, u_correct, *,
                 stream=None, events=None, row_stats=None):
        """row_stats: optional uint8 device tensor holding [B][K][2L+1] statistics
        (16 bytes each, e.g. from LmHead); the statistics pass is then skipped."""
        B, K, L, V = self.shape
        checks = [(target, (B, K, L + 1, V), self.dtype), (draft, (B, K, L, V), self.dtype),
                  (tokens, (B, K, L), torch.int32), (temperature, (B,), torch.float32),
                  (u_accept, (B, K, L), torch.float32), (u_correct, (B,), torch.float32)]
        for t, shp, dt in checks:
            if tuple(t.shape) != shp or t.dtype != dt or not t.is_contiguous():
                raise ValueError(f"expected contiguous {dt} tensor of shape {shp}, "
                                 f"got {t.dtype} {tuple(t.shape)}")
            if t.device.type != "cuda":
                raise ValueError("inputs must live in GPU memory")
        if row_stats is not None:
            _check_bytes(row_stats, B * K * (2 * L + 1) * 16, "row_stats")
        ins = SvInputs(B, K, L, V, _dtype_code(target), target.data_ptr(), draft.data_ptr(),
                       tokens.data_ptr(), temperature.data_ptr(), u_accept.data_ptr(),
                       u_correct.data_ptr(), _ptr(row_stats))
        if stream is None:
            stream = torch.cuda.current_stream(target.device).cuda_stream
        if self.noalloc:
            rc = self._fn(ctypes.byref(ins), ctypes.byref(self._outs), stream)
            name = "spec_verify_multidraft_noalloc"
        else:
            ev = (_vp * N_PHASE_EVENTS)(*(events or (None,) * N_PHASE_EVENTS))
            ln = SvLaunch(stream, self.workspace.data_ptr(), self.workspace.numel(), ev)
            rc = self._fn(ctypes.byref(ins), ctypes.byref(self._outs), ctypes.byref(ln))
            name = self._ENTRY[self.method]
        if rc != SV_OK:
            msg = load_library().sv_status_string(rc).decode()
            raise SpecVerifyError(f"{name} failed: {msg} ({rc})")
        return self.out


class Drafter:
    """Holds outputs and workspace for repeated draft sampling on one shape:
    K i.i.d. draft blocks of length L per request from [B][K][L][V] draft logits
    (see spec_draft_sample in include/spec_verify.h)."""

    def __init__(self, B, K, L, V, dtype, device="cuda"):
        lib = load_library()
        self.shape, self.dtype = (B, K, L, V), dtype
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.out = {"draft_tokens": torch.empty((B, K, L), **i32),
                    "flags": torch.empty(B, **i32), "rows_streamed": torch.empty(B, **i32)}
        code = SV_BF16 if dtype == torch.bfloat16 else SV_F32
        nbytes = int(lib.sv_draft_workspace_size(B, K, L, V, code))
        if nbytes == 0:
            raise ValueError(f"sizes out of range: B={B} K={K} L={L} V={V}")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self._outs = SvDraftOutputs(*[_ptr(self.out[k]) for k in
                                      ("draft_tokens", "flags", "rows_streamed")])

    def __call__(self, draft_logits, temperature, u_draft, *, stream=None, events=None):
        B, K, L, V = self.shape
        checks = [(draft_logits, (B, K, L, V), self.dtype), (temperature, (B,), torch.float32),
                  (u_draft, (B, K, L), torch.float32)]
        for t, shp, dt in checks:
            if tuple(t.shape) != shp or t.dtype != dt or not t.is_contiguous():
                raise ValueError(f"expected contiguous {dt} tensor of shape {shp}, "
                                 f"got {t.dtype} {tuple(t.shape)}")
            if t.device.type != "cuda":
                raise ValueError("inputs must live in GPU memory")
        ins = SvDraftInputs(B, K, L, V, _dtype_code(draft_logits), draft_logits.data_ptr(),
                            temperature.data_ptr(), u_draft.data_ptr())
        if stream is None:
            stream = torch.cuda.current_stream(draft_logits.device).cuda_stream
        ev = (_vp * N_PHASE_EVENTS)(*(events or (None,) * N_PHASE_EVENTS))
        ln = SvLaunch(stream, self.workspace.data_ptr(), self.workspace.numel(), ev)
        lib = load_library()
        rc = lib.spec_draft_sample(ctypes.byref(ins), ctypes.byref(self._outs), ctypes.byref(ln))
        if rc != SV_OK:
            raise SpecVerifyError(f"spec_draft_sample failed: "
                                  f"{lib.sv_status_string(rc).decode()} ({rc})")
        return self.out


class LmHead:
    """The LM head logits = h W^T (bf16 in, fp32 or bf16 logits out) with every
    row's temperature-softmax statistics computed in the same kernel
    (spec_lm_head in include/spec_verify.h).  Holds the logits output and the
    workspace."""

    STAT_BYTES = 16

    def __init__(self, R, d, V, device="cuda", logits_dtype=torch.float32):
        lib = load_library()
        self.shape = (R, d, V)
        dev = torch.device(device)
        self.logits = torch.empty((R, V), dtype=logits_dtype, device=dev)
        self._dt = _dtype_code(self.logits)
        nbytes = int(lib.sv_lm_workspace_size(R, d, V))
        if nbytes == 0:
            raise ValueError(f"sizes out of range: R={R} d={d} V={V} (d a multiple of 64, at least 128)")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def __call__(self, hidden, weight, temperature, *, stats=None, group=1, stride=1, offset=0,
                 stream=None, events=None):
        """hidden [R][d] and weight [V][d] bf16, temperature [R] fp32 (the row's
        request temperature).  stats: optional uint8 device tensor receiving
        row r's statistics at slot (r // group) * stride + offset + r % group."""
        R, d, V = self.shape
        for t, shp, dt in [(hidden, (R, d), torch.bfloat16), (weight, (V, d), torch.bfloat16),
                           (temperature, (R,), torch.float32)]:
            if tuple(t.shape) != shp or t.dtype != dt or not t.is_contiguous():
                raise ValueError(f"expected contiguous {dt} tensor of shape {shp}, "
                                 f"got {t.dtype} {tuple(t.shape)}")
            if t.device.type != "cuda":
                raise ValueError("inputs must live in GPU memory")
        if stats is not None:
            if not (group >= 1 and stride >= group and offset >= 0):
                raise ValueError("stats slots need group >= 1, stride >= group, offset >= 0")
            last = ((R - 1) // group) * stride + offset + (R - 1) % group if R > 0 else -1
            _check_bytes(stats, (last + 1) * self.STAT_BYTES, "stats")
        ins = SvLmInputs(R, d, V, hidden.data_ptr(), weight.data_ptr(), temperature.data_ptr())
        outs = SvLmOutputs(self.logits.data_ptr(), _ptr(stats), group, stride, offset, self._dt)
        if stream is None:
            stream = torch.cuda.current_stream(hidden.device).cuda_stream
        ev = (_vp * N_PHASE_EVENTS)(*(events or (None,) * N_PHASE_EVENTS))
        ln = SvLaunch(stream, self.workspace.data_ptr(), self.workspace.numel(), ev)
        lib = load_library()
        rc = lib.spec_lm_head(ctypes.byref(ins), ctypes.byref(outs), ctypes.byref(ln))
        if rc != SV_OK:
            raise SpecVerifyError(f"spec_lm_head failed: {lib.sv_status_string(rc).decode()} ({rc})")
        return self.logits


def spec_draft_sample(draft_logits, temperature, u_draft, **kw):
    """Draw K i.i.d. draft blocks per request.  See include/spec_verify.h."""
    B, K, L, V = draft_logits.shape
    d = Drafter(B, K, L, V, draft_logits.dtype, device=draft_logits.device)
    return dict(d(draft_logits, temperature, u_draft, **kw))


def _run(method, target, draft, tokens, temperature, u_accept, u_correct, diagnostics, **kw):
    B, K, L1, V = target.shape
    v = Verifier(method, B, K, L1 - 1, V, target.dtype, device=target.device,
                 diagnostics=diagnostics)
    return dict(v(target, draft, tokens, temperature, u_accept, u_correct, **kw))


def spec_verify_token(target, draft, tokens, temperature, u_accept, u_correct, *,
                      diagnostics=False, **kw):
    """Token-level speculative sampling (K = 1).  See include/spec_verify.h."""
    return _run("token", target, draft, tokens, temperature, u_accept, u_correct,
                diagnostics, **kw)


def spec_verify_block(target, draft, tokens, temperature, u_accept, u_correct, *,
                      diagnostics=False, **kw):
    """Greedy block verification of one draft (K = 1).  See include/spec_verify.h."""
    return _run("block", target, draft, tokens, temperature, u_accept, u_correct,
                diagnostics, **kw)


def spec_verify_multidraft(target, draft, tokens, temperature, u_accept, u_correct, *,
                           diagnostics=False, **kw):
    """Block verification over K i.i.d. drafts.  See include/spec_verify.h."""
    return _run("multidraft", target, draft, tokens, temperature, u_accept, u_correct,
                diagnostics, **kw)


def spec_verify_spectr(target, draft, tokens, temperature, u_accept, u_correct, *,
                       diagnostics=False, **kw):
    """SpecTr's position-by-position verification of K i.i.d. drafts.  See
    include/spec_verify.h."""
    return _run("spectr", target, draft, tokens, temperature, u_accept, u_correct,
                diagnostics, **kw)


__all__ = ["spec_verify_token", "spec_verify_block", "spec_verify_multidraft",
           "spec_verify_spectr", "spec_draft_sample", "Verifier", "Drafter", "LmHead",
           "workspace_size", "load_library", "SpecVerifyError"]
