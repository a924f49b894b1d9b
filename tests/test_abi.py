"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/spec_verify.h declares,
and reject bad arguments on the host before any device call.
"""
import ctypes
import os
import re

import pytest

import draft_token_verification_online_amd as sv
from draft_token_verification_online_amd import build as svbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


@pytest.fixture(scope="module")
def lib():
    if svbuild.stale():
        svbuild.build()
    return sv.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("spec_verify_token", "spec_verify_block", "spec_verify_multidraft",
              "spec_verify_spectr", "spec_draft_sample", "spec_lm_head", "sv_workspace_size",
              "sv_draft_workspace_size", "sv_lm_workspace_size", "sv_status_string",
              "sv_version"):
        assert n in names


def test_flag_bits_match_the_header():
    text = open(HEADER).read()
    for name in ("SV_FLAG_DEGENERATE", "SV_FLAG_INVALID", "SV_FLAG_NEAR_TIE", "SV_FLAG_REDONE",
                 "SV_NEAR_TIE"):
        m = re.search(rf"^#define {name} (\S+)", text, flags=re.M)
        assert m, name
        assert float(m.group(1)) == float(getattr(sv, name)), name


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.sv_status_string(0) == b"ok"
    assert b"invalid" in lib.sv_status_string(1)
    assert lib.sv_status_string(99) == b"unknown status"
    assert lib.sv_version().count(b".") == 2


def test_workspace_size(lib):
    ws = sv.workspace_size
    big = ws(512, 8, 8, 151936, sv.SV_BF16)
    # row statistics (16 B per row) + per-request walk state, flag bytes and list entries,
    # 256-aligned,
    # + a 196 608-byte node list per request when K >= 3
    node_lists = 512 * 196608
    assert big % 256 == 0
    assert 512 * 8 * 17 * 16 + 512 * 8 * 8 + node_lists <= big < 2 * 512 * 8 * 17 * 16 + node_lists
    two = ws(512, 2, 8, 151936, sv.SV_BF16)
    assert two % 256 == 0 and 512 * 2 * 17 * 16 <= two < big - node_lists   # no node lists for K = 2
    assert ws(1, 1, 4, 32, sv.SV_F32) % 256 == 0 and ws(1, 1, 4, 32, sv.SV_F32) >= 9 * 16
    # the two list counters, and 256 command (344 B) and partial (24 B) slots of the
    # fp64 re-evaluation's teams
    assert ws(0, 1, 1, 1, sv.SV_F32) == 512 + 256 * (344 + 24)
    for bad in [(1, 0, 4, 32), (1, 65, 4, 32), (1, 1, 0, 32), (1, 1, 17, 32), (1, 1, 4, 0),
                (1, 1, 4, (1 << 22) + 1), (-1, 1, 4, 32)]:
        assert ws(*bad, sv.SV_F32) == 0, bad
    assert ws(1, 1, 4, 32, 7) == 0


def _call(lib, name, ins, outs, ln):
    f = getattr(lib, name)
    return f(ctypes.byref(ins) if ins is not None else None,
             ctypes.byref(outs) if outs is not None else None,
             ctypes.byref(ln) if ln is not None else None)


def _fake(B=2, K=1, L=4, V=32, dtype=sv.SV_F32, align=256):
    # host addresses are never dereferenced: every case below fails validation first
    base = 1 << 20
    ins = sv.SvInputs(B, K, L, V, dtype, base, base + 4096, base + 8192, base + 8448,
                      base + 8704, base + 8960)
    outs = sv.SvOutputs(base + 9216, base + 9472, base + 9728, None, None, None, None, None)
    ln = sv.SvLaunch(None, base * 2 + (0 if align == 256 else align), 1 << 20,
                     (ctypes.c_void_p * sv.N_PHASE_EVENTS)())
    return ins, outs, ln


@pytest.mark.parametrize("name", ["spec_verify_token", "spec_verify_block",
                                  "spec_verify_multidraft", "spec_verify_spectr"])
def test_host_validation_rejects_bad_arguments(lib, name):
    ins, outs, ln = _fake()
    assert _call(lib, name, None, outs, ln) == sv.SV_EINVAL
    assert _call(lib, name, ins, None, ln) == sv.SV_EINVAL
    assert _call(lib, name, ins, outs, None) == sv.SV_EINVAL
    for field, value in [("K", 0), ("L", 0), ("L", 17), ("V", 0), ("B", -3), ("dtype", 5),
                         ("K", 65)]:
        ins, outs, ln = _fake()
        setattr(ins, field, value)
        assert _call(lib, name, ins, outs, ln) == sv.SV_EINVAL, (field, value)
    for field in ("target_logits", "draft_logits", "draft_tokens", "temperature", "u_accept",
                  "u_correct"):
        ins, outs, ln = _fake()
        setattr(ins, field, None)
        assert _call(lib, name, ins, outs, ln) == sv.SV_EINVAL, field
    for field in ("accept_len", "draft_index", "correction"):
        ins, outs, ln = _fake()
        setattr(outs, field, None)
        assert _call(lib, name, ins, outs, ln) == sv.SV_EINVAL, field
    ins, outs, ln = _fake()
    ins.target_logits += 2                       # fp32 logits must be 4-byte aligned
    assert _call(lib, name, ins, outs, ln) == sv.SV_EINVAL
    ins, outs, ln = _fake()
    ln.workspace = None
    assert _call(lib, name, ins, outs, ln) == sv.SV_EWORKSPACE
    ins, outs, ln = _fake(align=64)
    assert _call(lib, name, ins, outs, ln) == sv.SV_EWORKSPACE
    ins, outs, ln = _fake()
    ln.workspace_bytes = 16
    assert _call(lib, name, ins, outs, ln) == sv.SV_EWORKSPACE
    ins, outs, ln = _fake(B=0)
    assert _call(lib, name, ins, outs, ln) == sv.SV_OK          # empty batch: nothing to do


@pytest.mark.parametrize("name", ["spec_verify_token", "spec_verify_block"])
def test_single_draft_entries_need_k1(lib, name):
    ins, outs, ln = _fake(K=2)
    assert _call(lib, name, ins, outs, ln) == sv.SV_EINVAL


def test_python_binding_refuses_host_tensors(lib):
    import torch
    B, K, L, V = 2, 1, 3, 16
    v = sv.Verifier.__new__(sv.Verifier)
    v.method, v.shape, v.dtype = "block", (B, K, L, V), torch.float32
    with pytest.raises(ValueError):
        sv.Verifier.__call__(v, torch.zeros(B, K, L + 1, V), torch.zeros(B, K, L, V),
                             torch.zeros(B, K, L, dtype=torch.int32), torch.ones(B),
                             torch.zeros(B, K, L), torch.zeros(B))


class _Arg:
    """What the binding inspects of a tensor argument before it passes a pointer
    on: shape, dtype, layout and device (no GPU is needed to check them)."""

    def __init__(self, shape, dtype, contiguous=True, device="cuda"):
        import types
        self.shape, self.dtype, self._c = tuple(shape), dtype, contiguous
        self.device = types.SimpleNamespace(type=device)

    def is_contiguous(self):
        return self._c

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for d in self.shape:
            n *= d
        return n


def test_python_binding_checks_every_argument(lib):
    """Shape, dtype, layout and device are checked for every argument of the
    three callable objects before anything reaches the library."""
    import torch
    f32, bf16, i32 = torch.float32, torch.bfloat16, torch.int32
    B, K, L, V = 2, 2, 3, 16
    v = sv.Verifier.__new__(sv.Verifier)
    v.method, v.shape, v.dtype = "multidraft", (B, K, L, V), f32
    vargs = [((B, K, L + 1, V), f32), ((B, K, L, V), f32), ((B, K, L), i32), ((B,), f32),
             ((B, K, L), f32), ((B,), f32)]
    d = sv.Drafter.__new__(sv.Drafter)
    d.shape, d.dtype = (B, K, L, V), bf16
    dargs = [((B, K, L, V), bf16), ((B,), f32), ((B, K, L), f32)]
    R, dm = 4, 64
    h = sv.LmHead.__new__(sv.LmHead)
    h.shape = (R, dm, V)
    hargs = [((R, dm), bf16), ((V, dm), bf16), ((R,), f32)]
    for obj, spec in ((v, vargs), (d, dargs), (h, hargs)):
        # good arguments pass every check: the call goes on to take their pointers
        with pytest.raises(AttributeError, match="data_ptr"):
            type(obj).__call__(obj, *[_Arg(s_, t_) for s_, t_ in spec])
        for i, (shp, dt) in enumerate(spec):
            other = torch.float64 if dt != torch.float64 else f32
            bad = [(_Arg(shp[:-1] + (shp[-1] + 1,), dt), "expected contiguous"),
                   (_Arg(shp, other), "expected contiguous"),
                   (_Arg(shp, dt, contiguous=False), "expected contiguous"),
                   (_Arg(shp, dt, device="cpu"), "GPU memory")]
            for b, msg in bad:
                a = [_Arg(s_, t_) for s_, t_ in spec]
                a[i] = b
                with pytest.raises(ValueError, match=msg):
                    type(obj).__call__(obj, *a)
    # the raw statistics buffers: dtype, layout, device and size
    u8 = torch.uint8
    good_h = [_Arg(s_, t_) for s_, t_ in hargs]
    need = ((R - 1) // 2 * 5 + 1 + (R - 1) % 2 + 1) * 16     # group 2, stride 5, offset 1
    with pytest.raises(AttributeError, match="data_ptr"):
        h(*good_h, stats=_Arg((need,), u8), group=2, stride=5, offset=1)
    for b, msg in [(_Arg((need - 1,), u8), "bytes"), (_Arg((need,), f32), "uint8"),
                   (_Arg((need,), u8, contiguous=False), "uint8"),
                   (_Arg((need,), u8, device="cpu"), "GPU memory")]:
        with pytest.raises(ValueError, match=msg):
            h(*good_h, stats=b, group=2, stride=5, offset=1)
    for grp, strd, off in [(0, 5, 1), (3, 2, 0), (2, 5, -1)]:
        with pytest.raises(ValueError, match="group"):
            h(*good_h, stats=_Arg((1 << 20,), u8), group=grp, stride=strd, offset=off)
    good_v = [_Arg(s_, t_) for s_, t_ in vargs]
    nst = B * K * (2 * L + 1) * 16
    with pytest.raises(AttributeError, match="data_ptr"):
        v(*good_v, row_stats=_Arg((nst,), u8))
    for b, msg in [(_Arg((nst - 16,), u8), "bytes"), (_Arg((nst,), i32), "uint8"),
                   (_Arg((nst,), u8, device="cpu"), "GPU memory")]:
        with pytest.raises(ValueError, match=msg):
            v(*good_v, row_stats=b)


def test_missing_library_fails_loudly(tmp_path):
    saved = sv._lib
    try:
        sv._lib = None
        with pytest.raises(sv.SpecVerifyError):
            sv.load_library(str(tmp_path / "nope.so"))
    finally:
        sv._lib = saved


def _fake_draft(B=2, K=2, L=3, V=32, dtype=sv.SV_F32):
    base = 1 << 20
    ins = sv.SvDraftInputs(B, K, L, V, dtype, base, base + 4096, base + 8192)
    outs = sv.SvDraftOutputs(base + 12288, None, None)
    ln = sv.SvLaunch(None, base * 2, 1 << 20, (ctypes.c_void_p * sv.N_PHASE_EVENTS)())
    return ins, outs, ln


def test_draft_host_validation(lib):
    f = lambda i, o, l: lib.spec_draft_sample(ctypes.byref(i) if i is not None else None,
                                              ctypes.byref(o) if o is not None else None,
                                              ctypes.byref(l) if l is not None else None)
    ins, outs, ln = _fake_draft()
    assert f(None, outs, ln) == sv.SV_EINVAL
    assert f(ins, None, ln) == sv.SV_EINVAL
    assert f(ins, outs, None) == sv.SV_EINVAL
    for field, value in [("K", 0), ("K", 65), ("L", 0), ("L", 17), ("V", 0), ("B", -1),
                         ("dtype", 3)]:
        ins, outs, ln = _fake_draft()
        setattr(ins, field, value)
        assert f(ins, outs, ln) == sv.SV_EINVAL, (field, value)
    for field in ("draft_logits", "temperature", "u_draft"):
        ins, outs, ln = _fake_draft()
        setattr(ins, field, None)
        assert f(ins, outs, ln) == sv.SV_EINVAL, field
    ins, outs, ln = _fake_draft()
    outs.draft_tokens = None
    assert f(ins, outs, ln) == sv.SV_EINVAL
    ins, outs, ln = _fake_draft()
    ins.draft_logits += 2
    assert f(ins, outs, ln) == sv.SV_EINVAL
    ins, outs, ln = _fake_draft()
    ln.workspace = None
    assert f(ins, outs, ln) == sv.SV_EWORKSPACE
    ins, outs, ln = _fake_draft()
    ln.workspace_bytes = 4
    assert f(ins, outs, ln) == sv.SV_EWORKSPACE
    ins, outs, ln = _fake_draft(B=0)
    assert f(ins, outs, ln) == sv.SV_OK
    # flags, list lengths, two list buffers (by position parity) and slots, then per node
    # row 38 tile shifts and tile sums
    big = lib.sv_draft_workspace_size(512, 8, 8, 151936, sv.SV_BF16)
    assert big % 256 == 0 and 4096 * 38 * 12 <= big < 4096 * 38 * 12 + 65536
    assert lib.sv_draft_workspace_size(1, 0, 8, 16, sv.SV_BF16) == 0


def test_row_stats_must_be_aligned(lib):
    ins, outs, ln = _fake(K=2)
    ins.row_stats = (1 << 20) + 8
    assert _call(lib, "spec_verify_multidraft", ins, outs, ln) == sv.SV_EINVAL


def test_lm_head_host_validation(lib):
    base = 1 << 20
    f = lambda i, o, l: lib.spec_lm_head(ctypes.byref(i) if i is not None else None,
                                         ctypes.byref(o) if o is not None else None,
                                         ctypes.byref(l) if l is not None else None)

    def fake(R=4, d=128, V=100):
        ins = sv.SvLmInputs(R, d, V, base, base + 4096, base + 8192)
        outs = sv.SvLmOutputs(base + 12288, None, 1, 1, 0)
        ln = sv.SvLaunch(None, base * 2, 1 << 24, (ctypes.c_void_p * sv.N_PHASE_EVENTS)())
        return ins, outs, ln

    ins, outs, ln = fake()
    assert f(None, outs, ln) == sv.SV_EINVAL and f(ins, None, ln) == sv.SV_EINVAL
    assert f(ins, outs, None) == sv.SV_EINVAL
    for field, value in [("d", 0), ("d", 64), ("d", 96), ("d", 70000), ("V", 0), ("R", -1)]:
        ins, outs, ln = fake()
        setattr(ins, field, value)
        assert f(ins, outs, ln) == sv.SV_EINVAL, (field, value)
    for field in ("hidden", "weight", "temperature"):
        ins, outs, ln = fake()
        setattr(ins, field, None)
        assert f(ins, outs, ln) == sv.SV_EINVAL, field
    ins, outs, ln = fake()
    ins.hidden += 8                                  # not 16-byte aligned
    assert f(ins, outs, ln) == sv.SV_EINVAL
    ins, outs, ln = fake()
    outs.logits = None
    assert f(ins, outs, ln) == sv.SV_EINVAL
    ins, outs, ln = fake()
    outs.row_stats, outs.stats_group, outs.stats_stride = base + 20480, 3, 2   # stride < group
    assert f(ins, outs, ln) == sv.SV_EINVAL
    ins, outs, ln = fake()
    ln.workspace_bytes = 16
    assert f(ins, outs, ln) == sv.SV_EWORKSPACE
    ins, outs, ln = fake(R=0)
    assert f(ins, outs, ln) == sv.SV_OK
    # partial (max, sum) per row and 256-column block
    assert lib.sv_lm_workspace_size(36864, 3584, 151936) >= 36864 * 594 * 12
    assert lib.sv_lm_workspace_size(4, 100, 16) == 0


def test_noalloc_entry_checks_sizes_on_the_host(lib):
    """spec_verify_multidraft_noalloc refuses null arguments and sizes whose
    workspace exceeds its scratch before any device call."""
    f = lib.spec_verify_multidraft_noalloc
    ins, outs, _ = _fake(B=2, K=4, L=4, V=64)
    assert f(None, ctypes.byref(outs), None) == sv.SV_EINVAL
    assert f(ctypes.byref(ins), None, None) == sv.SV_EINVAL
    ins.K = 0
    assert f(ctypes.byref(ins), ctypes.byref(outs), None) == sv.SV_EINVAL
    big = sv.SvInputs(1024, 4, 8, 151936, sv.SV_BF16, 1, 1, 1, 1, 1, 1, None)
    assert sv.workspace_size(1024, 4, 8, 151936, sv.SV_BF16) > sv.SV_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), ctypes.byref(outs), None) == sv.SV_EUNSUPPORTED
    text = open(HEADER).read()
    m = re.search(r"^#define SV_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text, flags=re.M)
    assert m and int(m.group(1)) << int(m.group(2)) == sv.SV_NOALLOC_SCRATCH_BYTES
