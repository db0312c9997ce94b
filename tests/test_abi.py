"""The C-ABI library loads, exports what include/deformagg.h declares, and
rejects malformed calls on the host before any HIP call (no GPU needed).

Pointers passed here are fake, suitably aligned addresses: every call in
this file fails a host-side check, so nothing is dereferenced or launched.
"""
import ctypes

import numpy as np
import pytest

from view_deformable_feature_amd import _lib
from view_deformable_feature_amd.build import LIB_PATH, build, is_stale


@pytest.fixture(scope="module")
def lib():
    if is_stale():
        build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _lib.declared_functions()
    assert set(names) >= {"da_forward", "da_backward", "da_backward_accumulate",
                          "da_backward_atomic", "da_backward_workspace_size",
                          "da_forward_workspace_size", "da_status_string", "da_last_error",
                          "da_version"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in deformagg.h but not exported"


def test_version_and_status_strings(lib):
    assert lib.da_version() == 120
    for code in range(4):
        assert lib.da_status_string(code)
    assert b"unknown" in lib.da_status_string(99)


FAKE = 0x10000000          # 256-byte aligned fake device address
HOST_SHAPE = np.array([[[16, 16]]], np.int32)
HOST_START = np.array([[0]], np.int32)


def _prob(**kw):
    d = dict(bs=1, num_feat=256, num_embeds=32, num_anchors=8, num_pts=4, num_cams=1,
             num_scale=1, num_groups=1, feat_dtype=0, flags=0, out_dtype=0, reserved=0)
    d.update(kw)
    return _lib.DAProblem(**d)


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _fwd(lib, prob, feat=FAKE, shape=HOST_SHAPE, start=HOST_START, loc=FAKE, w=FAKE, out=FAKE,
         ws=0, ws_bytes=0):
    vp = ctypes.c_void_p
    return lib.da_forward(ctypes.byref(prob) if prob is not None else None, vp(feat),
                          _i32p(shape) if shape is not None else None,
                          _i32p(start) if start is not None else None,
                          vp(loc), vp(w), vp(out), vp(ws), ws_bytes, None)


def _bwd(lib, prob, name="da_backward", feat=FAKE, loc=FAKE, w=FAKE, go=FAKE, gf=FAKE, gl=FAKE,
         gw=FAKE, shape=HOST_SHAPE, start=HOST_START, ws=FAKE, ws_bytes=1 << 40):
    vp = ctypes.c_void_p
    args = [ctypes.byref(prob), vp(feat), _i32p(shape), _i32p(start), vp(loc), vp(w), vp(go),
            vp(gf), vp(gl), vp(gw)]
    if name in ("da_backward_atomic", "da_backward_noalloc"):
        return getattr(lib, name)(*args, None)
    return getattr(lib, name)(*args, vp(ws), ws_bytes, None)


def _msg(lib):
    return lib.da_last_error().decode()


@pytest.mark.parametrize("kw, code, needle", [
    (dict(num_embeds=30, num_groups=4), 1, "multiple of num_groups"),
    (dict(num_cams=0), 1, ">= 1"),
    (dict(num_scale=0), 1, ">= 1"),
    (dict(num_groups=0), 1, ">= 1"),
    (dict(num_feat=0), 1, ">= 1"),
    (dict(bs=-1), 1, ">= 0"),
    (dict(num_anchors=-2), 1, ">= 0"),
    (dict(num_pts=-1), 1, ">= 0"),
    (dict(feat_dtype=7), 1, "feat_dtype"),
    (dict(feat_dtype=-1), 1, "feat_dtype"),
    (dict(out_dtype=3), 1, "out_dtype"),
    (dict(reserved=1), 1, "reserved"),
    (dict(flags=3), 1, "flags"),
    (dict(flags=7), 1, "flags"),
    (dict(flags=12), 1, "flags"),
    (dict(flags=32), 1, "flags"),
    (dict(flags=-1), 1, "flags"),
    (dict(num_feat=255), 1, "inside num_feat"),
    (dict(num_cams=9, num_scale=8), 1, "DA_MAX_LEVELS"),
])
def test_forward_rejects_malformed_problem(lib, kw, code, needle):
    prob = _prob(**kw)
    shape, start = HOST_SHAPE, HOST_START
    if prob.num_cams * prob.num_scale > 1 and prob.num_cams * prob.num_scale <= 64:
        shape = np.tile(HOST_SHAPE, (prob.num_cams, prob.num_scale, 1))
        start = np.zeros((prob.num_cams, prob.num_scale), np.int32)
    elif prob.num_cams * prob.num_scale > 64:
        shape = np.ones((prob.num_cams, prob.num_scale, 2), np.int32)
        start = np.zeros((prob.num_cams, prob.num_scale), np.int32)
    assert _fwd(lib, prob, shape=shape, start=start) == code
    assert needle in _msg(lib)


@pytest.mark.parametrize("H, W, st, needle", [
    (0, 16, 0, "outside [1"),
    (16, 0, 0, "outside [1"),
    (40000, 1, 0, "outside [1"),
    (16, 16, -1, "inside num_feat"),
    (16, 16, 1, "inside num_feat"),
])
def test_rejects_bad_level_table(lib, H, W, st, needle):
    shape = np.array([[[H, W]]], np.int32)
    start = np.array([[st]], np.int32)
    assert _fwd(lib, _prob(num_feat=40000 if H == 40000 else 256), shape=shape, start=start) == 1
    assert needle in _msg(lib)
    assert _bwd(lib, _prob(num_feat=40000 if H == 40000 else 256), shape=shape, start=start) == 1


def test_rejects_null_pointers(lib):
    p = _prob()
    assert lib.da_forward(None, None, None, None, None, None, None, None, 0, None) == 1
    assert "problem is NULL" in _msg(lib)
    assert _fwd(lib, p, shape=None) == 1
    assert _fwd(lib, p, feat=0) == 1 and "mc_ms_feat" in _msg(lib)
    assert _fwd(lib, p, loc=0) == 1 and "sampling_location" in _msg(lib)
    assert _fwd(lib, p, w=0) == 1
    assert _fwd(lib, p, out=0) == 1 and "out is NULL" in _msg(lib)
    for kw, needle in ((dict(go=0), "grad_out"), (dict(gf=0), "grad_feat"),
                       (dict(gl=0), "grad_loc"), (dict(gw=0), "grad_loc / grad_weights")):
        for name in ("da_backward", "da_backward_accumulate", "da_backward_atomic"):
            assert _bwd(lib, p, name, **kw) == 1
            assert needle in _msg(lib)


def test_rejects_misaligned_pointers(lib):
    p = _prob()
    assert _fwd(lib, p, feat=FAKE + 2) == 1 and "element aligned" in _msg(lib)
    assert _fwd(lib, p, loc=FAKE + 4) == 1 and "8-byte" in _msg(lib)
    assert _fwd(lib, p, w=FAKE + 1) == 1
    assert _fwd(lib, p, out=FAKE + 2) == 1
    assert _bwd(lib, p, gl=FAKE + 4) == 1 and "grad_loc" in _msg(lib)
    assert _bwd(lib, p, gf=FAKE + 1) == 1
    # 16-bit features, out and grad_out need 2-byte alignment only
    for dt in (1, 2):
        assert _fwd(lib, _prob(feat_dtype=dt), feat=FAKE + 1) == 1
        assert _fwd(lib, _prob(out_dtype=dt), out=FAKE + 1) == 1 and "out" in _msg(lib)
        assert _bwd(lib, _prob(out_dtype=dt), go=FAKE + 1) == 1 and "grad_out" in _msg(lib)
        assert _bwd(lib, _prob(out_dtype=dt), "da_backward_atomic", go=FAKE + 1) == 1


def test_rejects_unsupported_sizes(lib):
    # a batch image beyond the 32-bit buffer range
    n = (1 << 32) // (256 * 4)
    shape = np.array([[[n // 8, 8]]], np.int32)
    p = _prob(num_feat=n, num_embeds=256, num_groups=8)
    assert _fwd(lib, p, shape=np.array([[[16, 16]]], np.int32)) == 2
    assert "4 GiB" in _msg(lib)
    # backward: too many channels per lane (C / pow2-part-of-group-width > 16)
    p = _prob(num_embeds=192, num_groups=8)
    assert _bwd(lib, p) == 2 and "exceeds 16" in _msg(lib)
    # too many channels
    p = _prob(num_embeds=(1 << 20) + 8, num_groups=1)
    assert _fwd(lib, p) == 2
    # LDS: one (point, camera) pair with a huge S * G does not fit
    p = _prob(num_embeds=4096, num_groups=4096, num_scale=64)
    shape = np.tile(HOST_SHAPE, (1, 64, 1))
    start = np.zeros((1, 64), np.int32)
    assert _fwd(lib, p, shape=shape, start=start) == 2 and "LDS" in _msg(lib)


def test_last_error_is_per_thread(lib):
    import threading
    assert _fwd(lib, _prob(num_embeds=30, num_groups=4)) == 1
    seen = {}

    def other():
        seen["msg"] = lib.da_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "multiple" in _msg(lib)


def test_binding_refuses_cpu_tensors():
    import torch
    import view_deformable_feature_amd as vdf
    wl_shape = np.array([[[4, 4]]], np.int32)
    feat = torch.zeros(1, 16, 4)
    loc = torch.zeros(1, 1, 1, 1, 2)
    w = torch.zeros(1, 1, 1, 1, 1, 1)
    with pytest.raises(ValueError, match="no CPU path"):
        vdf.da_forward(feat, wl_shape, np.zeros((1, 1), np.int32), loc, w)


def test_workspace_size_and_checks(lib):
    n = ctypes.c_size_t(0)
    p = _prob()
    assert lib.da_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    # scan counter + counts + local prefix + tile prefix + ranks + 16-byte entries + location
    # partials + per-corner group dot products (row-ordered form, G = 1), each 256-aligned
    n_rows, n_samples = 256, 8 * 4
    expect = 256 + 2 * 4 * n_rows + 256 + n_samples * 16 + n_samples * 4 * 16 + 256 + 512
    assert lib.da_backward_workspace_size(ctypes.byref(_prob(flags=4)), ctypes.byref(n)) == 0
    assert n.value == expect - 512                       # per-anchor form: no dot products
    # C/G = 24 channels per group: 6 lanes per group, not a power of two -> per-anchor form
    assert lib.da_backward_workspace_size(ctypes.byref(_prob(num_embeds=48, num_groups=2)),
                                          ctypes.byref(n)) == 0
    assert n.value == 256 + 2 * 4 * n_rows + 256 + n_samples * 16 + n_samples * 4 * 16 + 256
    # deterministic form: + one 64-bit row of C and a row index per possible long row
    # (4 * 32 // 65 + 1 = 2), + two words per counting block (one), 256-byte aligned
    assert lib.da_backward_workspace_size(ctypes.byref(_prob(flags=16)), ctypes.byref(n)) == 0
    assert n.value == expect + -(-(2 * (32 * 8 + 4) + 8) // 256) * 256
    assert _bwd(lib, _prob(flags=16), "da_backward_atomic") == 2 and "deterministic" in _msg(lib)
    # a 16-bit grad_out: + its binary32 copy, bs * A * C * 4 bytes
    for dt in (1, 2):
        assert lib.da_backward_workspace_size(ctypes.byref(_prob(out_dtype=dt)),
                                              ctypes.byref(n)) == 0
        assert n.value == expect + 8 * 32 * 4
        assert _bwd(lib, _prob(out_dtype=dt), ws_bytes=expect + 8 * 32 * 4 - 1) == 1
        assert "needed" in _msg(lib)
    assert lib.da_backward_workspace_size(ctypes.byref(_prob(out_dtype=9)), ctypes.byref(n)) == 1
    assert lib.da_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value == expect
    assert lib.da_backward_workspace_size(ctypes.byref(_prob(num_pts=0)), ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.da_backward_workspace_size(None, ctypes.byref(n)) == 1
    assert lib.da_backward_workspace_size(ctypes.byref(p), None) == 1
    big = _prob(bs=1 << 12, num_anchors=1 << 12, num_pts=1 << 7)
    assert lib.da_backward_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 2
    for name in ("da_backward", "da_backward_accumulate"):
        assert _bwd(lib, p, name, ws=0) == 1 and "workspace is NULL" in _msg(lib)
        assert _bwd(lib, p, name, ws=FAKE + 16) == 1 and "256-byte" in _msg(lib)
        assert _bwd(lib, p, name, ws_bytes=expect - 1) == 1 and "needed" in _msg(lib)


def _fws(lib, prob):
    n = ctypes.c_size_t(123)
    assert lib.da_forward_workspace_size(ctypes.byref(prob), ctypes.byref(n)) == 0
    return n.value


def test_forward_workspace_size_follows_the_slicing_rule(lib):
    # nuScenes-shaped: 6 cameras x 4 scales, 89,760 rows of 256 floats (92 MB)
    nus = dict(num_feat=89760, num_embeds=256, num_groups=8, num_anchors=900, num_pts=13,
               num_cams=6, num_scale=4)
    assert _fws(lib, _prob(**nus)) == 8 * 900 * 256 * 4
    assert _fws(lib, _prob(bs=2, **nus)) == 8 * 2 * 900 * 256 * 4
    assert _fws(lib, _prob(flags=2, **nus)) == 0                  # slices never
    # features within twice one die's L2: no slices unless forced
    assert _fws(lib, _prob(**dict(nus, num_feat=8000))) == 0
    assert _fws(lib, _prob(flags=1, **dict(nus, num_feat=8000))) == 8 * 900 * 256 * 4
    # 12 levels leave a third of the 16 slots idle; 20 leave a sixth
    assert _fws(lib, _prob(**dict(nus, num_cams=3))) == 0
    assert _fws(lib, _prob(**dict(nus, num_cams=5))) == 8 * 900 * 256 * 4
    assert _fws(lib, _prob(**dict(nus, num_cams=1))) == 0         # 4 levels
    assert _fws(lib, _prob(flags=1)) == 8 * 8 * 32 * 4            # forced, one level
    assert _fws(lib, _prob()) == 0
    assert _fws(lib, _prob(num_anchors=0, flags=1)) == 0
    n = ctypes.c_size_t(0)
    assert lib.da_forward_workspace_size(None, ctypes.byref(n)) == 1
    assert lib.da_forward_workspace_size(ctypes.byref(_prob()), None) == 1


def test_backward_sample_limit(lib):
    # the gather form keeps entry positions (4 per sample) below 2^31: a flag takes
    # their top bit, so 2^29 samples are refused and one fewer is sized
    n = ctypes.c_size_t(0)
    # 4 channels: grad_out (2 GiB) and weights (2 GiB) stay under the 4 GiB buffer range
    below = _prob(num_anchors=(1 << 27) - 1, num_pts=4, num_embeds=4)   # 2^29 - 4 samples
    assert lib.da_backward_workspace_size(ctypes.byref(below), ctypes.byref(n)) == 0
    assert n.value > 88 * ((1 << 29) - 4)
    at = _prob(num_anchors=1 << 27, num_pts=4, num_embeds=4)            # 2^29 samples
    assert lib.da_backward_workspace_size(ctypes.byref(at), ctypes.byref(n)) == 2
    assert "sample count" in _msg(lib)


def test_forward_workspace_checks(lib):
    p = _prob(flags=1)
    need = 8 * 8 * 32 * 4
    assert _fwd(lib, p, ws=FAKE + 16, ws_bytes=need) == 1 and "256-byte" in _msg(lib)
    assert _fwd(lib, p, ws=FAKE, ws_bytes=need - 1) == 1 and "needed" in _msg(lib)
    # a malformed problem is reported before the workspace is looked at
    assert _fwd(lib, _prob(flags=3), ws=FAKE + 16, ws_bytes=0) == 1 and "flags" in _msg(lib)


# ---------------------------------------------------------------------------------------
# deformable convolution (include/dcn.h): host-side checks only
# ---------------------------------------------------------------------------------------

def _dprob(**kw):
    d = dict(batch=2, height=8, width=9, channels=16, groups=4, kernel_h=3, kernel_w=3,
             stride_h=1, stride_w=1, pad_h=1, pad_w=1, dilation_h=1, dilation_w=1,
             in_dtype=0, out_dtype=0, flags=0, reserved=0)
    d.update(kw)
    return _lib.DCNProblem(**d)


def _dcn_fwd(lib, prob, inp=FAKE, om=FAKE, out=FAKE):
    vp = ctypes.c_void_p
    return lib.dcn_forward(ctypes.byref(prob), vp(inp), vp(om), vp(out), None)


def _dcn_bwd(lib, prob, inp=FAKE, om=FAKE, go=FAKE, gi=FAKE, gom=FAKE):
    vp = ctypes.c_void_p
    return lib.dcn_backward(ctypes.byref(prob), vp(inp), vp(om), vp(go), vp(gi), vp(gom),
                            None, 0, None)


def test_dcn_out_size(lib):
    ho, wo = ctypes.c_int64(0), ctypes.c_int64(0)
    for kw, expect in ((dict(), (8, 9)), (dict(stride_h=2, stride_w=2), (4, 5)),
                       (dict(kernel_h=3, kernel_w=5, pad_h=1, pad_w=2, dilation_h=2), (6, 9)),
                       (dict(kernel_h=1, kernel_w=1, pad_h=0, pad_w=0), (8, 9))):
        assert lib.dcn_out_size(ctypes.byref(_dprob(**kw)), ctypes.byref(ho), ctypes.byref(wo)) == 0
        assert (ho.value, wo.value) == expect, kw


@pytest.mark.parametrize("kw, code, needle", [
    (dict(channels=18), 1, "multiple of groups"),
    (dict(groups=0), 1, ">= 1"),
    (dict(height=0), 1, ">= 1"),
    (dict(batch=-1), 1, "batch"),
    (dict(stride_h=0), 1, "stride"),
    (dict(dilation_w=0), 1, "dilation"),
    (dict(pad_h=-1), 1, "padding"),
    (dict(kernel_h=11, pad_h=0), 1, "does not fit"),
    (dict(in_dtype=3), 1, "da_dtype"),
    (dict(out_dtype=-1), 1, "da_dtype"),
    (dict(flags=1), 1, "flags"),
    (dict(reserved=2), 1, "reserved"),
    (dict(channels=1 << 17, groups=1), 2, "2^16"),
    (dict(channels=2048, groups=4), 2, "channels per group"),
    (dict(batch=64, height=1024, width=1024, channels=64, groups=4), 2, "4 GiB"),
    # a 1x1 input padded to a 39999x39999 output: out and offset_mask reach 4 GiB
    (dict(batch=1, height=1, width=1, channels=1, groups=1, pad_h=20000, pad_w=20000), 2,
     "offset_mask"),
])
def test_dcn_rejects_malformed_problem(lib, kw, code, needle):
    assert _dcn_fwd(lib, _dprob(**kw)) == code
    assert needle in _msg(lib)
    assert _dcn_bwd(lib, _dprob(**kw)) == code


def test_dcn_rejects_null_and_misaligned(lib):
    p = _dprob()
    assert _dcn_fwd(lib, p, inp=0) == 1 and "NULL" in _msg(lib)
    assert _dcn_fwd(lib, p, om=0) == 1
    assert _dcn_fwd(lib, p, out=0) == 1
    assert _dcn_fwd(lib, p, out=FAKE + 2) == 1 and "aligned" in _msg(lib)
    assert _dcn_fwd(lib, _dprob(in_dtype=2), inp=FAKE + 1) == 1
    assert _dcn_bwd(lib, p, gi=0) == 1 and "grad_input" in _msg(lib)
    assert _dcn_bwd(lib, p, gom=0) == 1
    assert _dcn_bwd(lib, p, go=FAKE + 2) == 1 and "aligned" in _msg(lib)
    assert _dcn_bwd(lib, _dprob(out_dtype=1), go=FAKE + 1) == 1
    assert lib.dcn_forward(None, None, None, None, None) == 1 and "NULL" in _msg(lib)
    n = ctypes.c_size_t(7)
    assert lib.dcn_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    assert lib.dcn_backward_workspace_size(ctypes.byref(p), None) == 1


def _elf_exported_functions(path):
    """Defined global (or weak) function symbols of an ELF64 little-endian shared
    object's dynamic symbol table, read from the section headers and .dynsym."""
    import struct
    with open(path, "rb") as f:
        data = f.read()
    assert data[:4] == b"\x7fELF" and data[4] == 2 and data[5] == 1, "not an ELF64 LE file"
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum = struct.unpack_from("<HH", data, 0x3A)
    sections = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize)
                for i in range(shnum)]
    names = set()
    for sh in sections:
        if sh[1] != 11:                       # SHT_DYNSYM
            continue
        _, _, _, _, off, size, link, _, _, entsize = sh
        str_off = sections[link][4]
        for j in range(size // entsize):
            st_name, st_info, _, st_shndx, _, _ = struct.unpack_from("<IBBHQQ", data,
                                                                      off + j * entsize)
            if st_shndx == 0 or (st_info & 0xF) != 2 or (st_info >> 4) not in (1, 2):
                continue                      # undefined, not a function, or local
            end = data.index(b"\0", str_off + st_name)
            names.add(data[str_off + st_name:end].decode())
    return names


def test_exports_only_the_declared_c_abi(lib):
    """The library's dynamic symbol table holds the C ABI and nothing else (read from
    the ELF file directly, and cross-checked with nm where it is installed)."""
    import shutil
    import subprocess
    exported = _elf_exported_functions(LIB_PATH)
    assert exported == set(_lib.declared_functions())
    if shutil.which("nm") is not None:
        out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True,
                             text=True, check=True).stdout
        assert {ln.split()[-1] for ln in out.splitlines() if " T " in ln} == exported


@pytest.mark.parametrize("C, G, dtype", [(2048, 8, 0), (2048, 8, 1), (4096, 8, 1), (1028, 4, 0)])
@pytest.mark.parametrize("name", ["da_backward", "da_backward_accumulate", "da_backward_atomic"])
def test_backward_rejects_more_than_1024_channels(lib, C, G, dtype, name):
    """Every backward form handles at most 1024 channels; wider rows are refused on the
    host, before any launch (the forward still takes them)."""
    prob = _prob(num_embeds=C, num_groups=G, feat_dtype=dtype)
    assert _bwd(lib, prob, name=name) == 2
    assert "1024" in _msg(lib) or "exceeds 16" in _msg(lib)


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """da_backward_noalloc refuses, on the host and before any HIP call, a problem whose
    workspace exceeds the static scratch array (4 images of 160x400 levels here)."""
    from view_deformable_feature_amd import workloads as W
    wl = W.WORKLOADS["large"]
    prob = _prob(bs=wl.bs, num_feat=wl.num_feat, num_embeds=wl.C, num_anchors=wl.anchors,
                 num_pts=wl.pts, num_cams=wl.num_cams, num_scale=len(wl.levels),
                 num_groups=wl.groups)
    need = ctypes.c_size_t(0)
    assert lib.da_backward_workspace_size(ctypes.byref(prob), ctypes.byref(need)) == 0
    assert need.value > _lib.DA_NOALLOC_SCRATCH_BYTES
    shape = np.tile(np.array([[[1, 1]]], np.int32), (wl.num_cams, len(wl.levels), 1))
    start = np.zeros((wl.num_cams, len(wl.levels)), np.int32)
    assert _bwd(lib, prob, name="da_backward_noalloc", shape=shape, start=start) == 2
    assert "da_backward_noalloc" in _msg(lib) and str(need.value) in _msg(lib)
    # malformed problems are reported as by da_backward
    assert _bwd(lib, _prob(num_groups=0), name="da_backward_noalloc") == 1
