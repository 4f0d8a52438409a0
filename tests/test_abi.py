"""The C-ABI library loads and exports every entry point include/brq.h
declares; host-side argument checks return their status codes without
touching a GPU (no compute calls here)."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "brq.h")
LIB = os.path.join(ROOT, "bitwise_reproducible_int8_amd", "libbrq.so")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(brq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libbrq.so is not built: run __graft_entry__.build()")
    return C.CDLL(LIB)


def test_header_declares_the_path():
    names = declared()
    for n in ["brq_quantize_lsq", "brq_qgemm_fwd", "brq_qgemm_bwd_dx", "brq_qgemm_bwd_dw_wht",
              "brq_rmsnorm_fixed_fwd", "brq_rmsnorm_fixed_bwd", "brq_grad_norm", "brq_hash_state"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (brq_\w+)", out))
    missing = [n for n in declared() if n not in exported]
    assert not missing, missing
    for n in declared():
        getattr(lib, n)


def test_binding_symbol_list_matches_header():
    import bitwise_reproducible_int8_amd as brq
    assert sorted(brq.SYMBOLS) == declared()


def test_host_side_status_codes(lib):
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
    lib.brq_status_string.restype = C.c_char_p
    lib.brq_spec_version.restype = i32
    assert lib.brq_spec_version() == 1
    assert lib.brq_status_string(0) == b"ok"
    q = lib.brq_quantize_lsq
    q.restype = i32
    q.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp, C.c_size_t, vp, vp, vp]
    fake = 0x1000
    # bad dtype, negative shape, NULL output, misalignment, missing workspace
    assert q(fake, 7, 4, 8, 0, None, fake, None, fake, None, None, 0, None, None, None) == -2
    assert q(fake, 1, -1, 8, 0, None, fake, None, fake, None, None, 0, None, None, None) == -3
    assert q(fake, 1, 4, 8, 0, None, fake, None, None, None, None, 0, None, None, None) == -1
    assert q(fake + 2, 1, 4, 8, 0, None, fake, None, fake, None, None, 0, None, None, None) == -4
    assert q(fake, 1, 4, 12, 0, None, fake, None, fake, None, None, 0, None, None, None) == -5
    assert q(fake, 1, 4, 8, 0, None, fake, None, fake, None, None, 0, None, None, None) == -7
    g = lib.brq_qgemm_fwd
    g.restype = i32
    g.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, vp, vp, C.c_size_t, vp, vp]
    assert g(fake, fake, fake, fake, 1, 64, 64, 24, fake, None, 0, None, None) == -5   # K % 16
    assert g(fake, fake, fake, fake, 1, 64, 64, 133152, fake, None, 0, None, None) == -6  # int32 range
    assert g(fake, fake, fake, fake, 1, 64, 64, 131072, fake, None, 0, None, None) == -6  # 128*128*K
    d = lib.brq_qgemm_bwd_dw_wht
    d.restype = i32
    d.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, vp, vp, vp, vp, C.c_size_t, vp, vp, vp]
    assert d(fake, fake, fake, 1, 128, 64, 64, 96, fake, None, None, fake, 1 << 30, None, None, None) == -5
    assert d(fake, fake, fake, 1, 96, 64, 64, 64, fake, None, None, fake, 1 << 30, None, None, None) == -5


def test_workspace_sizes_are_monotone(lib):
    lib.brq_workspace_size.restype = C.c_size_t
    lib.brq_workspace_size.argtypes = [C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_void_p]
    a = lib.brq_workspace_size(1, 4096, 2048, 0, 0, None)
    b = lib.brq_workspace_size(1, 16384, 8192, 0, 0, None)
    assert 0 < a < b
    assert lib.brq_workspace_size(3, 16384, 8192, 2048, 128, None) > 16384 * (8192 + 2048)


def test_adamw_bias_corrections_host_matches_oracle():
    """The library's host-side bias corrections (no GPU involved) equal the
    oracle's, an independent implementation of the same definition."""
    import bitwise_reproducible_int8_amd as brq
    import oracle as orc
    for t in (1, 2, 3, 10, 99, 1000, 50000, 200000):
        for b1, b2 in ((0.9, 0.95), (0.8, 0.999)):
            got = brq.adamw_bias_corrections(t, b1, b2)
            want = orc.adamw_bias_corrections(t, b1, b2)
            assert np.float32(got[0]) == want[0] and np.float32(got[1]) == want[1], (t, b1, b2)


def test_static_quantiser_rejects_what_its_scratch_cannot_hold(lib):
    """brq_quantize_lsq_static refuses, before any device call, a per-tensor
    input whose tree partials exceed the static scratch (so this runs
    without a GPU)."""
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
    f = lib.brq_quantize_lsq_static
    f.restype = i32
    f.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    fake = 0x1000
    assert f(fake, 1, 1 << 20, 1 << 14, 0, None, fake, None, fake, None, None, None, None) == -10
    assert f(fake, 1, -1, 8, 0, None, fake, None, fake, None, None, None, None) == -3
    lib.brq_status_string.restype = C.c_char_p
    assert b"static scratch" in lib.brq_status_string(-10)


def test_rows_multi_argument_checks(lib):
    """brq_quantize_lsq_rows_multi checks every job before anything runs
    (these return without a device call)."""
    class Job(C.Structure):
        _fields_ = [("x", C.c_void_p), ("x_dtype", C.c_int), ("rows", C.c_int64),
                    ("cols", C.c_int64), ("q", C.c_void_p), ("q_t", C.c_void_p),
                    ("scale", C.c_void_p), ("amax", C.c_void_p)]
    f = lib.brq_quantize_lsq_rows_multi
    f.restype = C.c_int
    f.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]
    fake = 0x1000
    jobs = (Job * 2)(Job(fake, 1, 16, 64, fake, None, fake, None),
                     Job(fake, 1, 16, 64, fake, None, fake, None))
    assert f(None, 0, None, None) == 0          # nothing to do
    assert f(jobs, -1, None, None) == -9        # count out of range
    assert f(jobs, 1025, None, None) == -9
    assert f(None, 2, None, None) == -1         # no job array
    jobs[1].cols = 20000                        # wider than a per-row group may be
    assert f(jobs, 2, None, None) == -5
    jobs[1].cols = 60                           # not a whole bf16 vector
    assert f(jobs, 2, None, None) == -5
    jobs[1].cols, jobs[1].x_dtype = 64, 2       # int8 input
    assert f(jobs, 2, None, None) == -2
    jobs[1].x_dtype, jobs[1].rows = 1, -1
    assert f(jobs, 2, None, None) == -3
    jobs[1].rows, jobs[1].q_t, jobs[1].cols = 8, fake, 64   # transpose needs rows % 16
    assert f(jobs, 2, None, None) == -5
    jobs[1].q_t, jobs[1].x = None, fake + 4     # misaligned input
    assert f(jobs, 2, None, None) == -4
    jobs[1].x, jobs[1].scale = fake, None
    assert f(jobs, 2, None, None) == -1


def test_hash_stage_argument_checks(lib):
    """The two stages of the tensor digests check their arguments before
    any device call (a missing workspace, a missing or misaligned digest
    buffer)."""
    class Ref(C.Structure):
        _fields_ = [("data", C.c_void_p), ("dtype", C.c_int), ("ndim", C.c_int),
                    ("dims", C.c_int64 * 8), ("name", C.c_char_p)]
    refs = (Ref * 1)()
    refs[0].data, refs[0].dtype, refs[0].ndim, refs[0].name = 0x1000, 0, 1, b"a"
    refs[0].dims[0] = 4096
    vp, i32, sz = C.c_void_p, C.c_int, C.c_size_t
    lib.brq_hash_digests_workspace_size.restype = sz
    lib.brq_hash_digests_workspace_size.argtypes = [vp, i32]
    need = lib.brq_hash_digests_workspace_size(refs, 1)
    assert need > 0
    lv = lib.brq_hash_tensor_leaves
    lv.restype = i32
    lv.argtypes = [vp, i32, vp, sz, vp]
    fn = lib.brq_hash_tensor_finish
    fn.restype = i32
    fn.argtypes = [vp, i32, vp, vp, sz, vp]
    assert lv(refs, 1, None, 0, None) == -7
    assert lv(refs, 1, 0x2000, need - 1, None) == -7
    assert fn(refs, 1, None, 0x2000, need, None) == -1
    assert fn(refs, 1, 0x3008, 0x2000, need, None) == -4
    assert fn(refs, 1, 0x3000, 0x2000, need - 1, None) == -7
