"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and rejects
bad arguments on the host before any HIP call (fake, never-dereferenced pointers)."""
import ctypes
import os
import re

import pytest

import exact_io_aware_68_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULL, SHAPE, DTYPE, HEADDIM, GQA, SCALE, ALIGN, WORKSPACE, DEVICE, LAUNCH, TOO_LARGE = range(12)
A = 0x10000            # a 16-byte-aligned fake device address (never dereferenced here)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return fa.load()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_prep", "fa_bwd_dkdv", "fa_bwd_dq",
            "fa_bwd_workspace_size", "fa_status_str", "fa_abi_version", "fa_fwd_splitkv",
            "fa_fwd_splitkv_splits", "fa_fwd_splitkv_workspace_size", "fa_fwd_window",
            "fa_fwd_blocksparse"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+FA_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert fa.fa_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for s in range(12):
        assert fa.fa_status_str(s) and fa.fa_status_str(s) != "unknown status"
    assert fa.fa_status_str(99) == "unknown status"


def test_workspace_is_linear_in_N(lib):
    assert fa.fa_bwd_workspace_size(2, 16, 4096) == 2 * 16 * 4096 * 8
    assert fa.fa_bwd_workspace_size(2, 16, 8192) == 2 * fa.fa_bwd_workspace_size(2, 16, 4096)
    assert fa.fa_bwd_workspace_size(-1, 16, 8) == 0
    assert fa.fa_bwd_workspace_size(1, 0, 8) == 0


# Launch grids: HIP limits a 1-D grid to fewer than 2^32 work-items, so shapes whose grid would
# reach that are FA_ERR_SHAPE on the host, never a failed launch.
@pytest.mark.parametrize("call,code", [
    # forward bf16: B * Hq * ceil(N / 128) workgroups of 256
    (lambda lib: fwd(lib, B=1, Hq=16384, Hkv=1, N=128 * 1024, d=64), SHAPE),
    (lambda lib: fwd(lib, B=2, Hq=8192, Hkv=1, N=128 * 1024, d=64), SHAPE),
    # forward fp32: B * Hq * ceil(N / 64) workgroups of 64
    (lambda lib: fwd(lib, B=1, Hq=1 << 20, Hkv=1, N=64 * 64, d=1, dtype=fa.FA_F32), SHAPE),
    # window and block-sparse share the forward's grid
    (lambda lib: win(lib, B=1, Hq=16384, Hkv=1, N=128 * 1024, d=64), SHAPE),
    (lambda lib: bsp(lib, B=256, Hq=256, Hkv=1, N=65536, d=64), SHAPE),
    # backward: dK/dV B * Hkv * ceil(N / 128) workgroups of 512
    (lambda lib: bwd(lib, B=1, Hq=8192, Hkv=8192, N=128 * 1024, d=64), SHAPE),
    # split-KV merge: one workgroup of 256 per query row
    (lambda lib: skv(lib, B=1, Hq=1, Hkv=1, Nq=1 << 24, Nk=1), SHAPE),
])
def test_grids_past_2_32_work_items_are_shape_errors(lib, call, code):
    assert call(lib) == code


@pytest.mark.skipif("_gpu_present()", reason="fake pointers must never reach a real GPU")
def test_grids_just_below_the_limit_pass_the_shape_checks(lib):
    # 16384 * 1023 workgroups of 256 = 2^32 - 2^22 work-items: valid, so the call reaches the
    # device check (no GPU in this process)
    assert fwd(lib, B=1, Hq=16384, Hkv=1, N=128 * 1023, d=64) == DEVICE
    assert skv(lib, B=1, Hq=1, Hkv=1, Nq=(1 << 24) - 1, Nk=1, wsb=1 << 40) == DEVICE


def test_kernel_names(lib):
    assert fa.fa_fwd_kernel_name(128, True, False, fa.FA_BF16) == "fwd_bf16<d128,causal>"
    assert fa.fa_fwd_kernel_name(64, False, True, fa.FA_BF16) == "fwd_bf16<d64>"
    assert fa.fa_fwd_kernel_name(96, False, False, fa.FA_BF16) == "none"
    assert fa.fa_fwd_kernel_name(64, False, False, fa.FA_F32) == "fwd_f32<dmax64>"
    assert fa.fa_bwd_dkdv_kernel_name(128, True, False, fa.FA_BF16) == "bwd_dkdv_bf16<d128,causal>"
    assert fa.fa_bwd_dq_kernel_name(64, False, False, fa.FA_BF16) == "bwd_dq_bf16<d64>"
    assert fa.fa_bwd_dq_kernel_name(128, True, False, fa.FA_F32) == "none"


def fwd(lib, q=A, k=A, v=A, o=A, lse=A, kl=None, B=1, Hq=2, Hkv=1, N=8, d=64, scale=0.125,
        causal=0, dtype=fa.FA_BF16):
    return lib.fa_fwd(q, k, v, o, lse, kl, B, Hq, Hkv, N, d, ctypes.c_float(scale), causal,
                      dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), DTYPE),
    (dict(d=96), HEADDIM), (dict(d=32), HEADDIM), (dict(d=256, dtype=fa.FA_F32), HEADDIM),
    (dict(Hq=3, Hkv=2), GQA), (dict(Hkv=0), SHAPE), (dict(N=-1), SHAPE), (dict(B=-2), SHAPE),
    (dict(d=0), SHAPE),
    (dict(scale=float("nan")), SCALE), (dict(scale=float("inf")), SCALE), (dict(scale=0.0), SCALE),
    (dict(scale=-0.1), SCALE),
    (dict(q=None), NULL), (dict(o=None), NULL),
    (dict(k=A + 8), ALIGN), (dict(lse=A + 2), ALIGN), (dict(kl=A + 1), ALIGN),
    (dict(B=0), OK), (dict(N=0), OK), (dict(B=0, q=None, o=None), OK),
])
def test_fwd_argument_errors_before_any_hip_call(lib, kw, code):
    assert fwd(lib, **kw) == code


def test_fwd_f32_alignment_is_4_bytes(lib):
    assert fwd(lib, q=A + 4, dtype=fa.FA_F32, d=33) != ALIGN
    assert fwd(lib, q=A + 2, dtype=fa.FA_F32, d=33) == ALIGN


def bwd(lib, q=A, k=A, v=A, o=A, do=A, lse=A, kl=None, dq=A, dk=A, dv=A, ws=A, wsb=1 << 20,
        B=1, Hq=2, Hkv=1, N=8, d=128, scale=0.1, causal=1, dtype=fa.FA_BF16):
    return lib.fa_bwd(q, k, v, o, do, lse, kl, dq, dk, dv, ws, wsb, B, Hq, Hkv, N, d,
                      ctypes.c_float(scale), causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=fa.FA_F32), DTYPE), (dict(dtype=3), DTYPE), (dict(d=96), HEADDIM),
    (dict(Hq=4, Hkv=3), GQA), (dict(ws=None), WORKSPACE), (dict(wsb=2 * 8 * 8 - 1), WORKSPACE),
    (dict(scale=float("nan")), SCALE), (dict(do=None), NULL), (dict(lse=None), NULL),
    (dict(dq=A + 4), ALIGN), (dict(dk=A + 8), ALIGN), (dict(ws=A + 2), ALIGN),
    (dict(B=0, ws=None), OK),
])
def test_bwd_argument_errors_before_any_hip_call(lib, kw, code):
    assert bwd(lib, **kw) == code


def noalloc(lib, q=A, k=A, v=A, o=A, do=A, lse=A, kl=None, dq=A, dk=A, dv=A, B=1, Hq=2, Hkv=1,
            N=8, d=128, scale=0.1, causal=1, dtype=fa.FA_BF16):
    return lib.fa_bwd_noalloc(q, k, v, o, do, lse, kl, dq, dk, dv, B, Hq, Hkv, N, d,
                              ctypes.c_float(scale), causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=1, Hq=64, Hkv=1, N=65537, d=64), TOO_LARGE),          # 4194368 rows > 4194304
    (dict(B=2, Hq=32, Hkv=8, N=65536 + 1, d=128), TOO_LARGE),
    (dict(dtype=fa.FA_F32), DTYPE), (dict(dtype=3), DTYPE), (dict(d=96), HEADDIM),
    (dict(Hq=4, Hkv=3), GQA), (dict(N=-1), SHAPE), (dict(scale=float("nan")), SCALE),
    (dict(do=None), NULL), (dict(lse=None), NULL), (dict(dq=None), NULL), (dict(dv=None), NULL),
    (dict(dq=A + 4), ALIGN), (dict(o=A + 8), ALIGN), (dict(kl=A + 2), ALIGN),
    (dict(B=0), OK), (dict(N=0, q=None), OK),
])
def test_noalloc_argument_errors_before_any_hip_call(lib, kw, code):
    assert noalloc(lib, **kw) == code


@pytest.mark.skipif("_gpu_present()", reason="fake pointers must never reach a real GPU")
def test_noalloc_largest_problem_passes_the_checks(lib):
    assert noalloc(lib, B=1, Hq=64, Hkv=1, N=65536, d=64) == DEVICE      # exactly 2^22 rows


def test_bwd_stage_argument_errors(lib):
    f = ctypes.c_float(0.1)
    # fa_bwd_prep(o, dO, lse, ws, wsb, B, Hq, N, d, dtype, stream)
    assert lib.fa_bwd_prep(A, A, None, A, 1 << 20, 1, 2, 8, 128, fa.FA_BF16, None) == NULL
    assert lib.fa_bwd_prep(A, A, A, A, 8, 1, 2, 8, 128, fa.FA_BF16, None) == WORKSPACE
    assert lib.fa_bwd_prep(A, A, A, A, 1 << 20, 1, 2, 8, 96, fa.FA_BF16, None) == HEADDIM
    # fa_bwd_dkdv(q, k, v, dO, kl, dk, dv, ws, wsb, B, Hq, Hkv, N, d, scale, causal, dtype, s)
    assert lib.fa_bwd_dkdv(A, A, A, A, None, None, A, A, 1 << 20, 1, 2, 1, 8, 128, f, 1,
                           fa.FA_BF16, None) == NULL
    assert lib.fa_bwd_dkdv(A, A, A, A, None, A, A + 4, A, 1 << 20, 1, 2, 1, 8, 128, f, 1,
                           fa.FA_BF16, None) == ALIGN
    assert lib.fa_bwd_dkdv(A, A, A, A, None, A, A, A, 1 << 20, 1, 3, 2, 8, 128, f, 1,
                           fa.FA_BF16, None) == GQA
    # fa_bwd_dq(q, k, v, dO, kl, dq, ws, wsb, B, Hq, Hkv, N, d, scale, causal, dtype, s)
    assert lib.fa_bwd_dq(A, A, A, A, None, None, A, 1 << 20, 1, 2, 1, 8, 128, f, 1,
                         fa.FA_BF16, None) == NULL
    assert lib.fa_bwd_dq(A, A, A, A, None, A, None, 1 << 20, 1, 2, 1, 8, 128, f, 1,
                         fa.FA_BF16, None) == WORKSPACE
    assert lib.fa_bwd_dq(A, A, A, A, None, A, A, 1 << 20, 1, 2, 1, 8, 128, ctypes.c_float(0.0),
                         1, fa.FA_BF16, None) == SCALE


def skv(lib, q=A, k=A, v=A, o=A, lse=A, kl=None, ws=A, wsb=1 << 24, B=2, Hq=8, Hkv=2, Nq=1,
        Nk=1000, d=128, scale=0.1, splits=0, dtype=fa.FA_BF16):
    return lib.fa_fwd_splitkv(q, k, v, o, lse, kl, ws, wsb, B, Hq, Hkv, Nq, Nk, d,
                              ctypes.c_float(scale), splits, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=fa.FA_F32), DTYPE), (dict(dtype=5), DTYPE), (dict(d=96), HEADDIM),
    (dict(Hq=6, Hkv=4), GQA), (dict(Hkv=0), SHAPE), (dict(Nq=-1), SHAPE), (dict(Nk=-3), SHAPE),
    (dict(splits=-1), SHAPE), (dict(scale=float("nan")), SCALE),
    (dict(q=None), NULL), (dict(o=None), NULL), (dict(k=None), NULL),
    (dict(ws=None), WORKSPACE), (dict(wsb=100), WORKSPACE),
    (dict(v=A + 8), ALIGN), (dict(ws=A + 4), ALIGN), (dict(lse=A + 1), ALIGN),
    (dict(B=0, q=None, ws=None), OK), (dict(Nq=0, ws=None), OK),
])
def test_splitkv_argument_errors_before_any_hip_call(lib, kw, code):
    assert skv(lib, **kw) == code


def test_splitkv_plan_and_workspace(lib):
    # automatic: enough ranges for ~1024 workgroups, each a multiple of 128 keys
    assert fa.fa_fwd_splitkv_splits(4, 32, 8, 1, 16384) == 32
    assert fa.fa_fwd_splitkv_splits(1, 1, 1, 1, 100) == 1
    assert fa.fa_fwd_splitkv_splits(1, 1, 1, 1, 0) == 1
    assert fa.fa_fwd_splitkv_splits(2, 16, 16, 4, 4096, 3) == 3        # requested
    assert fa.fa_fwd_splitkv_splits(2, 16, 16, 4, 300, 50) == 3        # capped at ceil(Nk/128)
    s = fa.fa_fwd_splitkv_splits(4, 32, 8, 1, 16384)
    assert fa.fa_fwd_splitkv_workspace_size(4, 32, 8, 1, 16384, 128) == s * 4 * 32 * 1 * 129 * 4
    assert fa.fa_fwd_splitkv_workspace_size(4, 32, 8, 1, 16384, 128, -1) == 0
    assert fa.fa_fwd_splitkv_splits(4, 30, 8, 1, 16384) == 0           # Hq % Hkv != 0


def win(lib, q=A, k=A, v=A, o=A, lse=A, kl=None, B=1, Hq=2, Hkv=1, N=64, d=128, scale=0.1,
        left=16, right=16, dtype=fa.FA_BF16):
    return lib.fa_fwd_window(q, k, v, o, lse, kl, B, Hq, Hkv, N, d, ctypes.c_float(scale), left,
                             right, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(left=-2), SHAPE), (dict(right=-7), SHAPE), (dict(dtype=fa.FA_F32), DTYPE),
    (dict(dtype=9), DTYPE), (dict(d=96), HEADDIM), (dict(Hq=3, Hkv=2), GQA),
    (dict(scale=-1.0), SCALE), (dict(q=None), NULL), (dict(v=None), NULL), (dict(o=A + 8), ALIGN),
    (dict(kl=A + 2), ALIGN), (dict(B=0, q=None), OK), (dict(N=0), OK),
])
def test_window_argument_errors_before_any_hip_call(lib, kw, code):
    assert win(lib, **kw) == code


def bsp(lib, q=A, k=A, v=A, o=A, lse=A, kl=None, bm=A, B=1, Hq=2, Hkv=1, N=256, d=128,
        scale=0.1, causal=0, dtype=fa.FA_BF16):
    return lib.fa_fwd_blocksparse(q, k, v, o, lse, kl, bm, B, Hq, Hkv, N, d, ctypes.c_float(scale),
                                  causal, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(bm=None), NULL), (dict(q=None), NULL), (dict(N=65537), SHAPE), (dict(N=-1), SHAPE),
    (dict(dtype=fa.FA_F32), DTYPE), (dict(d=32), HEADDIM), (dict(Hq=5, Hkv=2), GQA),
    (dict(scale=0.0), SCALE), (dict(k=A + 4), ALIGN), (dict(lse=A + 2), ALIGN),
    (dict(B=0, bm=None), OK), (dict(N=0), OK),
])
def test_blocksparse_argument_errors_before_any_hip_call(lib, kw, code):
    assert bsp(lib, **kw) == code


def _gpu_present():
    import torch
    return torch.cuda.is_available()


@pytest.mark.skipif(_gpu_present(), reason="fake pointers must never reach a real GPU")
def test_valid_call_without_device_reports_device_error(lib):
    assert fwd(lib) == DEVICE
    assert bwd(lib) == DEVICE
    assert noalloc(lib) == DEVICE
    assert skv(lib) == DEVICE
    assert win(lib) == DEVICE
    assert bsp(lib) == DEVICE
    assert fwd(lib, B=0) == OK              # empty problems never touch HIP at all
