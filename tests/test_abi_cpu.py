"""The C-ABI library without a GPU: it loads, exports every symbol include/mm.h
declares, and validates arguments completely before any HIP call.

Every call here is either invalid (validation returns before touching HIP), of
zero size (nothing is launched), or made with MM_TEST_FORCE_FAIL=launch (the
library returns MM_ERR_DEVICE right after validation): none launches a kernel,
so the fake device pointers are never dereferenced, here or on a GPU machine.
"""
import ctypes
import os
import re

import pytest

import block_scaled_gemm_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mm.h")
P = 0x10000          # a fake, 64 KiB-aligned device address
P8 = P + 8           # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mm_status|const char\*)\s+(mm_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == {"mm_scaled_gemm", "mm_scaled_gemm_bias", "mm_scaled_gemm_batched", "mm_scaled_gemm_grouped",
                          "mm_scaled_gemm_grouped_layout", "mm_scaled_gemm_grouped_layout_noalloc",
                          "mm_grouped_workspace_bytes", "mm_transpose_u8",
                          "mm_blockscaled_gemm_amax", "mm_blockscaled_gemm_amax_atom", "mm_last_error",
                          "mm_version", "mm_debug_convert", "mm_debug_mfma_gemm"}
    lib = ctypes.CDLL(mm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(mm.EXPORTED) == set(names)


def test_version():
    assert mm.mm_version().startswith("mmfp8 ") and "gfx950" in mm.mm_version()


def gemm(**kw):
    args = dict(M=64, N=64, K=128, a=P, a_type=0, lda=128, b=P, b_type=0, ldb=128, scale_a=P, sa_mode=0,
                scale_b=P, sb_mode=0, scale_result=0, d=P, d_type=2, ldd=64, use_fast_accum=0, stream=0)
    args.update(kw)
    return mm.mm_scaled_gemm(**args)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(M=-1), mm.MM_ERR_INVALID_ARGUMENT, "must be >= 0"),
    (dict(K=-5), mm.MM_ERR_INVALID_ARGUMENT, "must be >= 0"),
    (dict(N=1 << 31), mm.MM_ERR_UNSUPPORTED, "below 2^31"),
    (dict(a_type=2), mm.MM_ERR_INVALID_ARGUMENT, "a_type and b_type"),
    (dict(b_type=7), mm.MM_ERR_INVALID_ARGUMENT, "a_type and b_type"),
    (dict(d_type=5), mm.MM_ERR_INVALID_ARGUMENT, "unknown d_type"),
    (dict(sa_mode=3), mm.MM_ERR_INVALID_ARGUMENT, "unknown scale mode"),
    (dict(sa_mode=0, sb_mode=1), mm.MM_ERR_UNSUPPORTED, "scale pair"),
    (dict(sa_mode=2, sb_mode=2), mm.MM_ERR_UNSUPPORTED, "scale pair"),
    (dict(sa_mode=1, sb_mode=0), mm.MM_ERR_UNSUPPORTED, "scale pair"),
    (dict(lda=64), mm.MM_ERR_INVALID_ARGUMENT, "lda and ldb"),
    (dict(ldd=63), mm.MM_ERR_INVALID_ARGUMENT, "ldd"),
    (dict(lda=(1 << 22) + 8, ldb=(1 << 22) + 8), mm.MM_ERR_UNSUPPORTED, "2^22"),
    (dict(d=0), mm.MM_ERR_INVALID_ARGUMENT, "d is NULL"),
    (dict(a=0), mm.MM_ERR_INVALID_ARGUMENT, "a or b is NULL"),
    (dict(scale_b=0), mm.MM_ERR_INVALID_ARGUMENT, "scale_a or scale_b"),
    (dict(a=P8), mm.MM_ERR_MISALIGNED, "16-byte"),
    (dict(lda=132, ldb=132), mm.MM_ERR_MISALIGNED, "multiples of 8"),
    (dict(d=P + 2), mm.MM_ERR_MISALIGNED, "element size"),
    (dict(d=P + 1, d_type=3), mm.MM_ERR_MISALIGNED, "element size"),
    (dict(scale_a=P + 2), mm.MM_ERR_MISALIGNED, "4-byte"),
])
def test_scaled_gemm_validation(kw, status, msg):
    assert gemm(**kw) == status
    assert msg in mm.mm_last_error()


def test_scaled_gemm_zero_sizes_launch_nothing():
    assert gemm(M=0, d=0, a=0) == mm.MM_OK
    assert gemm(N=0, d=0, b=0) == mm.MM_OK
    assert mm.mm_last_error() == ""


def gemm_bias(**kw):
    args = dict(M=64, N=64, K=128, a=P, a_type=0, lda=128, b=P, b_type=0, ldb=128, scale_a=P, sa_mode=0,
                scale_b=P, sb_mode=0, bias=P, d=P, d_type=3, ldd=64, use_fast_accum=0, stream=0)
    args.update(kw)
    return mm.mm_scaled_gemm_bias(**args)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d_type=0), mm.MM_ERR_UNSUPPORTED, "bias needs an f32, bf16 or f16 output"),
    (dict(d_type=1), mm.MM_ERR_UNSUPPORTED, "bias needs an f32, bf16 or f16 output"),
    (dict(bias=P + 1), mm.MM_ERR_MISALIGNED, "bias must be aligned"),
    (dict(d_type=2, bias=P + 2), mm.MM_ERR_MISALIGNED, "bias must be aligned"),
    (dict(sa_mode=1, sb_mode=0), mm.MM_ERR_UNSUPPORTED, "scale pair"),
    (dict(M=-1), mm.MM_ERR_INVALID_ARGUMENT, "must be >= 0"),
])
def test_scaled_gemm_bias_validation(kw, status, msg):
    assert gemm_bias(**kw) == status
    assert msg in mm.mm_last_error()


def test_scaled_gemm_bias_zero_sizes_launch_nothing():
    assert gemm_bias(M=0, d=0, a=0) == mm.MM_OK
    assert gemm_bias(N=0, d=0, b=0, bias=0) == mm.MM_OK


def bmm(**kw):
    args = dict(L=4, M=64, N=64, K=128, a=P, a_type=0, lda=128, stride_a=64 * 128, b=P, b_type=0, ldb=128,
                stride_b=64 * 128, scale_a=P, scale_b=P, scale_result=0, d=P, d_type=3, ldd=64,
                stride_d=64 * 64, use_fast_accum=0, stream=0)
    args.update(kw)
    return mm.mm_scaled_gemm_batched(**args)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(L=-1), mm.MM_ERR_INVALID_ARGUMENT, "must be >= 0"),
    (dict(L=1 << 31), mm.MM_ERR_UNSUPPORTED, "below 2^31"),
    (dict(stride_a=-16), mm.MM_ERR_INVALID_ARGUMENT, "batch strides"),
    (dict(stride_d=-1), mm.MM_ERR_INVALID_ARGUMENT, "batch strides"),
    (dict(stride_a=64 * 128 + 8), mm.MM_ERR_MISALIGNED, "multiples of 16 bytes"),
    (dict(stride_b=8), mm.MM_ERR_MISALIGNED, "multiples of 16 bytes"),
    (dict(L=1 << 20, M=1 << 16, N=1 << 16, ldd=1 << 16), mm.MM_ERR_UNSUPPORTED, "too many output tiles"),
    (dict(a_type=4), mm.MM_ERR_INVALID_ARGUMENT, "a_type and b_type"),
    (dict(ldd=63), mm.MM_ERR_INVALID_ARGUMENT, "ldd"),
    (dict(scale_a=0), mm.MM_ERR_INVALID_ARGUMENT, "scale_a or scale_b"),
])
def test_scaled_gemm_batched_validation(kw, status, msg):
    assert bmm(**kw) == status
    assert msg in mm.mm_last_error()


def test_scaled_gemm_batched_zero_sizes_launch_nothing():
    assert bmm(L=0, a=0, b=0, d=0) == mm.MM_OK
    assert bmm(M=0, a=0, d=0) == mm.MM_OK
    # one item: the strides are not used, so they need no alignment
    assert bmm(L=1, M=0, stride_a=8, d=0) == mm.MM_OK


def grouped(**kw):
    args = dict(batch_sum=300, N=64, K=256, G=4, a=P, a_type=0, lda=256, b=P, b_type=0, ldb=256, stride_b=64 * 256,
                batch_sizes=P, batch_offsets=P, scale_a=P, scale_b=P, scale_result=0, d=P, d_type=3, ldd=64,
                use_fast_accum=0, stream=0)
    args.update(kw)
    return mm.mm_scaled_gemm_grouped(**args)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(G=-1), mm.MM_ERR_INVALID_ARGUMENT, "group count"),
    (dict(G=1 << 31), mm.MM_ERR_UNSUPPORTED, "too many groups"),
    (dict(batch_sizes=0), mm.MM_ERR_INVALID_ARGUMENT, "batch_sizes or batch_offsets is NULL"),
    (dict(batch_offsets=P + 2), mm.MM_ERR_MISALIGNED, "4-byte"),
    (dict(stride_b=64 * 256 + 8), mm.MM_ERR_MISALIGNED, "multiples of 16"),
    (dict(stride_b=-16), mm.MM_ERR_INVALID_ARGUMENT, "strides must be >= 0"),
    (dict(a_type=2), mm.MM_ERR_INVALID_ARGUMENT, "a_type and b_type"),
    (dict(ldb=128), mm.MM_ERR_INVALID_ARGUMENT, "lda and ldb must be >= K"),
    (dict(d=0), mm.MM_ERR_INVALID_ARGUMENT, "d is NULL"),
])
def test_grouped_validation(kw, status, msg):
    assert grouped(**kw) == status
    assert msg in mm.mm_last_error()


def test_grouped_nothing_to_do_launches_nothing():
    assert grouped(G=0, batch_sizes=0, batch_offsets=0) == mm.MM_OK
    assert grouped(batch_sum=0, d=0) == mm.MM_OK
    assert grouped(N=0, d=0) == mm.MM_OK
    # no groups: the stride is not used
    assert grouped(G=0, stride_b=8) == mm.MM_OK


def amax_call(**kw):
    args = dict(M=64, N=64, K=256, L=2, a=P, b=P, ab_type=0, sfa=P, sfb=P, sf_vec_size=32, c=P, c_type=2,
                amax=P, amax_index=P, stream=0)
    args.update(kw)
    return mm.mm_blockscaled_gemm_amax(**args)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(L=-1), mm.MM_ERR_INVALID_ARGUMENT, "must be >= 0"),
    (dict(ab_type=3), mm.MM_ERR_INVALID_ARGUMENT, "ab_type"),
    (dict(sf_vec_size=16), mm.MM_ERR_UNSUPPORTED, "sf_vec_size 16"),
    (dict(sf_vec_size=64), mm.MM_ERR_INVALID_ARGUMENT, "sf_vec_size must be 32"),
    (dict(c_type=0), mm.MM_ERR_UNSUPPORTED, "FP8 C"),
    (dict(c_type=9), mm.MM_ERR_INVALID_ARGUMENT, "unknown c_type"),
    (dict(K=1 << 23), mm.MM_ERR_UNSUPPORTED, "2^22"),
    (dict(M=1 << 17, N=1 << 17, L=1), mm.MM_ERR_UNSUPPORTED, "2^33"),
    (dict(c=0), mm.MM_ERR_INVALID_ARGUMENT, "c is NULL"),
    (dict(sfb=0), mm.MM_ERR_INVALID_ARGUMENT, "NULL"),
    (dict(a=P8), mm.MM_ERR_MISALIGNED, "16-byte"),
    (dict(K=264), mm.MM_ERR_MISALIGNED, "multiple of 16"),
    (dict(amax=P + 2), mm.MM_ERR_MISALIGNED, "4-byte"),
    (dict(amax_index=P + 4), mm.MM_ERR_MISALIGNED, "8-byte"),
])
def test_amax_validation(kw, status, msg):
    assert amax_call(**kw) == status
    assert msg in mm.mm_last_error()


def test_amax_zero_size_without_outputs_launches_nothing():
    assert amax_call(M=0, amax=0, amax_index=0, c=0) == mm.MM_OK


def atom_call(**kw):
    args = dict(M=64, N=64, K=256, L=2, a=P, b=P, ab_type=0, sfa=P, sfb=P, sf_type=mm.MM_SF_E8M0, sf_vec_size=32,
                c=P, c_type=2, amax=P, amax_index=P, stream=0)
    args.update(kw)
    return mm.mm_blockscaled_gemm_amax_atom(**args)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(sf_type=mm.MM_SF_E4M3FN), mm.MM_ERR_UNSUPPORTED, "E4M3 scale factors"),  # FP8 operands
    (dict(sf_type=mm.MM_SF_E4M3FN, ab_type=mm.MM_F4_E2M1), mm.MM_ERR_UNSUPPORTED, "sf_vec_size 16"),
    (dict(sf_type=5), mm.MM_ERR_INVALID_ARGUMENT, "unknown sf_type"),
    (dict(L=-1), mm.MM_ERR_INVALID_ARGUMENT, "must be >= 0"),
    (dict(ab_type=2), mm.MM_ERR_INVALID_ARGUMENT, "ab_type"),
    (dict(sf_vec_size=16), mm.MM_ERR_UNSUPPORTED, "sf_vec_size 16"),
    (dict(c_type=1), mm.MM_ERR_UNSUPPORTED, "FP8 C"),
    (dict(sfa=0), mm.MM_ERR_INVALID_ARGUMENT, "NULL"),
    (dict(sfb=P + 2), mm.MM_ERR_MISALIGNED, "4-byte"),
    (dict(K=264), mm.MM_ERR_MISALIGNED, "multiple of 16"),
    # ceil(M/128) * ceil(K/128) * 512 bytes per item must stay below 2^31
    (dict(M=1 << 20, K=1 << 16, L=1), mm.MM_ERR_UNSUPPORTED, "below 2^31 bytes"),
    (dict(N=1 << 20, K=1 << 16, L=1, amax_index=0), mm.MM_ERR_UNSUPPORTED, "below 2^31 bytes"),
    # FP4 operands
    (dict(ab_type=mm.MM_F4_E2M1, K=272), mm.MM_ERR_MISALIGNED, "multiple of 32"),
    (dict(ab_type=mm.MM_F4_E2M1, sf_vec_size=64), mm.MM_ERR_INVALID_ARGUMENT, "32 or 16"),
    (dict(c_type=mm.MM_F4_E2M1), mm.MM_ERR_UNSUPPORTED, "FP4 C needs FP4 operands"),
    (dict(ab_type=mm.MM_F4_E2M1, c_type=7), mm.MM_ERR_INVALID_ARGUMENT, "unknown c_type"),
    (dict(ab_type=6), mm.MM_ERR_INVALID_ARGUMENT, "MM_F4_E2M1"),
])
def test_atom_validation(kw, status, msg):
    assert atom_call(**kw) == status
    assert msg in mm.mm_last_error()


def test_fp4_needs_the_atom_entry():
    assert amax_call(ab_type=mm.MM_F4_E2M1) == mm.MM_ERR_UNSUPPORTED
    assert "_atom entry" in mm.mm_last_error()


@pytest.mark.parametrize("kw", [dict(ab_type=mm.MM_F4_E2M1), dict(ab_type=mm.MM_F4_E2M1, sf_vec_size=16),
                                dict(ab_type=mm.MM_F4_E2M1, c_type=mm.MM_F8_E4M3FN, K=32),
                                dict(ab_type=mm.MM_F4_E2M1, c_type=mm.MM_F8_E5M2, sf_vec_size=16, K=4096),
                                dict(ab_type=mm.MM_F4_E2M1, sf_type=mm.MM_SF_E4M3FN, sf_vec_size=16),
                                dict(ab_type=mm.MM_F4_E2M1, c_type=mm.MM_F4_E2M1, N=63)])
def test_fp4_calls_pass_validation(kw, monkeypatch):
    # a launch failure forced after validation shows the call was accepted
    monkeypatch.setenv("MM_TEST_FORCE_FAIL", "launch")
    assert atom_call(**kw) == mm.MM_ERR_DEVICE
    assert "forced" in mm.mm_last_error()


def test_atom_zero_sizes_launch_nothing():
    assert atom_call(L=0, amax=0, amax_index=0, c=0) == mm.MM_OK
    assert atom_call(N=0, amax=0, amax_index=0, c=0, sfa=0, sfb=0) == mm.MM_OK


def test_forced_launch_failure(monkeypatch):
    monkeypatch.setenv("MM_TEST_FORCE_FAIL", "launch")
    assert gemm() == mm.MM_ERR_DEVICE
    assert "forced" in mm.mm_last_error()
    assert amax_call() == mm.MM_ERR_DEVICE
    assert atom_call() == mm.MM_ERR_DEVICE
    assert gemm_bias() == mm.MM_ERR_DEVICE
    assert bmm() == mm.MM_ERR_DEVICE
    assert grouped() == mm.MM_ERR_DEVICE
    assert mm.mm_debug_convert(P, P, 2, 16, 0) == mm.MM_ERR_DEVICE


def test_debug_convert_validation():
    assert mm.mm_debug_convert(P, P, 9, 16, 0) == mm.MM_ERR_INVALID_ARGUMENT
    assert mm.mm_debug_convert(P, P, 2, -1, 0) == mm.MM_ERR_INVALID_ARGUMENT
    assert mm.mm_debug_convert(P + 1, P, 2, 16, 0) == mm.MM_ERR_MISALIGNED
    assert mm.mm_debug_convert(0, 0, 2, 0, 0) == mm.MM_OK


def test_error_message_is_thread_local_and_cleared():
    assert gemm(M=-1) == mm.MM_ERR_INVALID_ARGUMENT
    assert mm.mm_last_error() != ""
    assert gemm(M=0, d=0) == mm.MM_OK
    assert mm.mm_last_error() == ""


def test_single_hip_runtime_after_import():
    """Importing the package must leave one HIP runtime in the process: torch's
    bundled runtime and the system one share a soname, and a second runtime
    initialised after the first finds no GPU."""
    import subprocess
    import sys
    code = ("import block_scaled_gemm_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "1", r.stdout


def layout_call(**kw):
    args = dict(batch_sum=300, N=64, K=96, G=3, transpose_a=1, transpose_b=0, a=P, a_type=0, lda=64, b=P, b_type=1,
                ldb=96, stride_b=0, batch_sizes=P, batch_offsets=P, scale_a=P, scale_b=P, scale_result=0, d=P,
                d_type=2, ldd=96, stride_d=64 * 96, workspace=P, workspace_bytes=1 << 30, use_fast_accum=0, stream=0)
    args.update(kw)
    return mm.mm_scaled_gemm_grouped_layout(**args)


def test_grouped_workspace_bytes():
    assert mm.mm_grouped_workspace_bytes(300, 64, 96, 3, 0, 1) == (mm.MM_OK, 0)      # NT: none
    assert mm.mm_grouped_workspace_bytes(300, 64, 90, 3, 0, 0) == (mm.MM_OK, 3 * 64 * 96)  # NN: b as [G][N][K16]
    st, n = mm.mm_grouped_workspace_bytes(300, 64, 96, 3, 1, 0)
    # TN / TT: both operands at a pitch holding every group 16-aligned, plus two int64 [G] tables
    assert st == mm.MM_OK and n >= (64 + 96) * (304 + 48) + 16 * 3
    assert mm.mm_grouped_workspace_bytes(300, 64, 96, 3, 1, 1) == (st, n)
    assert mm.mm_grouped_workspace_bytes(-1, 64, 96, 3, 1, 0)[0] == mm.MM_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw,status,msg", [
    (dict(transpose_a=2), mm.MM_ERR_INVALID_ARGUMENT, "0 or 1"),
    (dict(workspace_bytes=100), mm.MM_ERR_INVALID_ARGUMENT, "workspace needs"),
    (dict(workspace=0), mm.MM_ERR_INVALID_ARGUMENT, "workspace needs"),
    (dict(workspace=P + 8), mm.MM_ERR_MISALIGNED, "16-byte aligned"),
    (dict(a_type=2), mm.MM_ERR_INVALID_ARGUMENT, "a_type"),
    (dict(d_type=7), mm.MM_ERR_INVALID_ARGUMENT, "d_type"),
    (dict(lda=63), mm.MM_ERR_INVALID_ARGUMENT, "lda must be >= N"),
    (dict(ldb=95), mm.MM_ERR_INVALID_ARGUMENT, "ldb must be >= K"),
    (dict(transpose_b=1, ldb=299), mm.MM_ERR_INVALID_ARGUMENT, "ldb must be >= batch_sum"),
    (dict(ldd=95), mm.MM_ERR_INVALID_ARGUMENT, "ldd must be >= K"),
    (dict(stride_d=-1), mm.MM_ERR_INVALID_ARGUMENT, "stride_d"),
    (dict(batch_sum=1 << 22, ldb=1 << 22), mm.MM_ERR_UNSUPPORTED, "2^22"),
    (dict(batch_sizes=0), mm.MM_ERR_INVALID_ARGUMENT, "NULL"),
    (dict(batch_offsets=P + 2), mm.MM_ERR_MISALIGNED, "4-byte aligned"),
    (dict(d=0), mm.MM_ERR_INVALID_ARGUMENT, "d is NULL"),
    (dict(b=0), mm.MM_ERR_INVALID_ARGUMENT, "a or b is NULL"),
    (dict(scale_b=0), mm.MM_ERR_INVALID_ARGUMENT, "scale_a or scale_b is NULL"),
    (dict(d=P + 2), mm.MM_ERR_MISALIGNED, "aligned to its element size"),
    # NN: b is [G][K][ldb]
    (dict(transpose_a=0, lda=96, ldb=63, ldd=64), mm.MM_ERR_INVALID_ARGUMENT, "ldb must be >= N"),
    (dict(transpose_a=0, lda=96, ldb=64, ldd=64, stride_b=-16), mm.MM_ERR_INVALID_ARGUMENT, "stride_b"),
    (dict(transpose_a=0, lda=96, ldb=64, ldd=64, G=1 << 16), mm.MM_ERR_UNSUPPORTED, "NN packing"),
    (dict(transpose_a=0, lda=96, ldb=64, ldd=64, b=0), mm.MM_ERR_INVALID_ARGUMENT, "b is NULL"),
    (dict(transpose_a=0, lda=96, ldb=64, ldd=63), mm.MM_ERR_INVALID_ARGUMENT, "ldd must be >= N"),
])
def test_grouped_layout_validation(kw, status, msg):
    assert layout_call(**kw) == status
    assert msg in mm.mm_last_error()


def test_grouped_layout_nothing_to_do_launches_nothing():
    assert layout_call(G=0, batch_sizes=0, batch_offsets=0, workspace=0, workspace_bytes=0) == mm.MM_OK
    assert layout_call(N=0, d=0) == mm.MM_OK
    assert layout_call(K=0, d=0, ldd=0) == mm.MM_OK
    # NT needs no workspace and is the plain grouped entry
    assert layout_call(transpose_a=0, transpose_b=1, lda=96, ldb=96, ldd=64, workspace=0, workspace_bytes=0,
                       batch_sum=0, d=0) == mm.MM_OK


@pytest.mark.parametrize("kw", [dict(), dict(transpose_b=1, ldb=300), dict(batch_sum=0, a=0, b=0, ldb=96),
                                dict(transpose_a=0, lda=96, ldb=64, ldd=64, stride_b=96 * 64),
                                dict(transpose_a=0, transpose_b=1, lda=96, ldb=96, ldd=64, stride_b=96 * 64,
                                     workspace=0, workspace_bytes=0)],
                         ids=["TN", "TT", "TN-empty", "NN", "NT"])
def test_grouped_layout_calls_pass_validation(kw, monkeypatch):
    monkeypatch.setenv("MM_TEST_FORCE_FAIL", "launch")
    assert layout_call(**kw) == mm.MM_ERR_DEVICE
    assert "forced" in mm.mm_last_error()


@pytest.mark.parametrize("args,status,msg", [
    ((-1, 4, 4, P, 4, 0, P, 4, 0), mm.MM_ERR_INVALID_ARGUMENT, ">= 0"),
    ((1, 4, 8, P, 7, 0, P, 4, 0), mm.MM_ERR_INVALID_ARGUMENT, "ld_src"),
    ((1, 8, 4, P, 4, 0, P, 7, 0), mm.MM_ERR_INVALID_ARGUMENT, "ld_dst"),
    ((1, 4, 4, P, 4, -1, P, 4, 0), mm.MM_ERR_INVALID_ARGUMENT, "strides"),
    ((1 << 16, 4, 4, P, 4, 16, P, 4, 16), mm.MM_ERR_UNSUPPORTED, "2^16"),
    ((1, 4, 1 << 22, P, 1 << 22, 0, P, 4, 0), mm.MM_ERR_UNSUPPORTED, "2^22"),
    ((1, 4, 4, 0, 4, 0, P, 4, 0), mm.MM_ERR_INVALID_ARGUMENT, "NULL"),
])
def test_transpose_validation(args, status, msg):
    assert mm.mm_transpose_u8(*args, 0) == status
    assert msg in mm.mm_last_error()


def test_transpose_zero_sizes_and_forced_failure(monkeypatch):
    assert mm.mm_transpose_u8(0, 4, 4, 0, 4, 0, 0, 4, 0, 0) == mm.MM_OK
    assert mm.mm_transpose_u8(2, 0, 4, 0, 4, 0, 0, 0, 0, 0) == mm.MM_OK
    monkeypatch.setenv("MM_TEST_FORCE_FAIL", "launch")
    assert mm.mm_transpose_u8(2, 4, 4, P, 4, 16, P, 4, 16, 0) == mm.MM_ERR_DEVICE


def noalloc(**kw):
    args = dict(batch_sum=600, N=136, K=520, G=5, transpose_a=0, transpose_b=0, a=P, a_type=0, lda=520, b=P,
                b_type=0, ldb=136, stride_b=520 * 136, batch_sizes=P, batch_offsets=P, scale_a=P, scale_b=P,
                scale_result=0, d=P, d_type=3, ldd=136, stride_d=0, use_fast_accum=0, stream=0)
    args.update(kw)
    return mm.mm_scaled_gemm_grouped_layout_noalloc(**args)


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define MM_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mm.MM_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,status,msg", [
    (dict(transpose_a=2), mm.MM_ERR_INVALID_ARGUMENT, "must be 0 or 1"),
    (dict(batch_sum=-1), mm.MM_ERR_INVALID_ARGUMENT, "must be >= 0"),
    # NN with G N K above the scratch array: refused before any HIP call
    (dict(G=64, N=2048, K=2048, ldb=2048, stride_b=2048 * 2048), mm.MM_ERR_UNSUPPORTED, "scratch array"),
    (dict(transpose_a=1, batch_sum=1 << 21, N=4096, K=4096, lda=4096, ldb=4096, G=2), mm.MM_ERR_UNSUPPORTED,
     "scratch array"),
])
def test_noalloc_rejects_before_any_hip_call(kw, status, msg):
    assert noalloc(**kw) == status
    assert msg in mm.mm_last_error()


def test_noalloc_nt_layout_needs_no_scratch(monkeypatch):
    # NT packs nothing: the call goes straight to the grouped GEMM's validation (forced failure after it)
    monkeypatch.setenv("MM_TEST_FORCE_FAIL", "launch")
    assert noalloc(transpose_b=1, ldb=520) == mm.MM_ERR_DEVICE
    assert "forced" in mm.mm_last_error()
