"""The C-ABI library loads, exports every function include/fp8fg.h declares,
and rejects invalid arguments on the host (no kernel is launched by any call
here: each one fails validation, or is a documented no-op)."""

import ctypes

import pytest

from fp8_fine_grained_amd import binding as fp8

BAD = ctypes.c_void_p(0x1008)   # 8-byte aligned, not 16: never dereferenced
GOOD = ctypes.c_void_p(0x10000)  # aligned stand-in: only used where validation fails first
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def L():
    return fp8.lib()


def test_exports_every_declared_function(L):
    names = fp8.declared_functions()
    assert set(names) == {"fp8_quant_act_1x128", "fp8_quant_act_1x128_pow2", "fp8_quant_weight_128x128",
                          "fp8_quant_weight_128x128_pow2", "fp8_quant_weight_128x128_dual",
                          "fp8_quant_weight_128x128_dual_pow2", "fp8_quant_per_tensor",
                          "fp8_quant_act_weight",
                          "fp8_block_gemm", "fp8_block_gemm_accum", "fp8_block_gemm_quant", "fp8_block_grouped_gemm",
                          "fp8_block_grouped_gemm_accum", "fp8_block_grouped_gemm_gather",
                          "fp8fg_status_string", "fp8fg_abi_version"}
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.fp8fg_abi_version() == 9
    for st in range(0, 6):
        assert L.fp8fg_status_string(st)
    assert b"unknown" in L.fp8fg_status_string(99)


@pytest.mark.parametrize("fn", ["fp8_quant_act_1x128", "fp8_quant_act_1x128_pow2"])
def test_quant_act_validation(L, fn):
    f = getattr(L, fn)
    assert f(GOOD, 7, 4, 128, 128, 1, GOOD, GOOD, NULL) == fp8.ERR_INVALID_ARG  # dtype
    assert f(GOOD, fp8.BF16, -1, 128, 128, 1, GOOD, GOOD, NULL) == fp8.ERR_INVALID_ARG
    assert f(NULL, fp8.BF16, 0, 128, 128, 1, NULL, NULL, NULL) == fp8.OK  # M == 0: no-op
    assert f(GOOD, fp8.BF16, 4, 100, 100, 1, GOOD, GOOD, NULL) == fp8.ERR_UNSUPPORTED
    assert f(NULL, fp8.BF16, 4, 128, 128, 1, GOOD, GOOD, NULL) == fp8.ERR_INVALID_ARG
    assert f(BAD, fp8.BF16, 4, 128, 128, 1, GOOD, GOOD, NULL) == fp8.ERR_MISALIGNED
    assert f(GOOD, fp8.BF16, 4, 128, 128, 1, BAD, GOOD, NULL) == fp8.ERR_MISALIGNED
    assert f(GOOD, fp8.BF16, 4, 128, 129, 1, GOOD, GOOD, NULL) == fp8.ERR_MISALIGNED  # row pitch
    assert f(GOOD, fp8.BF16, 4, 128, 2, 3, GOOD, GOOD, NULL) == fp8.ERR_UNSUPPORTED   # strided both ways
    assert f(GOOD, fp8.BF16, 12, 128, 1, 16, GOOD, GOOD, NULL) == fp8.ERR_UNSUPPORTED  # transposed, M % 8


@pytest.mark.parametrize("fn", ["fp8_quant_weight_128x128", "fp8_quant_weight_128x128_pow2"])
def test_quant_weight_validation(L, fn):
    f = getattr(L, fn)
    assert f(GOOD, fp8.BF16, 100, 128, 128, GOOD, GOOD, NULL) == fp8.ERR_UNSUPPORTED
    assert f(GOOD, fp8.BF16, 128, 130, 130, GOOD, GOOD, NULL) == fp8.ERR_UNSUPPORTED
    assert f(GOOD, fp8.BF16, 128, 128, 64, GOOD, GOOD, NULL) == fp8.ERR_INVALID_ARG  # ld < K
    assert f(GOOD, fp8.F32, 128, 128, 128, NULL, GOOD, NULL) == fp8.ERR_INVALID_ARG
    assert f(GOOD, fp8.F32, 128, 128, 128, GOOD, ctypes.c_void_p(0x10002), NULL) == fp8.ERR_MISALIGNED
    assert f(NULL, fp8.F32, 0, 128, 128, NULL, NULL, NULL) == fp8.OK


def test_quant_per_tensor_validation(L):
    f = L.fp8_quant_per_tensor
    ok = dict(x=GOOD, dt=fp8.BF16, M=128, K=256, ld=256, q=GOOD, s=GOOD, layout=fp8.B_ROW_1x128, stream=NULL)
    args = lambda **kw: [kw.get(k, v) for k, v in ok.items()]
    assert f(*args(x=NULL, M=0, q=NULL, s=NULL)) == fp8.OK  # M == 0: no-op
    assert f(*args(M=-1)) == fp8.ERR_INVALID_ARG
    assert f(*args(dt=7)) == fp8.ERR_INVALID_ARG
    assert f(*args(layout=5)) == fp8.ERR_INVALID_ARG
    assert f(*args(K=200, ld=200)) == fp8.ERR_UNSUPPORTED
    assert f(*args(M=100, layout=fp8.B_BLOCK_128x128)) == fp8.ERR_UNSUPPORTED  # weight layout: M % 128
    assert f(*args(ld=128)) == fp8.ERR_INVALID_ARG  # ld < K
    assert f(*args(x=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(s=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(x=BAD)) == fp8.ERR_MISALIGNED
    assert f(*args(s=ctypes.c_void_p(0x10002))) == fp8.ERR_MISALIGNED
    assert f(*args(ld=260)) == fp8.ERR_MISALIGNED  # row pitch 520 B


def test_quant_act_weight_validation(L):
    """Each part is checked as in its separate call; an invalid part launches
    nothing (every call here either fails validation or has two empty parts)."""
    f = L.fp8_quant_act_weight
    ok = dict(x=GOOD, xdt=fp8.BF16, M=4, Kx=256, ldx=256, qx=GOOD, sx=GOOD,
              w=GOOD, wdt=fp8.BF16, N=128, Kw=256, ldw=256, qw=GOOD, sw=GOOD, pow2=0, stream=NULL)
    args = lambda **kw: [kw.get(k, v) for k, v in ok.items()]
    assert f(*args(x=NULL, M=0, qx=NULL, sx=NULL, w=NULL, N=0, qw=NULL, sw=NULL)) == fp8.OK  # both empty
    assert f(*args(pow2=2)) == fp8.ERR_INVALID_ARG
    assert f(*args(xdt=7)) == fp8.ERR_INVALID_ARG
    assert f(*args(wdt=7)) == fp8.ERR_INVALID_ARG
    assert f(*args(M=-1)) == fp8.ERR_INVALID_ARG
    assert f(*args(Kx=200, ldx=200)) == fp8.ERR_UNSUPPORTED
    assert f(*args(N=100)) == fp8.ERR_UNSUPPORTED
    assert f(*args(x=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(sw=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(ldx=128)) == fp8.ERR_INVALID_ARG  # ld_x < K_x
    assert f(*args(ldw=128)) == fp8.ERR_INVALID_ARG  # ld_w < K_w
    assert f(*args(qx=BAD)) == fp8.ERR_MISALIGNED
    assert f(*args(sw=ctypes.c_void_p(0x10002))) == fp8.ERR_MISALIGNED
    assert f(*args(ldw=260)) == fp8.ERR_MISALIGNED  # row pitch 520 B
    # an invalid part is reported even when the other part is empty
    assert f(*args(w=NULL, N=0, qw=NULL, sw=NULL, Kx=200, ldx=200)) == fp8.ERR_UNSUPPORTED
    assert f(*args(x=NULL, M=0, qx=NULL, sx=NULL, N=100)) == fp8.ERR_UNSUPPORTED


@pytest.mark.parametrize("fn", ["fp8_quant_weight_128x128_dual", "fp8_quant_weight_128x128_dual_pow2"])
def test_quant_weight_dual_validation(L, fn):
    f = getattr(L, fn)
    ok = dict(w=GOOD, dt=fp8.BF16, N=128, K=256, ld=256, q=GOOD, s=GOOD, qt=GOOD, st=GOOD, stream=NULL)
    args = lambda **kw: [kw.get(k, v) for k, v in ok.items()]
    assert f(*args(dt=7)) == fp8.ERR_INVALID_ARG
    assert f(*args(N=-128)) == fp8.ERR_INVALID_ARG
    assert f(*args(w=NULL, N=0, q=NULL, s=NULL, qt=NULL, st=NULL)) == fp8.OK  # N == 0: no-op
    assert f(*args(N=100)) == fp8.ERR_UNSUPPORTED
    assert f(*args(K=200, ld=200)) == fp8.ERR_UNSUPPORTED
    assert f(*args(qt=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(st=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(ld=128)) == fp8.ERR_INVALID_ARG  # ld < K
    assert f(*args(qt=BAD)) == fp8.ERR_MISALIGNED
    assert f(*args(st=ctypes.c_void_p(0x10002))) == fp8.ERR_MISALIGNED
    assert f(*args(ld=260)) == fp8.ERR_MISALIGNED  # row pitch 520 B


def test_basic_gemm_signatures_take_no_accumulation_argument(L):
    """fp8_block_gemm and fp8_block_grouped_gemm have the boundary's argument
    lists; their validation matches the *_accum forms with the default mode."""
    g = L.fp8_block_gemm
    assert len(g.argtypes) == 11
    base = [GOOD, GOOD, GOOD, GOOD, fp8.B_BLOCK_128x128, GOOD, fp8.BF16, 4, 128, 256, NULL]
    assert g(*[5 if i == 4 else v for i, v in enumerate(base)]) == fp8.ERR_INVALID_ARG
    assert g(*[200 if i == 9 else v for i, v in enumerate(base)]) == fp8.ERR_UNSUPPORTED
    assert g(*[BAD if i == 5 else v for i, v in enumerate(base)]) == fp8.ERR_MISALIGNED
    assert g(*[NULL if i == 0 else (0 if i == 7 else v) for i, v in enumerate(base)]) == fp8.OK
    h = L.fp8_block_grouped_gemm
    assert len(h.argtypes) == 12
    gb = [GOOD, GOOD, GOOD, 4, GOOD, GOOD, GOOD, fp8.BF16, 64, 128, 256, NULL]
    assert h(*[-1 if i == 3 else v for i, v in enumerate(gb)]) == fp8.ERR_INVALID_ARG
    assert h(*[NULL if i == 2 else v for i, v in enumerate(gb)]) == fp8.ERR_INVALID_ARG
    assert h(*[192 if i == 9 else v for i, v in enumerate(gb)]) == fp8.ERR_UNSUPPORTED
    assert h(*[0 if i == 3 else v for i, v in enumerate(gb)]) == fp8.OK


def test_gemm_validation(L):
    f = L.fp8_block_gemm_accum
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("a", GOOD), ("sa", GOOD), ("b", GOOD), ("sb", GOOD), ("mode", fp8.B_BLOCK_128x128),
        ("accum", fp8.ACCUM_FP8_MFMA), ("y", GOOD), ("ydt", fp8.BF16), ("M", 4), ("N", 128),
        ("K", 256), ("s", NULL))]
    assert f(*args(mode=5)) == fp8.ERR_INVALID_ARG
    assert f(*args(accum=9)) == fp8.ERR_INVALID_ARG
    assert f(*args(ydt=3)) == fp8.ERR_INVALID_ARG
    assert f(*args(M=-2)) == fp8.ERR_INVALID_ARG
    assert f(*args(a=NULL, M=0)) == fp8.OK
    assert f(*args(K=200)) == fp8.ERR_UNSUPPORTED
    assert f(*args(N=100)) == fp8.ERR_UNSUPPORTED
    assert f(*args(K=0)) == fp8.ERR_UNSUPPORTED
    assert f(*args(sb=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(y=BAD)) == fp8.ERR_MISALIGNED
    assert f(*args(sa=ctypes.c_void_p(0x10001))) == fp8.ERR_MISALIGNED
    # power-of-two scales on the matrix cores: 128x128 B scales and N % 256 == 0 only
    assert f(*args(accum=fp8.ACCUM_SCALED_MFMA)) == fp8.ERR_UNSUPPORTED  # N = 128
    assert f(*args(accum=fp8.ACCUM_SCALED_MFMA, N=256, mode=fp8.B_ROW_1x128)) == fp8.ERR_UNSUPPORTED
    assert f(*args(accum=fp8.ACCUM_SCALED_MFMA, a=NULL, M=0)) == fp8.OK


def test_grouped_validation(L):
    f = L.fp8_block_grouped_gemm_accum
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("a", GOOD), ("sa", GOOD), ("off", GOOD), ("G", 4), ("b", GOOD), ("sb", GOOD),
        ("accum", fp8.ACCUM_FP8_MFMA), ("y", GOOD), ("ydt", fp8.BF16), ("M", 64), ("N", 128),
        ("K", 256), ("s", NULL))]
    assert f(*args(G=-1)) == fp8.ERR_INVALID_ARG
    assert f(*args(off=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(off=ctypes.c_void_p(0x10002))) == fp8.ERR_MISALIGNED
    assert f(*args(N=192)) == fp8.ERR_UNSUPPORTED
    assert f(*args(G=0)) == fp8.OK
    assert f(*args(M=0, a=NULL)) == fp8.OK


def test_grouped_gather_validation(L):
    f = L.fp8_block_grouped_gemm_gather
    ok = dict(a=GOOD, sa=GOOD, T=32, idx=GOOD, off=GOOD, G=4, b=GOOD, sb=GOOD, accum=fp8.ACCUM_FP8_MFMA,
              y=GOOD, ydt=fp8.BF16, M=64, N=256, K=256, s=NULL)
    args = lambda **kw: [kw.get(k, v) for k, v in ok.items()]
    assert f(*args(G=-1)) == fp8.ERR_INVALID_ARG
    assert f(*args(T=-1)) == fp8.ERR_INVALID_ARG
    assert f(*args(T=0)) == fp8.ERR_INVALID_ARG
    assert f(*args(idx=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(off=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(idx=ctypes.c_void_p(0x10002))) == fp8.ERR_MISALIGNED
    assert f(*args(N=128)) == fp8.ERR_UNSUPPORTED  # gathering needs N % 256 == 0
    assert f(*args(T=1 << 20, K=1 << 13)) == fp8.ERR_UNSUPPORTED  # T * K >= 2^32
    assert f(*args(G=0)) == fp8.OK
    assert f(*args(M=0, a=NULL, idx=NULL)) == fp8.OK


def test_gemm_quant_validation(L):
    f = L.fp8_block_gemm_quant
    ok = dict(a=GOOD, sa=GOOD, b=GOOD, sb=GOOD, accum=fp8.ACCUM_FP8_MFMA, pow2=0, q=GOOD, s=GOOD,
              M=4, N=256, K=256, stream=NULL)
    args = lambda **kw: [kw.get(k, v) for k, v in ok.items()]
    assert f(*args(accum=fp8.ACCUM_EXACT)) == fp8.ERR_UNSUPPORTED
    assert f(*args(accum=7)) == fp8.ERR_INVALID_ARG
    assert f(*args(pow2=2)) == fp8.ERR_INVALID_ARG
    assert f(*args(s=NULL)) == fp8.ERR_INVALID_ARG
    assert f(*args(s=ctypes.c_void_p(0x10002))) == fp8.ERR_MISALIGNED
    assert f(*args(q=BAD)) == fp8.ERR_MISALIGNED
    assert f(*args(N=128)) == fp8.ERR_UNSUPPORTED
    assert f(*args(K=200)) == fp8.ERR_UNSUPPORTED
    assert f(*args(M=0, a=NULL, q=NULL, s=NULL)) == fp8.OK
