"""GPU parity of the quantisers against the oracle: codes and scales bit-exact."""

import numpy as np
import pytest
import torch

import workloads
from fp8_fine_grained_amd import binding as fp8
from oracle import e4m3, quant
from tests.gpu_util import assert_codes_equal, assert_scales_equal, check_guard, f32, guarded, say

pytestmark = pytest.mark.gpu


def _act_rows(x_cpu, what):
    say(f"quant_act rows {what} {tuple(x_cpu.shape)} {x_cpu.dtype}")
    M, K = x_cpu.shape
    x = x_cpu.cuda()
    qb, q = guarded((M, K), torch.uint8)
    sbuf, s = guarded((M, K // 128), torch.float32)
    fp8.fp8_quant_act_1x128(x, q, s)
    torch.cuda.synchronize()
    check_guard(qb)
    check_guard(sbuf)
    q_ref, s_ref = quant.quant_1x128(f32(x_cpu))
    assert_codes_equal(q, q_ref, what)
    assert_scales_equal(s, s_ref, what)
    return q, s


def _special_tiles():
    """Rows built to hit the corners of the cast: zero and -0 tiles, exact E4M3
    tiles, ties, power-of-two scaled copies, subnormal-range values."""
    rng = np.random.default_rng(99)
    rows = []
    z = np.zeros(1024, np.float32)
    rows.append(z.copy())
    nz = z.copy()
    nz[::3] = -0.0
    rows.append(nz)
    codes = rng.integers(0, 256, size=1024).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A
    codes[::128] = 0x7E
    rows.append(e4m3.DECODE_TABLE[codes].astype(np.float32))
    base = rng.standard_normal(1024).astype(np.float32)
    for j in (-30, -8, 0, 7, 40):
        rows.append(base * np.float32(2.0 ** j))
    tiny_range = base.copy()
    tiny_range[::2] *= np.float32(1e-4)  # many elements fall to E4M3 subnormals / zero
    rows.append(tiny_range)
    ties = np.zeros(1024, np.float32)
    ties[::128] = 896.0  # scale 2: grid midpoints below map to exact ties
    mids = (e4m3.DECODE_TABLE[:0x7E] + e4m3.DECODE_TABLE[1:0x7F]) / 2
    for g in range(8):
        ties[g * 128 + 1: g * 128 + 126] = (2 * mids[g * 16: g * 16 + 125] if g * 16 + 125 <= mids.size
                                            else 2 * np.resize(mids, 125)).astype(np.float32)
    rows.append(ties)
    rows.append(-ties)
    for j in (-1, 3, 12, -60, 90):
        rows.append(rng.standard_t(2.5, size=1024).astype(np.float32) * np.float32(2.0 ** j))
    # The ends of the scale range the contract allows: every group's amax exactly
    # 448 * 2^-126 (s = 2^-126, the smallest normal fp32, its other elements down
    # in the fp32 subnormals), and exactly the largest finite bf16, 0x7F7F (so
    # that the bf16 copy of the row is finite too).
    for top in (np.float32(448.0 * 2.0 ** -126), np.uint32(0x7F7F0000).view(np.float32)):
        r = base.copy().reshape(8, 128)
        r = r / np.abs(r).max(axis=1, keepdims=True)
        r = (r.astype(np.float64) * np.float64(top)).astype(np.float32)
        i = np.abs(r).argmax(axis=1)
        r[np.arange(8), i] = np.copysign(top, r[np.arange(8), i])
        rows.append(r.reshape(1024))
    for j in (-5, 20, 60, -100, 110, 1):  # pad to 24 rows (the transposed path needs M % 8 == 0)
        rows.append(rng.standard_t(2.5, size=1024).astype(np.float32) * np.float32(2.0 ** j))
    return np.stack(rows)


def test_act_rows_tiny_fp32():
    _act_rows(workloads.tiny()["x"], "tiny fp32")


def test_act_rows_ragged_bf16():
    _act_rows(workloads.dense(M=300, N=128, K=1024)["x"], "dense-like ragged")


def test_act_rows_student_t():
    _act_rows(workloads.quant_act(M=517, K=7168), "student-t")


def test_act_rows_special_tiles_fp32_and_bf16():
    x = _special_tiles()
    _act_rows(torch.from_numpy(x), "special fp32")
    _act_rows(workloads.to_bf16(x), "special bf16")


def test_act_rows_single_row_and_padded_pitch():
    x = workloads.dense(M=1, N=128, K=256)["x"]
    _act_rows(x, "M=1")
    big = workloads.dense(M=40, N=128, K=512)["x"]
    view = big[:, :384]  # pitch 512 elements, logical K 384
    say("quant_act rows with pitch > K")
    q, s = fp8.fp8_quant_act_1x128(big.cuda()[:, :384])
    q_ref, s_ref = quant.quant_1x128(f32(view))
    assert_codes_equal(q, q_ref, "pitch")
    assert_scales_equal(s, s_ref, "pitch")


def test_act_rows_deterministic():
    x = workloads.quant_act(M=256, K=2048).cuda()
    q1, s1 = fp8.fp8_quant_act_1x128(x)
    q2, s2 = fp8.fp8_quant_act_1x128(x)
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def _act_cols(x_phys_cpu, what):
    """x_phys [T, C]: quantise along T (the gradient-operand layout)."""
    say(f"quant_act transposed {what} {tuple(x_phys_cpu.shape)}")
    T, C = x_phys_cpu.shape
    x = x_phys_cpu.cuda()
    qb, q = guarded((C, T), torch.uint8)
    sbuf, s = guarded((C, T // 128), torch.float32)
    fp8.fp8_quant_act_1x128(x.t(), q, s)
    torch.cuda.synchronize()
    check_guard(qb)
    check_guard(sbuf)
    q_ref, s_ref = quant.quant_1x128_along_rows(f32(x_phys_cpu))
    assert_codes_equal(q, q_ref, what)
    assert_scales_equal(s, s_ref, what)
    return q, s


def test_act_cols_small():
    d = workloads.wgrad(T=384, C=200, Cin=136)
    _act_cols(d["dy"], "dY")
    _act_cols(d["x"], "X")
    _act_cols(torch.from_numpy(_special_tiles().T.copy()), "special fp32")


def test_act_cols_xcd_ordered_grid():
    # 8 token groups x 2 or 3 column blocks: block counts divisible by 8 take the
    # XCD-contiguous block order (the other tests' small grids do not)
    d = workloads.wgrad(T=1024, C=256, Cin=384)
    _act_cols(d["dy"], "dY 16 blocks")
    _act_cols(d["x"], "X 24 blocks")


def test_weight_small():
    for w, what in ((workloads.tiny()["w"], "tiny fp32"),
                    (workloads.dense(M=1, N=384, K=1024)["w"], "dense-like bf16"),
                    (torch.from_numpy(_special_tiles()[:8].reshape(8, 1024)[:, :].repeat(16, axis=0)[:128]), "special")):
        say(f"quant_weight {what} {tuple(w.shape)}")
        N, K = w.shape
        qb, q = guarded((N, K), torch.uint8)
        sbuf, s = guarded((N // 128, K // 128), torch.float32)
        fp8.fp8_quant_weight_128x128(w.cuda(), q, s)
        torch.cuda.synchronize()
        check_guard(qb)
        check_guard(sbuf)
        q_ref, s_ref = quant.quant_128x128(f32(w))
        assert_codes_equal(q, q_ref, what)
        assert_scales_equal(s, s_ref, what)


def _weight_dual(w, what):
    """Dual quantiser: row-major pair against the oracle on W, transposed pair
    against the oracle on W^T (computed independently from the transposed input)."""
    say(f"quant_weight dual {what} {tuple(w.shape)}")
    N, K = w.shape
    qb, q = guarded((N, K), torch.uint8)
    sbuf, s = guarded((N // 128, K // 128), torch.float32)
    qtb, qt = guarded((K, N), torch.uint8)
    stbuf, st = guarded((K // 128, N // 128), torch.float32)
    fp8.fp8_quant_weight_128x128_dual(w.cuda(), q, s, qt, st)
    torch.cuda.synchronize()
    for b in (qb, sbuf, qtb, stbuf):
        check_guard(b)
    wf = f32(w)
    q_ref, s_ref = quant.quant_128x128(wf)
    assert_codes_equal(q, q_ref, what)
    assert_scales_equal(s, s_ref, what)
    qt_ref, st_ref = quant.quant_128x128(np.ascontiguousarray(wf.T))
    assert_codes_equal(qt, qt_ref, what + " transposed")
    assert_scales_equal(st, st_ref, what + " transposed")


def test_weight_dual_small():
    _weight_dual(workloads.tiny()["w"], "tiny fp32")
    _weight_dual(workloads.dense(M=1, N=384, K=1024)["w"], "dense-like bf16")
    _weight_dual(workloads.dgrad(M=1, N=640, K=256)["w"], "dgrad-like bf16, N > K")
    _weight_dual(torch.from_numpy(_special_tiles()[:8].reshape(8, 1024).repeat(16, axis=0)[:128]), "special")


def _act_weight(x, w, pow2, what, oracle=False):
    """The one-launch pair against the two separate calls, bit for bit, with
    guard bands around all four outputs; optionally against the oracle too."""
    say(f"quant_act_weight {what}: x {tuple(x.shape)} {x.dtype}, w {tuple(w.shape)} {w.dtype}, pow2={pow2}")
    M, Kx = x.shape
    N, Kw = w.shape
    bufs = [guarded((M, Kx), torch.uint8), guarded((M, Kx // 128), torch.float32),
            guarded((N, Kw), torch.uint8), guarded((N // 128, Kw // 128), torch.float32)]
    xd, wd = x.cuda(), w.cuda()
    fp8.fp8_quant_act_weight(xd, wd, *[v for _, v in bufs], pow2=pow2)
    torch.cuda.synchronize()
    for b, _ in bufs:
        check_guard(b)
    qx, sx, qw, sw = (v for _, v in bufs)
    if M:
        rx, rsx = fp8.fp8_quant_act_1x128(xd, pow2=pow2)
        assert torch.equal(qx, rx) and torch.equal(sx.view(torch.int32), rsx.view(torch.int32)), what + " act"
    if N:
        rw, rsw = fp8.fp8_quant_weight_128x128(wd, pow2=pow2)
        assert torch.equal(qw, rw) and torch.equal(sw.view(torch.int32), rsw.view(torch.int32)), what + " weight"
    if oracle:
        q_ref, s_ref = quant.quant_1x128(f32(x))
        assert_codes_equal(qx, q_ref, what + " act")
        assert_scales_equal(sx, s_ref, what + " act")
        q_ref, s_ref = quant.quant_128x128(f32(w))
        assert_codes_equal(qw, q_ref, what + " weight")
        assert_scales_equal(sw, s_ref, what + " weight")


def test_act_weight_one_launch():
    d = workloads.dense(seed=21, M=300, N=256, K=512)  # 1200 activation tiles: a partial last workgroup
    x, w = d["x"], d["w"]
    _act_weight(x, w, False, "bf16 / bf16", oracle=True)
    _act_weight(x, w, True, "bf16 / bf16, power-of-two scales")
    _act_weight(x.float(), w, False, "fp32 / bf16")
    _act_weight(x, w.float(), False, "bf16 / fp32")
    t = workloads.tiny()
    _act_weight(t["x"], t["w"], False, "tiny fp32 / fp32", oracle=True)
    _act_weight(torch.from_numpy(_special_tiles()), w[:, :384].contiguous(), False, "special tiles, K 1024 / 384",
                oracle=True)
    _act_weight(x[:0], w, False, "no activation rows")
    _act_weight(x, w[:0], False, "no weight rows")


def test_act_weight_one_launch_dense_shape():
    d = workloads.dense()
    _act_weight(d["x"], d["w"], False, "X [4096,7168] + W [7168,7168] bf16")


def test_cast_exhaustive_through_the_act_quantiser():
    """Every fp32 in [0, 448] and its negation through the 1x128 kernel's cast.

    Each tile holds +-448 followed by 127 probe values, so amax = 448, s = 1 and
    1/s = 1: the kernel casts the probe values unscaled.  The expected codes come
    from torch's CPU float8_e4m3fn codec, which the oracle pins (tests/
    test_oracle_e4m3.py) show equal to the oracle's encoder on this whole range."""
    top = int(np.float32(448.0).view(np.uint32))
    per = 127
    tiles_per_call = 1 << 20
    total = top + 1
    for sign in (1.0, -1.0):
        say(f"cast sweep, sign {sign:+.0f}: {total} values in tiles of 448 + 127 probes")
        for lo in range(0, total, tiles_per_call * per):
            n = min(tiles_per_call * per, total - lo)
            T = (n + per - 1) // per
            bits = torch.clamp(torch.arange(lo, lo + T * per, dtype=torch.int32), max=top)
            vals = bits.view(torch.float32) * sign
            x = torch.empty((T, 128), dtype=torch.float32)
            x[:, 0] = 448.0 * sign
            x[:, 1:] = vals.view(T, per)
            q, s = fp8.fp8_quant_act_1x128(x.cuda())
            got = q[:, 1:].reshape(-1).cpu()
            torch.cuda.synchronize()
            assert bool(torch.all(s == 1.0)), "scale of an amax-448 tile"
            assert bool(torch.all(q[:, 0] == (0x7E if sign > 0 else 0xFE)))
            want = vals.to(torch.float8_e4m3fn).view(torch.uint8)
            if not torch.equal(got, want):
                bad = torch.nonzero(got != want).flatten()[:5].tolist()
                raise AssertionError([(float(vals[i]), hex(int(got[i])), hex(int(want[i]))) for i in bad])


def test_validation_errors_reported():
    x = torch.zeros((4, 100), device="cuda")
    with pytest.raises(fp8.Fp8fgError) as e:
        fp8.fp8_quant_act_1x128(x)
    assert e.value.status == fp8.ERR_UNSUPPORTED
    w = torch.zeros((100, 128), device="cuda")
    with pytest.raises(fp8.Fp8fgError) as e:
        fp8.fp8_quant_weight_128x128(w)
    assert e.value.status == fp8.ERR_UNSUPPORTED


# ------------------------------------------------------------ full sizes

def test_full_dense_activation():
    _act_rows(workloads.dense()["x"], "dense X [4096,7168]")


def test_full_quant_act():
    _act_rows(workloads.quant_act(), "act [16384,7168]")


def test_full_quant_weight():
    w = workloads.quant_weight()
    say("quant_weight full [7168,18432]")
    q, s = fp8.fp8_quant_weight_128x128(w.cuda())
    q_ref, s_ref = quant.quant_128x128(f32(w))
    assert_codes_equal(q, q_ref, "weight full")
    assert_scales_equal(s, s_ref, "weight full")


def test_full_dgrad_weight():
    _weight_dual(workloads.dgrad()["w"], "dgrad W [7168,7168]")


def test_full_wgrad_operands():
    d = workloads.wgrad()
    _act_cols(d["dy"], "dY [16384,7168]")
    _act_cols(d["x"], "X [16384,7168]")
