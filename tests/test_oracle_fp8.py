"""Pins of the 8-bit (E4M3) cache oracle: the value table, rounding, the
per-row scale, the pool layout and attention over the dequantised cache.

The independent references are torch's ``float8_e4m3fn`` conversions (a
library routine for the same OCP format), closed-form code values, and a
brute-force attention over logical tensors quantised through torch, which
shares nothing with the oracle's table, rounding or pool layout.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from helpers import bits, brute_force, oracle_run
from oracle import fp8
from oracle.pool import Pool, to_f64

E4M3 = torch.float8_e4m3fn


def torch_values():
    return torch.arange(256, dtype=torch.uint8).view(E4M3).to(torch.float64).numpy()


def test_value_table_matches_library():
    ref = torch_values()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(fp8.VALUES))
    assert np.array_equal(ref[~nan], fp8.VALUES[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(fp8.VALUES[~nan]))


def test_value_table_closed_forms():
    assert fp8.value(0x7E) == 448.0 and fp8.value(0xFE) == -448.0
    assert fp8.value(0x38) == 1.0                      # exponent field 7 = bias
    assert fp8.value(0x08) == 2.0 ** -6                # smallest normal
    assert fp8.value(0x01) == 2.0 ** -9                # smallest subnormal
    assert fp8.value(0x07) == 7 * 2.0 ** -9            # largest subnormal
    assert fp8.value(0x00) == 0.0 and math.copysign(1, fp8.value(0x80)) == -1
    assert [c for c in range(256) if math.isnan(fp8.value(c))] == [0x7F, 0xFF]


def test_encode_roundtrip_every_code():
    finite = [c for c in range(256) if not math.isnan(fp8.VALUES[c])]
    got = fp8.encode(fp8.VALUES[finite])
    assert list(got) == finite


def test_encode_ties_to_even_and_range():
    pos = fp8.VALUES[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2                  # exact in fp64 and fp32
    codes = fp8.encode(mids)
    lo = np.arange(0x7E)
    assert np.all((codes == lo) | (codes == lo + 1))
    assert np.all(codes % 2 == 0)
    assert fp8.encode(np.array([464.0]))[0] == 0x7E   # the 448 | (480) tie
    assert fp8.encode(np.array([464.0001]))[0] == 0x7F
    assert fp8.encode(np.array([-500.0]))[0] == 0xFF
    assert fp8.encode(np.array([-0.0]))[0] == 0x80


def test_encode_matches_library_rounding():
    rng = np.random.default_rng(0)
    pos = fp8.VALUES[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    f32 = np.float32
    ys = np.concatenate([
        rng.uniform(-464, 464, 20000), rng.standard_normal(20000) * 3,
        rng.uniform(-2 ** -5, 2 ** -5, 5000), mids, -mids,
        np.nextafter(mids.astype(f32), f32(np.inf)), np.nextafter(mids.astype(f32), f32(-np.inf)),
    ]).astype(np.float32)
    ref = torch.from_numpy(ys).to(E4M3).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(ys.astype(np.float64)), ref)


def test_grid_rounding_equals_table_search():
    """``encode`` (rounding onto the format's grid) gives the codes of the
    plain nearest-value search ``encode_nearest`` on every fp32 value of
    whole binades around the subnormal, normal and overflow ranges, on
    midpoints and their neighbours, and on random values of both signs."""
    rng = np.random.default_rng(7)
    f32 = np.float32
    pos = fp8.VALUES[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    binades = []
    for lo in (2.0 ** -12, 2.0 ** -9, 2.0 ** -7, 2.0 ** -6, 0.75, 1.0, 256.0):   # every fp32 in [lo, 2 lo)
        a = np.float32(lo).view(np.uint32)
        binades.append(np.arange(a, a + (1 << 23), 64, dtype=np.uint32).view(np.float32))
    ys = np.concatenate(binades + [
        rng.uniform(-600, 600, 200000).astype(f32), (rng.standard_normal(200000) * 2.0 ** -7).astype(f32),
        mids.astype(f32), np.nextafter(mids.astype(f32), f32(np.inf)), np.nextafter(mids.astype(f32), f32(-np.inf)),
        pos.astype(f32), np.array([0.0, 464.0, 464.00003, 479.99997, 480.0, 1e30, np.nan, np.inf], dtype=f32),
    ]).astype(np.float64)
    ys = np.concatenate([ys, -ys])
    assert np.array_equal(fp8.encode(ys), fp8.encode_nearest(ys))


def test_quantize_row_scale_and_error_bound():
    rng = np.random.default_rng(1)
    for trial in range(200):
        x = (rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 4)).astype(np.float32)
        codes, s = fp8.quantize_row(x)
        amax = np.float32(np.abs(x).max())
        assert s == np.float32(amax / np.float32(448))
        # the largest element lands on +-448
        assert abs(fp8.VALUES[codes[np.argmax(np.abs(x))]]) == 448.0
        y = np.abs(x.astype(np.float64)) / np.float64(s)
        err = np.abs(fp8.dequantize_row(codes, s) - x)
        # half a step of the E4M3 grid at |y| (2^-4 relative for normals,
        # 2^-10 absolute below 2^-6), plus the fp32 rounding of the quotient
        half_step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 1e-300))) - 4), 2.0 ** -10)
        assert np.all(err <= (half_step + y * 2.0 ** -23) * np.float64(s) * (1 + 1e-12))


def test_quantize_zero_row():
    codes, s = fp8.quantize_row(np.zeros(64, dtype=np.float32))
    assert s == 0 and not codes.any()
    assert not fp8.dequantize_row(codes, s).any()


def test_pool_layout_positions():
    """Each code lands where the documented layout puts it."""
    rng = np.random.default_rng(2)
    d, Hkv = 128, 2
    pl = Pool(6, Hkv, d, "fp8")
    k = torch.randn(3, Hkv, d, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(3, Hkv, d, dtype=torch.float32).to(torch.bfloat16)
    slots = [5 * 16 + 13, 0 * 16 + 2, 3 * 16 + 7]
    pl.scatter(0, slots, bits(k), bits(v))
    for i, slot in enumerate(slots):
        b, o = divmod(slot, 16)
        for h in range(Hkv):
            kc, ks = fp8.quantize_row(k[i, h].float().numpy())
            vc, vs = fp8.quantize_row(v[i, h].float().numpy())
            for j in rng.choice(d, 16, replace=False):
                assert pl.K[0][b, h, j // 16, o, j % 16] == kc[j]
                a, r = divmod(int(j), 64)
                assert pl.V[0][b, h, a, o // 4, r // 4, r % 4, o % 4] == vc[j]
            assert pl.KS[0][b, h, o] == np.float32(ks).view(np.uint32)
            assert pl.VS[0][b, h, o] == np.float32(vs).view(np.uint32)
    # untouched slots keep the poison
    assert pl.K[0][1].max() == 0x7F and np.all(pl.VS[0][1] == 0x7FC00000)


def torch_quantized(x: torch.Tensor) -> torch.Tensor:
    """Dequantised fp64 copy of bf16 rows [..][d] through torch: per-row
    fp32 scale amax/448, codes by torch's E4M3 conversion."""
    x32 = x.to(torch.float32)
    amax = x32.abs().amax(dim=-1, keepdim=True)
    s = amax / torch.tensor(448.0, dtype=torch.float32)
    y = torch.where(s > 0, x32 / torch.where(s > 0, s, torch.ones_like(s)), torch.zeros_like(x32))
    return y.to(E4M3).to(torch.float64) * s.to(torch.float64)


@pytest.mark.parametrize("make", [
    lambda: workloads.random_small(21, S=4, Hq=8, Hkv=2, d=64, dtype="bf16", max_len=70),
    lambda: workloads.random_small(22, S=3, Hq=6, Hkv=3, d=128, dtype="bf16", max_len=40),
])
def test_paged_fp8_attention_matches_brute_force(make):
    wl = workloads.fp8_cache(make())
    q, k, v = wl.tensors()
    _, out = oracle_run(wl, q, k, v)
    ref = brute_force(wl, q, torch_quantized(k), torch_quantized(v))
    assert np.abs(out - ref).max() <= 1e-13


def test_fp8_cache_stays_close_to_bf16():
    """Quantisation error of the 8-bit cache on N(0,1) data, against the
    same batch with a bf16 cache (a format property, not a parity bar)."""
    base = workloads.random_small(23, S=4, Hq=8, Hkv=2, d=128, dtype="bf16", max_len=300)
    q, k, v = base.tensors()
    _, o16 = oracle_run(base, q, k, v)
    _, o8 = oracle_run(workloads.fp8_cache(base), q, k, v)
    # E4M3 keeps 3 mantissa bits: a value's relative rounding error is at most
    # 2^-4 and its RMS about 2^-4 / sqrt(3) = 0.036; the outputs average such
    # errors (measured: 0.026 - 0.043), so 0.06 leaves room and still fails
    # for any wrong scale or misplaced code.
    rel_rms = math.sqrt(((o8 - o16) ** 2).mean() / (o16 ** 2).mean())
    assert rel_rms < 0.06
