"""Pins of the oracle's fp8 E4M3FN codec: exhaustive against torch's
float8_e4m3fn (a library implementation of the same OCP format), against
values fixed by the format's definition, and against a brute-force
nearest-value search with ties to even."""
import numpy as np
import torch

import oracle


def _torch_decode_all():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_all_256_codes_match_torch():
    ours = oracle.fp8_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_decode_landmarks_of_the_format():
    """Values the E4M3FN definition fixes: bias 7, 3 mantissa bits,
    subnormals below 2^-6, max 448, S.1111.111 is NaN, no infinity."""
    d = lambda c: float(oracle.fp8_decode(np.array([c], np.uint8))[0])
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert d(0x38) == 1.0  # e=7, m=0
    assert d(0x01) == 2.0 ** -9  # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert d(0x08) == 2.0 ** -6  # smallest normal
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x77) == 240.0  # e=14, m=7: 1.875 * 2^7
    assert np.all(np.isfinite(oracle.fp8_decode(np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8))))


def _all_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32) << 16
    return bits.view(np.float32)


def test_encode_all_bf16_inputs_match_torch_in_range():
    """torch rounds to nearest-even and overflows to NaN past 464; the
    reading taken here saturates instead. Inside +-464 both must agree."""
    for scale in (1.0, 0.5, 3.7, 1.0 / 448.0, 2.0 ** -7, 100.0):
        x = (_all_bf16_as_f32() / np.float32(scale)).astype(np.float32)
        ours = oracle.fp8_encode(x)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        finite = np.isfinite(x)
        inr = finite & (np.abs(x) <= 464.0)
        assert np.array_equal(ours[inr], ref[inr]), f"scale {scale}"
        big = finite & (np.abs(x) > 464.0)
        assert np.all(ours[big] & 0x7F == 0x7E)
        assert np.array_equal(ours[big] >> 7, np.signbit(x[big]).astype(np.uint8))
        assert np.all(ours[np.isnan(x)] == 0x7F)
        inf = np.isinf(x)
        assert np.all(ours[inf] & 0x7F == 0x7E)


def test_encode_is_nearest_with_ties_to_even_by_brute_force():
    """Exact nearest-value search over all 127 non-negative finite codes,
    ties broken toward the even code, on a random sample plus every exact
    midpoint between neighbouring codes."""
    vals = oracle.fp8_decode(np.arange(0x7F, dtype=np.uint8))  # 0x00..0x7E ascending
    mids = (vals[:-1] + vals[1:]) / 2.0
    rng = np.random.default_rng(0)
    sample = np.concatenate([mids, rng.uniform(0, 448, 20000), rng.uniform(0, 0.02, 20000),
                             vals]).astype(np.float32)
    sample = sample[np.abs(sample.astype(np.float64)) <= 448.0]
    ours = oracle.fp8_encode(sample)
    for x, c in zip(sample.astype(np.float64), ours):
        dist = np.abs(vals - x)
        best = np.flatnonzero(dist == dist.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want, (x, c, want)
    neg = oracle.fp8_encode(-sample)
    assert np.array_equal(neg & 0x7F, ours)
    assert np.all((neg >> 7)[sample != 0] == 1)


def test_round_trip_of_every_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = oracle.fp8_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.fp8_encode(vals), codes)


def test_block_encoder_divides_by_the_block_scale():
    rng = np.random.default_rng(3)
    src = rng.standard_normal((5, 2, 16, 8)).astype(np.float32)
    scales = (np.abs(src).max(axis=(2, 3)) / 448.0).astype(np.float32)
    codes = oracle.fp8_encode_blocks(src, scales)
    want = oracle.fp8_encode((src / scales[:, :, None, None]).astype(np.float32))
    assert np.array_equal(codes, want)
    # the block maximum lands on +-448 exactly
    dec = oracle.fp8_decode(codes)
    assert np.allclose(np.abs(dec).max(axis=(2, 3)), 448.0)
