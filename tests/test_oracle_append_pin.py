"""Pins of the oracle's KV append against an independent model of it.

The append is the block table's logical-to-physical mapping run forwards
("03 -- Engines Papers", section 2: a token's slot s names physical block
s // 16 at offset s % 16), plus, for an FP8 cache, quantization with a
scale per (block, KV head) ("The LLM inference engine playbook", Themes 3
and 6: E4M3 values with a scale).

The expected cache images here are built without the oracle: a numpy
scatter into the K layout [block][head][offset][dim] and the V layout
[block][head][dim][offset], and, for fp8, torch's own float8_e4m3fn
conversion of fp32(x) / scale. Inputs are chosen so that each plausible
slip in the oracle fails at least one test: heads swapped or reversed,
tokens shifted, the K scale used for V (or the V scale for K), the block
and offset of a slot exchanged, K and V layouts exchanged, and a skipped
slot written anyway."""
import numpy as np
import pytest
import torch

import oracle

NAN_BF16 = 0x7FC0
NAN_FP8 = 0x7F


def _bf16_bits(x32):
    """float32 -> bf16 bit patterns, round to nearest even (torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _fp8_codes_torch(x32):
    """float32 -> e4m3fn codes by torch's conversion (|x| must stay <= 448)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _case(rng, T, H, D, NB, dtype):
    """Random new rows and a slot mapping over several blocks, with a -1."""
    kn = rng.standard_normal((T, H, D)).astype(np.float32)
    vn = (3.0 * rng.standard_normal((T, H, D))).astype(np.float32)
    # distinct slots spread over the pool; one token skipped
    slots = rng.choice(NB * 16, size=T, replace=False).astype(np.int32)
    slots[T // 2] = -1
    return kn, vn, slots


def _expected_images(kn, vn, slots, H, D, NB, fill, enc_k, enc_v):
    """Scatter with numpy fancy indexing (no loops over heads or dims)."""
    kc = np.full((NB, H, 16, D), fill, dtype=enc_k.dtype)
    vc = np.full((NB, H, D, 16), fill, dtype=enc_v.dtype)
    keep = slots >= 0
    t = np.nonzero(keep)[0]
    b = slots[keep] // 16
    o = slots[keep] % 16
    # K[b][g][o][:] = new[t][g][:]; V[b][g][:][o] = new[t][g][:]
    kc[b, :, o, :] = enc_k[t]
    vc[b, :, :, o] = enc_v[t]
    return kc, vc


@pytest.mark.parametrize("H,D", [(3, 16), (4, 64), (2, 128)])
def test_append_f32_matches_numpy_scatter(H, D):
    """Catches: head or token index slips, block/offset exchanged, the V
    layout written token-major, a skipped slot written."""
    rng = np.random.default_rng(11 * H + D)
    T, NB = 21, 9
    kn, vn, slots = _case(rng, T, H, D, NB, "f32")
    kc_ref, vc_ref = _expected_images(kn, vn, slots, H, D, NB, np.float32(np.nan), kn, vn)
    kc = np.full((NB, H, 16, D), np.nan, np.float32)
    vc = np.full((NB, H, D, 16), np.nan, np.float32)
    oracle.kv_append(kc, vc, kn, vn, slots, kv_dtype="f32", new_dtype="f32",
                     num_kv_heads=H, head_dim=D)
    assert np.array_equal(kc.view(np.uint32), kc_ref.view(np.uint32))
    assert np.array_equal(vc.view(np.uint32), vc_ref.view(np.uint32))


@pytest.mark.parametrize("H,D", [(4, 64), (8, 128)])
def test_append_bf16_matches_numpy_scatter(H, D):
    """Same, for bf16 caches: the bits move unchanged."""
    rng = np.random.default_rng(5 * H + D)
    T, NB = 37, 12
    kn32, vn32, slots = _case(rng, T, H, D, NB, "bf16")
    kn, vn = _bf16_bits(kn32), _bf16_bits(vn32)
    kc_ref, vc_ref = _expected_images(kn, vn, slots, H, D, NB, np.uint16(NAN_BF16), kn, vn)
    kc = np.full((NB, H, 16, D), NAN_BF16, np.uint16)
    vc = np.full((NB, H, D, 16), NAN_BF16, np.uint16)
    oracle.kv_append(kc, vc, kn, vn, slots, kv_dtype="bf16", new_dtype="bf16",
                     num_kv_heads=H, head_dim=D)
    assert np.array_equal(kc, kc_ref)
    assert np.array_equal(vc, vc_ref)


@pytest.mark.parametrize("new_dtype", ["bf16", "f32"])
def test_append_fp8_quantizes_with_the_blocks_own_scales(new_dtype):
    """fp8 caches: byte = e4m3fn(fp32(x) / scale[block][head]), with
    different K and V scales for every (block, head), by torch's
    conversion. Catches: k_scale used for V (or v_scale for K), the scale
    of the wrong block or head, multiplication in place of division, and
    every index slip of the bf16 test."""
    rng = np.random.default_rng(2024)
    H, D, T, NB = 4, 64, 29, 10
    kn32, vn32, slots = _case(rng, T, H, D, NB, new_dtype)
    if new_dtype == "bf16":
        kn, vn = _bf16_bits(kn32), _bf16_bits(vn32)
        kx, vx = _bf16_value(kn), _bf16_value(vn)
    else:
        kn, vn = kn32, vn32
        kx, vx = kn32, vn32
    # scales per (block, head), K and V apart by a factor that is not a
    # power of two, all large enough that |x / scale| stays below 448
    ks = (0.02 + 0.01 * rng.random((NB, H))).astype(np.float32)
    vs = (0.07 + 0.03 * rng.random((NB, H))).astype(np.float32)
    keep = slots >= 0
    b = np.where(keep, slots // 16, 0)
    # fp32 division per element by the destination's (block, head) scale
    kq = (kx / ks[b][:, :, None]).astype(np.float32)
    vq = (vx / vs[b][:, :, None]).astype(np.float32)
    assert np.abs(kq[keep]).max() < 448 and np.abs(vq[keep]).max() < 448
    enc_k, enc_v = _fp8_codes_torch(kq), _fp8_codes_torch(vq)
    kc_ref, vc_ref = _expected_images(kn, vn, slots, H, D, NB, np.uint8(NAN_FP8), enc_k, enc_v)
    kc = np.full((NB, H, 16, D), NAN_FP8, np.uint8)
    vc = np.full((NB, H, D, 16), NAN_FP8, np.uint8)
    oracle.kv_append(kc, vc, kn, vn, slots, kv_dtype="fp8", new_dtype=new_dtype,
                     k_scale=ks, v_scale=vs, num_kv_heads=H, head_dim=D)
    assert np.array_equal(kc, kc_ref)
    assert np.array_equal(vc, vc_ref)


def test_append_then_gather_returns_the_rows():
    """The append followed by a plain Python gather through a block table
    gives back each token's row: slot = table[pos // 16] * 16 + pos % 16,
    the mapping of the first page's section 2, walked by hand here."""
    H, D = 3, 8
    table = [5, 2, 7]  # logical block j -> physical block
    L = 40
    rng = np.random.default_rng(3)
    rows_k = rng.standard_normal((L, H, D)).astype(np.float32)
    rows_v = rng.standard_normal((L, H, D)).astype(np.float32)
    slots = np.array([table[p // 16] * 16 + p % 16 for p in range(L)], np.int32)
    kc = np.full((8, H, 16, D), np.nan, np.float32)
    vc = np.full((8, H, D, 16), np.nan, np.float32)
    oracle.kv_append(kc, vc, rows_k, rows_v, slots, kv_dtype="f32", new_dtype="f32",
                     num_kv_heads=H, head_dim=D)
    for p in range(L):
        blk, off = table[p // 16], p % 16
        for g in range(H):
            for d in range(D):
                assert kc[blk, g, off, d] == rows_k[p, g, d]
                assert vc[blk, g, d, off] == rows_v[p, g, d]
    # blocks the table never names stay untouched
    for blk in set(range(8)) - set(table):
        assert np.isnan(kc[blk]).all() and np.isnan(vc[blk]).all()
