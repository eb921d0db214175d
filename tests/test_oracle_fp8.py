"""Pins for the oracle's FP8 E4M3 codec (CPU only): hand-decoded codes from the format's
definition, ties, saturation, the exhaustive code round trip, and agreement with torch's
float8_e4m3fn cast (a library routine) on in-range values."""
import math

import numpy as np
import pytest
import torch

from oracle import fp8 as F8


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0), (0x08, 2.0 ** -6),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x00, 0.0), (0xB8, -1.0), (0xFE, -448.0),
    (0x30, 0.5), (0x28, 0.25), (0x57, 15.0),
])
def test_decode_known_codes(code, value):
    assert F8.e4m3_decode(np.array([code], np.uint8))[0] == value


def test_decode_nan_and_negative_zero():
    d = F8.e4m3_decode(np.array([0x7F, 0xFF, 0x80], np.uint8))
    assert np.isnan(d[0]) and np.isnan(d[1])
    assert d[2] == 0.0 and math.copysign(1.0, d[2]) == -1.0


def test_every_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(F8.e4m3_encode(F8.e4m3_decode(codes)), codes)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),        # halfway 1.0 / 1.125: even mantissa 0
    (1.1875, 0x3A),        # halfway 1.125 / 1.25: even mantissa 2
    (2.0 ** -10, 0x00),    # halfway 0 / 2^-9: even 0
    (3 * 2.0 ** -10, 0x02),  # halfway 2^-9 / 2^-8: even 2
    (15.5 * 2.0 ** -10, 0x08),  # rounds up out of the subnormals
    (440.0, 0x7E), (-0.0, 0x80),
])
def test_encode_ties_to_even(x, code):
    assert F8.e4m3_encode(np.array([x]))[0] == code


def test_quantize_saturates_and_divides_in_float32():
    q = F8.quantize(np.array([1e6, -500.0, 448.0, 3.0], np.float32), 1.0)
    assert list(q) == [0x7E, 0xFE, 0x7E, 0x44]
    # x / scale rounded to float32 first: 1/3 in float32, then to E4M3
    assert F8.quantize(np.array([1.0], np.float32), 3.0)[0] == F8.e4m3_encode(np.array([np.float32(1.0) / np.float32(3.0)]))[0]


def test_agrees_with_torch_cast_in_range():
    g = np.random.default_rng(5)
    x = np.concatenate([g.uniform(-448, 448, 50000), g.normal(0, 1, 50000),
                        g.uniform(-2.0 ** -5, 2.0 ** -5, 20000)]).astype(np.float32)
    ours = F8.e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


# ---------------------------------------------------------------- 8-bit KV cache attention

def _torch_dequant(codes: np.ndarray, scale: float) -> torch.Tensor:
    """Independent dequantisation: torch's float8_e4m3fn -> float64 conversion, times the scale."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    return t * float(np.float32(scale))


def test_fp8_paged_decode_equals_sdpa_on_dequantised_kv():
    from oracle import attention as OA
    g = np.random.default_rng(9)
    B, Hq, Hkv, D, bs, x = 3, 4, 2, 32, 8, 16
    lens = [5, 17, 24]
    ks, vs = 0.0125, 0.02
    nblk = [(L + bs - 1) // bs for L in lens]
    NB = sum(nblk) + 3
    perm = g.permutation(NB)
    tables = np.full((B, max(nblk)), -1, np.int32)
    o = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    kc = np.full((NB, Hkv, D // x, bs, x), 0x7F, np.uint8)   # NaN codes in unused slots
    vc = np.full((NB, Hkv, D, bs), 0x7F, np.uint8)
    dense_k, dense_v = [], []
    for b, L in enumerate(lens):
        kcodes = F8.quantize(g.normal(0, 1, (Hkv, L, D)).astype(np.float32), ks)
        vcodes = F8.quantize(g.normal(0, 1, (Hkv, L, D)).astype(np.float32), vs)
        for t in range(L):
            blk, off = tables[b, t // bs], t % bs
            for h in range(Hkv):
                for d in range(D):
                    kc[blk, h, d // x, off, d % x] = kcodes[h, t, d]
                    vc[blk, h, d, off] = vcodes[h, t, d]
        dense_k.append(_torch_dequant(kcodes, ks))
        dense_v.append(_torch_dequant(vcodes, vs))
    q = torch.from_numpy(g.normal(0, 1, (B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
    qbits = q.view(torch.int16).numpy().view(np.uint16)
    scale = 1.0 / math.sqrt(D)
    got = OA.paged_decode(qbits, kc, vc, "bf16", tables, np.array(lens), scale, kv_dtype="e4m3",
                          k_scale=ks, v_scale=vs)
    for b in range(B):
        qq = q[b].to(torch.float64).view(Hkv, Hq // Hkv, 1, D)
        kk = dense_k[b].view(Hkv, 1, lens[b], D)
        vv = dense_v[b].view(Hkv, 1, lens[b], D)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, scale=float(np.float32(scale))).view(Hq, D).numpy()
        assert np.max(np.abs(got[b] - ref)) <= 1e-12


def test_fp8_reshape_and_cache_matches_torch_quantisation():
    from oracle import cache_ops as OC
    g = np.random.default_rng(10)
    N, H, D, bs, NB = 5, 2, 32, 16, 6
    key = torch.from_numpy(g.normal(0, 3, (N, H, D)).astype(np.float32)).to(torch.bfloat16)
    val = torch.from_numpy(g.normal(0, 3, (N, H, D)).astype(np.float32)).to(torch.bfloat16)
    kc = np.zeros((NB, H, D // 16, bs, 16), np.uint8)
    vc = np.zeros((NB, H, D, bs), np.uint8)
    slots = np.array([3, -1, 40, 95, 17])
    ks, vs = 0.01, 0.03
    OC.reshape_and_cache_fp8(kc, vc, key.view(torch.int16).numpy().view(np.uint16),
                             val.view(torch.int16).numpy().view(np.uint16), "bf16", slots, ks, vs)

    def tq(x, s):  # torch: x / s in float32, clamp, cast
        y = torch.clamp(x.to(torch.float32) / torch.tensor(s, dtype=torch.float32), -448, 448)
        return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    kq, vq = tq(key, ks), tq(val, vs)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = slot // bs, slot % bs
        assert np.array_equal(kc[blk, :, :, off, :].reshape(H, D), kq[i])
        assert np.array_equal(vc[blk, :, :, off], vq[i])
    assert not kc[3:5].any() and not vc[3:5].any()   # blocks no slot names stay untouched
