"""Pins for the oracle's INT8 codec of the 8-bit KV cache (CPU only): two's-complement decoding,
ties to even, saturation at +-127, the float32 division, agreement with torch's round-half-even
quantisation (a library routine), and paged decode / cache write over INT8 codes against torch's
own dequantisation and SDPA."""
import math

import numpy as np
import pytest
import torch

from oracle import int8 as I8


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 1.0), (0x7F, 127.0), (0x80, -128.0), (0x81, -127.0), (0xFF, -1.0),
    (0xC0, -64.0), (0x40, 64.0),
])
def test_decode_known_codes(code, value):
    assert I8.i8_decode(np.array([code], np.uint8))[0] == value


def test_every_written_code_round_trips():
    vals = np.arange(-127, 128, dtype=np.float32)
    codes = I8.quantize(vals, 1.0)
    assert np.array_equal(I8.i8_decode(codes), vals.astype(np.float64))
    assert 0x80 not in set(codes.tolist())   # -128 is never written


@pytest.mark.parametrize("y,q", [
    (0.5, 0), (1.5, 2), (2.5, 2), (-0.5, 0), (-1.5, -2), (-2.5, -2), (126.5, 126), (-126.5, -126),
    (0.49999997, 0), (0.50000006, 1),
])
def test_ties_to_even(y, q):
    assert I8.i8_decode(I8.quantize(np.array([y], np.float32), 1.0))[0] == q


def test_saturation_and_nan():
    x = np.array([127.5, 1e6, -1e6, np.inf, -np.inf, np.nan, -127.5], np.float32)
    assert list(I8.i8_decode(I8.quantize(x, 1.0))) == [127, 127, -127, 127, -127, 0, -127]


def test_division_is_float32():
    # x / s is 2.5 + 3e-8 in exact arithmetic but exactly 2.5 once rounded to float32, where the
    # tie goes to the even code 2 (a float64 division would give 3)
    x, s = np.float32(0.07618216425180435), np.float32(0.03047286532819271)
    assert float(x) / float(s) > 2.5 and x / s == np.float32(2.5)
    assert I8.i8_decode(I8.quantize(np.array([x]), s))[0] == 2


def test_agrees_with_torch_rounding():
    g = np.random.default_rng(7)
    x = np.concatenate([g.normal(0, 1, 50000), g.uniform(-6, 6, 50000),
                        np.arange(-300, 300) * 0.5]).astype(np.float32)
    for s in (0.0313, 1.0, 0.5):
        ours = I8.quantize(x, s)
        y = torch.from_numpy(x) / torch.tensor(s, dtype=torch.float32)
        theirs = torch.round(y).clamp(-127, 127).to(torch.int8).view(torch.uint8).numpy()
        assert np.array_equal(ours, theirs)


# ---------------------------------------------------------------- 8-bit integer KV cache attention

def _torch_dequant(codes: np.ndarray, scale: float) -> torch.Tensor:
    """Independent dequantisation: torch's int8 -> float64 conversion, times the scale."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.int8).to(torch.float64)
    return t * float(np.float32(scale))


def test_int8_paged_decode_equals_sdpa_on_dequantised_kv():
    from oracle import attention as OA
    g = np.random.default_rng(19)
    B, Hq, Hkv, D, bs, x = 3, 4, 2, 32, 8, 16
    lens = [5, 17, 24]
    ks, vs = 0.0313, 0.0297
    nblk = [(L + bs - 1) // bs for L in lens]
    NB = sum(nblk) + 3
    perm = g.permutation(NB)
    tables = np.full((B, max(nblk)), -1, np.int32)
    o = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    kc = np.full((NB, Hkv, D // x, bs, x), 0x80, np.uint8)   # -128 in unused slots
    vc = np.full((NB, Hkv, D, bs), 0x80, np.uint8)
    dense_k, dense_v = [], []
    for b, L in enumerate(lens):
        kcodes = I8.quantize(g.normal(0, 1, (Hkv, L, D)).astype(np.float32), ks)
        vcodes = I8.quantize(g.normal(0, 1, (Hkv, L, D)).astype(np.float32), vs)
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
    got = OA.paged_decode(qbits, kc, vc, "bf16", tables, np.array(lens), scale, kv_dtype="i8",
                          k_scale=ks, v_scale=vs)
    for b in range(B):
        qq = q[b].to(torch.float64).view(Hkv, Hq // Hkv, 1, D)
        kk = dense_k[b].view(Hkv, 1, lens[b], D)
        vv = dense_v[b].view(Hkv, 1, lens[b], D)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, scale=float(np.float32(scale))).view(Hq, D).numpy()
        assert np.max(np.abs(got[b] - ref)) <= 1e-12


def test_int8_reshape_and_cache_matches_torch_quantisation():
    from oracle import cache_ops as OC
    g = np.random.default_rng(20)
    N, H, D, bs, NB = 5, 2, 32, 16, 6
    key = torch.from_numpy(g.normal(0, 3, (N, H, D)).astype(np.float32)).to(torch.bfloat16)
    val = torch.from_numpy(g.normal(0, 3, (N, H, D)).astype(np.float32)).to(torch.bfloat16)
    kc = np.zeros((NB, H, D // 16, bs, 16), np.uint8)
    vc = np.zeros((NB, H, D, bs), np.uint8)
    slots = np.array([3, -1, 40, 95, 17])
    ks, vs = 0.02, 0.05
    OC.reshape_and_cache_int8(kc, vc, key.view(torch.int16).numpy().view(np.uint16),
                              val.view(torch.int16).numpy().view(np.uint16), "bf16", slots, ks, vs)

    def tq(x, s):  # torch: x / s in float32, round half to even, clamp, cast
        y = x.to(torch.float32) / torch.tensor(s, dtype=torch.float32)
        return torch.round(y).clamp(-127, 127).to(torch.int8).view(torch.uint8).numpy()
    kq, vq = tq(key, ks), tq(val, vs)
    assert np.abs(kq.view(np.int8)).max() == 127   # some elements saturate
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = slot // bs, slot % bs
        assert np.array_equal(kc[blk, :, :, off, :].reshape(H, D), kq[i])
        assert np.array_equal(vc[blk, :, :, off], vq[i])
    assert not kc[3:5].any() and not vc[3:5].any()   # blocks no slot names stay untouched
