"""Pins for the oracle's MXFP4-weight variant (OCP Microscaling Formats
specification v1.0: E2M1 elements, E8M0 block scales over 32 elements):

* every E2M1 code against the specification's value list, every E8M0 byte
  against 2^(e - 127) (255: NaN);
* the packing: a row whose only non-zero element is element i (the low
  nibble of byte i / 2 when i is even) selects activation i alone, for every i
  of a 256-wide row, with its block's scale;
* the grouped GEMM against exact rationals (Fraction) rounded once to BF16;
* the whole layer equals the pinned block-FP8 layer bit for bit where the two
  readings coincide: E2M1 values re-encoded as E4M3 codes, and every scale of
  a 128 x 128 block the same power of two.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests import exact

# the E2M1 values of codes 0..7 as the specification lists them (codes 8..15:
# the same values negated)
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_every_code():
    for c in range(16):
        v = O.e2m1_decode(c)
        want = E2M1_SPEC[c & 7] * (-1.0 if c & 8 else 1.0)
        assert v == want and np.signbit(v) == bool(c & 8), c


def test_e8m0_every_byte():
    for e in range(255):
        assert O.e8m0_decode(e) == 2.0 ** (e - 127), e
    assert np.isnan(O.e8m0_decode(255))


def _pack(codes: np.ndarray) -> np.ndarray:
    """[..., K] E2M1 codes -> [..., K/2] bytes, even element in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _e4m3(v: float) -> int:
    c = int(torch.tensor([v]).to(torch.float8_e4m3fn).view(torch.uint8)[0])
    assert O.e4m3_decode(c) == v
    return c


def test_packing_selects_one_element():
    K, N = 256, 256
    a = np.array([_e4m3(float(1 + (i % 7))) for i in range(K)], np.uint8)[None, :]   # distinct values 1..7
    a_s = np.ones((1, K // 128), np.float32)
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), np.arange(K)] = 2                                            # element i of row i: 1.0
    ws = np.full((N, K // 32), 127, np.uint8)
    ws[np.arange(N), np.arange(K) // 32] = 127 + 3                                  # its block: 2^3
    acc, _ = O.grouped_gemm_mxfp4(a, a_s, 1, _pack(codes)[None], ws[None], np.zeros((1, 1), np.int32), 0, 1,
                                  exact=True)
    want = np.array([(1 + (i % 7)) * 8.0 for i in range(K)])
    assert np.array_equal(acc[0], want)


def _frac_gemm_row(a, a_s, codes, ws):
    K = codes.size
    tot = Fraction(0)
    for b in range(K // 32):
        p = sum(exact.e4m3_spec_value(int(a[i])) * Fraction(E2M1_SPEC[codes[i] & 7]) * (-1 if codes[i] & 8 else 1)
                for i in range(b * 32, b * 32 + 32))
        tot += Fraction(float(a_s[b // 4])) * Fraction(2) ** (int(ws[b]) - 127) * p
    return tot


def test_grouped_gemm_against_exact_rationals():
    rng = np.random.default_rng(7)
    M, k, E, N, K = 3, 2, 4, 8, 256
    hidden = synth.hidden_states(M, K, "mx_exact", 0)
    aq, as_ = O.quant_fp8(hidden)
    codes = rng.integers(0, 16, (E, N, K)).astype(np.uint8)
    ws = rng.integers(120, 132, (E, N, K // 32)).astype(np.uint8)
    ids = np.array([[0, 3], [2, -1], [1, 1]], np.int32)
    C = O.grouped_gemm_mxfp4(aq, as_, k, _pack(codes), ws, ids, 0, E)
    acc, mag = O.grouped_gemm_mxfp4(aq, as_, k, _pack(codes), ws, ids, 0, E, exact=True)
    for r in range(M * k):
        e = ids.reshape(-1)[r]
        if e < 0:
            assert np.isnan(acc[r]).all() and (C[r] == 0).all()
            continue
        for n in range(N):
            x = _frac_gemm_row(aq[r // k], as_[r // k], codes[e, n], ws[e, n])
            assert C[r, n] == exact.bf16_bits_of(exact.round_bf16(x)), (r, n)
            assert abs(Fraction(float(acc[r, n])) - x) <= Fraction(float(mag[r, n])) * Fraction(1, 2 ** 50)


@pytest.mark.parametrize("fmt,clamp", [(O.SCALE_FP32, float("inf")), (O.SCALE_UE8M0, 7.0)])
def test_layer_equals_block_layer_where_they_coincide(fmt, clamp):
    M, E, k, H, I = 3, 5, 3, 512, 256
    rng = np.random.default_rng(11)
    hidden = synth.hidden_states(M, H, "mx_layer", 0)
    ids, w = synth.uniform_routing(M, E, k, "mx_layer")
    c13 = rng.integers(0, 16, (E, 2 * I, H)).astype(np.uint8)
    c2 = rng.integers(0, 16, (E, H, I)).astype(np.uint8)
    b13 = rng.integers(120, 126, (E, 2 * I // 128, H // 128))          # one exponent per 128 x 128 block
    b2 = rng.integers(120, 126, (E, H // 128, I // 128))
    e13 = np.repeat(np.repeat(b13, 128, axis=1), 4, axis=2).astype(np.uint8)   # [E, 2I, H/32]
    e2 = np.repeat(np.repeat(b2, 128, axis=1), 4, axis=2).astype(np.uint8)
    lut = np.array([_e4m3(E2M1_SPEC[c & 7] * (-1.0 if c & 8 else 1.0)) if c & 7 else (0x80 if c & 8 else 0)
                    for c in range(16)], np.uint8)
    f13 = np.exp2(b13.astype(np.float64) - 127).astype(np.float32)
    f2 = np.exp2(b2.astype(np.float64) - 127).astype(np.float32)
    ref = O.fused_moe(hidden, ids, w, lut[c13], f13, lut[c2], f2, scale_fmt=fmt, clamp=clamp)
    got = O.fused_moe_mxfp4(hidden, ids, w, _pack(c13), e13, _pack(c2), e2, scale_fmt=fmt, clamp=clamp)
    assert np.array_equal(got, ref)
    assert np.abs(exact_f32(ref)).max() > 0


def exact_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)
