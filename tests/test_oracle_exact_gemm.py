"""Pins of the oracle's unrounded GEMM (oracle_grouped_gemm_f64) and of the
parity helpers' BF16 rounding, against exact integer arithmetic.

On the exact-arithmetic workload (synth.exact_layer_inputs) every code is a
small integer or +-448 and every scale a power of two, so each GEMM output is
an integer multiple of a power of two that numpy's int64 products give
exactly.  The oracle must reproduce those values exactly (its fp64 sums are
exact on them), its BF16 outputs must be their one rounding, and its
magnitudes must be the sums of |terms|.  A transposed operand, a wrong block
scale index or a dropped group changes these integers."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from block_fp8_mixture_route_amd import synth
from oracle import oracle as O
from tests import exact
from tests.parity import bf16_bits_rne, f32_of_bits, n_between

E4M3 = {c: exact.e4m3_spec_value(c) for c in range(256)}


def _int_codes(codes: np.ndarray) -> np.ndarray:
    """Integer values of E4M3 codes that hold integers (the workload's)."""
    lut = np.zeros(256, np.int64)
    for c, v in E4M3.items():
        if v is not None and v.denominator == 1:
            lut[c] = int(v)
    vals = lut[codes]
    # every code used must be an integer one
    nz = codes & 0x7F
    assert (vals != 0).sum() == (nz != 0).sum()
    return vals


def test_bf16_rounding_helper_matches_exact_rounding():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-40, 38, 4000),
                        # exact BF16 midpoints and their neighbours
                        f32_of_bits(rng.integers(0, 0x7F00, 500).astype(np.uint16)).astype(np.float64)
                        * (1 + 2.0 ** -8),
                        np.ldexp(1.0, -133) * np.arange(1, 50),  # subnormal quanta
                        [0.0, -0.0, 1.0, -1.0]])
    got = bf16_bits_rne(x)
    for v, g in zip(x, got):
        ref = exact.round_bf16(Fraction(float(v)))
        assert exact.bf16_value(int(g)) == float(ref), v
    assert (got[np.signbit(x)] & 0x8000).all()


def test_n_between_counts_values_across_zero():
    lo = bf16_bits_rne(np.array([-2.0 ** -130, 1.0, -1.0]))
    hi = bf16_bits_rne(np.array([2.0 ** -130, 1.0, 1.0]))
    # 2^-130 is 8 subnormal quanta (2^-133); 1.0 is pattern 0x3F80
    assert list(n_between(lo, hi)) == [2 * 8 + 1, 1, 2 * 0x3F80 + 1]


@pytest.mark.parametrize("M,E,k,H,I", [(3, 6, 4, 1024, 256), (2, 5, 3, 2560, 128), (1, 9, 8, 7168, 256)])
def test_exact_workload_gemms(M, E, k, H, I):
    hidden, ids, w, W = synth.exact_layer_inputs(M, E, k, H, I, "pin")
    ids_np = ids.numpy()
    hid = hidden.view(torch.int16).numpy().view(np.uint16)
    out, inter = O.fused_moe(hidden, ids, w, W.w13, W.w13_s, W.w2, W.w2_s, scale_fmt=O.SCALE_UE8M0,
                             want_intermediates=True)
    # the hidden quantisation is exact: codes are the integers and +-448,
    # scales 2^m
    aq, as_ = O.quant_fp8(hid, O.SCALE_UE8M0)
    x = f32_of_bits(hid).astype(np.float64)
    xi = _int_codes(aq).reshape(M, H)
    assert np.array_equal(xi * as_.repeat(128, axis=1), x)

    acc, mag = O.grouped_gemm_f64(aq, as_, k, W.w13, W.w13_s, ids, 0, E)
    w13 = _int_codes(W.w13.numpy()).reshape(E, 2 * I, H)
    s13 = W.w13_s.numpy().astype(np.float64)
    for r in range(M * k):
        e = ids_np.reshape(-1)[r]
        if e < 0:
            assert np.isnan(acc[r]).all()
            continue
        t = r // k
        # integer group sums, then exact power-of-two scales
        grp = (w13[e].reshape(2 * I, H // 128, 128) * xi[t].reshape(1, H // 128, 128)).sum(-1)
        gabs = np.abs(w13[e].reshape(2 * I, H // 128, 128) * xi[t].reshape(1, H // 128, 128)).sum(-1)
        sc = np.repeat(s13[e], 128, axis=0) * as_[t].astype(np.float64)[None, :]
        ref = (grp * sc).sum(-1)
        assert np.array_equal(acc[r], ref)
        assert np.array_equal(mag[r], (gabs * sc).sum(-1))
        assert np.array_equal(inter["h13"][r], bf16_bits_rne(ref))

    # down projection on the oracle's own SwiGLU codes: two non-zero integer
    # weights per row, so the sum is exact in float64 too
    q, s = inter["q"], inter["s"]
    accy, magy = O.grouped_gemm_f64(q, s, 1, W.w2, W.w2_s, ids, 0, E)
    w2 = _int_codes(W.w2.numpy()).reshape(E, H, I)
    s2 = W.w2_s.numpy().astype(np.float64)
    qv = np.array([float(E4M3[c]) if E4M3[c] is not None else np.nan for c in range(256)])[q]
    for r in range(M * k):
        e = ids_np.reshape(-1)[r]
        if e < 0:
            continue
        sc = np.repeat(np.repeat(s2[e], 128, axis=0), 128, axis=1) * np.repeat(s[r].astype(np.float64), 128)[None]
        ref = (w2[e] * qv[r][None, :] * sc).sum(-1)
        assert np.array_equal(accy[r], ref)
        assert np.array_equal(inter["y"][r], bf16_bits_rne(ref))
