"""Pins for the oracle's single-group top-k router.

* selection: brute force with Python's sorted() over (-key, expert id) on every
  token of seeded inputs, with BF16-valued logits so that equal keys occur;
  all-equal logits choose experts 0..k-1; -0 and +0 are equal keys;
* softmax weights: scipy's softmax over the chosen logits (renormalised) or
  over the whole row (not renormalised) to within one fp32 ulp, the closed
  forms 1/k and 1/E for equal logits, and logits near +-800 where exp without
  the max subtracted overflows or underflows;
* sigmoid weights: scipy's expit of the chosen logits, renormalised or not;
  the selection bias moves an expert into the top-k without changing any
  weight's formula;
* scale multiplies every weight.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

from block_fp8_mixture_route_amd import synth
from oracle import oracle as O


def ulps(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float64)
    sp = np.spacing(np.abs(a)).astype(np.float64)
    return np.abs(a.astype(np.float64) - b) / sp


def sig32(x):
    # fp32 sigmoid from scipy's fp64 expit, rounded once
    return np.float32(expit(np.float64(x)))


def brute_ids(lg, k, score_fn, bias):
    E = len(lg)
    if score_fn == O.SCORE_SOFTMAX:
        keys = [float(lg[e]) for e in range(E)]
    else:
        keys = [float(sig32(lg[e]) + (np.float32(bias[e]) if bias is not None else np.float32(0)))
                for e in range(E)]
    return [e for _, e in sorted((-keys[e], e) for e in range(E))[:k]]


@pytest.mark.parametrize("score_fn", [O.SCORE_SOFTMAX, O.SCORE_SIGMOID])
@pytest.mark.parametrize("M,E,k", [(16, 256, 8), (8, 72, 6), (4, 8, 8), (5, 130, 1)])
def test_selection_brute_force(M, E, k, score_fn):
    lg = synth.router_logits(M, E, "pin", score_fn, bf16_valued=True, std=0.5).numpy()
    bias = synth.router_bias(E, "pin").numpy() if score_fn == O.SCORE_SIGMOID else None
    ids, _ = O.router_topk(lg, k, score_fn, bias)
    assert E < 64 or any(len(set(r.tolist())) < E for r in lg)  # ties present
    for t in range(M):
        assert ids[t].tolist() == brute_ids(lg[t], k, score_fn, bias)


def test_ties_and_signed_zero():
    lg = np.zeros((1, 16), np.float32)
    ids, w = O.router_topk(lg, 4)
    assert ids[0].tolist() == [0, 1, 2, 3] and np.all(w == np.float32(0.25))
    _, w = O.router_topk(lg, 4, renormalize=False)
    assert np.all(w == np.float32(1 / 16))
    lg = np.full((1, 8), -1.0, np.float32)
    lg[0, 5] = -0.0
    lg[0, 2] = 0.0
    lg[0, 6] = 3.0
    ids, _ = O.router_topk(lg, 3)
    assert ids[0].tolist() == [6, 2, 5]


@pytest.mark.parametrize("std,shift", [(1.0, 0.0), (4.0, 0.0), (1.0, 800.0), (1.0, -800.0)])
def test_softmax_weights_against_scipy(std, shift):
    lg = (synth.router_logits(32, 256, "sm", std=std).numpy() + np.float32(shift)).astype(np.float32)
    for renorm in (True, False):
        ids, w = O.router_topk(lg, 8, renormalize=renorm)
        for t in range(32):
            row = lg[t].astype(np.float64)
            ref = softmax(row[ids[t]]) if renorm else softmax(row)[ids[t]]
            assert ulps(w[t], ref).max() <= 1.0
        if renorm:
            assert np.abs(w.astype(np.float64).sum(1) - 1).max() < 1e-6
        assert np.all(np.diff(w, axis=1) <= 0)  # largest first


def test_softmax_all_experts_sum_to_one():
    lg = synth.router_logits(4, 64, "all").numpy()
    _, w = O.router_topk(lg, 64, renormalize=False)
    assert np.abs(w.astype(np.float64).sum(1) - 1).max() < 1e-6


@pytest.mark.parametrize("renorm", [True, False])
def test_sigmoid_weights_against_scipy(renorm):
    lg = synth.router_logits(16, 256, "sg", std=2.0).numpy()
    bias = synth.router_bias(256, "sg", std=0.3).numpy()
    ids, w = O.router_topk(lg, 8, O.SCORE_SIGMOID, bias, renormalize=renorm, scale=2.5)
    for t in range(16):
        s = expit(lg[t].astype(np.float64)[ids[t]])
        ref = (s / s.sum() if renorm else s) * 2.5
        assert ulps(w[t], ref).max() <= 1.0


def test_bias_moves_selection_not_weights():
    lg = np.linspace(-2, 2, 32, dtype=np.float32)[None, :].copy()
    bias = np.zeros(32, np.float32)
    ids0, _ = O.router_topk(lg, 4, O.SCORE_SIGMOID, bias, renormalize=False)
    assert ids0[0].tolist() == [31, 30, 29, 28]
    bias[3] = 1.0  # sigmoid(lg[3]) + 1 beats every unbiased score
    ids1, w1 = O.router_topk(lg, 4, O.SCORE_SIGMOID, bias, renormalize=False)
    assert ids1[0].tolist() == [3, 31, 30, 29]
    assert w1[0, 0] == sig32(lg[0, 3])


def test_sigmoid_rn_and_scale():
    for x in (-30.0, -1.5, 0.0, 0.25, 7.0, 40.0):
        assert O.sigmoid_rn(x) == sig32(np.float32(x))
    lg = synth.router_logits(8, 64, "scale").numpy()
    _, w1 = O.router_topk(lg, 6)
    _, w2 = O.router_topk(lg, 6, scale=4.0)
    assert np.array_equal(w1 * np.float32(4), w2)


def test_rejects_k_above_e():
    with pytest.raises(ValueError):
        O.router_topk(np.zeros((1, 4), np.float32), 5)
