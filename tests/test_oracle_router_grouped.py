"""Pins for the oracle's group-limited noaux-TC router (oracle_router_noaux_tc).

* selection: brute force with Python's sorted() -- group scores as the fp32
  sum of each group's two largest keys, the best groups by (-score, group),
  the experts by (-key, id) among them -- on seeded BF16-valued logits whose
  equal keys and equal group scores are common;
* one group, or every group kept, is the single-group sigmoid router exactly
  (ids and weights); groups of one expert keep the single-group choice when
  k <= topk_group;
* a hand-built token where the best expert sits in a group that loses: it is
  not chosen;
* weights come from the unbiased scores (the bias steers the choice only).
"""
import numpy as np
import pytest

from block_fp8_mixture_route_amd import synth
from oracle import oracle as O


def _keys(lg, bias):
    s = np.array([O.sigmoid_rn(float(x)) for x in lg], np.float32)
    return s + bias if bias is not None else s  # numpy float32 add: one fp32 rounding


def brute_ids(lg, k, n_group, topk_group, bias):
    E = len(lg)
    gs = E // n_group
    key = _keys(lg, bias)
    gscore = []
    for g in range(n_group):
        top = sorted(key[g * gs:(g + 1) * gs].tolist(), reverse=True)
        gscore.append(np.float32(top[0]) + np.float32(top[1]) if gs > 1 else np.float32(top[0]))
    groups = [g for _, g in sorted((-float(s), g) for g, s in enumerate(gscore))][:topk_group]
    allowed = [e for e in range(E) if e // gs in groups]
    return [e for _, e in sorted((-float(key[e]), e) for e in allowed)][:k]


@pytest.mark.parametrize("E,k,n_group,topk_group", [(256, 8, 8, 4), (160, 6, 8, 3), (64, 6, 4, 2), (16, 4, 16, 6),
                                                    (72, 8, 9, 2)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_selection_matches_brute_force(E, k, n_group, topk_group, with_bias):
    lg = synth.router_logits(24, E, "noaux", bf16_valued=True, std=0.5).numpy()
    bias = synth.router_bias(E, "noaux", std=0.05).numpy() if with_bias else None
    ids, _ = O.router_noaux_tc(lg, k, n_group, topk_group, bias)
    for t in range(lg.shape[0]):
        assert ids[t].tolist() == brute_ids(lg[t], k, n_group, topk_group, bias), t


@pytest.mark.parametrize("renorm", [True, False])
def test_one_group_or_all_groups_is_the_single_group_router(renorm):
    lg = synth.router_logits(16, 256, "noaux1", std=2.0).numpy()
    bias = synth.router_bias(256, "noaux1", std=0.3).numpy()
    ref_ids, ref_w = O.router_topk(lg, 8, O.SCORE_SIGMOID, bias, renormalize=renorm, scale=2.5)
    for n_group, topk_group in ((1, 1), (8, 8), (256, 256)):
        ids, w = O.router_noaux_tc(lg, 8, n_group, topk_group, bias, renormalize=renorm, scale=2.5)
        assert np.array_equal(ids, ref_ids) and np.array_equal(w.view(np.uint32), ref_w.view(np.uint32))
    # groups of one expert, topk_group >= k: the same choice
    ids, _ = O.router_noaux_tc(lg, 8, 256, 12, bias, renormalize=renorm)
    assert np.array_equal(ids, ref_ids)


def test_best_expert_in_a_losing_group_is_not_chosen():
    # 4 groups of 2: group 0 holds the largest key (sigmoid(2.2) ~ 0.90) but its
    # pair sums to ~1.0; group 1's pair sums to ~1.2
    lg = np.array([[2.2, -2.2, 0.4, 0.4, -1.0, -1.0, -3.0, -3.0]], np.float32)
    ids, w = O.router_noaux_tc(lg, 2, 4, 1)
    assert ids[0].tolist() == [2, 3]
    assert np.allclose(w[0], [0.5, 0.5])
    ids, _ = O.router_noaux_tc(lg, 2, 4, 2)
    assert ids[0].tolist() == [0, 2]


def test_bias_steers_the_choice_not_the_weights():
    lg = np.array([[0.0, 0.1, 0.2, 0.3]], np.float32)
    bias = np.array([0.5, 0.0, 0.0, 0.0], np.float32)
    ids, w = O.router_noaux_tc(lg, 1, 2, 1, bias, renormalize=False)
    assert ids[0, 0] == 0  # group 0 (1.0 + 0.525) beats group 1 (0.550 + 0.574)
    assert w[0, 0] == np.float32(0.5)  # sigmoid(0), no bias


def test_rejects_bad_grouping():
    lg = np.zeros((1, 12), np.float32)
    for args in ((4, 5, 2), (4, 4, 5), (7, 4, 1), (4, 4, 0)):
        with pytest.raises(ValueError):
            O.router_noaux_tc(lg, *args)
