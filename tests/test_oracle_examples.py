"""Pins of the oracle to the worked examples printed on the MoE page.

Values come from tests/golden/page_examples.json, each with its section of
"How Mixture of Experts Scales Model Parameters".
"""

import json
import os

import numpy as np
import torch

import oracle
from mixture_experts_layer_wave_amd import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def test_top1_example_choice_and_scale():
    ex = GOLD["top1_routing"]
    p = np.array([ex["probs"]])
    z = np.log(p) + 3.7  # any shift: softmax is shift invariant
    pp = oracle.softmax_rows(z)
    np.testing.assert_allclose(pp, p, rtol=1e-12)
    idx = oracle.topk_select(z, 1)
    assert idx[0, 0] + 1 == ex["chosen_expert_1based"]
    w = oracle.topk_weights(pp, idx, renorm=False)
    assert abs(w[0, 0] - ex["output_scale"]) < 1e-12


def test_top2_example_renormalisation():
    ex = GOLD["top2_renormalisation"]
    p = np.array([ex["probs"]])
    z = np.log(p) - 1.25
    pp = oracle.softmax_rows(z)
    idx = oracle.topk_select(z, ex["k"])
    assert (idx[0] + 1).tolist() == ex["chosen_experts_1based"]
    w = oracle.topk_weights(pp, idx, renorm=True)
    assert abs(pp[0, idx[0]].sum() - ex["sum_of_chosen"]) < 1e-12
    assert np.round(w[0], 2).tolist() == ex["weights_printed_2dp"]
    np.testing.assert_allclose(w[0], [0.45 / 0.76, 0.31 / 0.76], rtol=1e-12)


def _rows_with_argmax(argmax0, maxp, E, rng):
    """Probability rows whose largest entry is at argmax0 with value maxp."""
    rows = []
    for a, m in zip(argmax0, maxp):
        rest = rng.dirichlet(np.ones(E - 1)) * (1 - m)
        while rest.max() >= m:
            rest = rng.dirichlet(np.ones(E - 1)) * (1 - m)
        r = np.insert(rest, a, m)
        rows.append(r)
    return np.array(rows)


def test_dispatch_six_token_example():
    ex = GOLD["dispatch_six_tokens"]
    E = ex["E"]
    am = np.array(ex["argmax_expert_1based"]) - 1
    rng = np.random.default_rng(5)
    maxp = [ex["max_prob"]["t1"], ex["max_prob"]["t2"], 0.5, 0.55, 0.6, 0.45]
    p = _rows_with_argmax(am, maxp, E, rng)
    z = np.log(p)
    idx = oracle.topk_select(z, 1)
    assert idx[:, 0].tolist() == am.tolist()
    assert abs(oracle.softmax_rows(z)[0, 1] - 0.62) < 1e-12
    assert abs(oracle.softmax_rows(z)[1, 0] - 0.70) < 1e-12
    dp = oracle.dispatch(idx, E)
    piles = {str(e + 1): (dp["perm"][dp["offsets"][e]:dp["offsets"][e + 1]] + 1).tolist() for e in range(E)}
    assert piles == ex["piles_1based"]
    assert dp["counts"].tolist() == [2, 3, 0, 1]
    assert dp["offsets"].tolist() == [0, 2, 5, 5, 6]


def test_top1_example_through_the_whole_layer():
    """A token of the tiny float32 layer whose router probabilities are the
    page's (0.45, 0.19, 0.05, 0.31): the layer output must be 0.45 times
    expert 1's FFN, which is computed here with torch's own SiLU."""
    layer = W.make_layer(W.TINY)
    wg = oracle.decode_f32(layer["wg"])  # [E][d] = [4][3]
    p = np.array(GOLD["top1_routing"]["probs"])
    # Solve wg x + c = ln p for (x, c): d + 1 = E unknowns.
    A = np.concatenate([wg, np.ones((4, 1))], axis=1)
    sol = np.linalg.solve(A, np.log(p))
    x = sol[:3].astype(np.float32)
    one = dict(layer, x=x[None, :], n=1)
    out = oracle.forward(one, k=1)
    assert out["idx"][0, 0] == 0
    assert abs(out["w"][0, 0] - 0.45) < 1e-6
    xt = torch.tensor(x, dtype=torch.float64)[None]
    w1 = torch.tensor(layer["w1"][0], dtype=torch.float64)
    w3 = torch.tensor(layer["w3"][0], dtype=torch.float64)
    w2 = torch.tensor(layer["w2"][0], dtype=torch.float64)
    ffn = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(xt, w1))
                                     * torch.nn.functional.linear(xt, w3), w2)
    np.testing.assert_allclose(out["y"], out["w"][0, 0] * ffn.numpy(), rtol=1e-12, atol=1e-15)


def test_aux_loss_tables():
    ex = GOLD["aux_loss"]
    # Four tokens that always pick expert 1 and whose mean p_1 is 0.5825.
    p = np.array([[0.60, 0.20, 0.10, 0.10],
                  [0.55, 0.15, 0.15, 0.15],
                  [0.63, 0.07, 0.20, 0.10],
                  [0.55, 0.25, 0.10, 0.10]])
    idx = oracle.topk_select(np.log(p), 1)
    r = oracle.aux_loss(p, idx)
    assert abs(r["P"][0] - ex["unbalanced"]["P1"]) < 1e-12
    assert r["f"].tolist() == ex["unbalanced"]["f"]
    assert round(r["loss"], 2) == ex["unbalanced"]["loss_over_alpha_2dp"]
    assert abs(oracle.aux_loss(p, idx, alpha=ex["alpha"])["loss"] - ex["terms_added"][0]) < 1e-12
    # Balanced: every expert is the argmax once.
    pb = np.full((4, 4), 0.2) + 0.2 * np.eye(4)
    rb = oracle.aux_loss(pb, oracle.topk_select(np.log(pb), 1))
    assert rb["f"].tolist() == ex["balanced"]["f"]
    assert abs(rb["loss"] - ex["balanced"]["loss_over_alpha"]) < 1e-12
    rnd = np.random.default_rng(0).dirichlet(np.ones(4), size=4)
    rnd = rnd[:, [0, 1, 2, 3]]
    # any distribution with one argmax per expert gives exactly 1 (P sums to 1)
    perm_rows = np.array([np.roll(np.sort(r)[::-1], i) for i, r in enumerate(rnd)])
    rr = oracle.aux_loss(perm_rows, oracle.topk_select(np.log(perm_rows), 1))
    assert abs(rr["loss"] - 1.0) < 1e-12
    assert abs(oracle.aux_loss(pb, oracle.topk_select(np.log(pb), 1), alpha=ex["alpha"])["loss"]
               - ex["terms_added"][1]) < 1e-15


def test_active_experts_on_the_page_dispatch_example():
    """[MoE] forward-pass example: argmax experts (2, 1, 4, 2, 1, 2) use
    experts 1, 2 and 4; expert 3 gets no tokens."""
    am = np.array(GOLD["dispatch_six_tokens"]["argmax_expert_1based"]) - 1
    assert oracle.active_experts(am.reshape(-1, 1), 4).tolist() == [0, 1, 3]


def test_active_experts_is_the_nonempty_piles():
    """Brute force: the deduplicated choices are the experts whose pile (built
    by the oracle's pile scan) is non-empty, for random and degenerate inputs."""
    rng = np.random.default_rng(5)
    for E, shape in ((8, (40, 2)), (1, (9, 1)), (130, (3, 4)), (6, (50, 6))):
        idx = rng.integers(0, E, size=shape)
        want = np.nonzero(oracle.dispatch(idx, E)["counts"] > 0)[0]
        assert np.array_equal(oracle.active_experts(idx, E), want)


def test_resolve_slots_is_a_gather():
    """Slots given by a permutation bring each expert's stored rows back;
    the identity table changes nothing."""
    rng = np.random.default_rng(6)
    E = 5
    w = rng.standard_normal((E, 3, 4))
    same = oracle.resolve_slots({"w1": w, "w3": None, "w2": None}, np.arange(E))
    assert np.array_equal(same["w1"], w)
    pos = rng.permutation(E + 2)[:E]
    phys2 = np.zeros((E + 2, 3, 4))
    phys2[pos] = w
    assert np.array_equal(oracle.resolve_slots({"w1": phys2}, pos)["w1"], w)
