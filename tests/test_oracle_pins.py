"""Pins that hold the oracle to facts other than its own code.

Each test fixes the oracle against a closed form, an invariant, a special case
or brute force, chosen so that a dropped term, a wrong sign, index, scale or
operand, or pooling probabilities instead of logits, fails at least one.
Passages: the long-form digest "LycheeDecode: Accelerating Long-Context LLM
Inference via Hybrid-Head Sparse Decoding", section 3.4 (Eq. 1-3, S
propagation, layer-0 rule, Algorithm 1, GQA pooling line).
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest

import oracle
import synth
from goldens import cases as golden_cases

TIGHT = 1e-12


def _f32_case(rng, B, Hq, Hkv, d, max_ctx, n=None, dyadic=False):
    def draw(shape):
        x = rng.standard_normal(shape)
        if dyadic:                       # multiples of 2^-10: sums stay exact
            x = np.round(x * 1024) / 1024
        return x.astype(np.float32)
    q = draw((B, Hq, d))
    kc = draw((B, Hkv, max_ctx, d))
    vc = draw((B, Hkv, max_ctx, d))
    n_ctx = np.full(B, max_ctx if n is None else n, dtype=np.int32)
    return q, kc, vc, n_ctx


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_golden_worked_examples(case):
    """Hand-derived closed forms (tests/golden/*.json), S chained over layers."""
    S = None
    n_ctx = np.array(case["n_ctx"], dtype=np.int32)
    for li, lay in enumerate(case["layers"]):
        out, S, _ = oracle.layer(lay["q"], lay["k"], lay["v"], lay["role"], S, n_ctx, case["k"])
        np.testing.assert_allclose(out, lay["expect_out"], rtol=0, atol=TIGHT,
                                   err_msg=f"{case['file']} layer {li}")
        np.testing.assert_array_equal(S, lay["expect_S"], err_msg=f"{case['file']} layer {li}")


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("G", [1, 4])
def test_identical_keys_give_mean_of_values_and_lowest_indices(G):
    """All keys equal -> uniform weights -> out = mean of V rows; every score
    ties, so S = {0..k-1} (lower index wins)."""
    rng = np.random.default_rng(7)
    Hkv, d, n, k = 2, 64, 300, 37
    q, kc, vc, n_ctx = _f32_case(rng, 1, Hkv * G, Hkv, d, n)
    kc[:] = kc[:, :, :1, :]
    out, S, _ = oracle.layer(q, kc, vc, np.ones(Hkv, np.uint8), None, n_ctx, k)
    for h in range(Hkv * G):
        expect = vc[0, h // G].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(out[0, h], expect, rtol=0, atol=TIGHT)
    np.testing.assert_array_equal(S, np.broadcast_to(np.arange(k, dtype=np.int32), S.shape))


def test_planted_dominant_key_selected_and_returned():
    """A key aligned with the group's queries with logit gap D >= 40 over all
    others: it is selected, and |out - V[j*]| <= 2 (n-1) e^-D max|V|."""
    rng = np.random.default_rng(11)
    G, d, n, k = 4, 64, 1000, 16
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = (u[None, :] + 0.05 * rng.standard_normal((G, d))).astype(np.float32)[None]
    kc = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    vc = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    jstar = 617
    kc[0, 0, jstar] = (500.0 * u).astype(np.float32)
    out, S, _ = oracle.layer(q, kc, vc, np.ones(1, np.uint8), None, np.array([n], np.int32), k)
    c = 1 / math.sqrt(d)
    z = c * np.einsum("hd,nd->hn", q[0].astype(np.float64), kc[0, 0].astype(np.float64))
    gap = min(z[h, jstar] - np.max(np.delete(z[h], jstar)) for h in range(G))
    assert gap >= 40.0, "precondition: planted gap"
    assert jstar in S[0, 0]
    bound = 2 * (n - 1) * math.exp(-gap) * np.abs(vc).max()
    for h in range(G):
        assert np.abs(out[0, h] - vc[0, 0, jstar]).max() <= max(bound, 1e-15)


def test_constant_value_rows_reproduce_the_constant():
    """Weights sum to one: V rows all equal to w give out = w, for both kinds."""
    rng = np.random.default_rng(3)
    q, kc, vc, n_ctx = _f32_case(rng, 1, 8, 2, 64, 500)
    w = rng.standard_normal(64).astype(np.float32)
    vc[:] = w
    out, S, _ = oracle.layer(q, kc, vc, np.ones(2, np.uint8), None, n_ctx, 40)
    np.testing.assert_allclose(out[0], np.broadcast_to(w.astype(np.float64), (8, 64)), rtol=0, atol=1e-12)
    out2, _, _ = oracle.layer(q, kc, vc, np.array([0, 0], np.uint8), S, n_ctx, 40)
    np.testing.assert_allclose(out2[0], np.broadcast_to(w.astype(np.float64), (8, 64)), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- brute force

def _brute_force_topk(s, k):
    """Max score-sum subset; among those the lexicographically smallest sorted
    index tuple.  Equals 'larger score first, then lower index'."""
    best_sum, best = None, None
    for comb in itertools.combinations(range(len(s)), k):
        tot = sum(s[j] for j in comb)
        if best_sum is None or tot > best_sum or (tot == best_sum and comb < best):
            best_sum, best = tot, comb
    return list(best)


@pytest.mark.parametrize("G", [1, 2])
def test_topk_matches_brute_force_with_ties(G):
    """Integer-valued logits full of ties (d = 4, q = 2 e_i so logit = K[j, i]);
    with G = 2 the pooled score is the mean of the two heads' logits."""
    rng = np.random.default_rng(100 + G)
    for trial in range(150):
        n = int(rng.integers(1, 13))
        k = int(rng.integers(1, 6))
        q = np.zeros((1, G, 4), np.float32)
        for h in range(G):
            q[0, h, h] = 2.0
        kc = np.zeros((1, 1, n, 4), np.float32)
        kc[0, 0, :, :G] = rng.integers(-2, 3, size=(n, G))
        vc = rng.standard_normal((1, 1, n, 4)).astype(np.float32)
        _, S, _ = oracle.layer(q, kc, vc, np.ones(1, np.uint8), None, np.array([n], np.int32), k)
        pooled = [sum(float(kc[0, 0, j, h]) for h in range(G)) / G for j in range(n)]
        ke = min(k, n)
        expect = _brute_force_topk(pooled, ke) + [-1] * (k - ke)
        assert S[0, 0].tolist() == expect, (trial, pooled, k)


# ---------------------------------------------------------------- special cases

def test_sparse_over_all_positions_equals_dense():
    """S = all n positions (k = n): Eq. 3 reduces to Eq. 1."""
    rng = np.random.default_rng(5)
    n = 257
    q, kc, vc, n_ctx = _f32_case(rng, 2, 8, 2, 64, n)
    dense, _, _ = oracle.layer(q, kc, vc, np.ones(2, np.uint8), None, n_ctx, n)
    S = np.broadcast_to(np.arange(n, dtype=np.int32), (2, 2, n)).copy()
    sparse, S_out, _ = oracle.layer(q, kc, vc, np.zeros(2, np.uint8), S, n_ctx, n)
    np.testing.assert_allclose(sparse, dense, rtol=0, atol=TIGHT)
    np.testing.assert_array_equal(S_out, S)


def test_masked_softmax_identity():
    """Sparse attention over S equals dense attention after every key outside S
    is moved to logit <= -1000 (exp underflows to exactly 0 in fp64)."""
    rng = np.random.default_rng(9)
    G, d, n, k = 4, 64, 400, 50
    base = rng.standard_normal(d)
    q = (base[None] + 0.1 * rng.standard_normal((G, d))).astype(np.float32)[None]
    kc = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    vc = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    S = np.sort(rng.choice(n, size=k, replace=False)).astype(np.int32)[None, None]
    out_sparse, _, _ = oracle.layer(q, kc, vc, np.zeros(1, np.uint8), S, np.array([n], np.int32), k)
    qbar = q[0].astype(np.float64).mean(axis=0)
    far = (-1e5 * qbar / np.dot(qbar, qbar)).astype(np.float32)
    k2 = kc.copy()
    outside = np.setdiff1d(np.arange(n), S[0, 0])
    k2[0, 0, outside] = far
    z_far = (q[0].astype(np.float64) @ far.astype(np.float64)) / math.sqrt(d)
    assert np.all(z_far <= -1000), "precondition: pushed keys are far below"
    out_dense, _, _ = oracle.layer(q, k2, vc, np.ones(1, np.uint8), None, np.array([n], np.int32), k)
    np.testing.assert_allclose(out_sparse, out_dense, rtol=0, atol=TIGHT)


def test_gqa_head_map_matches_expanded_cache():
    """Query head h reads KV head floor(h/G): running GQA equals running MHA on
    a cache with each KV head repeated G times (outputs)."""
    rng = np.random.default_rng(21)
    G, Hkv, d, n = 4, 2, 64, 333
    q, kc, vc, n_ctx = _f32_case(rng, 1, G * Hkv, Hkv, d, n)
    out_gqa, _, _ = oracle.layer(q, kc, vc, np.ones(Hkv, np.uint8), None, n_ctx, 8)
    kx = np.repeat(kc, G, axis=1)
    vx = np.repeat(vc, G, axis=1)
    out_mha, _, _ = oracle.layer(q, kx, vx, np.ones(G * Hkv, np.uint8), None, n_ctx, 8)
    np.testing.assert_allclose(out_gqa, out_mha, rtol=0, atol=TIGHT)


def test_pooled_score_is_mean_of_head_logits_and_single_head_is_own():
    """With G identical query heads the pooled score equals each head's logit,
    so S is the top-k of that one head (checked against G = 1)."""
    rng = np.random.default_rng(22)
    d, n, k = 64, 500, 33
    q1, kc, vc, n_ctx = _f32_case(rng, 1, 1, 1, d, n)
    q4 = np.repeat(q1, 4, axis=1)
    _, S1, s1 = oracle.layer(q1, kc, vc, np.ones(1, np.uint8), None, n_ctx, k, want_scores=True)
    _, S4, s4 = oracle.layer(q4, kc, vc, np.ones(1, np.uint8), None, n_ctx, k, want_scores=True)
    np.testing.assert_array_equal(S1, S4)
    np.testing.assert_allclose(s4, s1, rtol=1e-15, atol=0)


# ---------------------------------------------------------------- invariants

def test_outputs_lie_in_the_value_hull():
    rng = np.random.default_rng(13)
    q, kc, vc, n_ctx = _f32_case(rng, 1, 8, 2, 64, 700)
    out, S, _ = oracle.layer(q, kc, vc, np.ones(2, np.uint8), None, n_ctx, 64)
    for h in range(8):
        v = vc[0, h // 4].astype(np.float64)
        assert np.all(out[0, h] >= v.min(axis=0) - 1e-12) and np.all(out[0, h] <= v.max(axis=0) + 1e-12)
    out2, _, _ = oracle.layer(q, kc, vc, np.zeros(2, np.uint8), S, n_ctx, 64)
    for h in range(8):
        v = vc[0, h // 4][S[0, h // 4]].astype(np.float64)
        assert np.all(out2[0, h] >= v.min(axis=0) - 1e-12) and np.all(out2[0, h] <= v.max(axis=0) + 1e-12)


def test_logit_shift_invariance():
    """Adding one vector w to every key shifts each head's logits by a constant
    (q_h.w/sqrt(d)): outputs unchanged, pooled ranking unchanged.  Dyadic
    inputs keep K + w exact in fp32."""
    rng = np.random.default_rng(17)
    q, kc, vc, n_ctx = _f32_case(rng, 1, 8, 2, 64, 600, dyadic=True)
    w = np.round(rng.standard_normal(64) * 4).astype(np.float32)
    out, S, _ = oracle.layer(q, kc, vc, np.ones(2, np.uint8), None, n_ctx, 50)
    out2, S2, _ = oracle.layer(q, kc + w, vc, np.ones(2, np.uint8), None, n_ctx, 50)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-11)
    np.testing.assert_array_equal(S2, S)


def test_row_permutation_equivariance():
    """Permuting cache rows by pi leaves outputs unchanged and maps S by pi."""
    rng = np.random.default_rng(19)
    n, k = 512, 40
    q, kc, vc, n_ctx = _f32_case(rng, 1, 8, 2, 64, n)
    pi = rng.permutation(n)
    out, S, _ = oracle.layer(q, kc, vc, np.ones(2, np.uint8), None, n_ctx, k)
    out2, S2, _ = oracle.layer(q, kc[:, :, pi], vc[:, :, pi], np.ones(2, np.uint8), None, n_ctx, k)
    np.testing.assert_allclose(out2, out, rtol=0, atol=TIGHT)
    for g in range(2):
        assert sorted(pi[S2[0, g]].tolist()) == S[0, g].tolist()


def test_batch_rows_are_independent():
    """A batch of two sequences with different contexts equals two runs of one."""
    rng = np.random.default_rng(23)
    max_ctx, k = 300, 20
    q, kc, vc, _ = _f32_case(rng, 2, 8, 2, 64, max_ctx)
    n_ctx = np.array([300, 171], np.int32)
    kc[1, :, 171:] = np.nan
    vc[1, :, 171:] = np.nan
    role = np.array([1, 0], np.uint8)
    S_in = np.stack([np.stack([np.arange(k), np.arange(k) * 3]) for _ in range(2)]).astype(np.int32)
    out, S, _ = oracle.layer(q, kc, vc, role, S_in, n_ctx, k)
    for b in range(2):
        o1, s1, _ = oracle.layer(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], role, S_in[b:b + 1], n_ctx[b:b + 1], k)
        np.testing.assert_array_equal(out[b:b + 1], o1)
        np.testing.assert_array_equal(S[b:b + 1], s1)
    assert np.all(np.isfinite(out))


# ---------------------------------------------------------------- propagation

def test_sparse_head_forwards_S_bitwise_and_retrieval_ignores_S_in():
    rng = np.random.default_rng(29)
    q, kc, vc, n_ctx = _f32_case(rng, 1, 8, 2, 64, 256)
    S_in = np.stack([np.sort(rng.choice(256, 16, replace=False)) for _ in range(2)])[None].astype(np.int32)
    _, S_out, _ = oracle.layer(q, kc, vc, np.array([0, 1], np.uint8), S_in, n_ctx, 16)
    np.testing.assert_array_equal(S_out[0, 0], S_in[0, 0])
    garbage = S_in.copy()
    garbage[0, 1] = np.arange(16)[::-1]
    _, S_out2, _ = oracle.layer(q, kc, vc, np.array([0, 1], np.uint8), garbage, n_ctx, 16)
    np.testing.assert_array_equal(S_out2[0, 1], S_out[0, 1])


def test_all_sparse_chain_returns_layer0_S():
    """Layers 1..L-1 all sparse: S after the last layer is the layer-0 S."""
    w = synth.WORKLOADS["tiny_gqa"].replace(layers=4, n_retrieval=0)
    layers = []
    roles = synth.roles(w)
    assert roles[1:].sum() == 0
    for l in range(w.layers):
        x = synth.layer_inputs(w, l)
        layers.append((x["q"], x["k"], x["v"], roles[l]))
    outs, Ss = oracle.step(layers, synth.n_ctx(w), w.k)
    for S in Ss[1:]:
        np.testing.assert_array_equal(S, Ss[0])


def test_short_context_pads_with_minus_one():
    rng = np.random.default_rng(31)
    q, kc, vc, _ = _f32_case(rng, 1, 4, 1, 64, 40)
    n_ctx = np.array([9], np.int32)
    kc[0, 0, 9:] = np.nan
    vc[0, 0, 9:] = np.nan
    out, S, _ = oracle.layer(q, kc, vc, np.ones(1, np.uint8), None, n_ctx, 16)
    assert S[0, 0, :9].tolist() == list(range(9)) and S[0, 0, 9:].tolist() == [-1] * 7
    assert np.all(np.isfinite(out))


# ---------------------------------------------------------------- error paths

def test_oracle_rejects_bad_arguments():
    rng = np.random.default_rng(37)
    q, kc, vc, n_ctx = _f32_case(rng, 1, 4, 1, 64, 32)
    with pytest.raises(ValueError):
        oracle.layer(q, kc, vc, np.zeros(1, np.uint8), None, n_ctx, 4)       # sparse without S
    with pytest.raises(ValueError):
        oracle.layer(q, kc, vc, np.zeros(1, np.uint8), np.array([[[0, 1, 2, 32]]], np.int32), n_ctx, 4)
    with pytest.raises(ValueError):
        oracle.layer(q, kc, vc, np.ones(1, np.uint8), None, np.array([33], np.int32), 4)
    with pytest.raises(ValueError):
        oracle.step([(q, kc, vc, np.zeros(1, np.uint8))], n_ctx, 4)


# ---------------------------------------------------------------- selection rules (reading R16)

def _pooled_scores_by_hand(q, kc, b, g, n, G):
    """Mean over the group's G heads of q_h . k_j / sqrt(d), in float64 loops."""
    d = q.shape[2]
    s = np.zeros(n)
    for j in range(n):
        acc = 0.0
        for i in range(G):
            acc += float(np.dot(q[b, g * G + i].astype(np.float64), kc[b, g, j].astype(np.float64))) / math.sqrt(d)
        s[j] = acc / G
    return s


def test_ratio_rule_is_topk_of_ceil_theta_n():
    """Ratio(theta) keeps min(k, ceil(theta * n)) tokens; theta with
    ceil(theta * n) = k' reduces to top-k', theta = 1 with k >= n keeps all."""
    rng = np.random.default_rng(31)
    G, Hkv, d, n = 4, 2, 32, 200
    q, kc, vc, n_ctx = _f32_case(rng, 1, Hkv * G, Hkv, d, n)
    ones = np.ones(Hkv, np.uint8)
    for theta, kprime in ((0.1, 20), (0.2525, 51), (0.005, 1), (0.0001, 1)):
        _, S_r, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, 64, rule="ratio", param=theta)
        _, S_k, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, kprime)
        np.testing.assert_array_equal(S_r[:, :, :kprime], S_k, err_msg=f"theta={theta}")
        assert np.all(S_r[:, :, kprime:] == -1)
    _, S_all, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, 256, rule="ratio", param=1.0)
    np.testing.assert_array_equal(S_all[0, 0, :n], np.arange(n))
    assert np.all(S_all[:, :, n:] == -1)
    # the budget cap k still applies
    _, S_cap, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, 16, rule="ratio", param=0.5)
    _, S_16, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, 16)
    np.testing.assert_array_equal(S_cap, S_16)


def test_threshold_rule_matches_scores_computed_by_hand():
    """Threshold(tau) keeps the tokens with pooled score >= tau (the k highest
    if more): checked against scores computed in plain loops, plus the closed
    forms tau = -inf (top-k) and tau = +inf (empty)."""
    rng = np.random.default_rng(32)
    G, Hkv, d, n, k = 2, 2, 16, 60, 40
    q, kc, vc, n_ctx = _f32_case(rng, 1, Hkv * G, Hkv, d, n)
    ones = np.ones(Hkv, np.uint8)
    for g in range(Hkv):
        s = _pooled_scores_by_hand(q, kc, 0, g, n, G)
        for tau in (np.sort(s)[-5], np.sort(s)[-25], np.median(s), np.sort(s)[-50]):
            _, S, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, k, rule="threshold", param=float(tau))
            keep = [j for j in sorted(range(n), key=lambda j: (-s[j], j)) if s[j] >= tau][:k]
            got = S[0, g]
            np.testing.assert_array_equal(got[:len(keep)], np.sort(keep), err_msg=f"g={g} tau={tau}")
            assert np.all(got[len(keep):] == -1)
    _, S_lo, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, k, rule="threshold", param=-math.inf)
    _, S_k, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, k)
    np.testing.assert_array_equal(S_lo, S_k)
    _, S_hi, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, k, rule="threshold", param=math.inf)
    assert np.all(S_hi == -1)


def test_sparse_head_skips_padding_and_empty_set_gives_zero():
    """-1 entries of S_in are padding: a sparse head over S with padding equals
    the sparse head over the valid entries alone; an all-padding S gives 0."""
    rng = np.random.default_rng(33)
    G, Hkv, d, n, k = 4, 2, 32, 100, 10
    q, kc, vc, n_ctx = _f32_case(rng, 1, Hkv * G, Hkv, d, n)
    sparse = np.zeros(Hkv, np.uint8)
    S_pad = np.full((1, Hkv, k), -1, np.int32)
    S_pad[0, 0, :4] = [3, 17, 50, 99]
    S_pad[0, 1, :1] = [42]
    out_pad, S_fwd, _ = oracle.layer(q, kc, vc, sparse, S_pad, n_ctx, k)
    np.testing.assert_array_equal(S_fwd, S_pad)
    # head 0 over rows {3, 17, 50, 99} equals dense attention restricted to them by hand
    for i in range(G):
        h = i
        z = np.array([float(np.dot(q[0, h].astype(np.float64), kc[0, 0, j].astype(np.float64))) / math.sqrt(d)
                      for j in (3, 17, 50, 99)])
        w = np.exp(z - z.max())
        w /= w.sum()
        ref = sum(w[r] * vc[0, 0, j].astype(np.float64) for r, j in enumerate((3, 17, 50, 99)))
        np.testing.assert_allclose(out_pad[0, h], ref, rtol=0, atol=1e-12)
    # head 1 over a single row returns that V row
    for i in range(G):
        np.testing.assert_allclose(out_pad[0, G + i], vc[0, 1, 42].astype(np.float64), rtol=0, atol=1e-12)
    S_empty = np.full((1, Hkv, k), -1, np.int32)
    out_e, _, _ = oracle.layer(q, kc, vc, sparse, S_empty, n_ctx, k)
    assert np.all(out_e == 0.0)


def test_topp_rule_identical_keys_keeps_ceil_p_n():
    """Identical keys: every pooled share is 1/n, so Top-p keeps ceil(p n)
    tokens, the lowest indices (ties), for p n away from an integer."""
    rng = np.random.default_rng(34)
    G, Hkv, d, n = 2, 1, 16, 200
    q, kc, vc, n_ctx = _f32_case(rng, 1, G * Hkv, Hkv, d, n)
    kc[0, 0, :] = kc[0, 0, 7]
    for p, r in ((0.3025, 61), (0.0001, 1), (0.9975, 200)):
        _, S, _ = oracle.layer(q, kc, vc, np.ones(Hkv, np.uint8), None, n_ctx, 256, rule="topp", param=p)
        np.testing.assert_array_equal(S[0, 0, :r], np.arange(r), err_msg=f"p={p}")
        assert np.all(S[0, 0, r:] == -1), f"p={p}"


def test_topp_rule_two_level_profile_closed_form():
    """m heavy tokens with pooled score a, n - m light ones with score 0: each
    heavy share is e^a / Z and each light share 1 / Z with Z = m e^a + n - m,
    so Top-p keeps ceil(p Z / e^a) heavy tokens (lowest indices first), or all
    m heavy plus ceil((p - m e^a / Z) Z) light ones (lowest indices)."""
    d, n = 16, 120
    heavy = np.array([5, 17, 40, 41, 99])
    m = heavy.size
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 8.0
    kc = np.zeros((1, 1, n, d), np.float32)
    kc[0, 0, :, 1] = 1.0                      # light rows: orthogonal to q, score 0
    kc[0, 0, heavy, 1] = 0.0
    kc[0, 0, heavy, 0] = 1.0                  # heavy rows: score 8 / sqrt(16) = 2
    vc = np.random.default_rng(35).standard_normal((1, 1, n, d)).astype(np.float32)
    n_ctx = np.array([n], np.int32)
    a = 2.0
    Z = m * math.exp(a) + (n - m)
    light = np.setdiff1d(np.arange(n), heavy)
    for p in (0.1, 0.2, 0.25, 0.3):
        x = p * Z / math.exp(a)
        if x <= m:
            assert abs(x - round(x)) > 1e-3
            keep = heavy[:math.ceil(x)]
        else:
            y = (p - m * math.exp(a) / Z) * Z
            assert abs(y - round(y)) > 1e-3
            keep = np.concatenate([heavy, light[:math.ceil(y)]])
        _, S, _ = oracle.layer(q, kc, vc, np.ones(1, np.uint8), None, n_ctx, 64, rule="topp", param=p)
        np.testing.assert_array_equal(S[0, 0, :keep.size], np.sort(keep), err_msg=f"p={p}")
        assert np.all(S[0, 0, keep.size:] == -1), f"p={p}"


def test_topp_rule_limits():
    """A tiny p keeps the argmax alone (top-1); p = 1 with k < n is capped by
    k (the shares of the other n - k tokens keep the sum below 1): top-k."""
    rng = np.random.default_rng(36)
    G, Hkv, d, n, k = 4, 2, 32, 100, 40
    q, kc, vc, n_ctx = _f32_case(rng, 1, Hkv * G, Hkv, d, n)
    ones = np.ones(Hkv, np.uint8)
    _, S_p, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, k, rule="topp", param=1e-12)
    _, S_1, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, 1)
    np.testing.assert_array_equal(S_p[:, :, :1], S_1)
    assert np.all(S_p[:, :, 1:] == -1)
    _, S_p, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, k, rule="topp", param=1.0)
    _, S_k, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, k)
    np.testing.assert_array_equal(S_p, S_k)
    with pytest.raises(ValueError):
        oracle.layer(q, kc, vc, ones, None, n_ctx, k, rule="topp", param=0.0)


# ---------------------------------------------------------------- block-granular selection (reading R17)

def test_block_rule_with_one_token_blocks_is_topk():
    rng = np.random.default_rng(37)
    G, Hkv, d, n, k = 4, 2, 32, 150, 24
    q, kc, vc, n_ctx = _f32_case(rng, 1, Hkv * G, Hkv, d, n)
    ones = np.ones(Hkv, np.uint8)
    _, S_b, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, k, rule="block", param=1)
    _, S_k, _ = oracle.layer(q, kc, vc, ones, None, n_ctx, k)
    np.testing.assert_array_equal(S_b, S_k)


def test_block_rule_planted_maxima_closed_form():
    """Light tokens score 0 (K orthogonal to q); planted tokens score 2, 1.5,
    1.5 (a tie between two blocks) and 1 in known blocks of 8.  With
    floor(k / 8) = 3 blocks kept: the block of the 2, then of the tied 1.5s
    the two of them, i.e. blocks {5, 1, 9} - the 1's block (3) is out; with
    2 blocks the tie goes to the lower block (1 before 9)."""
    d, n, bs = 16, 84, 8                      # 11 blocks, the last one 4 tokens long
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 4.0
    kc = np.zeros((1, 1, n, d), np.float32)
    kc[0, 0, :, 1] = 1.0
    plant = {43: 2.0, 12: 1.5, 77: 1.5, 30: 1.0}   # token -> score (blocks 5, 1, 9, 3)
    for j, sc in plant.items():
        kc[0, 0, j, 1] = 0.0
        kc[0, 0, j, 0] = sc                   # score = 4 * sc / sqrt(16) = sc
    vc = np.random.default_rng(38).standard_normal((1, 1, n, d)).astype(np.float32)
    n_ctx = np.array([n], np.int32)
    for k, blocks in ((24, [1, 5, 9]), (16, [1, 5]), (31, [1, 5, 9]), (32, [1, 3, 5, 9])):
        _, S, _ = oracle.layer(q, kc, vc, np.ones(1, np.uint8), None, n_ctx, k, rule="block", param=bs)
        want = np.concatenate([np.arange(b * bs, min(n, b * bs + bs)) for b in blocks])
        np.testing.assert_array_equal(S[0, 0, :want.size], want, err_msg=f"k={k}")
        assert np.all(S[0, 0, want.size:] == -1), f"k={k}"
    # the short last block (tokens 80..83) scores 0 like the other light blocks
    # and, tied with them, comes last: it is kept only when every block is
    _, S, _ = oracle.layer(q, kc, vc, np.ones(1, np.uint8), None, n_ctx, 88, rule="block", param=bs)
    np.testing.assert_array_equal(S[0, 0, :n], np.arange(n))
    assert np.all(S[0, 0, n:] == -1)
    _, S, _ = oracle.layer(q, kc, vc, np.ones(1, np.uint8), None, n_ctx, 80, rule="block", param=bs)
    np.testing.assert_array_equal(S[0, 0, :80], np.arange(80))


def test_block_rule_rejects_bad_block_sizes():
    rng = np.random.default_rng(39)
    q, kc, vc, n_ctx = _f32_case(rng, 1, 2, 1, 16, 40)
    for bs in (0, 2.5, 64):                   # 64 > k = 32
        with pytest.raises(ValueError):
            oracle.layer(q, kc, vc, np.ones(1, np.uint8), None, n_ctx, 32, rule="block", param=bs)


# ---------------------------------------------------------------- multi-step loop (reading R18)

def test_kv_append_writes_the_new_rows_and_grows_n():
    rng = np.random.default_rng(40)
    B, Hkv, d, max_ctx = 2, 3, 16, 10
    for dtype in ("f32", "bf16"):
        kc = rng.standard_normal((B, Hkv, max_ctx, d)).astype(np.float32)
        vc = rng.standard_normal((B, Hkv, max_ctx, d)).astype(np.float32)
        kn = rng.standard_normal((B, Hkv, d)).astype(np.float32)
        vn = rng.standard_normal((B, Hkv, d)).astype(np.float32)
        if dtype == "bf16":
            kc, vc, kn, vn = (synth.to_bf16_bits(a) for a in (kc, vc, kn, vn))
        k0, v0 = kc.copy(), vc.copy()
        n = np.array([4, 9], np.int32)
        n2 = oracle.kv_append(kn, vn, kc, vc, n)
        np.testing.assert_array_equal(n2, n + 1)
        for b in range(B):
            np.testing.assert_array_equal(kc[b, :, n[b]], kn[b])
            np.testing.assert_array_equal(vc[b, :, n[b]], vn[b])
            others = np.ones(max_ctx, bool)
            others[n[b]] = False
            np.testing.assert_array_equal(kc[b][:, others], k0[b][:, others])
            np.testing.assert_array_equal(vc[b][:, others], v0[b][:, others])
        with pytest.raises(ValueError):           # the second sequence is now full
            oracle.kv_append(kn, vn, kc, vc, n2)


def _corr_case(rng, B, T, Hq, Hkv, d, max_ctx, n):
    q = rng.standard_normal((B, T, Hq, d)).astype(np.float32)
    kc = rng.standard_normal((B, Hkv, max_ctx, d)).astype(np.float32)
    vc = rng.standard_normal((B, Hkv, max_ctx, d)).astype(np.float32)
    return q, kc, vc, np.asarray(n, np.int32)


def test_correction_attention_one_row_is_the_dense_decode_output():
    rng = np.random.default_rng(41)
    B, Hq, Hkv, d, max_ctx = 2, 8, 2, 32, 90
    q, kc, vc, n = _corr_case(rng, B, 1, Hq, Hkv, d, max_ctx, [90, 57])
    out = oracle.correction_attention(q, kc, vc, n)
    ref, _, _ = oracle.layer(q[:, 0], kc, vc, np.ones(Hkv, np.uint8), None, n, 4)
    np.testing.assert_allclose(out[:, 0], ref, rtol=0, atol=1e-13)


def test_correction_attention_identical_keys_average_the_v_prefix():
    rng = np.random.default_rng(42)
    B, T, Hq, Hkv, d, max_ctx = 1, 5, 4, 2, 16, 40
    q, kc, vc, n = _corr_case(rng, B, T, Hq, Hkv, d, max_ctx, [33])
    kc[:] = kc[:, :, :1]                           # every key equal: uniform weights
    out = oracle.correction_attention(q, kc, vc, n)
    for t in range(T):
        p = 33 - T + t
        for h in range(Hq):
            np.testing.assert_allclose(out[0, t, h], vc[0, h // 2, :p + 1].astype(np.float64).mean(axis=0),
                                       rtol=0, atol=1e-12)


def test_correction_attention_is_causal():
    """Rows after a position never change its output; a row at or before it does."""
    rng = np.random.default_rng(43)
    B, T, Hq, Hkv, d, max_ctx = 1, 6, 4, 1, 16, 30
    q, kc, vc, n = _corr_case(rng, B, T, Hq, Hkv, d, max_ctx, [30])
    base = oracle.correction_attention(q, kc, vc, n)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[0, 0, 27:] += 3.0                          # positions 27..29
    vc2[0, 0, 27:] -= 2.0
    out = oracle.correction_attention(q, kc2, vc2, n)
    # row t sits at position 24 + t: rows 0..2 (positions 24..26) see no change
    np.testing.assert_array_equal(out[0, :3], base[0, :3])
    assert np.all(np.abs(out[0, 3:] - base[0, 3:]).max(axis=-1) > 1e-3)


def test_correction_attention_matches_torch_sdpa_with_a_causal_mask():
    import torch
    rng = np.random.default_rng(44)
    B, T, Hq, Hkv, d, max_ctx = 2, 7, 8, 2, 32, 50
    q, kc, vc, n = _corr_case(rng, B, T, Hq, Hkv, d, max_ctx, [50, 23])
    out = oracle.correction_attention(q, kc, vc, n)
    G = Hq // Hkv
    for b in range(B):
        nb = int(n[b])
        Q = torch.from_numpy(q[b].astype(np.float64)).permute(1, 0, 2)          # [Hq, T, d]
        K = torch.from_numpy(kc[b, :, :nb].astype(np.float64)).repeat_interleave(G, dim=0)   # [Hq, n, d]
        V = torch.from_numpy(vc[b, :, :nb].astype(np.float64)).repeat_interleave(G, dim=0)
        pos = torch.arange(nb - T, nb)[:, None]
        mask = torch.arange(nb)[None, :] <= pos                                   # [T, n]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
