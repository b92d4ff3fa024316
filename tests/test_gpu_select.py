"""Selection rules other than top-k on the GPU, against the oracle (reading R16
of the oracle: the ratio, threshold and Top-p rules of the digest's ablation
of selection methods, section 4.4.1 / Figure 6; reading R17: block-granular
selection).

Each case runs layer 0 (all retrieval) under a rule and a layer 1 with half
of the KV heads sparse under the same rule, so the sparse heads attend to a
set padded with -1.  Ragged contexts (one not a multiple of 32) and, at the
end, a context shorter than k (every token is a candidate) and the 128K
context (several passes per workgroup) are covered.  Hand-made S_in rows with
-1 entries anywhere, and a row of padding only, check the sparse path alone."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, make_handle, run_layer
from parity import compare_layer

pytestmark = pytest.mark.gpu

RAGGED = synth.Workload("select_ragged", 31, 2, 2, 32, 8, 128, 16384, 1024, "bf16", 4,
                        ctx_list=(16384, 9001), hh_frac=0.01)
SHORT = synth.Workload("select_short", 32, 2, 2, 32, 8, 128, 4096, 4096, "bf16", 4,
                       ctx_list=(3001, 4096), hh_frac=0.01)
HALF = np.array([0, 1, 0, 1, 0, 1, 0, 1], np.uint8)


def _two_layers(w: synth.Workload, rule: str, param: float, role1=HALF):
    import torch
    handle = make_handle(w)
    lens = synth.n_ctx(w)
    n_ctx_dev = torch.from_numpy(lens).cuda()
    role0 = np.ones(w.n_kv_heads, np.uint8)
    x0 = synth.layer_inputs(w, 0)
    out0, S0, S0_dev = run_layer(handle, x0, role0, None, n_ctx_dev, w.k, rule=rule, param=param)
    err0, band0 = compare_layer(out0, S0, x0, role0, None, lens, w.k, w.dtype, rule=rule, param=param)
    kept = (S0 != -1).sum(axis=2)
    log(f"[{w.name}] {rule}({param:g}) layer 0: kept per head {kept.min()}..{kept.max()}, "
        f"max|err|={err0:.2e} band-diffs={band0}")
    x1 = synth.layer_inputs(w, 1)
    out1, S1, _ = run_layer(handle, x1, role1, S0_dev, n_ctx_dev, w.k, rule=rule, param=param)
    err1, band1 = compare_layer(out1, S1, x1, role1, S0, lens, w.k, w.dtype, rule=rule, param=param)
    log(f"[{w.name}] {rule}({param:g}) layer 1 roles={list(role1)}: max|err|={err1:.2e} band-diffs={band1}")
    handle.check_device_errors()
    return S0, out1


def _tau_keeping(w: synth.Workload, rank: int) -> float:
    """A tau between the rank-th and (rank+1)-th pooled scores of layer 0's
    first head (so about `rank` tokens per head pass it)."""
    lens = synth.n_ctx(w)
    x0 = synth.layer_inputs(w, 0)
    _, _, scores = oracle.layer(x0["q"], x0["k"], x0["v"], np.ones(w.n_kv_heads, np.uint8), None, lens, w.k,
                                want_scores=True)
    s = np.sort(scores[0, 0, :int(lens[0])])[::-1]
    return float(0.5 * (s[rank - 1] + s[rank]))


def test_ratio_rule_below_k():
    # ceil(0.03 n) = 492 and 271 < k = 1024
    S0, _ = _two_layers(RAGGED, "ratio", 0.03)
    for b, n in enumerate(synth.n_ctx(RAGGED)):
        assert np.all((S0[b] != -1).sum(axis=1) == math.ceil(0.03 * int(n)))


def test_ratio_rule_above_k_equals_topk():
    S0, _ = _two_layers(RAGGED, "ratio", 0.5)
    assert np.all((S0 != -1).sum(axis=2) == RAGGED.k)


def test_ratio_rule_whole_context():
    # theta = 1 and k >= n: every token, in order
    S0, _ = _two_layers(SHORT, "ratio", 1.0)
    for b, n in enumerate(synth.n_ctx(SHORT)):
        assert np.all(S0[b, :, :n] == np.arange(n)) and np.all(S0[b, :, n:] == -1)


def test_threshold_rule_below_k():
    _two_layers(RAGGED, "threshold", _tau_keeping(RAGGED, 300))


def test_threshold_rule_bound_by_k():
    _two_layers(RAGGED, "threshold", _tau_keeping(RAGGED, 6000))


def test_threshold_rule_every_token_a_candidate():
    # k >= n: the threshold alone cuts the set
    _two_layers(SHORT, "threshold", _tau_keeping(SHORT, 700))


def test_threshold_minus_infinity_is_topk_and_plus_infinity_is_empty():
    S0, _ = _two_layers(RAGGED, "threshold", -math.inf)
    assert np.all((S0 != -1).sum(axis=2) == RAGGED.k)
    S0, out1 = _two_layers(RAGGED, "threshold", math.inf)
    assert np.all(S0 == -1)
    # the sparse heads of layer 1 attend to nothing: output 0
    G = RAGGED.group
    for g in np.nonzero(HALF == 0)[0]:
        assert np.all(out1[:, g * G:(g + 1) * G, :] == 0.0)


def test_ratio_rule_at_128k_context():
    w = synth.Workload("select_128k", 33, 1, 2, 32, 8, 128, 131072, 4096, "bf16", 4, hh_frac=0.01)
    _two_layers(w, "ratio", 0.02)


def test_sparse_heads_skip_padding_anywhere():
    import torch
    w = RAGGED
    handle = make_handle(w)
    lens = synth.n_ctx(w)
    n_ctx_dev = torch.from_numpy(lens).cuda()
    role0 = np.ones(w.n_kv_heads, np.uint8)
    x0 = synth.layer_inputs(w, 0)
    _, S0, _ = run_layer(handle, x0, role0, None, n_ctx_dev, w.k)
    rng = np.random.default_rng(77)
    S_in = S0.copy()
    for b in range(w.batch):
        for g in range(w.n_kv_heads):
            hole = rng.random(w.k) < 0.3
            S_in[b, g, hole] = -1
    S_in[1, 2, :] = -1                  # a sparse head (g = 2) with nothing to attend to
    S_in_dev = torch.from_numpy(S_in).cuda()
    x1 = synth.layer_inputs(w, 1)
    out1, S1, _ = run_layer(handle, x1, HALF, S_in_dev, n_ctx_dev, w.k)
    err, _ = compare_layer(out1, S1, x1, HALF, S_in, lens, w.k, w.dtype)
    log(f"[{w.name}] padded S_in: max|err|={err:.2e}")
    G = w.group
    assert np.all(out1[1, 2 * G:3 * G, :] == 0.0)
    handle.check_device_errors()


# Top-p needs logits large enough for the pooled softmax to concentrate:
# q, K ~ N(0, 1) (unscaled) with 1% heavy hitters
LOUD = synth.Workload("select_topp", 34, 2, 2, 32, 8, 128, 16384, 4096, "bf16", 4,
                      ctx_list=(16384, 9001), qk_scaled=False, hh_frac=0.01)
LOUD_SHORT = synth.Workload("select_topp_short", 35, 2, 2, 32, 8, 128, 4096, 4096, "bf16", 4,
                            ctx_list=(3001, 4096), qk_scaled=False, hh_frac=0.01)


@pytest.mark.parametrize("p", [0.05, 0.3, 0.6])
def test_topp_rule(p):
    S0, _ = _two_layers(LOUD, "topp", p)
    kept = (S0 != -1).sum(axis=2)
    assert kept.min() >= 1 and kept.max() <= LOUD.k


def test_topp_rule_limits():
    # a tiny p keeps the argmax alone; p = 1 keeps min(k, n)
    S0, _ = _two_layers(LOUD, "topp", 1e-12)
    assert np.all((S0 != -1).sum(axis=2) == 1)
    S0, _ = _two_layers(LOUD, "topp", 1.0)
    assert np.all((S0 != -1).sum(axis=2) == LOUD.k)


def test_topp_rule_every_token_a_candidate():
    # k >= n: the shares of the whole context decide alone
    _two_layers(LOUD_SHORT, "topp", 0.4)


@pytest.mark.parametrize("bs", [16, 64, 256])
def test_block_rule(bs):
    # 9001 = 140 * 64 + 41: a short last block
    S0, _ = _two_layers(RAGGED, "block", bs)
    for b, n in enumerate(synth.n_ctx(RAGGED)):
        kb = min(RAGGED.k // bs, -(-int(n) // bs))
        assert np.all(np.unique(S0[b, 0][S0[b, 0] >= 0] // bs).size == kb)


def test_block_rule_every_block_and_short_context():
    # k >= n: every block kept, S lists all tokens
    S0, _ = _two_layers(SHORT, "block", 64)
    for b, n in enumerate(synth.n_ctx(SHORT)):
        assert np.all(S0[b, :, :n] == np.arange(n)) and np.all(S0[b, :, n:] == -1)


def test_block_rule_at_128k_context():
    w = synth.Workload("select_block_128k", 36, 1, 2, 32, 8, 128, 131072, 4096, "bf16", 4, hh_frac=0.01)
    _two_layers(w, "block", 64)


# A 2^18-token context: layer 0 gives each workgroup 8192 rows, so it makes
# two passes (the Top-p normaliser parts and the block maxima are merged
# across passes), and 16-token blocks give 16384 block words per head, the
# most the block resolve holds in LDS; the Top-p kernel holds more than 16
# of a head's 4096 entries per thread outside its registers.
LONG = synth.Workload("select_256k", 37, 1, 2, 32, 8, 128, 262144, 4096, "bf16", 4, qk_scaled=False,
                      hh_frac=0.01)


def test_topp_rule_two_passes_per_workgroup():
    S0, _ = _two_layers(LONG, "topp", 0.05)
    kept = (S0 != -1).sum(axis=2)
    assert kept.min() >= 1 and kept.max() <= LONG.k


def test_block_rule_16384_blocks_and_two_passes():
    _two_layers(LONG.replace(name="select_256k_block", seed=38), "block", 16)


@pytest.mark.parametrize("n", [9001, 40000])
def test_block_rule_tied_block_maxima(n):
    """Every key ties, so every block's largest key ties: the floor(k / bs)
    lowest blocks are kept (reading R17: ties go to the lower block).  In
    16-token blocks, 9001 tokens give 563 blocks, cut by counting ranks within
    the threshold digit; 40000 give 2500, more than that count takes, cut by
    radix passes over the digit's composites."""
    import torch
    k, bs = 1024, 16
    w = synth.Workload(f"block_ties_{n}", 39, 1, 1, 8, 2, 128, n, k, "bf16", 0, ctx_list=(n,))
    x = synth.layer_inputs(w, 0)
    x["k"][:] = x["k"][:, :, :1, :]
    handle = make_handle(w)
    lens = synth.n_ctx(w)
    n_ctx_dev = torch.from_numpy(lens).cuda()
    role = np.ones(2, np.uint8)
    log(f"[block ties] n={n} k={k} bs={bs}")
    out, S, _ = run_layer(handle, x, role, None, n_ctx_dev, k, rule="block", param=bs)
    m = min(k // bs, -(-n // bs))
    for g in range(2):
        np.testing.assert_array_equal(S[0, g, :m * bs], np.arange(m * bs))
        assert np.all(S[0, g, m * bs:] == -1)
    compare_layer(out, S, x, role, None, lens, k, "bf16", rule="block", param=bs)
    handle.check_device_errors()


def test_topp_rule_no_cut_decided_from_the_normaliser():
    """p above k_eff / Z for every head, with Z the pooled softmax's
    normaliser relative to its largest term: no share exceeds 1 / Z, so no
    prefix of the top-k set reaches p and the cut keeps the whole set.  The
    kernel decides this from the normaliser alone, before reading the set
    back.  The case is checked to satisfy the bound (oracle scores), then S
    and the outputs are compared with the oracle as for every rule, and
    every retrieval head keeps min(k, n) tokens."""
    lens = synth.n_ctx(RAGGED)
    for layer in (0, 1):
        x = synth.layer_inputs(RAGGED, layer)
        _, _, s = oracle.layer(x["q"], x["k"], x["v"], np.ones(RAGGED.n_kv_heads, np.uint8), None, lens,
                               RAGGED.k, want_scores=True)
        for b, n in enumerate(lens):
            sb = s[b, :, :int(n)]
            z = np.exp(sb - sb.max(axis=1, keepdims=True)).sum(axis=1)
            assert np.all(min(RAGGED.k, int(n)) / z < 0.25), "the case must satisfy the no-cut bound at p = 0.3"
    S0, _ = _two_layers(RAGGED, "topp", 0.3)
    for b, n in enumerate(lens):
        assert np.all((S0[b] != -1).sum(axis=1) == min(RAGGED.k, int(n)))


@pytest.mark.parametrize("rule,param", [("topp", 0.02), ("topp", 0.3), ("block", 16), ("ratio", 0.05)])
def test_rules_on_many_short_heads(rule, param):
    """Batch 16 x 8 KV heads, contexts 2000-8192: the Top-p cut (p = 0.02
    cuts; p = 0.3 is decided from the normaliser) and the block cut run on
    heads of one to three workgroups, resolved by the head's own first
    workgroup or its last arrival."""
    w = synth.Workload("select_many_heads", 42, 16, 2, 32, 8, 128, 8192, 512, "bf16", 4, ctx_range=(2000, 8192))
    S0, _ = _two_layers(w, rule, param)
    kept = (S0 != -1).sum(axis=2)
    assert kept.min() >= 1 and kept.max() <= w.k
