"""Edge cases of the HIP path against the oracle (GPU): ragged and tiny
contexts around k, k = 1, every supported head_dim / group / dtype variant,
in-place S, identical keys (LDS and global resolution paths of the top-k),
determinism, out-of-range S entries, the dense baseline, the maximum
context, and many sequences."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, make_handle, run_layer, to_device
from parity import OUT_TOL, check_relative, compare_layer

pytestmark = pytest.mark.gpu


def _w(name, seed, B, L, Hq, Hkv, d, max_ctx, k, dtype, n_retr, ctx_list=None, **kw):
    return synth.Workload(name, seed, B, L, Hq, Hkv, d, max_ctx, k, dtype, n_retr, ctx_list=ctx_list, **kw)


def _chain(w, n_layers=None, inplace=False):
    import torch
    handle = make_handle(w)
    roles = synth.roles(w)
    lens = synth.n_ctx(w)
    n_ctx_dev = torch.from_numpy(lens).cuda()
    S_prev_dev, S_prev = None, None
    for l in range(n_layers or w.layers):
        log(f"[{w.name}] layer {l} roles={roles[l].tolist()} n={lens.tolist()[:8]} k={w.k}")
        x = synth.layer_inputs(w, l)
        S_out_dev = S_prev_dev if (inplace and S_prev_dev is not None) else None
        out, S, S_dev = run_layer(handle, x, roles[l], S_prev_dev, n_ctx_dev, w.k, S_out_dev=S_out_dev)
        compare_layer(out, S, x, roles[l], S_prev, lens, w.k, w.dtype)
        S_prev_dev, S_prev = S_dev, S
    handle.check_device_errors()


@pytest.mark.parametrize("k", [1, 16, 17, 64])
def test_ragged_contexts_around_k(k):
    ctx = (1, k - 1 if k > 1 else 2, k, k + 1, 600)
    _chain(_w(f"ragged_k{k}", 50 + k, 5, 3, 32, 8, 128, 600, k, "bf16", 6, ctx_list=ctx, hh_frac=0.01))


@pytest.mark.parametrize("dtype,d,Hq,Hkv", [
    ("f32", 128, 32, 8), ("bf16", 64, 16, 8), ("bf16", 128, 64, 8), ("bf16", 128, 8, 8),
    ("f32", 64, 16, 8), ("bf16", 64, 8, 1),
])
def test_every_variant(dtype, d, Hq, Hkv):
    w = _w(f"var_{dtype}_{d}_{Hq}_{Hkv}", 70, 2, 3, Hq, Hkv, d, 3000, 100, dtype, max(1, Hkv // 2),
           ctx_list=(3000, 1777), hh_frac=0.01)
    _chain(w)


def test_in_place_S():
    _chain(_w("inplace", 80, 2, 5, 32, 8, 128, 5000, 300, "bf16", 8, ctx_list=(5000, 2345), hh_frac=0.01),
           inplace=True)


def test_all_sparse_then_all_retrieval_layers():
    import torch
    w = _w("roles", 81, 1, 4, 32, 8, 128, 4000, 256, "bf16", 0, ctx_list=(4000,), hh_frac=0.01)
    roles = [np.ones(8, np.uint8), np.zeros(8, np.uint8), np.ones(8, np.uint8), np.zeros(8, np.uint8)]
    handle = make_handle(w)
    lens = synth.n_ctx(w)
    n_ctx_dev = torch.from_numpy(lens).cuda()
    S_dev, S = None, None
    for l in range(4):
        x = synth.layer_inputs(w, l)
        out, S_new, S_dev_new = run_layer(handle, x, roles[l], S_dev, n_ctx_dev, w.k)
        compare_layer(out, S_new, x, roles[l], S, lens, w.k, w.dtype)
        if l == 1:
            np.testing.assert_array_equal(S_new, S)
        S_dev, S = S_dev_new, S_new


@pytest.mark.parametrize("n,k", [(3000, 100), (3000, 3000), (20000, 64), (20000, 5000)])
def test_identical_keys_select_lowest_indices(n, k):
    """Every score ties: S must be exactly {0..k-1}; out = mean of V rows.
    n = 20000 exceeds the LDS candidate buffer and takes the global passes."""
    import torch
    w = _w(f"ident_{n}_{k}", 90, 1, 1, 8, 2, 128, n, k, "bf16", 0, ctx_list=(n,))
    x = synth.layer_inputs(w, 0)
    x["k"][:] = x["k"][:, :, :1, :]
    handle = make_handle(w)
    n_ctx_dev = torch.from_numpy(synth.n_ctx(w)).cuda()
    log(f"[identical] n={n} k={k}")
    out, S, _ = run_layer(handle, x, np.ones(2, np.uint8), None, n_ctx_dev, k)
    ke = min(k, n)
    for g in range(2):
        np.testing.assert_array_equal(S[0, g, :ke], np.arange(ke))
    compare_layer(out, S, x, np.ones(2, np.uint8), None, synth.n_ctx(w), k, "bf16")
    handle.check_device_errors()


def test_bitwise_determinism():
    import torch
    w = _w("determinism", 95, 2, 2, 32, 8, 128, 20000, 512, "bf16", 4, ctx_list=(20000, 12345), hh_frac=0.01)
    handle = make_handle(w)
    n_ctx_dev = torch.from_numpy(synth.n_ctx(w)).cuda()
    roles = synth.roles(w)
    runs = []
    for rep in range(2):
        x0 = synth.layer_inputs(w, 0)
        o0, S0, S0d = run_layer(handle, x0, roles[0], None, n_ctx_dev, w.k)
        x1 = synth.layer_inputs(w, 1)
        o1, S1, _ = run_layer(handle, x1, roles[1], S0d, n_ctx_dev, w.k)
        runs.append((o0, S0, o1, S1))
    for a, b in zip(runs[0], runs[1]):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)


def test_out_of_range_S_entries_are_skipped_and_reported():
    import torch
    import hybrid_head_sparse_amd as hhs
    w = _w("bad_S", 96, 1, 2, 8, 2, 128, 1000, 16, "bf16", 0, ctx_list=(1000,))
    handle = make_handle(w)
    n_ctx_dev = torch.from_numpy(synth.n_ctx(w)).cuda()
    x = synth.layer_inputs(w, 1)
    S_in = np.tile(np.arange(16, dtype=np.int32) * 7, (1, 2, 1))
    S_in[0, 0, 3] = -5
    S_in[0, 1, 9] = 1003
    S_dev = torch.from_numpy(S_in).cuda()
    out, S, _ = run_layer(handle, x, np.zeros(2, np.uint8), S_dev, n_ctx_dev, 16)
    assert np.all(np.isfinite(out))
    with pytest.raises(hhs.LycheeError) as ei:
        handle.check_device_errors()
    assert ei.value.status == hhs.LYCHEE_ERR_DEVICE_CHECK
    handle.check_device_errors()      # the flag was cleared


def test_dense_baseline_matches_oracle():
    import torch
    for w in (synth.WORKLOADS["tiny_gqa"],
              _w("dense_bf16", 97, 2, 1, 32, 8, 128, 9000, 64, "bf16", 0, ctx_list=(9000, 4321))):
        handle = make_handle(w)
        lens = synth.n_ctx(w)
        x = synth.layer_inputs(w, 0)
        dt = w.dtype
        q, kc, vc = to_device(x["q"], dt), to_device(x["k"], dt), to_device(x["v"], dt)
        out = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), device="cuda")
        handle.dense_decode_layer(q, kc, vc, out, torch.from_numpy(lens).cuda())
        torch.cuda.synchronize()
        ref, _, _ = oracle.layer(x["q"], x["k"], x["v"], np.ones(w.n_kv_heads, np.uint8), None, lens, 1)
        got = out.cpu().numpy()
        assert np.abs(got - ref).max() <= OUT_TOL[dt]
        rel = check_relative(got, ref, w.group, what="dense")
        log(f"[dense {w.name}] max|err| {np.abs(got - ref).max():.2e} normalised {rel:.2e}")


def test_maximum_context():
    w = _w("max_ctx", 98, 1, 2, 8, 2, 128, 1 << 18, 4096, "bf16", 0, ctx_list=(1 << 18,), hh_frac=0.01)
    _chain(w)


def test_many_sequences():
    w = _w("many_seq", 99, 64, 3, 32, 8, 128, 2000, 32, "bf16", 8, ctx_range=(1, 2000), hh_frac=0.01)
    _chain(w)


def test_clustered_top_keys_take_the_full_scan_path():
    """300 keys far above the rest, packed into the first rows of KV head 0.
    The workgroup streaming those rows holds ~300 of the head's top 1024 but
    bounds its candidates at twice its proportional share (tens of keys), so
    its bound lies above the head's threshold digit and the selector must
    detect that and re-read every key of the head.  Both heads must still
    match the oracle."""
    import torch
    w = _w("clustered", 90, 1, 1, 8, 2, 64, 65536, 1024, "f32", 0, ctx_list=(65536,))
    x = synth.layer_inputs(w, 0)
    qbar = x["q"][0, 0:4, :].astype(np.float64).mean(axis=0)
    direction = (qbar / np.linalg.norm(qbar)).astype(np.float32)
    rng = np.random.default_rng(91)
    x["k"][0, 0, :300, :] = 8.0 * direction + 0.1 * rng.standard_normal((300, 64), dtype=np.float32)
    role = np.ones(2, np.uint8)
    handle = make_handle(w)
    lens = synth.n_ctx(w)
    n_ctx_dev = torch.from_numpy(lens).cuda()
    log("[clustered] 300 planted keys in rows 0..299 of head 0, n=65536, k=1024")
    out, S, _ = run_layer(handle, x, role, None, n_ctx_dev, w.k)
    compare_layer(out, S, x, role, None, lens, w.k, w.dtype)
    assert set(range(300)) <= set(S[0, 0].tolist())
    handle.check_device_errors()


def test_context_outside_the_contract_is_clamped_and_flagged():
    """n_ctx = max_ctx + 1 is clamped to max_ctx (the output is the oracle's
    at max_ctx); n_ctx = 0 gives zeros, -1 retrieval rows and copied sparse
    rows; both latch the device flag."""
    import torch
    import hybrid_head_sparse_amd as hhs
    w = _w("bad_n", 92, 2, 2, 32, 8, 128, 1000, 64, "bf16", 4, ctx_list=(1000, 700), hh_frac=0.01)
    handle = make_handle(w)
    lens = synth.n_ctx(w)
    roles = synth.roles(w)
    good = torch.from_numpy(lens).cuda()
    bad = torch.tensor([1001, 0], dtype=torch.int32, device="cuda")
    x0 = synth.layer_inputs(w, 0)
    _, S0, S0_dev = run_layer(handle, x0, roles[0], None, good, w.k)
    handle.check_device_errors()
    row0 = {key: np.ascontiguousarray(v[:1]) for key, v in x0.items()}
    out, S, _ = run_layer(handle, x0, roles[0], None, bad, w.k)
    compare_layer(out[:1], S[:1], row0, roles[0], None, lens[:1], w.k, w.dtype)
    assert np.all(out[1] == 0.0) and np.all(S[1] == -1)
    with pytest.raises(hhs.LycheeError) as ei:
        handle.check_device_errors()
    assert ei.value.status == hhs.LYCHEE_ERR_DEVICE_CHECK
    x1 = synth.layer_inputs(w, 1)
    out1, S1, _ = run_layer(handle, x1, roles[1], S0_dev, bad, w.k)
    row1 = {key: np.ascontiguousarray(v[:1]) for key, v in x1.items()}
    compare_layer(out1[:1], S1[:1], row1, roles[1], S0[:1], lens[:1], w.k, w.dtype)
    assert np.all(out1[1] == 0.0)
    for g in range(w.n_kv_heads):
        want = np.full(w.k, -1, np.int32) if roles[1][g] else S0[1, g]
        np.testing.assert_array_equal(S1[1, g], want)
    with pytest.raises(hhs.LycheeError):
        handle.check_device_errors()
    handle.check_device_errors()      # cleared
    log(f"[bad_n] n_ctx [1001, 0] clamped to [1000, 0] and flagged; roles of layer 1 {roles[1].tolist()}")


@pytest.mark.parametrize("n,k,where", [(1000, 16, (5,)), (20000, 4096, (128, 1024, 2047, 2048, 3001))])
def test_duplicate_S_entries_are_flagged(n, k, where):
    """S_in rows whose entries (other than -1) are not strictly ascending --
    here a duplicate next to its twin, with and without -1 holes between --
    latch the device flag; the duplicated row is attended twice, as the
    oracle does, and a row with holes but no duplicate does not flag."""
    import torch
    import hybrid_head_sparse_amd as hhs
    w = _w(f"dup_S_{k}", 93, 1, 2, 8, 2, 128, n, k, "bf16", 0, ctx_list=(n,))
    handle = make_handle(w)
    lens = synth.n_ctx(w)
    n_ctx_dev = torch.from_numpy(lens).cuda()
    x = synth.layer_inputs(w, 1)
    base = (np.arange(k, dtype=np.int64) * (n // k)).astype(np.int32)
    S_in = np.stack([base, base])[None].copy()
    S_in[0, 1, ::3] = -1                         # holes, still ascending: no flag
    sparse = np.zeros(2, np.uint8)
    out, S, _ = run_layer(handle, x, sparse, torch.from_numpy(S_in).cuda(), n_ctx_dev, k)
    compare_layer(out, S, x, sparse, S_in, lens, k, w.dtype)
    handle.check_device_errors()
    dup = S_in.copy()
    for i in where:
        dup[0, 0, i] = dup[0, 0, i - 1]          # adjacent twin
    dup[0, 1, where[0] + 1] = -1                 # twin across a hole
    dup[0, 1, where[0] + 2] = dup[0, 1, where[0]] if dup[0, 1, where[0]] != -1 else dup[0, 1, where[0] - 1]
    out, S, _ = run_layer(handle, x, sparse, torch.from_numpy(dup).cuda(), n_ctx_dev, k)
    compare_layer(out, S, x, sparse, dup, lens, k, w.dtype)
    with pytest.raises(hhs.LycheeError) as ei:
        handle.check_device_errors()
    assert ei.value.status == hhs.LYCHEE_ERR_DEVICE_CHECK and "flag 0x20 " in str(ei.value)
    log(f"[dup_S k={k}] duplicates at {list(where)} flagged")
