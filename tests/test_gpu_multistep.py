"""The multi-step loop around the step on the GPU, against the oracle (reading
R18: Algorithm 1's cache append and the attention of Cache Correction, the
dense causal re-prefill over the last T <= 32 decoded tokens).

The append is compared byte for byte (it is a copy); the correction attention
to the oracle's fp64 output within the bf16 tolerance of the layer outputs."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, to_device
from parity import CORR_REL, check_relative, compare_layer

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2


def _handle(B, Hq, Hkv, d, max_ctx, dtype, k_max=64):
    import hybrid_head_sparse_amd as hhs
    return hhs.Handle(B, Hq, Hkv, d, max_ctx, min(k_max, max_ctx), dtype)


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_append_matches_the_oracle_bytewise(dtype):
    import torch
    rng = np.random.default_rng(50)
    B, Hq, Hkv, d, max_ctx = 3, 8, 2, 64 if dtype == "f32" else 128, 40
    kc = rng.standard_normal((B, Hkv, max_ctx, d)).astype(np.float32)
    vc = rng.standard_normal((B, Hkv, max_ctx, d)).astype(np.float32)
    if dtype == "bf16":
        kc, vc = synth.to_bf16_bits(kc), synth.to_bf16_bits(vc)
    n = np.array([0, 17, 38], np.int32)
    h = _handle(B, Hq, Hkv, d, max_ctx, dtype)
    kc_d, vc_d = to_device(kc, dtype), to_device(vc, dtype)
    n_d = torch.from_numpy(n.copy()).cuda()
    for step in range(2):                          # two tokens in a row
        kn = rng.standard_normal((B, Hkv, d)).astype(np.float32)
        vn = rng.standard_normal((B, Hkv, d)).astype(np.float32)
        if dtype == "bf16":
            kn, vn = synth.to_bf16_bits(kn), synth.to_bf16_bits(vn)
        h.kv_append(to_device(kn, dtype), to_device(vn, dtype), kc_d, vc_d, n_d)
        n = oracle.kv_append(kn, vn, kc, vc, n)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(n_d.cpu().numpy(), n)
        np.testing.assert_array_equal(_bits(kc_d), kc)
        np.testing.assert_array_equal(_bits(vc_d), vc)
    h.check_device_errors()
    log(f"[append {dtype}] two appends bytewise equal, n_ctx -> {n.tolist()}")


def test_kv_append_to_a_full_cache_is_flagged_and_changes_nothing():
    import torch
    import hybrid_head_sparse_amd as hhs
    B, Hq, Hkv, d, max_ctx = 2, 4, 1, 128, 16
    h = _handle(B, Hq, Hkv, d, max_ctx, "bf16")
    kc = torch.zeros((B, Hkv, max_ctx, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    n_d = torch.tensor([max_ctx, 3], dtype=torch.int32, device="cuda")
    kn = torch.ones((B, Hkv, d), dtype=torch.bfloat16, device="cuda")
    h.kv_append(kn, kn, kc, vc, n_d)
    torch.cuda.synchronize()
    assert n_d.cpu().tolist() == [max_ctx, 4]
    assert float(kc[0].abs().sum()) == 0.0 and float(kc[1, 0, 3].sum()) == d
    with pytest.raises(hhs.LycheeError):
        h.check_device_errors()


def _correction_case(w: synth.Workload, T: int, seed: int, lens):
    rng = np.random.default_rng(seed)
    x = synth.layer_inputs(w, 0)
    q = rng.standard_normal((w.batch, T, w.n_q_heads, w.head_dim)).astype(np.float32) / np.sqrt(w.head_dim)
    return synth.to_bf16_bits(q), x["k"], x["v"], np.asarray(lens, np.int32)


@pytest.mark.parametrize("T, G", [(32, 4), (7, 4), (1, 4), (32, 1), (32, 8), (32, 2), (13, 2)])
def test_correction_attention_matches_the_oracle(T, G):
    import torch
    Hkv = 8 if G < 8 else 4
    w = synth.Workload(f"corr_g{G}", 60 + G, 2, 1, Hkv * G, Hkv, 128, 4096, 64, "bf16", 0,
                       ctx_list=(4096, 1001), hh_frac=0.01)
    q, kc, vc, lens = _correction_case(w, T, 70 + T, w.ctx_list)
    h = _handle(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_ctx, "bf16")
    out = torch.full((w.batch, T, w.n_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    h.correction_attention(to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"),
                           torch.from_numpy(lens).cuda(), out)
    torch.cuda.synchronize()
    h.check_device_errors()
    ref = oracle.correction_attention(q, kc, vc, lens)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref).max()
    rel = check_relative(got, ref, G, CORR_REL, "correction")
    log(f"[correction T={T} G={G}] max|err| = {err:.2e} normalised {rel:.2e}")
    assert err <= OUT_TOL


def test_correction_attention_over_a_context_of_exactly_T():
    """n = T: the whole context is the causal triangle (row t sees rows 0..t),
    beside a longer sequence in the same call."""
    import torch
    T = 32
    w = synth.Workload("corr_tri", 68, 2, 1, 32, 8, 128, 4096, 64, "bf16", 0, ctx_list=(T, 300), hh_frac=0.01)
    q, kc, vc, lens = _correction_case(w, T, 78, w.ctx_list)
    h = _handle(2, 32, 8, 128, 4096, "bf16")
    out = torch.full((2, T, 32, 128), float("nan"), dtype=torch.float32, device="cuda")
    h.correction_attention(to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"),
                           torch.from_numpy(lens).cuda(), out)
    torch.cuda.synchronize()
    h.check_device_errors()
    got, ref = out.cpu().numpy(), oracle.correction_attention(q, kc, vc, lens)
    err = np.abs(got - ref).max()
    rel = check_relative(got, ref, 4, CORR_REL, "correction")
    log(f"[correction n = T = {T}] max|err| = {err:.2e} normalised {rel:.2e}")
    assert err <= OUT_TOL


def test_correction_attention_over_a_context_shorter_than_T_is_flagged():
    """n < T is outside the contract: the device flag latches (the rows are
    undefined, so only the flag is checked) and later calls run normally."""
    import torch
    import hybrid_head_sparse_amd as hhs
    T = 8
    w = synth.Workload("corr_short", 69, 1, 1, 32, 8, 128, 1024, 64, "bf16", 0, ctx_list=(600,), hh_frac=0.01)
    q, kc, vc, lens2 = _correction_case(w, T, 79, [600])
    h = _handle(1, 32, 8, 128, 1024, "bf16")
    q_d, kc_d, vc_d = to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16")
    out = torch.empty((1, T, 32, 128), dtype=torch.float32, device="cuda")
    h.correction_attention(q_d, kc_d, vc_d, torch.tensor([5], dtype=torch.int32, device="cuda"), out)
    with pytest.raises(hhs.LycheeError):
        h.check_device_errors()
    # the same cache and queries within the contract
    h.correction_attention(q_d, kc_d, vc_d, torch.from_numpy(lens2).cuda(), out)
    torch.cuda.synchronize()
    h.check_device_errors()
    got, ref = out.cpu().numpy(), oracle.correction_attention(q, kc, vc, lens2)
    err = np.abs(got - ref).max()
    rel = check_relative(got, ref, 4, CORR_REL, "correction")
    log(f"[correction n < T flagged, then n = 600] max|err| = {err:.2e} normalised {rel:.2e}")
    assert err <= OUT_TOL


def test_correction_attention_at_128k_context():
    """The full-size context (several chunks per head, each many tiles), a
    few positions so the oracle finishes in seconds."""
    import torch
    w = synth.Workload("corr_128k", 66, 1, 1, 32, 8, 128, 131072, 64, "bf16", 0, hh_frac=0.01)
    T = 4
    q, kc, vc, lens = _correction_case(w, T, 77, [131072])
    h = _handle(1, 32, 8, 128, 131072, "bf16")
    out = torch.empty((1, T, 32, 128), dtype=torch.float32, device="cuda")
    h.correction_attention(to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"),
                           torch.from_numpy(lens).cuda(), out)
    torch.cuda.synchronize()
    h.check_device_errors()
    ref = oracle.correction_attention(q, kc, vc, lens, threads=16)
    got = out.cpu().numpy()
    err = np.abs(got - ref).max()
    rel = check_relative(got, ref, 4, CORR_REL, "correction")
    log(f"[correction 128K T={T}] max|err| = {err:.2e} normalised {rel:.2e} (max|out| {np.abs(ref).max():.2e})")
    assert err <= OUT_TOL


def test_append_then_correct_then_decode_chain():
    """A short loop: append T tokens, run the correction over them, then one
    hybrid layer at the new length, each checked against the oracle."""
    import torch
    w = synth.Workload("loop", 67, 1, 1, 32, 8, 128, 2048, 256, "bf16", 0, ctx_list=(1500,), hh_frac=0.01)
    rng = np.random.default_rng(80)
    x = synth.layer_inputs(w, 0)
    kc, vc = x["k"].copy(), x["v"].copy()
    n = np.array([1500], np.int32)
    h = _handle(1, 32, 8, 128, 2048, "bf16", k_max=256)
    kc_d, vc_d = to_device(kc, "bf16"), to_device(vc, "bf16")
    n_d = torch.from_numpy(n.copy()).cuda()
    T = 5
    for _ in range(T):
        kn = synth.to_bf16_bits(rng.standard_normal((1, 8, 128)).astype(np.float32) / np.sqrt(128))
        vn = synth.to_bf16_bits(rng.standard_normal((1, 8, 128)).astype(np.float32))
        h.kv_append(to_device(kn, "bf16"), to_device(vn, "bf16"), kc_d, vc_d, n_d)
        n = oracle.kv_append(kn, vn, kc, vc, n)
    q = synth.to_bf16_bits(rng.standard_normal((1, T, 32, 128)).astype(np.float32) / np.sqrt(128))
    out = torch.empty((1, T, 32, 128), dtype=torch.float32, device="cuda")
    h.correction_attention(to_device(q, "bf16"), kc_d, vc_d, n_d, out)
    torch.cuda.synchronize()
    h.check_device_errors()
    assert n_d.cpu().tolist() == n.tolist() == [1505]
    got, ref = out.cpu().numpy(), oracle.correction_attention(q, kc, vc, n)
    err = np.abs(got - ref).max()
    rel = check_relative(got, ref, 4, CORR_REL, "correction")
    log(f"[loop] correction after {T} appends: max|err| = {err:.2e} normalised {rel:.2e}")
    assert err <= OUT_TOL
    # the next decode step's layer over the grown cache (all retrieval)
    q1 = synth.to_bf16_bits(rng.standard_normal((1, 32, 128)).astype(np.float32) / np.sqrt(128))
    role = np.ones(8, np.uint8)
    S = torch.empty((1, 8, 256), dtype=torch.int32, device="cuda")
    o1 = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
    h.decode_layer(to_device(q1, "bf16"), kc_d, vc_d, role, None, S, o1, n_d, 256)
    torch.cuda.synchronize()
    err1, band = compare_layer(o1.cpu().numpy(), S.cpu().numpy(), {"q": q1, "k": kc, "v": vc}, role, None, n, 256,
                               "bf16")
    log(f"[loop] decode layer at n = {int(n[0])}: max|err| = {err1:.2e}, band diffs {band}")
    h.check_device_errors()


def _raw(t):
    """The tensor's bit patterns (the cache holds NaN rows past the context,
    which compare unequal to themselves as floats)."""
    import torch
    return t.view({torch.bfloat16: torch.int16, torch.float32: torch.int32}.get(t.dtype, t.dtype))


def test_loop_kernels_replay_from_a_graph():
    """Append, correction, and a hybrid layer under the Top-p and the block
    rule (each cut in its own build of the attention kernel) and under the
    Ratio and Threshold rules, captured once into a HIP graph: three replays, with the cache and n_ctx
    restored eagerly between them, each reproduce the eager run bitwise, and
    the eager layers meet the parity bar against the oracle."""
    import torch
    w = synth.Workload("loop_graph", 71, 1, 1, 32, 8, 128, 4096, 256, "bf16", 0, ctx_list=(3000,), hh_frac=0.01)
    rng = np.random.default_rng(81)
    x = synth.layer_inputs(w, 0)
    h = _handle(1, 32, 8, 128, 4096, "bf16", k_max=256)
    kc0, vc0 = to_device(x["k"], "bf16"), to_device(x["v"], "bf16")
    n0 = torch.tensor([3000], dtype=torch.int32, device="cuda")
    kc, vc, n_d = kc0.clone(), vc0.clone(), n0.clone()
    T, k = 6, 256
    kn = to_device(synth.to_bf16_bits(rng.standard_normal((1, 8, 128)).astype(np.float32) / np.sqrt(128)), "bf16")
    vn = to_device(synth.to_bf16_bits(rng.standard_normal((1, 8, 128)).astype(np.float32)), "bf16")
    qc = to_device(synth.to_bf16_bits(rng.standard_normal((1, T, 32, 128)).astype(np.float32) / np.sqrt(128)), "bf16")
    q1_np = synth.to_bf16_bits(rng.standard_normal((1, 32, 128)).astype(np.float32) / np.sqrt(128))
    q1 = to_device(q1_np, "bf16")
    # S_in of the hybrid layers: an all-retrieval layer over the grown cache, outside the graph
    S0 = torch.empty((1, 8, k), dtype=torch.int32, device="cuda")
    o0 = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
    role = np.array([1, 0, 0, 0, 0, 1, 0, 0], np.uint8)
    oc = torch.empty((1, T, 32, 128), dtype=torch.float32, device="cuda")
    Sp, Sb, Sr, St = (torch.empty_like(S0) for _ in range(4))
    op, ob, orr, ot = (torch.empty_like(o0) for _ in range(4))

    def body():
        h.kv_append(kn, vn, kc, vc, n_d)
        h.correction_attention(qc, kc, vc, n_d, oc)
        h.decode_layer(q1, kc, vc, role, S0, Sp, op, n_d, k, rule="topp", param=0.05)
        h.decode_layer(q1, kc, vc, role, S0, Sb, ob, n_d, k, rule="block", param=32)
        h.decode_layer(q1, kc, vc, role, S0, Sr, orr, n_d, k, rule="ratio", param=0.02)
        h.decode_layer(q1, kc, vc, role, S0, St, ot, n_d, k, rule="threshold", param=0.01)

    def restore():
        kc.copy_(kc0)
        vc.copy_(vc0)
        n_d.copy_(n0)

    outs = (kc, n_d, oc, Sp, op, Sb, ob, Sr, orr, St, ot)
    # eager reference (S0 from the grown cache first)
    h.kv_append(kn, vn, kc, vc, n_d)
    h.decode_layer(q1, kc, vc, np.ones(8, np.uint8), None, S0, o0, n_d, k)
    restore()
    body()
    torch.cuda.synchronize()
    h.check_device_errors()
    ref = [t.cpu().clone() for t in outs]
    # capture on a side stream after a warm-up there, as torch requires
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        h.set_stream(cap)
        restore()
        body()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        h.set_stream(torch.cuda.current_stream())
        body()
    h.set_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        for t in (oc, op, ob, orr, ot):
            t.fill_(float("nan"))
        for t in (Sp, Sb, Sr, St):
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("k_cache", "n_ctx", "correction", "S topp", "out topp", "S block", "out block",
                               "S ratio", "out ratio", "S threshold", "out threshold"), outs, ref):
            assert torch.equal(_raw(t.cpu()), _raw(r)), f"replay {rep}: {name} differs from the eager run"
        log(f"[loop graph] replay {rep} bitwise equal to the eager run")
    h.check_device_errors()
    # the eager append byte for byte, and the eager layers against the oracle
    # over the grown cache
    kc_np, vc_np = x["k"].copy(), x["v"].copy()
    n_np = oracle.kv_append(_bits(kn), _bits(vn), kc_np, vc_np, np.array([3000], np.int32))
    np.testing.assert_array_equal(_bits(ref[0]), kc_np)
    np.testing.assert_array_equal(ref[1].numpy(), n_np)
    inputs = {"q": q1_np, "k": kc_np, "v": vc_np}
    S0_np = S0.cpu().numpy()
    for rule, param, S_t, o_t in (("topp", 0.05, ref[3], ref[4]), ("block", 32, ref[5], ref[6]),
                                  ("ratio", 0.02, ref[7], ref[8]), ("threshold", 0.01, ref[9], ref[10])):
        err, band = compare_layer(o_t.numpy(), S_t.numpy(), inputs, role, S0_np, n_np, k, "bf16", rule=rule,
                                  param=param)
        log(f"[loop graph] {rule} layer: max|err| = {err:.2e}, band diffs {band}")
