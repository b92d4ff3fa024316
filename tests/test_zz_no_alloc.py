"""The allocation-free entry point against the handle's entry point (GPU).

lychee_decode_layer_static runs the same kernel as lychee_decode_layer with
the library's per-GPU scratch in place of a caller's workspace, so on the same
inputs (the same S_in: the handle path's S of the previous layer) its out and
S_out must be bitwise equal.  Two workloads back to back, the second smaller
(fewer sequences, heads and rows, another dtype and head dim), so the second
call reuses the scratch the first one left."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import log, make_handle, to_device

pytestmark = pytest.mark.gpu

BIG = synth.Workload("static_big", 141, 2, 2, 32, 8, 128, 20000, 1024, "bf16", 4, ctx_list=(20000, 12345),
                     hh_frac=0.01)
SMALL = synth.Workload("static_small", 142, 1, 2, 8, 2, 64, 3000, 100, "f32", 1, ctx_list=(2900,), qk_scaled=False)


def _compare(w):
    import torch
    import hybrid_head_sparse_amd as hhs
    handle = make_handle(w)
    dims = hhs.make_dims(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_ctx, w.k, w.dtype)
    roles = synth.roles(w)
    n_ctx = torch.from_numpy(synth.n_ctx(w)).cuda()
    S_prev = None
    for l in range(w.layers):
        x = synth.layer_inputs(w, l)
        q, kc, vc = (to_device(x[key], w.dtype) for key in ("q", "k", "v"))
        shape_S = (w.batch, w.n_kv_heads, w.k)
        S_h = torch.full(shape_S, -7, dtype=torch.int32, device="cuda")
        S_s = torch.full(shape_S, -9, dtype=torch.int32, device="cuda")
        out_h = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), device="cuda")
        out_s = torch.full_like(out_h, float("inf"))
        handle.decode_layer(q, kc, vc, roles[l], S_prev, S_h, out_h, n_ctx, w.k)
        hhs.decode_layer_static(dims, q, kc, vc, roles[l], S_prev, S_s, out_s, n_ctx, w.k)
        torch.cuda.synchronize()
        assert torch.equal(out_h.view(torch.int32), out_s.view(torch.int32)), f"{w.name} layer {l}: out differs"
        assert torch.equal(S_h, S_s), f"{w.name} layer {l}: S differs"
        log(f"[{w.name}] layer {l} roles={roles[l].tolist()}: static entry bitwise equal to the handle's")
        S_prev = S_h
    handle.check_device_errors()


def test_static_entry_matches_the_handle_entry_twice_second_smaller():
    _compare(BIG)
    _compare(SMALL)
