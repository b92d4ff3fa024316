"""The kernel sweep in the shape of the pages' kernel-latency figure (GPU).

Parity at the figure's operating point (half the heads sparse, 90% sparsity:
k = n/10) against the oracle, parity at a large budget (k = n/10 at 128K, so
the resolver reads more candidates than its first load round holds), and the
figure's qualitative trends on a reduced grid of the sweep: the layer's time
grows with the batch and the context and falls as more heads are sparse
(between the ends of each axis, where bytes rather than the layer's fixed
latency set the time)."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import log, make_handle, run_layer
from parity import compare_layer

pytestmark = pytest.mark.gpu


def _two_layers(w: synth.Workload, role1):
    import torch
    handle = make_handle(w)
    lens = synth.n_ctx(w)
    n_ctx_dev = torch.from_numpy(lens).cuda()
    role0 = np.ones(w.n_kv_heads, np.uint8)
    x0 = synth.layer_inputs(w, 0)
    out0, S0, S0_dev = run_layer(handle, x0, role0, None, n_ctx_dev, w.k)
    err0, band0 = compare_layer(out0, S0, x0, role0, None, lens, w.k, w.dtype)
    log(f"[{w.name}] layer 0 all retrieval k={w.k}: max|err|={err0:.2e} band-diffs={band0}")
    if role1 is not None:
        x1 = synth.layer_inputs(w, 1)
        out1, S1, _ = run_layer(handle, x1, role1, S0_dev, n_ctx_dev, w.k)
        err1, band1 = compare_layer(out1, S1, x1, role1, S0, lens, w.k, w.dtype)
        log(f"[{w.name}] layer 1 roles={list(role1)}: max|err|={err1:.2e} band-diffs={band1}")
    handle.check_device_errors()


def test_half_sparse_at_ninety_percent_sparsity():
    w = synth.Workload("sweep_b2_16k", 21, 2, 2, 32, 8, 128, 16384, 1638, "bf16", 4, hh_frac=0.01)
    _two_layers(w, np.array([0, 0, 0, 0, 1, 1, 1, 1], np.uint8))


def test_large_budget_all_retrieval():
    w = synth.Workload("sweep_b1_128k_k13107", 22, 1, 1, 32, 8, 128, 131072, 13107, "bf16", 0, hh_frac=0.01)
    _two_layers(w, None)


def test_multi_pass_ranges_at_ninety_percent_sparsity():
    # 2 x 8 heads of 128K rows over the grid: every workgroup streams its part
    # of a retrieval head in several passes, and the ranges split heads at
    # arbitrary rows (short boundary passes)
    w = synth.Workload("sweep_b2_128k", 23, 2, 2, 32, 8, 128, 131072, 13107, "bf16", 4, hh_frac=0.01)
    _two_layers(w, np.array([0, 0, 0, 0, 1, 1, 1, 1], np.uint8))


def test_sweep_trends_on_a_reduced_grid():
    import torch
    import hybrid_head_sparse_amd as hhs
    from hybrid_head_sparse_amd import sweep
    rows = []
    # contexts and batches far enough apart that bytes, not the layer's fixed
    # latency (about 15-20 us), separate the points
    for si, s in enumerate((4, 8)):
        for bi, B in enumerate((1, 4)):
            for ni, n in enumerate((32768, 131072)):
                r = sweep.run_point(hhs, torch, B, n, s, 5, 100 + si * 10 + bi * 5 + ni)
                log(f"[sweep] sparse {s}/8 batch {B} n {n}: {r['us']:.1f} us, dense {r['dense_us']:.1f} us")
                rows.append(r)
    for name, ok in sweep.checks(rows):
        log(f"[sweep] {'PASS' if ok else 'FAIL'}: {name}")
        assert ok, name
    # the pages' 4/8 claim is reported, not asserted (where it fails is measured, not hidden)
    name, ok, losers = sweep.half_sparse_claim(rows)
    log(f"[sweep] {'PASS' if ok else 'FAIL'}: {name}")
    for r in losers:
        log(f"[sweep]   4/8 loses: batch {r['batch']} n {r['n']}: {r['us']:.1f} vs dense {r['dense_us']:.1f} us")
