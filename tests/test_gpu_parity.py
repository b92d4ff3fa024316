"""Parity of the HIP path with the oracle on every workload (GPU).

Each layer runs through the C ABI (binding) on the device and through the
oracle on the host with the same inputs and the same S_in (the GPU's S_out of
the previous layer); the bar is the one in tests/parity.py.  The small
workloads run their whole step; the large ones run the first layers of the
step (the full-size launch configuration of the benchmark is covered by
test_gpu_fullsize.py)."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import log, make_handle, plant_boundary_groups, run_layer
from parity import compare_layer

pytestmark = pytest.mark.gpu


def _chain(w: synth.Workload, n_layers: int, plant: bool = False):
    import torch
    handle = make_handle(w)
    roles = synth.roles(w)
    lens = synth.n_ctx(w)
    n_ctx_dev = torch.from_numpy(lens).cuda()
    S_prev_dev, S_prev = None, None
    stats = []
    for l in range(n_layers):
        log(f"[{w.name}] layer {l} roles={roles[l].tolist()} k={w.k}")
        x = synth.layer_inputs(w, l, tie_info=bool(w.tie_frac) or plant)
        ties = x.pop("ties", None)
        if plant:
            plant_boundary_groups(w, x, w.k, ties)
        out, S, S_dev = run_layer(handle, x, roles[l], S_prev_dev, n_ctx_dev, w.k)
        err, band = compare_layer(out, S, x, roles[l], S_prev, lens, w.k, w.dtype, ties=ties)
        stats.append((l, err, band))
        log(f"    max|err|={err:.2e} band-diffs={band}")
        S_prev_dev, S_prev = S_dev, S
    handle.check_device_errors()
    return stats


def test_tiny_gqa_full_step():
    _chain(synth.WORKLOADS["tiny_gqa"], 2)


def test_tiny_mha_full_step():
    _chain(synth.WORKLOADS["tiny_mha"], 2)


def test_tiny_gqa_longer_chain_all_roles():
    # 6 layers, 5 retrieval slots spread over layers 1..5
    _chain(synth.WORKLOADS["tiny_gqa"].replace(layers=6, n_retrieval=5), 6)


def test_llama3_32k_full_step():
    _chain(synth.WORKLOADS["llama3_32k"], 32)


def test_llama3_128k_first_layers():
    _chain(synth.WORKLOADS["llama3_128k"], 6)


def test_llama3_ragged_b8_first_layers():
    _chain(synth.WORKLOADS["llama3_ragged_b8"], 4)


@pytest.mark.parametrize("name", ["qwen3_128k_k1024", "qwen3_128k_k4096"])
def test_qwen3_ties_with_planted_boundary_groups(name):
    _chain(synth.WORKLOADS[name], 4, plant=True)
