"""The headline workload at full size, in the launch configuration the
benchmark times (GPU): the 32-layer step of the Llama3-8B-shaped 128K
workload (k = 4096), all layers resident, chained through S on the device and
captured once into a HIP graph.

Checked:
  * every graph replay reproduces the eager step bitwise (out and S of every
    layer), with eager work and synchronisation between replays;
  * every layer matches the oracle to the parity bar, the oracle taking the
    same inputs and, for the sparse heads, the S_in the GPU produced for the
    previous layer (teacher forcing)."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import log, make_handle, to_device
from parity import compare_layer

pytestmark = pytest.mark.gpu


def test_llama3_128k_full_step_in_a_graph():
    import torch
    w = synth.WORKLOADS["llama3_128k"]
    roles = synth.roles(w)
    lens = synth.n_ctx(w)
    B, Hq, Hkv, d, k = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.k
    handle = make_handle(w)
    n_ctx = torch.from_numpy(lens).cuda()
    dev = []
    for l in range(w.layers):
        x = synth.layer_inputs(w, l, threads=16)
        dev.append({key: to_device(x[key], w.dtype) for key in ("q", "k", "v")})
    log(f"[{w.name}] {w.layers} layers resident")
    S = [torch.full((B, Hkv, k), -7, dtype=torch.int32, device="cuda") for _ in range(w.layers)]
    outs = [torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda") for _ in range(w.layers)]

    def step():
        for l in range(w.layers):
            x = dev[l]
            handle.decode_layer(x["q"], x["k"], x["v"], roles[l], S[l - 1] if l else None, S[l], outs[l],
                                n_ctx, k)

    step()
    torch.cuda.synchronize()
    handle.check_device_errors()
    ref_out = [o.cpu().numpy().copy() for o in outs]
    ref_S = [s.cpu().numpy().copy() for s in S]
    log(f"[{w.name}] eager step done")

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        handle.set_stream(torch.cuda.current_stream())
        step()
    handle.set_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        for s in S:
            s.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(w.layers):
            np.testing.assert_array_equal(outs[l].cpu().numpy(), ref_out[l], err_msg=f"replay {rep} layer {l}")
            np.testing.assert_array_equal(S[l].cpu().numpy(), ref_S[l], err_msg=f"replay {rep} layer {l}")
        log(f"[{w.name}] replay {rep} bitwise equal to the eager step")
    handle.check_device_errors()
    del dev
    torch.cuda.empty_cache()

    for l in range(w.layers):
        x = synth.layer_inputs(w, l, threads=16)
        st = compare_layer(ref_out[l], ref_S[l], x, roles[l], ref_S[l - 1] if l else None, lens, k, w.dtype,
                           threads=16)
        log(f"[{w.name}] layer {l} roles={int(roles[l].sum())} retrieval  max|err|={st[0]:.2e} "
            f"normalised={st.rel:.2e} band-diffs={st[1]}")
