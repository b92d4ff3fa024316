"""The seeded input generator: determinism and the planted structure."""
import hashlib

import numpy as np

import synth


def _digest(x):
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()


def test_generation_is_deterministic_and_seed_dependent():
    w = synth.WORKLOADS["tiny_gqa"]
    a = synth.layer_inputs(w, 1)
    b = synth.layer_inputs(w, 1, threads=1)
    for key in ("q", "k", "v"):
        assert _digest(a[key]) == _digest(b[key])
    c = synth.layer_inputs(w.replace(seed=99), 1)
    assert _digest(a["k"]) != _digest(c["k"])
    d = synth.layer_inputs(w, 0)
    assert _digest(a["k"]) != _digest(d["k"])


def test_roles_layer0_all_retrieval_and_budget():
    for name, w in synth.WORKLOADS.items():
        r = synth.roles(w)
        assert r.shape == (w.layers, w.n_kv_heads)
        assert np.all(r[0] == 1)
        assert int(r[1:].sum()) == w.n_retrieval, name


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1e-3], np.float32)
    bits = synth.to_bf16_bits(x)
    assert bits[0] == 0x3F80
    assert bits[1] == 0x3F80            # exactly half-way, rounds to even
    assert bits[2] == 0x3F82            # half-way, rounds up to even
    assert bits[3] == 0xC020
    back = synth.bf16_bits_to_f32(bits)
    assert abs(back[4] - 1e-3) <= 2**-9 * 1e-3


def test_ragged_lengths_heavy_hitters_ties_and_nan_tail():
    w = synth.WORKLOADS["llama3_ragged_b8"].replace(max_ctx=4096, ctx_range=(2000, 4096), layers=2,
                                                    tie_frac=0.1)
    lens = synth.n_ctx(w)
    assert lens.shape == (8,) and lens.min() >= 2000 and lens.max() <= 4096
    x = synth.layer_inputs(w, 1, tie_info=True)
    for b in range(w.batch):
        n = int(lens[b])
        kf = synth.bf16_bits_to_f32(x["k"][b, 0])
        assert np.all(np.isnan(kf[n:])) and np.all(np.isfinite(kf[:n]))
        hh = synth.heavy_positions(w, b, 0, n)
        assert hh.size == round(0.01 * n)
        grp = x["ties"][(b, 0)]
        assert grp.shape[1] == 8 and grp.shape[0] > 0
        assert not np.intersect1d(grp.ravel(), hh).size
        for row in grp[:5]:
            assert np.all(x["k"][b, 0, row] == x["k"][b, 0, row[0]])
    # heavy-hitter positions are shared across layers
    assert np.array_equal(synth.heavy_positions(w, 3, 2, 3000), synth.heavy_positions(w, 3, 2, 3000))
