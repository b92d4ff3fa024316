"""The parity bar can fail where it must (CPU only).

At the 128K shape a retrieval head's output is the mean of ~131072 V rows
weighted by a nearly flat softmax, of size ~1/sqrt(n): the absolute 2e-2 bar
of the bf16 outputs passes an all-zero output and a split merge that loses a
group of partial records.  The normalised bound (tests/parity.py) must reject
both.  The mistakes are planted in oracle-side outputs: the oracle run over
the whole context against the oracle run over the context with the rows of
one merge group (1/32 of the head) left out."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import OUT_REL, OUT_TOL, check_relative


def _one_head(n: int):
    w = synth.Workload("bar_128k", 123, 1, 1, 4, 1, 128, n, 64, "bf16", 0, hh_frac=0.01)
    return w, synth.layer_inputs(w, 0, threads=8)


def test_normalised_bound_rejects_zero_output_and_a_dropped_record_group():
    n = 131072
    w, x = _one_head(n)
    role = np.ones(1, np.uint8)
    full, _, _ = oracle.layer(x["q"], x["k"], x["v"], role, None, np.array([n], np.int32), 64, threads=8)
    cut = n // 32
    part = {key: (np.ascontiguousarray(x[key][:, :, cut:]) if key in ("k", "v") else x[key]) for key in x}
    dropped, _, _ = oracle.layer(part["q"], part["k"], part["v"], role, None, np.array([n - cut], np.int32), 64,
                                 threads=8)
    zero = np.zeros_like(full)
    # the absolute bar alone passes both mistakes at this size ...
    assert np.abs(full).max() < OUT_TOL["bf16"]
    assert np.abs(dropped - full).max() <= OUT_TOL["bf16"]
    # ... the normalised bound rejects them
    with pytest.raises(AssertionError):
        check_relative(zero, full, 4)
    with pytest.raises(AssertionError):
        check_relative(dropped, full, 4)
    # and accepts an error at the level fp32 arithmetic leaves (1e-6 relative)
    rng = np.random.default_rng(5)
    noisy = full * (1.0 + 1e-6 * rng.standard_normal(full.shape))
    assert check_relative(noisy, full, 4) < OUT_REL


def test_normalised_bound_blocks_are_kv_heads():
    """A wrong output in one KV head's block fails even when another block's
    outputs are far larger."""
    o = np.zeros((1, 8, 4))
    o[0, :4] = 100.0                 # KV head 0 (G = 4): large outputs
    o[0, 4:] = 1e-3                  # KV head 1: small outputs
    bad = o.copy()
    bad[0, 5, 0] += 1e-4             # 10% of head 1's scale, 1e-6 of head 0's
    with pytest.raises(AssertionError):
        check_relative(bad, o, 4)
    assert check_relative(o, o, 4) == 0.0
    # an exactly-zero block (an empty set) must stay exactly zero
    z = o.copy()
    z[0, 4:] = 0.0
    zb = z.copy()
    zb[0, 6, 1] = 1e-12
    with pytest.raises(AssertionError):
        check_relative(zb, z, 4)
