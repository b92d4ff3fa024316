"""Comparison rules between the HIP path and the oracle (test-side only).

Tolerances (stated for the method's parity bar):
  * outputs: max |out_gpu - out_oracle| <= 2e-2 for a bf16 KV cache and
    <= 1e-4 for fp32, per layer;
  * S: the GPU set must equal the oracle set except at positions whose oracle
    pooled score lies within 1e-3 (relative) of the oracle's k-th score;
  * exact ties: inside a group of bit-identical K rows every member has the
    same score on both sides, so where such a group straddles the boundary
    the selected members must be the lowest-indexed ones (checked exactly);
  * S rows are ascending, duplicate-free, inside [0, n), padded with -1.
The oracle receives the same S_in as the GPU (the GPU's S_out of the previous
layer), so a tolerated boundary swap upstream cannot move a downstream
sparse-head output.
"""
from __future__ import annotations

import numpy as np

import oracle

OUT_TOL = {"f32": 1e-4, "bf16": 2e-2}
BAND_REL = 1e-3


def check_S_row(S_gpu_row, n, k):
    ke = min(k, n)
    row = np.asarray(S_gpu_row)
    assert row.shape == (k,)
    assert np.all(row[ke:] == -1), "padding"
    sel = row[:ke]
    assert np.all(sel >= 0) and np.all(sel < n), "range"
    assert np.all(np.diff(sel) > 0), "ascending, no duplicates"
    return sel


def compare_S(S_gpu, S_or, scores, role, n_ctx, k, ties=None):
    """Returns the number of band positions that differ (informational)."""
    B, Hkv, _ = S_gpu.shape
    band_diffs = 0
    for b in range(B):
        n = int(n_ctx[b])
        ke = min(k, n)
        for g in range(Hkv):
            A = check_S_row(S_gpu[b, g], n, k)
            if not role[g]:
                continue
            O = S_or[b, g, :ke]
            s = scores[b, g, :n]
            s_k = s[O].min()
            tol = BAND_REL * abs(s_k) if abs(s_k) >= 1e-6 else 1e-9
            band = np.abs(s - s_k) <= tol
            a_set = set(A.tolist())
            o_set = set(O.tolist())
            a_out = {j for j in a_set if not band[j]}
            o_out = {j for j in o_set if not band[j]}
            assert a_out == o_out, f"S mismatch outside the band at b={b} g={g}: " \
                                   f"gpu-only {sorted(a_out - o_out)[:8]} oracle-only {sorted(o_out - a_out)[:8]}"
            band_diffs += len(a_set ^ o_set)
            if ties is not None and (b, g) in ties:
                for grp in ties[(b, g)]:
                    members = np.sort(np.asarray(grp))
                    picked = np.array([m in a_set for m in members])
                    cnt = int(picked.sum())
                    if 0 < cnt < members.size:
                        assert np.all(picked[:cnt]) and not np.any(picked[cnt:]), \
                            f"tie group {members.tolist()} at b={b} g={g}: not the lowest indices"
    return band_diffs


def compare_layer(out_gpu, S_gpu, inputs, role, S_in, n_ctx, k, dtype, ties=None, threads=0):
    """Run the oracle on the same inputs and S_in; assert the parity bar."""
    out_or, S_or, scores = oracle.layer(inputs["q"], inputs["k"], inputs["v"], role, S_in, n_ctx, k,
                                        want_scores=True, threads=threads)
    err = np.abs(out_gpu.astype(np.float64) - out_or)
    assert np.all(np.isfinite(out_gpu)), "non-finite output"
    assert err.max() <= OUT_TOL[dtype], f"max |out err| {err.max():.3e} > {OUT_TOL[dtype]}"
    for b in range(S_gpu.shape[0]):
        for g in range(S_gpu.shape[1]):
            if not role[g]:
                np.testing.assert_array_equal(S_gpu[b, g], S_in[b, g], err_msg="sparse head must forward S")
    band = compare_S(S_gpu, S_or, scores, role, n_ctx, k, ties)
    return float(err.max()), band
