"""Seeded synthetic inputs for the hybrid-head decode-attention step.

This module is shared by the oracle side (tests) and the HIP side (tests,
benchmark).  It draws random numbers and lays out tensors; it computes no
attention, softmax or selection.  Every array is a pure function of
(workload, layer, seed).

Workloads mirror the shapes the pages evaluate: Llama3-8B / Qwen3-8B-like
attention (32 query heads over 8 KV heads, head dim 128, bf16 KV cache,
16K-128K context, batch 1-8, k = 1024/2048/4096 critical tokens), plus two
tiny fp32 cases the oracle finishes in milliseconds.  The pages' datasets are
not used; these inputs only stand in for the attention shapes and the score
structure (heavy-hitter keys, exact ties, ragged lengths).

Recipe (per workload, per layer l):
  * RNG: numpy PCG64, one independent stream per (seed, layer, stream id,
    batch row, KV head); stream ids 0 q, 1 K, 2 V, 3 heavy-hitter positions
    (drawn with layer = 65535, so shared by every layer), 4 heavy-hitter
    noise, 5 tie groups, 6 roles, 7 ragged lengths.
  * q, K, V are drawn as float32 normals; q and K are scaled by 1/sqrt(d)
    when ``qk_scaled`` (the Llama/Qwen-like workloads), V stays N(0,1).
    bf16 workloads round to bfloat16 with round-to-nearest-even.
  * Heavy hitters: round(hh_frac * n_b) positions per (b, KV head), the same
    positions in every layer; their key is 4 * qbar/|qbar| + N(0,1)/sqrt(d),
    qbar being the mean of the group's query rows of that layer.
  * Tie groups: tie_frac of the remaining positions are split into groups of
    8; each member's K row is a bit-copy of the group's first member.
  * Rows at or beyond n_b hold NaN (they must never be read).
  * Roles: layer 0 is all retrieval; ``n_retrieval`` (layer, KV head) slots of
    layers 1..L-1 are drawn without replacement and made retrieval.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_HH_POS, STREAM_HH_NOISE, STREAM_TIES, STREAM_ROLES, STREAM_LEN = range(8)
SHARED_LAYER = 65535
BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    max_ctx: int
    k: int
    dtype: str                     # "f32" or "bf16"
    n_retrieval: int               # retrieval (layer, KV head) slots over layers 1..L-1
    ctx_range: tuple | None = None  # (lo, hi) inclusive for ragged batches, else n = max_ctx
    qk_scaled: bool = True         # q, K ~ N(0,1)/sqrt(d) when True, N(0,1) when False
    hh_frac: float = 0.0
    tie_frac: float = 0.0
    ctx_list: tuple | None = None   # explicit per-sequence contexts (edge cases)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny GQA 4:1 step, fp32, 2 layers: layer 1 has 1 retrieval KV head of 2
    "tiny_gqa": Workload("tiny_gqa", 1, 1, 2, 8, 2, 64, 2048, 128, "f32", 1, qk_scaled=False),
    # the same sizes in MHA form (G = 1): layer 1 has 2 retrieval heads of 8
    "tiny_mha": Workload("tiny_mha", 11, 1, 2, 8, 8, 64, 2048, 128, "f32", 2, qk_scaled=False),
    # Llama3-8B attention shape, 32 layers, 32K context, k = 4096
    "llama3_32k": Workload("llama3_32k", 2, 1, 32, 32, 8, 128, 32768, 4096, "bf16", 25, hh_frac=0.01),
    # the same at 128K context (the headline workload)
    "llama3_128k": Workload("llama3_128k", 3, 1, 32, 32, 8, 128, 131072, 4096, "bf16", 25, hh_frac=0.01),
    # batch 8, ragged contexts U{32768..65536}, k = 2048
    "llama3_ragged_b8": Workload("llama3_ragged_b8", 4, 8, 32, 32, 8, 128, 65536, 2048, "bf16", 25,
                                 ctx_range=(32768, 65536), hh_frac=0.01),
    # Qwen3-8B attention shape, 36 layers, 128K context, 5% retrieval, ties
    "qwen3_128k_k1024": Workload("qwen3_128k_k1024", 5, 1, 36, 32, 8, 128, 131072, 1024, "bf16", 14,
                                 hh_frac=0.005, tie_frac=0.10),
    "qwen3_128k_k4096": Workload("qwen3_128k_k4096", 5, 1, 36, 32, 8, 128, 131072, 4096, "bf16", 14,
                                 hh_frac=0.005, tie_frac=0.10),
}


def _rng(w: Workload, layer: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([w.seed, layer, stream, *extra])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def n_ctx(w: Workload) -> np.ndarray:
    if w.ctx_list is not None:
        assert len(w.ctx_list) == w.batch and max(w.ctx_list) <= w.max_ctx
        return np.asarray(w.ctx_list, dtype=np.int32)
    if w.ctx_range is None:
        return np.full(w.batch, w.max_ctx, dtype=np.int32)
    lo, hi = w.ctx_range
    return _rng(w, SHARED_LAYER, STREAM_LEN).integers(lo, hi + 1, size=w.batch).astype(np.int32)


def roles(w: Workload) -> np.ndarray:
    """[L, Hkv] uint8, 1 = retrieval.  Layer 0 is all retrieval."""
    r = np.zeros((w.layers, w.n_kv_heads), dtype=np.uint8)
    r[0, :] = 1
    slots = (w.layers - 1) * w.n_kv_heads
    if slots and w.n_retrieval:
        pick = _rng(w, SHARED_LAYER, STREAM_ROLES).choice(slots, size=w.n_retrieval, replace=False)
        r[1 + pick // w.n_kv_heads, pick % w.n_kv_heads] = 1
    return r


def heavy_positions(w: Workload, b: int, g: int, n: int) -> np.ndarray:
    cnt = int(round(w.hh_frac * n))
    if cnt == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(w, SHARED_LAYER, STREAM_HH_POS, b, g).choice(n, size=cnt, replace=False))


def tie_groups(w: Workload, layer: int, b: int, g: int, n: int, exclude: np.ndarray) -> np.ndarray:
    """[n_groups, 8] positions; member 0 is the source row of each group."""
    if w.tie_frac <= 0.0:
        return np.zeros((0, 8), dtype=np.int64)
    mask = np.ones(n, dtype=bool)
    mask[exclude] = False
    rest = np.nonzero(mask)[0]
    n_groups = int(round(w.tie_frac * rest.size)) // 8
    pick = _rng(w, layer, STREAM_TIES, b, g).choice(rest, size=n_groups * 8, replace=False)
    return pick.reshape(n_groups, 8)


def _normal(rng, shape, scale):
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def layer_inputs(w: Workload, layer: int, threads: int | None = None,
                 tie_info: bool = False):
    """Inputs of one layer.

    Returns dict(q [B,Hq,d], k [B,Hkv,max_ctx,d], v [B,Hkv,max_ctx,d]) as
    float32 arrays (f32 workloads) or uint16 bfloat16 bit patterns (bf16),
    plus ``ties`` = {(b,g): [groups,8] positions} when ``tie_info``.
    """
    B, Hq, Hkv, d, M = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_ctx
    G = w.group
    bf16 = w.dtype == "bf16"
    qk_scale = 1.0 / np.sqrt(d) if w.qk_scaled else 1.0
    store = np.uint16 if bf16 else np.float32
    lens = n_ctx(w)

    q32 = np.empty((B, Hq, d), dtype=np.float32)
    for b in range(B):
        for g in range(Hkv):
            q32[b, g * G:(g + 1) * G] = _normal(_rng(w, layer, STREAM_Q, b, g), (G, d), qk_scale)
    kc = np.empty((B, Hkv, M, d), dtype=store)
    vc = np.empty((B, Hkv, M, d), dtype=store)
    ties = {}

    def one(bg):
        b, g = divmod(bg, Hkv)
        n = int(lens[b])
        kf = _normal(_rng(w, layer, STREAM_K, b, g), (n, d), qk_scale)
        hh = heavy_positions(w, b, g, n)
        if hh.size:
            qbar = q32[b, g * G:(g + 1) * G].mean(axis=0)
            direction = (4.0 / np.linalg.norm(qbar)) * qbar
            noise = _normal(_rng(w, layer, STREAM_HH_NOISE, b, g), (hh.size, d), 1.0 / np.sqrt(d))
            kf[hh] = direction.astype(np.float32)[None, :] + noise
        grp = tie_groups(w, layer, b, g, n, hh)
        if grp.size:
            kf[grp[:, 1:]] = kf[grp[:, :1]]
        if tie_info:
            ties[(b, g)] = grp
        vf = _normal(_rng(w, layer, STREAM_V, b, g), (n, d), 1.0)
        if bf16:
            kc[b, g, :n] = to_bf16_bits(kf)
            vc[b, g, :n] = to_bf16_bits(vf)
            kc[b, g, n:] = BF16_NAN
            vc[b, g, n:] = BF16_NAN
        else:
            kc[b, g, :n] = kf
            vc[b, g, :n] = vf
            kc[b, g, n:] = np.nan
            vc[b, g, n:] = np.nan

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads <= 1 or B * Hkv == 1:
        for bg in range(B * Hkv):
            one(bg)
    else:
        with _cf.ThreadPoolExecutor(max_workers=nthreads) as ex:
            list(ex.map(one, range(B * Hkv)))
    q = to_bf16_bits(q32) if bf16 else q32
    res = {"q": q, "k": kc, "v": vc}
    if tie_info:
        res["ties"] = ties
    return res
