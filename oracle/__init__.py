"""Reference oracle for the hybrid-head decode-attention step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``; never by the product package.  It shares
no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation); this module
only marshals numpy arrays and chains layers.

Sources: the long-form digest "LycheeDecode: Accelerating Long-Context LLM
Inference via Hybrid-Head Sparse Decoding" (paper-graph-ui), section 3.4:
Eq. 1 (retrieval-head attention), Eq. 2 (argsTopK -> next layer's S), Eq. 3
(sparse-head attention over S), the rule that a sparse head forwards S
unchanged, the layer-0 all-retrieval rule, Algorithm 1 (the decoding loop) and
the hyper-parameter summary (GQA: queries average-pooled before selection).

Pins (the tests that hold the oracle to something other than itself; all in
``tests/test_oracle_pins.py`` unless noted):
  * hand-derived worked examples with closed-form outputs and S sets
    (``tests/golden/*.json``): scale 1/sqrt(d), exact softmax weights,
    GQA pooling of logits (not of probabilities), tie-break, propagation;
  * identical keys -> output = mean of V rows, S = {0..k-1};
  * planted dominant key -> selected and output within 2(n-1)e^-gap max|V|
    of its V row;
  * brute force over all C(n,k) subsets (max score-sum, then lexicographically
    smallest index tuple) for n <= 12 with integer scores full of ties;
  * sparse head with S = all positions equals the retrieval head's output;
  * masked-softmax identity: sparse output equals the dense output after the
    keys outside S are pushed to -inf logit by a planted direction;
  * invariants: constant V rows reproduce the constant; each output lies in
    the per-coordinate hull of V; logit shift and row permutation
    (in)variance; sparse S_out == S_in bitwise; an all-sparse chain returns
    the layer-0 S bitwise;
  * selection rules (reading R16 of oracle.c): Ratio equals top-k at
    k' = ceil(theta n); Threshold matches pooled scores computed in plain
    loops and reduces to top-k / the empty set at tau = -inf / +inf; Top-p
    over identical keys keeps ceil(p n) tokens, over a two-level score
    profile keeps the closed-form count of heavy tokens, keeps the argmax
    alone for a tiny p and equals top-k at p = 1; a sparse head skips -1
    padding and outputs zeros for an empty set;
  * block selection (reading R17): blocks of one token are top-k; planted
    heavy tokens pick their blocks in closed form, ties between blocks go
    to the lower block; a short last block and k covering every block list
    all tokens;
  * the multi-step loop (reading R18): the append writes exactly the new
    rows and grows n by one (bytes compared, the rest untouched, a full
    cache refused); the correction attention with T = 1 equals the layer's
    dense retrieval output, over identical keys gives the mean of the V
    prefix 0..p, ignores rows after p and not rows up to p, and matches
    torch's scaled_dot_product_attention with an explicit causal mask in
    float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

ERRORS = {
    -1: "invalid argument",
    -2: "S_in entry outside [0, n_ctx)",
    -3: "n_ctx outside [1, max_ctx]",
    -4: "out of host memory",
}


def build() -> str:
    """Compile oracle.c into liboracle.so (plain gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           _SRC, "-o", _LIB_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_layer.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, p, p, i, p, i]
        lib.oracle_layer.restype = i
        lib.oracle_layer_select.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, p, p, i, i, ctypes.c_double, p, i]
        lib.oracle_layer_select.restype = i
        lib.oracle_kv_append.argtypes = [i, i, i, i, i, p, p, p, p, p]
        lib.oracle_kv_append.restype = i
        lib.oracle_correction_attention.argtypes = [i, i, i, i, i, i, i, p, p, p, p, p, i]
        lib.oracle_correction_attention.restype = i
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:          # bfloat16 bit patterns
        return 1
    raise TypeError(f"oracle takes float32 or bf16-as-uint16 arrays, got {a.dtype}")


RULES = {"topk": 0, "ratio": 1, "threshold": 2, "topp": 3, "block": 4}


def layer(q, k_cache, v_cache, role, S_in, n_ctx, k, *, want_scores=False,
          threads=0, rule="topk", param=0.0):
    """One layer.  Returns (out[B,Hq,d] float64, S_out[B,Hkv,k] int32, scores).

    ``rule`` selects S (reading R16 of oracle.c): "topk" (the top min(k, n)),
    "ratio" (the top min(k, ceil(param * n)), param in (0, 1]) or
    "threshold" (the tokens with pooled score >= param, the k highest if
    more), "topp" (the shortest prefix of the ranking whose softmax share
    of the pooled scores reaches param in (0, 1], the k highest if longer)
    or "block" (blocks of param tokens scored by their largest pooled score,
    the floor(k / param) highest kept, reading R17); S rows are ascending
    and padded with -1, and a sparse head skips -1 entries.

    q: [B,Hq,d]; k_cache, v_cache: [B,Hkv,max_ctx,d] (float32, or uint16
    holding bfloat16 bits); role: [Hkv] (1 retrieval / 0 sparse); S_in:
    [B,Hkv,k] int32 or None (legal only when every role is 1); n_ctx: [B].
    ``scores`` is [B,Hkv,max_ctx] float64 with the pooled selection score of
    every retrieval head (NaN elsewhere) when ``want_scores``, else None.
    """
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    dt = _dtype_code(q)
    if _dtype_code(k_cache) != dt or _dtype_code(v_cache) != dt:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    B, Hq, d = q.shape
    _, Hkv, max_ctx, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or k_cache.shape[0] != B:
        raise ValueError("shape mismatch")
    role = np.ascontiguousarray(np.asarray(role, dtype=np.uint8))
    n_ctx = np.ascontiguousarray(np.asarray(n_ctx, dtype=np.int32))
    if S_in is not None:
        S_in = np.ascontiguousarray(np.asarray(S_in, dtype=np.int32))
        if S_in.shape != (B, Hkv, k):
            raise ValueError("S_in shape")
    out = np.zeros((B, Hq, d), dtype=np.float64)
    S_out = np.full((B, Hkv, k), -1, dtype=np.int32)
    scores = np.full((B, Hkv, max_ctx), np.nan, dtype=np.float64) if want_scores else None
    rc = _load().oracle_layer_select(B, Hq, Hkv, d, max_ctx, dt, _ptr(q), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(role), _ptr(S_in), _ptr(S_out),
                                     _ptr(out), _ptr(n_ctx), int(k), RULES[rule], float(param),
                                     _ptr(scores), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_layer: {ERRORS.get(rc, rc)}")
    return out, S_out, scores


def kv_append(k_new, v_new, k_cache, v_cache, n_ctx):
    """Algorithm 1's cache append (reading R18 of oracle.c), in place: row
    n_ctx[b] of each KV head receives k_new / v_new [B, Hkv, d]; returns the
    new n_ctx (a copy, each entry one larger)."""
    k_new = np.ascontiguousarray(k_new)
    v_new = np.ascontiguousarray(v_new)
    dt = _dtype_code(k_cache)
    if _dtype_code(k_new) != dt or _dtype_code(v_new) != dt or _dtype_code(v_cache) != dt:
        raise TypeError("one dtype for the new rows and the caches")
    if not (k_cache.flags.c_contiguous and v_cache.flags.c_contiguous):
        raise ValueError("caches must be contiguous (appended in place)")
    B, Hkv, max_ctx, d = k_cache.shape
    if k_new.shape != (B, Hkv, d) or v_new.shape != (B, Hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    n = np.array(n_ctx, dtype=np.int32, copy=True)
    rc = _load().oracle_kv_append(B, Hkv, d, max_ctx, dt, _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(n))
    if rc != 0:
        raise ValueError(f"oracle_kv_append: {ERRORS.get(rc, rc)}")
    return n


def correction_attention(q, k_cache, v_cache, n_ctx, *, threads=0):
    """Cache Correction's attention (reading R18 of oracle.c): q [B, T, Hq, d]
    holds the last T positions' queries; returns out [B, T, Hq, d] float64,
    row t attending causally to cache rows 0 .. n_ctx[b] - T + t."""
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    dt = _dtype_code(q)
    if _dtype_code(k_cache) != dt or _dtype_code(v_cache) != dt:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    B, T, Hq, d = q.shape
    _, Hkv, max_ctx, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape or k_cache.shape[0] != B:
        raise ValueError("shape mismatch")
    n_ctx = np.ascontiguousarray(np.asarray(n_ctx, dtype=np.int32))
    out = np.zeros((B, T, Hq, d), dtype=np.float64)
    rc = _load().oracle_correction_attention(B, T, Hq, Hkv, d, max_ctx, dt, _ptr(q), _ptr(k_cache),
                                             _ptr(v_cache), _ptr(n_ctx), _ptr(out), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_correction_attention: {ERRORS.get(rc, rc)}")
    return out


def step(layers, n_ctx, k, *, threads=0):
    """Chain a whole decode step (Algorithm 1, attention part).

    ``layers`` is a sequence of (q, k_cache, v_cache, role) per layer; layer 0
    must be all-retrieval.  Returns (list of outputs, list of S after each
    layer).
    """
    S = None
    outs, Ss = [], []
    for l, (q, kc, vc, role) in enumerate(layers):
        if l == 0 and not np.all(np.asarray(role) == 1):
            raise ValueError("layer 0 must be all retrieval")
        out, S, _ = layer(q, kc, vc, role, S, n_ctx, k, threads=threads)
        outs.append(out)
        Ss.append(S)
    return outs, Ss
