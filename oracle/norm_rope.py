"""Plain fp64 CPU oracle for the step that feeds the paged cache: per-head
RMSNorm of Q and K, rotary position embedding (RoPE), and the store of the
rotated K and the untouched V through ``slot_mapping``.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

Sources (the web pages this method is described on):

* "大模型推理入门与 nano-vLLM 源码详解" (duanmeng.github.io), cited [Intro §x]:
  §12.2 (Qwen3 normalises each Q and K head over its 128 features, then
  rotates Q and K by the tokens' real positions; V is neither normalised nor
  rotated), §19.3-19.4 (RMSNorm), §19.7 (RoPE: the pair rotation, the
  half-split pairing, rope_theta = 1e6, the cache holds rotated K).
* "nano-vllm 技术分析" (deepseek.csdn.net), cited [Analysis §4.x]: §4.2 (the
  q/k norm is applied when the projection has no bias), §4.4 (the frequency
  of pair i is one over theta to the power 2i/d).
* "Pico-vLLM 开发日志 #8 更多Triton Kernel和性能优化" on Fain's blog
  (koas-w.github.io), cited [Pico #8 §1]: the fused kernel rotates Q and K in
  registers, writes Q back contiguous, and writes rotated K and V straight
  into the paged cache through slot_mapping.

Everything is computed in float64 on the exact stored input values, following
the definitions; the only rounding of the product path this oracle does not
model is the final rounding to the storage type, which the tests bound.

Parity pins (tests marked "not gpu"): the RMSNorm example the pages print
(tests/golden/), scale invariance and unit mean square, the 90-degree pair
example, identity at position 0, the unit frequency of pair 0 and the
theta**-0.5 frequency of pair d/4, half-split (not adjacent) pairing, length
preservation, the relative-position property of rotated dot products,
norm-before-rope order, and the store's slot routing.  No function here is
"parity unpinned".
"""

from __future__ import annotations

import numpy as np

from .paged_attention import store, to_f64

__all__ = [
    "rms_norm",
    "rope_frequencies",
    "rotate_pair",
    "rope",
    "split_qkv",
    "qk_norm_rope",
    "qk_norm_rope_store",
]


def rms_norm(x: np.ndarray, weight: np.ndarray | None, eps: float) -> np.ndarray:
    """RMSNorm along the last axis [Intro §19.3].

    ``y_i = weight_i * x_i / sqrt(mean(x**2) + eps)``: the mean of squares is
    taken over the last axis only (for Q/K head norm, one head's features of
    one token [Intro §12.2, §19.3]); there is no mean subtraction and no bias.
    ``weight=None`` stands for all ones.
    """
    x = np.asarray(x, dtype=np.float64)
    mean_square = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(mean_square + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return y


def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """Angular frequency of each of the ``head_dim / 2`` pairs [Analysis §4.4].

    Pair ``i`` turns by ``omega_i = theta ** (-2 i / head_dim)`` radians per
    position, so pair 0 turns one radian per position and later pairs
    progressively slower [Intro §19.7].
    """
    assert head_dim % 2 == 0
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rotate_pair(a, b, phi):
    """Rotate the plane vector ``[a, b]`` by ``phi`` radians [Intro §19.7].

    ``a' = a cos(phi) - b sin(phi)``, ``b' = a sin(phi) + b cos(phi)``.
    """
    c, s = np.cos(phi), np.sin(phi)
    return a * c - b * s, a * s + b * c


def rope(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """Rotary embedding of ``x [T, H, d]`` at per-token ``positions [T]``.

    [Intro §19.7]: the head's features form ``d / 2`` pairs by halves --
    feature ``i`` pairs with feature ``i + d / 2`` -- and pair ``i`` of a token
    at position ``p`` is rotated by ``phi = p * omega_i`` with
    :func:`rope_frequencies`.  Every head of the token uses the same angles.
    """
    x = np.asarray(x, dtype=np.float64)
    t, h, d = x.shape
    half = d // 2
    pos = np.asarray(positions, dtype=np.float64).reshape(t, 1, 1)
    phi = pos * rope_frequencies(d, theta).reshape(1, 1, half)
    a, b = rotate_pair(x[..., :half], x[..., half:], phi)
    return np.concatenate([a, b], axis=-1)


def split_qkv(qkv: np.ndarray, num_q_heads: int, num_kv_heads: int, head_dim: int):
    """Split a fused projection row into Q, K, V heads [Analysis §4.2].

    Each token's row holds the Q heads, then the K heads, then the V heads,
    ``head_dim`` features each.
    """
    t = qkv.shape[0]
    q_size, kv_size = num_q_heads * head_dim, num_kv_heads * head_dim
    assert qkv.shape[1] >= q_size + 2 * kv_size
    q = qkv[:, :q_size].reshape(t, num_q_heads, head_dim)
    k = qkv[:, q_size:q_size + kv_size].reshape(t, num_kv_heads, head_dim)
    v = qkv[:, q_size + kv_size:q_size + 2 * kv_size].reshape(t, num_kv_heads, head_dim)
    return q, k, v


def qk_norm_rope(q, k, q_weight, k_weight, positions, eps: float, theta: float,
                 use_norm: bool = True):
    """Per-head RMSNorm of Q and K (when ``use_norm``), then RoPE of both.

    [Intro §12.2, §19.7]: the order is norm, then rotation; Q and K have their
    own norm weights; ``use_norm=False`` is the biased-projection model where
    no q/k norm exists [Analysis §4.2].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if use_norm:
        q = rms_norm(q, q_weight, eps)
        k = rms_norm(k, k_weight, eps)
    return rope(q, positions, theta), rope(k, positions, theta)


def qk_norm_rope_store(qkv_raw: np.ndarray, dtype: str, num_q_heads: int, num_kv_heads: int,
                       head_dim: int, q_weight_raw, k_weight_raw, positions, slot_mapping,
                       eps: float, theta: float, k_cache: np.ndarray, v_cache: np.ndarray):
    """The whole fused step [Pico #8 §1; Intro §12.2, §19.7].

    Inputs are raw stored bits (``dtype`` "bf16" or "f32"): ``qkv_raw [T, >=
    (Hq + 2 Hkv) d]``, weights ``[d]`` (both None: no q/k norm), caches
    ``[num_blocks, block_size, Hkv, d]``.  Returns ``(q_rot, k_rot, k_cache',
    v_cache')``: ``q_rot [T, Hq, d]`` and ``k_rot [T, Hkv, d]`` in float64, and
    the caches with rotated K (as float64) and the raw V bits written at each
    token's slot (-1: no write).  ``k_cache'`` is float64 (the cache widened,
    then the stored rows replaced); ``v_cache'`` stays raw bits, since V is
    copied unchanged.
    """
    if (q_weight_raw is None) != (k_weight_raw is None):
        raise ValueError("q and k norm weights are both given or both absent")
    q, k, v_raw = split_qkv(qkv_raw, num_q_heads, num_kv_heads, head_dim)
    use_norm = q_weight_raw is not None
    qw = to_f64(q_weight_raw, dtype) if use_norm else None
    kw = to_f64(k_weight_raw, dtype) if use_norm else None
    q_rot, k_rot = qk_norm_rope(to_f64(q, dtype), to_f64(k, dtype), qw, kw, positions, eps,
                                theta, use_norm)
    k_wide = to_f64(k_cache, dtype)
    k_out, v_out = store(k_wide, v_cache, k_rot, np.ascontiguousarray(v_raw), slot_mapping)
    return q_rot, k_rot, k_out, v_out
