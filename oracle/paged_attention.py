"""Plain, slow, fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library; its only
inputs are arrays (NumPy) holding the raw stored bits of the caches and the
queries, plus plain integers.

Sources (the web pages this method is described on):

* "大模型推理入门与 nano-vLLM 源码详解" (duanmeng.github.io; an introduction to
  LLM inference with a nano-vLLM source walk), cited below as [Intro §x].
* "Pico-vLLM 开发日志 #6" on Fain's blog (koas-w.github.io), cited [Pico #6].
* "对着日志读懂 nano-vllm" (juejin.cn), cited [Log-walk §x].

What is computed, and why the oracle is the plain definition: paging changes
where K/V rows live, never the attention formula [Intro §9.5, §9.6].  So every
function here gathers a sequence's K/V rows through its block table into a
contiguous array and runs textbook softmax attention in float64 on the exact
stored values (bf16 and fp32 widen to float64 without rounding).

Parity pins: every function below is checked by tests marked "not gpu"
against worked examples printed on the pages (tests/golden/), closed forms,
invariants and brute-force loops.  No function here is "parity unpinned".

Storage convention: a cache is a raw-bit array shaped
``[num_blocks, block_size, num_kv_heads, head_dim]`` of ``np.uint16`` (bf16)
or ``np.uint32`` (fp32) -- the per-layer slice of the nano-vLLM pool
[Intro §11.5].  Queries and new K/V use the same raw-bit convention.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "RAW_TYPES",
    "to_f64",
    "slot_of",
    "store",
    "gather",
    "softmax",
    "attend",
    "decode",
    "prefill",
    "split_partials",
    "merge",
]

# Raw storage type for each element type the path supports.
RAW_TYPES = {"f32": np.uint32, "bf16": np.uint16}


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored bits to float64, exactly.

    bf16 is the upper half of an IEEE binary32 pattern, so shifting it left by
    16 bits gives the binary32 value it encodes; binary32 -> binary64 is exact.
    """
    raw = np.asarray(raw)
    if dtype == "bf16":
        assert raw.dtype == np.uint16
        return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        assert raw.dtype == np.uint32
        return raw.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def slot_of(block_table_row, position: int, block_size: int) -> int:
    """Write/read slot of a logical token position.

    [Intro §9.2]: the logical block is ``position // block_size``, the block
    table maps it to a physical block, and the slot is that physical block
    times ``block_size`` plus the offset ``position % block_size``.
    """
    physical = int(block_table_row[position // block_size])
    return physical * block_size + position % block_size


def store(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray,
          v_new: np.ndarray, slot_mapping) -> tuple[np.ndarray, np.ndarray]:
    """KV store through ``slot_mapping``; returns updated copies of both caches.

    [Intro §13.1]: token ``i`` of this step writes all of its kv heads' K (and
    V) vectors into slot ``slot_mapping[i]``; a slot of -1 marks a padding row
    and writes nothing.  The copy is of raw bits (no arithmetic), so NaN
    patterns round-trip too.  Slots must be unique and in range (a repeated
    slot has no defined winner on the pages; the oracle refuses it).
    """
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    assert v_cache.shape == k_cache.shape
    assert k_new.shape[1:] == k_cache.shape[2:] and v_new.shape == k_new.shape
    kc = k_cache.copy()
    vc = v_cache.copy()
    seen = set()
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s == -1:
            continue
        if s < 0 or s >= nb * bs or s in seen:
            raise ValueError(f"invalid or repeated slot {s} for token {i}")
        seen.add(s)
        kc[s // bs, s % bs] = k_new[i]
        vc[s // bs, s % bs] = v_new[i]
    return kc, vc


def gather(cache: np.ndarray, block_table_row, length: int) -> np.ndarray:
    """Rows ``0..length-1`` of one sequence, in logical order: ``[L, Hkv, d]``.

    Uses the same slot formula as the store [Intro §9.2]; only the first
    ``ceil(length / block_size)`` block-table entries are looked at, so -1
    padding after them is never touched [Intro §11.3].
    """
    bs = cache.shape[1]
    flat = cache.reshape(cache.shape[0] * bs, *cache.shape[2:])
    idx = np.array([slot_of(block_table_row, j, bs) for j in range(length)], dtype=np.int64)
    return flat[idx]


def softmax(scores: np.ndarray) -> np.ndarray:
    """Softmax along the last axis, max-subtracted [Intro §19.1]."""
    shifted = scores - scores.max(axis=-1, keepdims=True)
    e = np.exp(shifted)
    return e / e.sum(axis=-1, keepdims=True)


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """One query against ``L`` readable keys: returns ``(output [d], weights [L])``.

    [Intro §1.4, §9.5]: scores ``s_j = scale * q . k_j``, weights
    ``w = softmax(s)`` over all readable positions, output ``sum_j w_j v_j``.
    """
    scores = scale * (keys @ q)
    w = softmax(scores)
    return w @ values, w


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           block_table: np.ndarray, context_lens, scale: float, dtype: str) -> np.ndarray:
    """Batched single-token decode over the paged cache; float64 ``[B, Hq, d]``.

    * ``q``: raw ``[B, Hq, d]``; one new query per sequence.
    * ``context_lens[b]``: readable keys of sequence ``b``, including the token
      stored this step [Intro §11.4; Pico #6 on context_lens].
    * GQA: query head ``h`` reads kv head ``h // (Hq / Hkv)``; consecutive
      query heads share one kv head [Intro §19.6].
    * A sequence with ``context_len == 0`` (a padding row of a captured
      batch [Intro §13.5]) has no readable key; its output is defined here as
      zeros.
    """
    qf = to_f64(q, dtype)
    nseq, hq, d = qf.shape
    hkv = k_cache.shape[2]
    assert hq % hkv == 0
    group = hq // hkv
    out = np.zeros((nseq, hq, d), dtype=np.float64)
    for b in range(nseq):
        length = int(context_lens[b])
        if length == 0:
            continue
        keys = to_f64(gather(k_cache, block_table[b], length), dtype)
        vals = to_f64(gather(v_cache, block_table[b], length), dtype)
        for h in range(hq):
            g = h // group
            out[b, h], _ = attend(qf[b, h], keys[:, g, :], vals[:, g, :], scale)
    return out


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, cu_seqlens_q,
            cu_seqlens_k, block_table: np.ndarray, scale: float, dtype: str) -> np.ndarray:
    """Variable-length causal prefill over the paged cache; float64 ``[Tq, Hq, d]``.

    Sequence ``b`` owns query rows ``cu_q[b]..cu_q[b+1]-1`` (``Lq`` rows) and
    ``Lk = cu_k[b+1]-cu_k[b]`` readable keys, all read from the paged pool
    through its block table [Intro §9.5, §13.2].  When a prefix of
    ``c = Lk - Lq`` tokens is cached, the first new query sits at position
    ``c`` and sees keys ``0..c``; query row ``i`` sees keys ``0..c+i``
    [Intro §10.2, §11.2] (a causal mask aligned to the bottom-right).

    Written in matrix form per (sequence, head): full score matrix, future
    positions set to -inf before the softmax [Intro §19.1, §18.2], then
    weights times V.
    """
    qf = to_f64(q, dtype)
    tq, hq, d = qf.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    out = np.zeros((tq, hq, d), dtype=np.float64)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    for b in range(len(cu_q) - 1):
        lq = int(cu_q[b + 1] - cu_q[b])
        lk = int(cu_k[b + 1] - cu_k[b])
        if lq == 0:
            continue
        c = lk - lq
        assert c >= 0, "a sequence cannot have more new queries than readable keys"
        keys = to_f64(gather(k_cache, block_table[b], lk), dtype)
        vals = to_f64(gather(v_cache, block_table[b], lk), dtype)
        pos_q = c + np.arange(lq)[:, None]
        pos_k = np.arange(lk)[None, :]
        future = pos_k > pos_q
        for h in range(hq):
            g = h // group
            scores = scale * (qf[cu_q[b]:cu_q[b + 1], h, :] @ keys[:, g, :].T)
            scores = np.where(future, -np.inf, scores)
            out[cu_q[b]:cu_q[b + 1], h] = softmax(scores) @ vals[:, g, :]
    return out


def split_partials(q_vec: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
                   bounds):
    """Per-split statistics of one query: list of ``(m_s, l_s, acc_s)``.

    [Intro §9.5, §13.3]: a split over key positions ``[a, b)`` keeps its own
    running maximum ``m_s``, exponential sum ``l_s = sum exp(s_j - m_s)`` and
    un-normalised output ``acc_s = sum exp(s_j - m_s) v_j``.  An empty split
    has ``m = -inf, l = 0, acc = 0``; a split reaching past the last key
    stops there (its positions beyond the context are not readable).
    """
    scores = scale * (keys @ q_vec)
    parts = []
    for a, b in bounds:
        b = min(b, len(scores))
        if b <= a:
            parts.append((-np.inf, 0.0, np.zeros(values.shape[1])))
            continue
        s = scores[a:b]
        m = s.max()
        e = np.exp(s - m)
        parts.append((m, e.sum(), e @ values[a:b]))
    return parts


def merge(ms, ls, accs) -> np.ndarray:
    """Combine split statistics into one normalised output [Intro §9.5].

    Splits are weighted by their exponential sums rescaled to a common
    maximum ``m* = max m_s``: ``o = sum_s acc_s e^{m_s-m*} / sum_s l_s e^{m_s-m*}``.
    Summing per-split *normalised* outputs would be wrong (each would weigh 1).
    If every split is empty the output is zeros (no readable key).
    """
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    accs = np.asarray(accs, dtype=np.float64)
    m_star = ms.max()
    if not np.isfinite(m_star):
        return np.zeros(accs.shape[-1])
    w = np.exp(ms - m_star)
    return (w @ accs) / (w @ ls)
