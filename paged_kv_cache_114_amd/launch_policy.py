"""Host-side launch policy: the split sizes a caller passes to the library.

The library takes the decode split size (``partition_tokens``) and the prefill
key-range size (``split_keys``) as arguments; an engine picks them from the
host-side sequence lengths it already holds.  These functions are that choice,
used by the benchmark and by the tests that check the benchmark's launches.
They do no attention arithmetic and need neither the GPU nor the library.
"""

from __future__ import annotations

import math

# Compute units of one MI355X.
CUS = 256


def decode_partition(num_seqs: int, num_kv_heads: int, max_context_len: int,
                     cus: int = CUS) -> int:
    """Decode split size in tokens.

    When (sequence, kv head) waves already give every SIMD four (16 per CU), one
    split per sequence.  Otherwise 512 tokens, long enough that the reduce is
    cheap, halved while there are fewer than 8 (sequence, kv head, split) waves
    per CU."""
    waves = num_seqs * num_kv_heads
    if waves >= 16 * cus:
        return 64 * max(1, math.ceil(max_context_len / 64))
    p = 512
    while p > 64 and waves * math.ceil(max(max_context_len, 1) / p) < 8 * cus:
        p //= 2
    return p


def prefill_rows_per_tile(num_q_heads: int, num_kv_heads: int) -> int:
    """Query positions per prefill work item (the library's tile height)."""
    group = num_q_heads // num_kv_heads
    return 32 * (1 if group >= 4 else 4 // group)


def prefill_split_keys(q_lens, context_lens, num_q_heads: int, num_kv_heads: int,
                       cus: int = CUS, wgs_per_cu: int = 2) -> int:
    """Keys per work item for long query tiles (0: no split).

    The prefill's workgroups take (query tile, kv head) items from a
    longest-first list, which balances a batch by itself once it has more
    items than workgroup slots; with fewer (one long sequence), long tiles are
    cut into key ranges of about 1.5x the mean key tiles per slot, so every
    slot gets work."""
    rows = prefill_rows_per_tile(num_q_heads, num_kv_heads)
    tiles = []
    for lq, lk in zip(q_lens, context_lens):
        lq, lk = int(lq), int(lk)
        for t in range(math.ceil(lq / rows)):
            tiles.append((lk - lq + min(lq, (t + 1) * rows) - 1) // 64 + 1)
    slots = cus * wgs_per_cu
    if not tiles or len(tiles) * num_kv_heads >= slots:
        return 0
    mean = num_kv_heads * sum(tiles) / slots
    keys = 64 * max(4, math.ceil(1.5 * mean))
    return 0 if keys >= 64 * max(tiles) else keys
