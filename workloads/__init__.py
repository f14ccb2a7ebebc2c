"""Seeded synthetic inputs for the paged-attention path.

Shared by the tests (both the oracle side and the HIP side), the smoke check
and the benchmark.  This module draws lengths, block placements and values
and lays them out the way an engine's model runner hands them to the
attention layer; it performs none of the attention arithmetic.

Shapes follow the workloads the pages describe (Qwen3-0.6B: 16 query heads,
8 kv heads, head_dim 128; nano-vLLM's engine limits of 16384 batched tokens,
512 sequences and 4096-token contexts).  The pages benchmark on 256 random-
length requests with no public dataset; these seeded draws stand in for it.

Recipe (fixed draw order per case):

1. integers: lengths and the shared or cached choices from
   ``numpy.random.default_rng(seed)``; then, from ``default_rng([seed, 1])``,
   a random permutation of the pool's physical block ids, dealt out in
   sequence order (shared prefix blocks first);
2. values from a ``torch.Generator`` seeded with the same seed on the device
   the tensors are made on: the whole pool, then the new tokens' K and V, then
   the queries, each ``N(0, 1)`` in float32 and rounded to the storage type
   (round-to-nearest-even for bf16);
3. every pool slot that holds no readable, already-stored token -- unused
   blocks, the unused tail of each last block, and the slots the new tokens
   will be written to -- is overwritten with a quiet-NaN bit pattern, so a
   kernel that reads outside a sequence's context, or skips a store, shows up.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

POISON_BITS = {"bf16": 0x7FC0, "f32": 0x7FC00000}


@dataclass
class Case:
    """Metadata of one synthetic workload (values are made by :func:`materialize`)."""

    name: str
    kind: str                    # "decode" or "prefill"
    dtype: str                   # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int              # physical blocks in the pool
    seed: int
    block_table: np.ndarray      # int32 [B, W], -1 past each sequence's blocks
    context_lens: np.ndarray     # int32 [B]: readable keys incl. this step's tokens
    num_cached: np.ndarray       # int32 [B]: tokens already stored before this step
    slot_mapping: np.ndarray     # int32 [T]: write slot of each new token (-1: padding)
    new_seq: np.ndarray          # int32 [T]: owning sequence of each new token (-1: padding)
    new_pos: np.ndarray          # int32 [T]: logical position of each new token
    shared_blocks: int = 0       # physical blocks shared by several sequences
    notes: dict = field(default_factory=dict)
    # prefix-cache groups: sequence b shares the first prefix_tokens[g] positions
    # (whole blocks, the same physical ids) with every sequence of group
    # g = prefix_group[b]; -1: no group
    prefix_group: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    prefix_tokens: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_new_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_dim), as the float32 the kernels receive."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    # prefill views (decode cases have one new token per live sequence)
    @property
    def q_lens(self) -> np.ndarray:
        return (self.context_lens - self.num_cached).astype(np.int32)

    @property
    def cu_seqlens_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def cu_seqlens_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.context_lens)]).astype(np.int32)

    @property
    def max_seqlen_q(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def elt_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def kv_bytes_logical(self) -> int:
        """K and V bytes every sequence reads for its whole context."""
        row = self.num_kv_heads * self.head_dim * self.elt_bytes
        return int(2 * row * int(self.context_lens.astype(np.int64).sum()))

    def kv_bytes_unique(self) -> int:
        """K and V bytes of distinct readable slots (shared prefix counted once)."""
        row = self.num_kv_heads * self.head_dim * self.elt_bytes
        return int(2 * row * len(self.readable_slots()))

    def readable_slots(self) -> np.ndarray:
        """Distinct pool slots that some sequence reads this step."""
        bs = self.block_size
        out = []
        for b in range(self.num_seqs):
            n = int(self.context_lens[b])
            pos = np.arange(n)
            out.append(self.block_table[b, pos // bs].astype(np.int64) * bs + pos % bs)
        return np.unique(np.concatenate(out)) if out else np.zeros(0, np.int64)

    def stored_slots(self) -> np.ndarray:
        """Slots holding tokens stored before this step (positions < num_cached)."""
        bs = self.block_size
        out = []
        for b in range(self.num_seqs):
            n = int(self.num_cached[b])
            pos = np.arange(n)
            out.append(self.block_table[b, pos // bs].astype(np.int64) * bs + pos % bs)
        return np.unique(np.concatenate(out)) if out else np.zeros(0, np.int64)

    def causal_pairs(self) -> int:
        """(query, key) pairs a causal prefill visits: sum over rows of visible keys."""
        total = 0
        for lq, lk in zip(self.q_lens.tolist(), self.context_lens.tolist()):
            c = lk - lq
            total += lq * (c + 1) + lq * (lq - 1) // 2
        return int(total)


def _place_blocks(rng, blocks_per_seq, groups, pool=None, pool_factor=1.25):
    """Random physical placement: returns (block_table, pool size).

    ``groups`` lists (shared block count, member sequences).  The pool holds
    ``pool`` blocks (default: 1.25x the blocks needed, rounded up); a random
    permutation of its ids is dealt out: each group's shared blocks first, then
    every sequence's own blocks in sequence order, a member's row starting with
    its group's shared blocks."""
    needed = sum(n for n, _ in groups) + int(sum(blocks_per_seq))
    if pool is None:
        pool = max(1, math.ceil(pool_factor * needed))
    assert pool >= needed
    perm = rng.permutation(pool).astype(np.int32)
    cursor = 0
    front = {}
    for n, members in groups:
        for b in members:
            assert b not in front, "a sequence belongs to one group at most"
            front[b] = perm[cursor:cursor + n]
        cursor += n
    nseq = len(blocks_per_seq)
    rows = []
    for b in range(nseq):
        own = perm[cursor:cursor + blocks_per_seq[b]]
        cursor += blocks_per_seq[b]
        rows.append(np.concatenate([front[b], own]) if b in front else own)
    width = max(1, max(len(r) for r in rows))
    table = np.full((nseq, width), -1, dtype=np.int32)
    for b, r in enumerate(rows):
        table[b, :len(r)] = r
    return table, pool


def _slots(table_row, positions, bs):
    positions = np.asarray(positions, dtype=np.int64)
    return (table_row[positions // bs].astype(np.int64) * bs + positions % bs).astype(np.int32)


def _finish(name, kind, dtype, hq, hkv, d, bs, seed, lengths, cached, shared_prefix_tokens=0,
            shared_seqs=(), pad_rows=0, notes=None, pool=None, prefix_groups=None):
    rng_place = np.random.default_rng([seed, 1])
    if prefix_groups is None:
        prefix_groups = [(shared_prefix_tokens, list(shared_seqs))] if shared_prefix_tokens and \
            len(shared_seqs) else []
    lengths = np.asarray(lengths, dtype=np.int64)
    cached = np.asarray(cached, dtype=np.int64)
    nseq = len(lengths)
    if len(cached) != nseq or np.any(cached < 0) or np.any(cached > lengths) or \
            (kind == "prefill" and np.any(cached >= lengths)):
        raise ValueError(f"{name}: cached positions must lie in [0, length) (prefill) or "
                         f"[0, length] (decode)")
    groups = [(int(tokens) // bs, [int(b) for b in members]) for tokens, members in prefix_groups]
    prefix_group = np.full(nseq, -1, np.int32)
    for g, (n, members) in enumerate(groups):
        for b in members:
            if n * bs > lengths[b]:
                raise ValueError(f"{name}: sequence {b} is shorter than its shared prefix")
            prefix_group[b] = g
    per_seq = []
    for b in range(nseq):
        total = math.ceil(int(lengths[b]) / bs)
        per_seq.append(total - (groups[prefix_group[b]][0] if prefix_group[b] >= 0 else 0))
    table, pool = _place_blocks(rng_place, per_seq, groups, pool)
    slots, seqs, poss = [], [], []
    for b in range(nseq):
        pos = np.arange(int(cached[b]), int(lengths[b]))
        slots.append(_slots(table[b], pos, bs))
        seqs.append(np.full(len(pos), b, np.int32))
        poss.append(pos.astype(np.int32))
    if pad_rows:
        table = np.concatenate([table, np.full((pad_rows, table.shape[1]), -1, np.int32)])
        lengths = np.concatenate([lengths, np.zeros(pad_rows, np.int64)])
        cached = np.concatenate([cached, np.zeros(pad_rows, np.int64)])
        prefix_group = np.concatenate([prefix_group, np.full(pad_rows, -1, np.int32)])
        slots.append(np.full(pad_rows, -1, np.int32))
        seqs.append(np.full(pad_rows, -1, np.int32))
        poss.append(np.zeros(pad_rows, np.int32))
    return Case(
        name=name, kind=kind, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=bs, num_blocks=pool, seed=seed, block_table=table,
        context_lens=lengths.astype(np.int32), num_cached=cached.astype(np.int32),
        slot_mapping=np.concatenate(slots).astype(np.int32),
        new_seq=np.concatenate(seqs).astype(np.int32),
        new_pos=np.concatenate(poss).astype(np.int32),
        shared_blocks=sum(n for n, _ in groups), notes=dict(notes or {}),
        prefix_group=prefix_group,
        prefix_tokens=np.array([n * bs for n, _ in groups], np.int32))


def decode_case(name, seed, *, lengths, hq=16, hkv=8, d=128, dtype="bf16", bs=256,
                shared_prefix_tokens=0, shared_seqs=(), pad_rows=0, notes=None,
                pool=None, prefix_groups=None) -> Case:
    """A decode step: each sequence stores its newest token (position L-1), then reads L keys.
    ``prefix_groups``: (prefix tokens, member sequences) pairs; members share the physical
    blocks of their group's first prefix tokens (rounded down to whole blocks)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cached = np.maximum(lengths - 1, 0)
    return _finish(name, "decode", dtype, hq, hkv, d, bs, seed, lengths, cached,
                   shared_prefix_tokens, shared_seqs, pad_rows, notes, pool, prefix_groups)


def prefill_case(name, seed, *, lengths, cached, hq=16, hkv=8, d=128, dtype="bf16",
                 bs=256, notes=None) -> Case:
    """A prefill step: sequence b stores positions cached[b]..L-1, then attends causally."""
    return _finish(name, "prefill", dtype, hq, hkv, d, bs, seed, lengths, cached, notes=notes)


# --------------------------------------------------------------------------------------
# The five workloads, and scaled-down twins the oracle finishes in seconds.
# --------------------------------------------------------------------------------------

def c1_tiny_decode() -> Case:
    """1 sequence, context 37, 2 query heads / 1 kv head, d=64, fp32, block 16, pool of 8."""
    return decode_case("c1_tiny_decode", 1141, lengths=[37], hq=2, hkv=1, d=64,
                       dtype="f32", bs=16, pool=8)


def c2_decode(batch=64, seed=1142, name="c2_decode_b64", bs=256) -> Case:
    """Qwen3-0.6B one-layer decode: contexts uniform in [128, 1024], block 256 (or ``bs``)."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(128, 1024, size=batch, endpoint=True)
    return decode_case(name, seed, lengths=lengths, bs=bs)


def _prefill_lengths(rng, nseq, lo, hi, n_cached, cached_choices):
    while True:
        lengths = rng.integers(lo, hi, size=nseq, endpoint=True)
        eligible = np.flatnonzero(lengths > min(cached_choices))
        if len(eligible) >= n_cached:
            break
    chosen = rng.choice(eligible, size=n_cached, replace=False)
    cached = np.zeros(nseq, dtype=np.int64)
    for b in chosen:
        options = [c for c in cached_choices if c < lengths[b]]
        cached[b] = options[int(rng.integers(0, len(options)))]
    return lengths, cached


def c3_prefill(nseq=8, lo=64, hi=2048, n_cached=3, seed=1143, name="c3_prefill_8seq") -> Case:
    """Varlen causal prefill: lengths uniform in [64, 2048]; 3 sequences have 256 or 512
    block-aligned cached tokens (drawn among sequences longer than the choice)."""
    rng = np.random.default_rng(seed)
    lengths, cached = _prefill_lengths(rng, nseq, lo, hi, n_cached, (256, 512))
    return prefill_case(name, seed, lengths=lengths, cached=cached)


def c4_heavy_decode(batch=512, ctx=4096, seed=1144, name="c4_heavy_decode_b512") -> Case:
    """512 sequences, every context 4096, block 256: the bandwidth-roofline decode."""
    return decode_case(name, seed, lengths=np.full(batch, ctx))


def c5_shared_prefix_decode(batch=256, n_shared=192, prefix=2048, tail_median=300.0,
                            tail_sigma=1.0, tail_cap=6000, private_lo=32, private_hi=8192,
                            seed=1145, name="c5_shared_prefix_b256") -> Case:
    """Block 16; 3/4 of sequences share the physical blocks of a common 2048-token prefix
    then a private lognormal tail (median 300, capped at 6000); the rest are private with
    lengths uniform in [32, 8192]."""
    rng = np.random.default_rng(seed)
    shared = np.sort(rng.permutation(batch)[:n_shared])
    tails = np.clip(np.rint(rng.lognormal(math.log(tail_median), tail_sigma, size=batch)),
                    1, tail_cap).astype(np.int64)
    private = rng.integers(private_lo, private_hi, size=batch, endpoint=True)
    shared_set = set(shared.tolist())
    lengths = np.array([prefix + tails[b] if b in shared_set else private[b]
                        for b in range(batch)], dtype=np.int64)
    return decode_case(name, seed, lengths=lengths, bs=16, shared_prefix_tokens=prefix,
                       shared_seqs=shared.tolist())


def mixed_batch(n_decode=48, n_chunks=4, chunk=512, n_fresh=2, seed=1146,
                name="mixed_chunked_b54") -> Case:
    """One engine step with chunked prefill, through the varlen prefill call: n_decode
    sequences decoding one token (contexts U[128, 1024], Lq = 1), n_chunks long
    prompts continuing by one chunk of `chunk` positions after a cached prefix
    U[100, 1500] that is generally not block aligned, and n_fresh new prompts
    U[64, 700].  Qwen3-0.6B head shapes, block 256."""
    rng = np.random.default_rng(seed)
    dec = rng.integers(128, 1024, size=n_decode, endpoint=True)
    cached_chunks = rng.integers(100, 1500, size=n_chunks, endpoint=True)
    fresh = rng.integers(64, 700, size=n_fresh, endpoint=True)
    lengths = np.concatenate([dec, cached_chunks + chunk, fresh])
    cached = np.concatenate([dec - 1, cached_chunks, np.zeros(n_fresh, np.int64)])
    return prefill_case(name, seed, lengths=lengths, cached=cached,
                        notes={"rows": "decode rows (Lq=1), chunked-prefill continuations, fresh prompts"})


def balanced_prefill(nseq=8, length=2048, seed=1147, name="prefill_8x2048") -> Case:
    """A balanced varlen prefill: nseq fresh prompts of one length (Qwen3-0.6B head
    shapes, block 256); the steady-state case of the tile loop."""
    return prefill_case(name, seed, lengths=np.full(nseq, length),
                        cached=np.zeros(nseq, np.int64))


FULL_CASES = {
    "c1": c1_tiny_decode,
    "c2": c2_decode,
    "c3": c3_prefill,
    "c4": c4_heavy_decode,
    "c5": c5_shared_prefix_decode,
    "mixed": mixed_batch,
    "p8x2048": balanced_prefill,
}

# Scaled-down twins: same head shapes, block sizes and length laws, several
# tiles each and ragged tails, small enough for the oracle to finish in seconds.
SMALL_CASES = {
    "c1": c1_tiny_decode,
    "c2s": lambda: c2_decode(batch=6, seed=2142, name="c2s_decode_b6"),
    "c3s": lambda: c3_prefill(nseq=4, lo=64, hi=700, n_cached=2, seed=2143,
                              name="c3s_prefill_4seq"),
    "c4s": lambda: c4_heavy_decode(batch=2, ctx=4096, seed=2144, name="c4s_decode_b2"),
    "c5s": lambda: c5_shared_prefix_decode(batch=12, n_shared=9, prefix=512, tail_cap=1500,
                                           private_hi=2048, seed=2145,
                                           name="c5s_shared_prefix_b12"),
    "mixeds": lambda: mixed_batch(n_decode=10, n_chunks=3, chunk=200, n_fresh=2, seed=2146,
                                  name="mixeds_chunked_b15"),
}


# --------------------------------------------------------------------------------------
# Values
# --------------------------------------------------------------------------------------

def _torch_dtype(dtype):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def _raw_view(t, dtype):
    import torch
    return t.view(torch.int16 if dtype == "bf16" else torch.int32)


def materialize(case: Case, device="cpu", chunk_blocks=None) -> dict:
    """Draw the values of ``case`` on ``device``; returns a dict of torch tensors.

    Keys: ``k_cache, v_cache`` ``[NB, bs, Hkv, d]`` (readable already-stored
    tokens hold values, every other slot holds the NaN poison), ``k_new,
    v_new`` ``[T, Hkv, d]`` (this step's tokens, to be stored), ``q``
    ``[T, Hq, d]`` (decode: one row per sequence), and the int32 metadata
    ``block_table, context_lens, slot_mapping, cu_seqlens_q, cu_seqlens_k``.
    """
    import torch
    dev = torch.device(device)
    tdt = _torch_dtype(case.dtype)
    gen = torch.Generator(device=dev)
    gen.manual_seed(case.seed)
    nb, bs, hkv, d = case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim
    shape = (nb, bs, hkv, d)
    if chunk_blocks is None:
        chunk_blocks = max(1, (256 << 20) // (bs * hkv * d))
    caches = []
    for _ in range(2):
        cache = torch.empty(shape, dtype=tdt, device=dev)
        for lo in range(0, nb, chunk_blocks):
            hi = min(nb, lo + chunk_blocks)
            cache[lo:hi] = torch.randn((hi - lo, bs, hkv, d), generator=gen, device=dev,
                                       dtype=torch.float32).to(tdt)
        caches.append(cache)
    t = case.num_new_tokens
    k_new = torch.randn((t, hkv, d), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    v_new = torch.randn((t, hkv, d), generator=gen, device=dev, dtype=torch.float32).to(tdt)
    q = torch.randn((t, case.num_q_heads, d), generator=gen, device=dev,
                    dtype=torch.float32).to(tdt)
    keep = np.zeros(nb * bs, dtype=bool)
    keep[case.stored_slots()] = True
    poison_idx = torch.from_numpy(np.flatnonzero(~keep)).to(dev)
    for cache in caches:
        raw = _raw_view(cache, case.dtype).view(nb * bs, hkv * d)
        raw.index_fill_(0, poison_idx, _signed(POISON_BITS[case.dtype], case.dtype))
    i32 = dict(dtype=torch.int32, device=dev)
    return {
        "k_cache": caches[0], "v_cache": caches[1], "k_new": k_new, "v_new": v_new, "q": q,
        "block_table": torch.tensor(case.block_table, **i32),
        "context_lens": torch.tensor(case.context_lens, **i32),
        "slot_mapping": torch.tensor(case.slot_mapping, **i32),
        "cu_seqlens_q": torch.tensor(case.cu_seqlens_q, **i32),
        "cu_seqlens_k": torch.tensor(case.cu_seqlens_k, **i32),
        "prefix_group": torch.tensor(case.prefix_group, **i32),
        "prefix_tokens": torch.tensor(case.prefix_tokens, **i32),
    }


def _signed(bits, dtype):
    width = 16 if dtype == "bf16" else 32
    return bits - (1 << width) if bits >= 1 << (width - 1) else bits


def raw_numpy(t, dtype) -> np.ndarray:
    """Raw stored bits of a torch tensor as NumPy (uint16 for bf16, uint32 for fp32)."""
    r = _raw_view(t.detach().contiguous(), dtype).cpu().numpy()
    return r.view(np.uint16 if dtype == "bf16" else np.uint32)


def from_raw(raw: np.ndarray, dtype, device="cpu"):
    """Torch tensor of the given storage type holding exactly the raw bits."""
    import torch
    signed = raw.view(np.int16 if dtype == "bf16" else np.int32)
    t = torch.from_numpy(np.ascontiguousarray(signed)).to(device)
    return t.view(_torch_dtype(dtype))


def projection_inputs(case: Case, device="cpu", row_pad=0) -> dict:
    """Draw the fused projection rows and q/k norm weights of ``case``'s new tokens.

    The input of the norm + rotary + store step: ``qkv`` ``[T, (Hq + 2 Hkv) d
    + row_pad]`` (Q heads, then K, then V, as a fused projection writes them;
    ``row_pad`` extra columns widen the row stride) with entries ``N(0, 1)``
    rounded to the storage type, and ``q_norm_weight, k_norm_weight`` ``[d]``
    uniform in [0.25, 2] (positive per-feature gains around one, as learned
    norm weights are), all from a ``torch.Generator`` seeded with
    ``case.seed + 7919`` on ``device`` in that order; ``positions`` are the new
    tokens' logical positions and ``slot_mapping`` their write slots (int32).
    """
    import torch
    dev = torch.device(device)
    tdt = _torch_dtype(case.dtype)
    gen = torch.Generator(device=dev)
    gen.manual_seed(case.seed + 7919)
    hq, hkv, d = case.num_q_heads, case.num_kv_heads, case.head_dim
    t = case.num_new_tokens
    width = (hq + 2 * hkv) * d
    qkv = torch.randn((t, width + row_pad), generator=gen, device=dev,
                      dtype=torch.float32).to(tdt)
    qw = (0.25 + 1.75 * torch.rand((d,), generator=gen, device=dev, dtype=torch.float32)).to(tdt)
    kw = (0.25 + 1.75 * torch.rand((d,), generator=gen, device=dev, dtype=torch.float32)).to(tdt)
    i32 = dict(dtype=torch.int32, device=dev)
    return {
        "qkv": qkv[:, :width] if row_pad else qkv,
        "q_norm_weight": qw, "k_norm_weight": kw,
        "positions": torch.tensor(case.new_pos, **i32),
        "slot_mapping": torch.tensor(case.slot_mapping, **i32),
    }
