"""Host-side checks of the seeded input generators (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_varlen_metadata_matches_round_two_example():
    """cu_seqlens of [Intro §11.2]: A has 188 new of 700 keys, B 32 of 32."""
    with open(os.path.join(GOLDEN, "intro_s11_2_varlen.json"), encoding="utf-8") as f:
        g = json.load(f)["round_two"]
    case = W.prefill_case("t", 1, lengths=g["k_lens"], cached=[512, 0], hq=2, hkv=1, d=4)
    assert case.cu_seqlens_q.tolist() == g["cu_seqlens_q"]
    assert case.cu_seqlens_k.tolist() == g["cu_seqlens_k"]
    assert case.max_seqlen_q == g["max_seqlen_q"] and case.max_context_len == g["max_seqlen_k"]
    # slot_mapping lists the new positions in input order, through each block table
    bt = case.block_table
    want = [oracle.slot_of(bt[0], p, 256) for p in range(512, 700)] + \
           [oracle.slot_of(bt[1], p, 256) for p in range(32)]
    assert case.slot_mapping.tolist() == want


@pytest.mark.parametrize("name", sorted(W.FULL_CASES))
def test_full_cases_are_consistent(name):
    case = W.FULL_CASES[name]()
    bs = case.block_size
    assert case.block_table.max() < case.num_blocks
    nblk = -(-case.context_lens // bs)
    for b in range(case.num_seqs):
        row = case.block_table[b]
        assert np.all(row[:nblk[b]] >= 0) and np.all(row[nblk[b]:] == -1)
    # new-token slots are unique, unwritten and readable by their own sequence
    slots = case.slot_mapping[case.slot_mapping >= 0]
    assert len(np.unique(slots)) == len(slots)
    assert not np.isin(slots, case.stored_slots()).any()
    assert np.isin(slots, case.readable_slots()).all()
    if case.kind == "decode":
        assert case.num_new_tokens == case.num_seqs
        assert np.array_equal(case.new_pos, case.context_lens - 1)


def test_config_shapes():
    c1 = W.c1_tiny_decode()
    assert (c1.num_blocks, c1.block_size, c1.head_dim, c1.dtype) == (8, 16, 64, "f32")
    assert c1.context_lens.tolist() == [37] and c1.block_table.shape == (1, 3)
    c2 = W.c2_decode()
    assert c2.num_seqs == 64 and c2.context_lens.min() >= 128 and c2.context_lens.max() <= 1024
    c3 = W.c3_prefill()
    assert c3.num_seqs == 8 and int(c3.q_lens.sum()) <= 16384
    assert sorted(c3.num_cached[c3.num_cached > 0].tolist()) in (
        [256, 256, 256], [256, 256, 512], [256, 512, 512], [512, 512, 512])
    c4 = W.c4_heavy_decode()
    assert c4.kv_bytes_logical() == 512 * 4096 * 4096
    c5 = W.c5_shared_prefix_decode()
    shared_rows = [b for b in range(256) if np.array_equal(
        c5.block_table[b, :128], c5.block_table[c5.block_table[:, 0] == c5.block_table[b, 0]][0, :128])]
    assert c5.shared_blocks == 128 and c5.block_size == 16
    assert c5.kv_bytes_unique() < c5.kv_bytes_logical()
    assert len(shared_rows) >= 192


def test_prefix_groups_share_exactly_their_prefix_blocks():
    """prefix_group / prefix_tokens describe the placement: members of a group hold the
    same physical ids in their first prefix_tokens / block_size entries, and no block
    is shared outside a group's prefix."""
    c5 = W.c5_shared_prefix_decode()
    assert c5.prefix_tokens.tolist() == [2048]
    members = np.flatnonzero(c5.prefix_group == 0)
    assert len(members) == 192 and np.all(c5.prefix_group[c5.prefix_group != 0] == -1)
    first = c5.block_table[members[0], :128]
    assert all(np.array_equal(c5.block_table[b, :128], first) for b in members)
    case = W.decode_case("groups", 77, bs=16, lengths=[100, 40, 300, 64, 64, 90, 5],
                         prefix_groups=[(32, [0, 2, 4]), (64, [3, 5])])
    assert case.prefix_group.tolist() == [0, -1, 0, 1, 0, 1, -1]
    assert case.prefix_tokens.tolist() == [32, 64]
    owners = {}
    for b in range(case.num_seqs):
        n = -(-int(case.context_lens[b]) // case.block_size)
        for j, blk in enumerate(case.block_table[b, :n].tolist()):
            owners.setdefault(blk, set()).add((b, j))
    for blk, uses in owners.items():
        if len(uses) > 1:  # shared: same column, within one group's prefix
            seqs = {b for b, _ in uses}
            cols = {j for _, j in uses}
            groups = {int(case.prefix_group[b]) for b in seqs}
            assert len(cols) == 1 and len(groups) == 1 and -1 not in groups
            g = groups.pop()
            assert next(iter(cols)) < case.prefix_tokens[g] // case.block_size
    with pytest.raises(ValueError):
        W.decode_case("short", 78, bs=16, lengths=[20, 40], prefix_groups=[(32, [0, 1])])


def test_materialize_poisons_everything_but_stored_tokens():
    case = W.SMALL_CASES["c5s"]()
    vals = W.materialize(case, "cpu")
    raw = W.raw_numpy(vals["k_cache"], case.dtype).reshape(case.num_blocks * case.block_size, -1)
    poisoned = np.all(raw == W.POISON_BITS[case.dtype], axis=1)
    stored = np.zeros(len(raw), bool)
    stored[case.stored_slots()] = True
    assert np.array_equal(~poisoned, stored)
    # the new tokens' slots start poisoned: the store must fill them
    assert poisoned[case.slot_mapping].all()
    # seeded: drawing again gives the same bits
    again = W.materialize(case, "cpu")
    for k in ("k_cache", "v_cache", "q", "k_new", "v_new"):
        assert np.array_equal(W.raw_numpy(vals[k], case.dtype), W.raw_numpy(again[k], case.dtype))


def test_raw_round_trip():
    x = np.array([0x7FC0, 0x8000, 0x3F80, 0x0001], np.uint16)
    t = W.from_raw(x, "bf16")
    assert np.array_equal(W.raw_numpy(t, "bf16"), x)
