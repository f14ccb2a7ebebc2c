"""Pins for the fp64 oracle: page worked examples, closed forms, invariants and
brute force.  CPU only.

Each test names the passage it follows.  The page titles are abbreviated:
[Intro] = "大模型推理入门与 nano-vLLM 源码详解"; [Log-walk] = "对着日志读懂 nano-vllm".
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def f32_raw(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def paged_pool_f32(rows, block_size, block_table, num_blocks):
    """Place per-position K (or V) rows [L, Hkv, d] into an fp32 raw pool via block_table.

    Built with plain indexing, not with the oracle, and NaN-poisoned elsewhere."""
    rows = np.asarray(rows, dtype=np.float32)
    pool = np.full((num_blocks, block_size) + rows.shape[1:], np.nan, dtype=np.float32)
    for j in range(rows.shape[0]):
        pool[block_table[j // block_size], j % block_size] = rows[j]
    return pool.view(np.uint32)


def tol(decimals):
    return 0.5 * 10.0 ** (-decimals) + 1e-12


# ----------------------------------------------------------------------------- worked examples

def test_single_head_weights_and_output_intro_s1_3():
    g = golden("intro_s1_3_single_head.json")
    q = np.array(g["q"], float)
    k = np.array(g["k"], float)
    v = np.array(g["v"], float)
    out, w = oracle.attend(q, k, v, g["scale"])
    assert np.all(np.abs(w - np.array(g["weights"])) <= tol(g["weights_decimals"]))
    assert abs(out[0] - g["output"][0]) <= tol(g["output_decimals"])


def test_single_head_through_paged_decode_intro_s1_3():
    """Same example, stored in a block-4... here block-2 pool at scattered blocks."""
    g = golden("intro_s1_3_single_head.json")
    bt = np.array([[5, 2]], np.int32)          # 3 positions over 2 blocks of size 2
    kc = paged_pool_f32(np.array(g["k"])[:, None, :], 2, bt[0], 6)
    vc = paged_pool_f32(np.array(g["v"])[:, None, :], 2, bt[0], 6)
    q = f32_raw(np.array(g["q"])[None, None, :])
    out = oracle.decode(q, kc, vc, bt, [3], g["scale"], "f32")
    assert abs(out[0, 0, 0] - g["output"][0]) <= tol(g["output_decimals"])


def test_softmax_intro_s19_1():
    g = golden("intro_s19_1_softmax.json")
    z = np.array(g["z"])
    assert np.all(np.abs(oracle.softmax(z) - g["softmax"]) <= tol(g["decimals"]))
    assert np.all(np.abs(np.exp(z - z.max()) - g["shifted_exp"]) <= tol(g["decimals"]))


def test_v_differs_example_intro_s18_2():
    g = golden("intro_s18_2_v_differs.json")
    k = np.array(g["k"])
    v = np.array(g["v"])
    scale = 1.0 / math.sqrt(2.0)
    out, w = oracle.attend(np.array(g["q_last"]), k, v, scale)
    assert np.all(np.abs(scale * (k @ np.array(g["q_last"])) - g["scaled_scores"])
                  <= tol(g["scores_decimals"]))
    assert np.all(np.abs(w - g["weights"]) <= tol(g["decimals"]))
    assert np.all(np.abs(out - g["output"]) <= tol(g["decimals"]))
    # the same numbers through the paged decode entry, blocks of 2 in reversed order
    bt = np.array([[1, 0]], np.int32)
    kc = paged_pool_f32(k[:, None, :], 2, bt[0], 2)
    vc = paged_pool_f32(v[:, None, :], 2, bt[0], 2)
    o = oracle.decode(f32_raw(np.array(g["q_last"])[None, None, :]), kc, vc, bt, [3], scale, "f32")
    assert np.all(np.abs(o[0, 0] - g["output"]) <= tol(g["decimals"]))


def test_causal_qkv_example_intro_s18_2():
    g = golden("intro_s18_2_causal_qkv.json")
    x = np.array(g["x"])
    scale = 1.0 / math.sqrt(2.0)
    bt = np.array([[0, 1]], np.int32)
    kc = paged_pool_f32(x[:, None, :], 2, bt[0], 2)
    out = oracle.prefill(f32_raw(x[:, None, :]), kc, kc, [0, 3], [0, 3], bt, scale, "f32")[:, 0, :]
    w_printed = np.array(g["weights"])
    # each printed weight is within half a unit of its last decimal; rows of V=X have |v|_1 <= 2
    assert np.all(np.abs(out - w_printed @ x) <= 2 * tol(g["weights_decimals"]))
    assert np.all(np.abs(out[-1] - g["last_output"]) <= tol(g["output_decimals"]))
    # weights sum to one on every row, and the first row reads only itself
    assert np.allclose(out[0], x[0], atol=0, rtol=0)


def test_masked_future_leaves_earlier_rows_unchanged_intro_s18_2():
    g = golden("intro_s18_2_causal_qkv.json")
    x = np.array(g["x"])
    x2 = x.copy()
    x2[-1] = g["future_change_last_row"]
    scale = 1.0 / math.sqrt(2.0)
    bt = np.array([[0, 1]], np.int32)
    outs = []
    for xx in (x, x2):
        kc = paged_pool_f32(xx[:, None, :], 2, bt[0], 2)
        outs.append(oracle.prefill(f32_raw(xx[:, None, :]), kc, kc, [0, 3], [0, 3], bt, scale,
                                   "f32"))
    delta = np.abs(outs[0][:2] - outs[1][:2]).max()
    assert delta == g["masked_earlier_delta"]
    assert np.abs(outs[0][2] - outs[1][2]).max() > 0


def test_merge_page_weights_intro_s9_5():
    g = golden("intro_s9_5_merge.json")
    l1, l2 = g["page_exp_sums"]
    # page 1 alone would output e0, page 2 alone e1: un-normalised accumulators l_s * e_s
    out = oracle.merge([0.0, 0.0], [l1, l2], [[l1, 0.0], [0.0, l2]])
    assert np.allclose(out, g["page_weights"], rtol=0, atol=1e-15)
    # the same sums expressed on different running maxima give the same weights
    out2 = oracle.merge([0.0, math.log(3.0)], [l1, l2 / 3.0], [[l1, 0.0], [0.0, l2 / 3.0]])
    assert np.allclose(out2, g["page_weights"], rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------- addresses

def test_slot_examples_intro_s9():
    g = golden("intro_s9_slots.json")
    for c in g["cases"]:
        bs, bt = c["block_size"], c["block_table"]
        if "positions" in c:
            got = [oracle.slot_of(bt, p, bs) for p in c["positions"]]
            assert got == c["slots"], c["where"]
        else:
            a, b = c["position_range"]
            got = [oracle.slot_of(bt, p, bs) for p in range(a, b)]
            assert got == list(range(*c["slot_range"])), c["where"]


def test_gather_reads_first_108_slots_of_tail_block_intro_s9_5():
    r = golden("intro_s9_slots.json")["read_620"]
    bs = r["block_size"]
    nb = max(r["block_table"]) + 1
    # every slot holds its own slot number, so the gathered rows name the slots read
    pool = np.arange(nb * bs, dtype=np.uint32).reshape(nb, bs, 1, 1)
    got = oracle.gather(pool, r["block_table"], r["length"]).reshape(-1)
    blocks, counts = np.unique(got // bs, return_counts=True)
    assert {str(b): int(c) for b, c in zip(blocks, counts)} == r["blocks_read"]
    assert np.all(got % bs == np.concatenate([np.arange(256), np.arange(256), np.arange(108)]))


def test_store_writes_slots_and_skips_padding_logwalk_s2_7():
    g = golden("logwalk_s2_7_metadata.json")
    bs = g["block_size"]
    nb, hkv, d = 2, 2, 3
    rng = np.random.default_rng(0)
    pool = np.full((nb, bs, hkv, d), 0x7FC0, np.uint16)
    slots = np.array(g["decode_slot_mapping"] + [-1], np.int32)       # one padding row
    k_new = rng.integers(0, 1 << 16, size=(3, hkv, d)).astype(np.uint16)
    v_new = rng.integers(0, 1 << 16, size=(3, hkv, d)).astype(np.uint16)
    kc, vc = oracle.store(pool, pool, k_new, v_new, slots)
    flat_k = kc.reshape(nb * bs, hkv, d)
    flat_v = vc.reshape(nb * bs, hkv, d)
    assert np.array_equal(flat_k[11], k_new[0]) and np.array_equal(flat_k[273], k_new[1])
    assert np.array_equal(flat_v[11], v_new[0]) and np.array_equal(flat_v[273], v_new[1])
    untouched = np.ones(nb * bs, bool)
    untouched[[11, 273]] = False
    assert np.all(flat_k[untouched] == 0x7FC0) and np.all(flat_v[untouched] == 0x7FC0)
    assert np.all(pool == 0x7FC0)                     # input not modified
    # the decode slots follow from the traced tables and positions
    for b, (pos, s) in enumerate(zip(g["decode_positions"], g["decode_slot_mapping"])):
        assert oracle.slot_of(g["block_tables"][b], pos, bs) == s
        assert g["decode_context_lens"][b] == pos + 1
    # prefill slots of the two sequences
    for b, (lo, hi) in enumerate(g["prefill_slot_mapping_ranges"]):
        got = [oracle.slot_of(g["block_tables"][b], p, bs) for p in range(g["prefill_lengths"][b])]
        assert got == list(range(lo, hi))


def test_store_rejects_repeated_slot():
    pool = np.zeros((2, 4, 1, 1), np.uint32)
    new = np.ones((2, 1, 1), np.uint32)
    with pytest.raises(ValueError):
        oracle.store(pool, pool, new, new, [3, 3])
    with pytest.raises(ValueError):
        oracle.store(pool, pool, new, new, [3, -2])


def test_store_is_raw_bit_copy():
    """NaN payloads and -0.0 survive the store bit for bit (a copy, not arithmetic)."""
    pool = np.zeros((1, 4, 1, 2), np.uint32)
    new = np.array([[[0x7FC00001, 0x80000000]]], np.uint32)
    kc, _ = oracle.store(pool, pool, new, new, [2])
    assert kc[0, 2, 0, 0] == 0x7FC00001 and kc[0, 2, 0, 1] == 0x80000000


# ----------------------------------------------------------------------------- invariants

def _rand_seq(rng, length, hkv, d):
    return (rng.standard_normal((length, hkv, d)).astype(np.float32),
            rng.standard_normal((length, hkv, d)).astype(np.float32))


def test_weights_sum_to_one_and_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    for length in (1, 2, 7, 50):
        k = rng.standard_normal((length, 5))
        v = rng.standard_normal((length, 5))
        out, w = oracle.attend(rng.standard_normal(5), k, v, 0.3)
        assert abs(w.sum() - 1.0) < 1e-14 and np.all(w >= 0)
        if length == 1:
            assert np.array_equal(out, v[0])


def test_paged_equals_contiguous_and_block_permutation_invariance():
    """Paged decode equals attention over a contiguous per-sequence cache (Pico-vLLM's
    naive cache), and relabelling physical blocks changes nothing, bit for bit."""
    rng = np.random.default_rng(2)
    bs, hq, hkv, d = 4, 4, 2, 8
    lengths = [1, 5, 12, 9]
    nb = sum(math.ceil(n / bs) for n in lengths) + 3
    perm = rng.permutation(nb)
    width = max(math.ceil(n / bs) for n in lengths)
    bt = np.full((len(lengths), width), -1, np.int32)
    kc = np.full((nb, bs, hkv, d), np.nan, np.float32)
    vc = kc.copy()
    contiguous = []
    cur = 0
    for b, n in enumerate(lengths):
        nblk = math.ceil(n / bs)
        bt[b, :nblk] = perm[cur:cur + nblk]
        cur += nblk
        k, v = _rand_seq(rng, n, hkv, d)
        contiguous.append((k, v))
        for j in range(n):
            kc[bt[b, j // bs], j % bs] = k[j]
            vc[bt[b, j // bs], j % bs] = v[j]
    q = rng.standard_normal((len(lengths), hq, d)).astype(np.float32)
    scale = 1 / math.sqrt(d)
    out = oracle.decode(q.view(np.uint32), kc.view(np.uint32), vc.view(np.uint32), bt, lengths,
                        scale, "f32")
    for b, (k, v) in enumerate(contiguous):
        for h in range(hq):
            g = h // (hq // hkv)
            ref, _ = oracle.attend(q[b, h].astype(float), k[:, g].astype(float),
                                   v[:, g].astype(float), scale)
            assert np.array_equal(out[b, h], ref)
    # relabel physical blocks: block p moves to sigma[p]
    sigma = rng.permutation(nb)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[sigma] = kc
    vc2[sigma] = vc
    bt2 = np.where(bt >= 0, sigma[np.maximum(bt, 0)], -1).astype(np.int32)
    out2 = oracle.decode(q.view(np.uint32), kc2.view(np.uint32), vc2.view(np.uint32), bt2,
                         lengths, scale, "f32")
    assert np.array_equal(out, out2)


def test_gqa_pairs_consecutive_query_heads_intro_s19_6():
    """Query heads 1,2 share kv head 1, 3,4 share kv head 2, ... (1-based on the page).

    Every value vector of kv head g is the constant g+1, so any weights give g+1."""
    bs, hq, hkv, d, n = 4, 16, 8, 4, 6
    rng = np.random.default_rng(3)
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    v = np.broadcast_to((np.arange(hkv) + 1.0)[None, :, None], (n, hkv, d)).astype(np.float32)
    bt = np.array([[1, 0]], np.int32)
    kc = paged_pool_f32(k, bs, bt[0], 2)
    vc = paged_pool_f32(v, bs, bt[0], 2)
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    out = oracle.decode(q.view(np.uint32), kc, vc, bt, [n], 0.5, "f32")
    expect = np.repeat(np.arange(hkv) + 1.0, hq // hkv)
    assert np.allclose(out[0, :, 0], expect, rtol=0, atol=1e-12)


def test_zero_context_gives_zero_output():
    kc = np.full((1, 4, 1, 2), 0x7FC00000, np.uint32)
    q = f32_raw(np.ones((2, 1, 2)))
    out = oracle.decode(q, kc, kc, np.array([[0], [-1]], np.int32), [1, 0], 1.0, "f32")
    assert np.all(np.isnan(out[0])) and np.array_equal(out[1], np.zeros((1, 2)))


def test_split_merge_equals_single_pass_and_identity():
    rng = np.random.default_rng(4)
    n, d = 37, 6
    k = rng.standard_normal((n, d)) * 3
    v = rng.standard_normal((n, d))
    q = rng.standard_normal(d)
    ref, _ = oracle.attend(q, k, v, 0.7)
    for bounds in ([(0, n)], [(0, 16), (16, 32), (32, n)], [(0, 1), (1, 1), (1, n), (n, n + 8)]):
        parts = oracle.split_partials(q, k, v, 0.7, bounds)
        out = oracle.merge([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
        assert np.allclose(out, ref, rtol=1e-13, atol=1e-14)
    m, l, acc = oracle.split_partials(q, k, v, 0.7, [(0, n)])[0]
    assert np.allclose(oracle.merge([m], [l], [acc]), acc / l, rtol=1e-15, atol=0)
    # all splits empty -> zeros
    parts = oracle.split_partials(q, k, v, 0.7, [(5, 5), (9, 9)])
    assert np.array_equal(oracle.merge([p[0] for p in parts], [p[1] for p in parts],
                                       [p[2] for p in parts]), np.zeros(d))


def _paged_fp32_case(rng, lengths, bs, hkv, d, extra_blocks=2):
    nb = sum(math.ceil(n / bs) for n in lengths) + extra_blocks
    perm = rng.permutation(nb)
    width = max(math.ceil(n / bs) for n in lengths)
    bt = np.full((len(lengths), width), -1, np.int32)
    kc = np.full((nb, bs, hkv, d), np.nan, np.float32)
    vc = kc.copy()
    cur = 0
    for b, n in enumerate(lengths):
        nblk = math.ceil(n / bs)
        bt[b, :nblk] = perm[cur:cur + nblk]
        cur += nblk
        k, v = _rand_seq(rng, n, hkv, d)
        for j in range(n):
            kc[bt[b, j // bs], j % bs] = k[j]
            vc[bt[b, j // bs], j % bs] = v[j]
    return kc.view(np.uint32), vc.view(np.uint32), bt


def test_prefill_equals_stepwise_decodes_intro_s3_4():
    """Prefill of positions c..L-1 equals one decode per position with context p+1
    (the cache-equivalence check of [Intro §15.2, §18.4])."""
    rng = np.random.default_rng(5)
    bs, hq, hkv, d = 4, 4, 2, 8
    lengths, cached = [9, 14, 3], [0, 8, 2]
    kc, vc, bt = _paged_fp32_case(rng, lengths, bs, hkv, d)
    q_lens = [n - c for n, c in zip(lengths, cached)]
    cu_q = np.concatenate([[0], np.cumsum(q_lens)])
    cu_k = np.concatenate([[0], np.cumsum(lengths)])
    q = rng.standard_normal((int(cu_q[-1]), hq, d)).astype(np.float32)
    scale = 0.35
    pre = oracle.prefill(q.view(np.uint32), kc, vc, cu_q, cu_k, bt, scale, "f32")
    for b, (n, c) in enumerate(zip(lengths, cached)):
        for i in range(n - c):
            row = cu_q[b] + i
            dec = oracle.decode(q[row:row + 1].view(np.uint32), kc, vc, bt[b:b + 1], [c + i + 1],
                                scale, "f32")
            assert np.allclose(pre[row], dec[0], rtol=1e-12, atol=1e-13)


def test_cached_prefix_prefill_equals_tail_of_full_prefill_intro_s10_2():
    g = golden("intro_s11_2_varlen.json")["prefix_hit"]
    rng = np.random.default_rng(6)
    bs, hq, hkv, d = 256, 2, 1, 4
    lk = g["cu_seqlens_k"][1]
    lq = g["cu_seqlens_q"][1]
    kc, vc, bt = _paged_fp32_case(rng, [lk], bs, hkv, d)
    q_full = rng.standard_normal((lk, hq, d)).astype(np.float32)
    full = oracle.prefill(q_full.view(np.uint32), kc, vc, [0, lk], [0, lk], bt, 0.5, "f32")
    part = oracle.prefill(q_full[lk - lq:].view(np.uint32), kc, vc, g["cu_seqlens_q"],
                          g["cu_seqlens_k"], bt, 0.5, "f32")
    assert np.allclose(part, full[lk - lq:], rtol=1e-12, atol=1e-13)


def test_first_new_query_sees_exactly_keys_up_to_its_position_intro_s11_2():
    """Round two of request A: 188 new queries over 700 keys; the first new query
    (position 512) reads keys 0..512 only, the last reads 0..699."""
    g = golden("intro_s11_2_varlen.json")["round_two"]
    rng = np.random.default_rng(7)
    bs, hq, hkv, d = 256, 1, 1, 2
    lengths = g["k_lens"]
    kc, vc, bt = _paged_fp32_case(rng, lengths, bs, hkv, d)
    q = rng.standard_normal((g["cu_seqlens_q"][-1], hq, d)).astype(np.float32)
    base = oracle.prefill(q.view(np.uint32), kc, vc, g["cu_seqlens_q"], g["cu_seqlens_k"], bt,
                          0.7, "f32")
    lo, hi = g["first_new_query_of_A_sees"]

    def perturbed(pos, seq=0):
        kc2 = kc.view(np.float32).copy()
        kc2[bt[seq, pos // bs], pos % bs] += 5.0
        return oracle.prefill(q.view(np.uint32), kc2.view(np.uint32), vc, g["cu_seqlens_q"],
                              g["cu_seqlens_k"], bt, 0.7, "f32")

    assert np.array_equal(perturbed(hi + 1)[0], base[0])        # key 513 is in the future
    assert not np.array_equal(perturbed(hi)[0], base[0])        # key 512 is visible
    assert not np.array_equal(perturbed(lengths[0] - 1)[187], base[187])
    # sequence B (rows 188..219) never sees A's keys
    assert np.array_equal(perturbed(5)[188:], base[188:])


# ----------------------------------------------------------------------------- brute force

def _brute_attention(q, keys, values, scale):
    """Scalar loops with math.exp, no NumPy reductions."""
    scores = []
    for j in range(len(keys)):
        s = 0.0
        for t in range(len(q)):
            s += float(q[t]) * float(keys[j][t])
        scores.append(scale * s)
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    tot = sum(e)
    return [sum(e[j] * float(values[j][t]) for j in range(len(keys))) / tot
            for t in range(len(q))]


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny_decode_and_prefill(seed):
    rng = np.random.default_rng(100 + seed)
    bs = int(rng.choice([1, 2, 4]))
    hkv = int(rng.integers(1, 3))
    hq = hkv * int(rng.integers(1, 3))
    d = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(1, 9, size=3)]
    kc, vc, bt = _paged_fp32_case(rng, lengths, bs, hkv, d)
    kf, vf = kc.view(np.float32), vc.view(np.float32)
    q = rng.standard_normal((3, hq, d)).astype(np.float32)
    scale = float(rng.uniform(0.1, 1.5))
    dec = oracle.decode(q.view(np.uint32), kc, vc, bt, lengths, scale, "f32")
    for b, n in enumerate(lengths):
        keys = [[kf[bt[b, j // bs], j % bs, h] for h in range(hkv)] for j in range(n)]
        vals = [[vf[bt[b, j // bs], j % bs, h] for h in range(hkv)] for j in range(n)]
        for h in range(hq):
            g = h // (hq // hkv)
            ref = _brute_attention(q[b, h], [r[g] for r in keys], [r[g] for r in vals], scale)
            assert np.allclose(dec[b, h], ref, rtol=1e-12, atol=1e-12)
    # prefill with a random cached prefix per sequence
    cached = [int(rng.integers(0, n)) for n in lengths]
    q_lens = [n - c for n, c in zip(lengths, cached)]
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    qp = rng.standard_normal((int(cu_q[-1]), hq, d)).astype(np.float32)
    pre = oracle.prefill(qp.view(np.uint32), kc, vc, cu_q, cu_k, bt, scale, "f32")
    for b, (n, c) in enumerate(zip(lengths, cached)):
        for i in range(n - c):
            p = c + i
            for h in range(hq):
                g = h // (hq // hkv)
                keys = [kf[bt[b, j // bs], j % bs, g] for j in range(p + 1)]
                vals = [vf[bt[b, j // bs], j % bs, g] for j in range(p + 1)]
                ref = _brute_attention(qp[cu_q[b] + i, h], keys, vals, scale)
                assert np.allclose(pre[cu_q[b] + i, h], ref, rtol=1e-12, atol=1e-12)


def test_bf16_widening_is_exact():
    """bf16 bits are the top half of binary32: 0x3F80 is 1.0, 0xC000 is -2.0, 0x3F81 is
    1 + 2^-7, 0x0001 is the smallest subnormal 2^-133, 0x7F80 is +inf."""
    raw = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80], np.uint16)
    got = oracle.to_f64(raw, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 1.0 + 2.0 ** -7
    assert got[3] == 2.0 ** -133 and got[4] == np.inf
