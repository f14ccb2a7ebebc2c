"""pa_decode + pa_decode_reduce on the GPU against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from pa_runner import (DEV, HostInputs, assert_close, decode_buffers, default_partition,
                       run_decode, run_store, sample_seqs, timed_partition, to_f64)

import paged_kv_cache_114_amd as pa

pytestmark = pytest.mark.gpu


def _decode_vs_oracle(case, partition_tokens, seqs=None):
    print(f"decode case={case.name} B={case.num_seqs} P={partition_tokens} "
          f"max_ctx={case.max_context_len}", flush=True)
    vals = W.materialize(case, DEV)
    host = HostInputs(case, vals, seqs)
    run_store(vals)
    out, ws, splits = run_decode(case, vals, partition_tokens)
    torch.cuda.synchronize()
    ref = host.decode()
    got = to_f64(out, case.dtype)[host.seqs]
    return assert_close(got, ref, case.dtype, case.name)


@pytest.mark.parametrize("name", ["c1", "c2s", "c4s", "c5s"])
@pytest.mark.parametrize("partition", [64, 512, None])
def test_decode_small_cases(name, partition):
    case = W.SMALL_CASES[name]()
    _decode_vs_oracle(case, partition or default_partition(case))


@pytest.mark.parametrize("policy", ["timed", "default"])
def test_decode_c2_full_all_sequences(policy):
    """Every sequence of the batch-64 workload, at the split size bench.py times
    (256 tokens) and at the tests' other split policy (128)."""
    case = W.c2_decode()
    p = timed_partition(case) if policy == "timed" else default_partition(case)
    _decode_vs_oracle(case, p)


@pytest.mark.parametrize("name", ["c4", "c5"])
@pytest.mark.parametrize("policy", ["timed", "default"])
def test_decode_full_size_sampled(name, policy):
    """Full-size pools at the split size bench.py times (C4: one split of 4096
    tokens; C5: 512-token splits) and at the tests' other policy; the oracle checks a
    spread of sequences (longest, shortest, random), all heads."""
    case = W.FULL_CASES[name]()
    p = timed_partition(case) if policy == "timed" else default_partition(case)
    _decode_vs_oracle(case, p, seqs=sample_seqs(case, 10, seed=1))


@pytest.mark.parametrize("hq,hkv,d,dtype,bs", [
    (8, 8, 128, "bf16", 256),    # MHA, group 1
    (16, 4, 128, "bf16", 64),    # group 4
    (16, 2, 128, "bf16", 16),    # group 8
    (16, 8, 64, "bf16", 32),     # head_dim 64
    (4, 2, 128, "f32", 16),      # fp32, head_dim 128
    (2, 1, 64, "f32", 256),      # fp32, head_dim 64
    (24, 3, 128, "bf16", 8),     # odd kv-head count, smallest block
])
def test_decode_shapes(hq, hkv, d, dtype, bs):
    lengths = [1, 63, 64, 65, 127, 129, 511, 512, 513, 1000]
    case = W.decode_case(f"shape_{hq}_{hkv}_{d}_{dtype}_{bs}", 300 + hq + bs, lengths=lengths,
                         hq=hq, hkv=hkv, d=d, dtype=dtype, bs=bs)
    for p in (64, 256):
        _decode_vs_oracle(case, p)


def test_decode_padding_rows_give_zeros():
    case = W.decode_case("pad", 81, lengths=[700, 3, 1], pad_rows=2)
    vals = W.materialize(case, DEV)
    run_store(vals)
    out, _, _ = run_decode(case, vals, 256)
    torch.cuda.synchronize()
    got = to_f64(out, case.dtype)
    assert np.array_equal(got[-2:], np.zeros_like(got[-2:]))
    ref = HostInputs(case, vals, [0, 1, 2]).decode()
    assert_close(got[:3], ref, case.dtype, "pad")


def test_single_key_context_returns_its_value_bit_exact():
    """With one readable key every weight is 1, so the output is v_0 exactly."""
    case = W.decode_case("one", 82, lengths=[1, 1, 1, 1], hq=16, hkv=8)
    vals = W.materialize(case, DEV)
    run_store(vals)
    out, _, _ = run_decode(case, vals, 64)
    torch.cuda.synchronize()
    v = W.raw_numpy(vals["v_new"], "bf16")               # [B, Hkv, d], the stored rows
    want = np.repeat(v, 2, axis=1)                       # query heads 2g, 2g+1 read kv head g
    assert np.array_equal(W.raw_numpy(out, "bf16"), want)


def test_block_permutation_leaves_output_bit_identical():
    """Relabel every physical block (moving its data): splits are in logical token
    space, so the summation order and the result do not change."""
    case = W.SMALL_CASES["c5s"]()
    vals = W.materialize(case, DEV)
    run_store(vals)
    out1, _, _ = run_decode(case, vals, 128)
    sigma = torch.randperm(case.num_blocks, generator=torch.Generator().manual_seed(5))
    sig = sigma.to(DEV)
    k2 = torch.empty_like(vals["k_cache"])
    v2 = torch.empty_like(vals["v_cache"])
    k2[sig] = vals["k_cache"]
    v2[sig] = vals["v_cache"]
    bt = vals["block_table"].long()
    bt2 = torch.where(bt >= 0, sig[bt.clamp(min=0)], bt).to(torch.int32)
    vals2 = dict(vals, k_cache=k2, v_cache=v2, block_table=bt2)
    out2, _, _ = run_decode(case, vals2, 128)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_page_examples_on_gpu():
    """The worked examples of [Intro §1.3] (d=1) and [Intro §18.2] (d=2, V differs),
    zero-padded to head_dim 64 in fp32: padding changes no dot product and no leading
    output element, so the printed numbers must come out."""
    cases = [
        dict(q=[1.0], k=[[0.0], [1.0], [2.0]], v=[[10.0], [20.0], [30.0]], scale=1.0,
             out=[25.75], tol=0.005),
        dict(q=[1.0, 1.0], k=[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]],
             v=[[1.0, 0.0], [0.0, 2.0], [1.0, 2.0]], scale=1 / math.sqrt(2.0),
             out=[0.75174492, 1.50348984], tol=5e-7),
    ]
    for c in cases:
        n, dd = len(c["k"]), len(c["q"])
        kc = torch.full((4, 16, 1, 64), float("nan"), device=DEV)
        vc = kc.clone()
        bt = torch.tensor([[3]], dtype=torch.int32, device=DEV)
        kpad = torch.zeros((n, 64), device=DEV)
        vpad = torch.zeros((n, 64), device=DEV)
        kpad[:, :dd] = torch.tensor(c["k"], device=DEV)
        vpad[:, :dd] = torch.tensor(c["v"], device=DEV)
        kc[3, :n, 0] = kpad
        vc[3, :n, 0] = vpad
        q = torch.zeros((1, 2, 64), device=DEV)
        q[0, :, :dd] = torch.tensor(c["q"], device=DEV)
        ctx = torch.tensor([n], dtype=torch.int32, device=DEV)
        nbytes, splits = pa.pa_decode_workspace_size(1, 2, 64, n, 64)
        ws = torch.empty(nbytes // 4, device=DEV)
        out = torch.empty((1, 2, 64), device=DEV)
        pa.pa_decode(q, kc, vc, bt, ctx, n, 64, c["scale"], ws)
        pa.pa_decode_reduce(ws, ctx, splits, 64, out)
        torch.cuda.synchronize()
        got = out[0].cpu().numpy()
        for h in range(2):
            assert np.all(np.abs(got[h, :dd] - c["out"]) <= c["tol"])
            assert np.all(got[h, dd:] == 0)


def test_workspace_partials_match_oracle_split_statistics():
    """The partition pass alone: (m, l, acc) of every split equals the oracle's split
    statistics, converted to the base-2 units the workspace uses."""
    case = W.SMALL_CASES["c2s"]()
    p = 128
    vals = W.materialize(case, DEV)
    host = HostInputs(case, vals)
    run_store(vals)
    ws, out, splits = decode_buffers(case, p)
    pa.pa_decode(vals["q"], vals["k_cache"], vals["v_cache"], vals["block_table"],
                 vals["context_lens"], case.max_context_len, p, case.scale, ws)
    torch.cuda.synchronize()
    b_, hq, d = case.num_seqs, case.num_q_heads, case.head_dim
    acc = ws[:b_ * hq * splits * d].view(b_, hq, splits, d).cpu().numpy().astype(np.float64)
    ml = ws[b_ * hq * splits * d:b_ * hq * splits * (d + 2)].view(b_, hq, splits, 2).cpu().numpy()
    kc, vc = host.stored()
    log2e = 1.0 / math.log(2.0)
    for b in range(b_):
        n = int(case.context_lens[b])
        keys = oracle.to_f64(oracle.gather(kc, host.block_table[b], n), "bf16")
        vals_ = oracle.to_f64(oracle.gather(vc, host.block_table[b], n), "bf16")
        qf = oracle.to_f64(host.q[b], "bf16")
        active = -(-n // p)
        for h in range(hq):
            g = h // (hq // case.num_kv_heads)
            parts = oracle.split_partials(qf[h], keys[:, g], vals_[:, g], case.scale,
                                          [(s * p, (s + 1) * p) for s in range(active)])
            for s, (m, l, a) in enumerate(parts):
                # base-e statistics -> base-2: m2 = m log2 e; l and acc are unchanged
                assert abs(ml[b, h, s, 0] - m * log2e) <= 1e-3 + 1e-4 * abs(m * log2e)
                assert abs(ml[b, h, s, 1] - l) <= 1e-4 * l + 1e-5
                assert np.all(np.abs(acc[b, h, s] - a) <= 1e-4 * (np.abs(a) + l) + 1e-5)


@pytest.mark.parametrize("s_,lens", [
    (7, [0, 1, 64, 65, 7 * 64]),
    # 40 splits: rows of 0, 1, 16 (the first two load batches), 17 and 29 (one and
    # two more batches) and 40 active splits
    (40, [0, 1, 16 * 64, 16 * 64 + 1, 28 * 64 + 5, 40 * 64]),
])
def test_reduce_on_synthetic_partials(s_, lens):
    """pa_decode_reduce alone, on random split statistics, against oracle.merge."""
    rng = np.random.default_rng(9 + s_)
    b_, hq, d, p = len(lens), 4, 128, 64
    ctx = np.array(lens, np.int32)
    m = rng.normal(0, 20, size=(b_, hq, s_)).astype(np.float32)
    l = rng.uniform(0.5, 64, size=(b_, hq, s_)).astype(np.float32)
    acc = (rng.normal(size=(b_, hq, s_, d)) * l[..., None]).astype(np.float32)
    ws = torch.from_numpy(np.concatenate([acc.reshape(-1),
                                          np.stack([m, l], -1).reshape(-1)])).to(DEV)
    ctx_t = torch.from_numpy(ctx).to(DEV)
    for dtype, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        out = torch.empty((b_, hq, d), dtype=tdt, device=DEV)
        pa.pa_decode_reduce(ws, ctx_t, s_, p, out)
        torch.cuda.synchronize()
        got = to_f64(out, dtype)
        for b in range(b_):
            active = min(s_, -(-int(ctx[b]) // p))
            for h in range(hq):
                # the workspace maxima are base 2: scale to base e for the oracle
                ref = oracle.merge(m[b, h, :active].astype(np.float64) * math.log(2.0),
                                   l[b, h, :active], acc[b, h, :active]) if active else np.zeros(d)
                assert_close(got[b, h], ref, dtype, f"reduce b={b} h={h}")


def _random_decode_case(seed):
    """A seeded random batch: group sizes 1 to 8, head_dim 64 or 128, bf16 or fp32, block
    sizes 8 to 512, 1 to 12 sequences of 1 to 2500 positions, a split size that is a
    random multiple of 64 up to 1024."""
    rng = np.random.default_rng(9200 + seed)
    hq, hkv = [(16, 8), (8, 8), (16, 4), (16, 2), (32, 4)][int(rng.integers(5))]
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    bs = int(rng.choice([8, 16, 32, 64, 128, 256, 512]))
    nseq = int(rng.integers(1, 13))
    lengths = rng.integers(1, 2501, size=nseq)
    if nseq > 1:
        lengths[int(rng.integers(nseq))] = 1
    partition = 64 * int(rng.integers(1, 17))
    case = W.decode_case(f"decode_rand_{seed}", 9200 + seed, lengths=lengths, hq=hq, hkv=hkv,
                         d=d, dtype=dtype, bs=bs)
    return case, partition


@pytest.mark.parametrize("seed", range(16))
def test_decode_random_batches(seed):
    """Seeded random batches (shapes, dtypes, block and split sizes, one-token contexts)
    element by element against the oracle."""
    case, partition = _random_decode_case(seed)
    _decode_vs_oracle(case, partition)
