"""pa_store_kv on the GPU against the oracle store: bit-exact over the whole pool."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from pa_runner import DEV, HostInputs, run_store

import paged_kv_cache_114_amd as pa

pytestmark = pytest.mark.gpu


def _store_and_compare(case, vals):
    host = HostInputs(case, vals)
    # the whole pool before the store, as the oracle sees it
    k_before = W.raw_numpy(vals["k_cache"], case.dtype)
    v_before = W.raw_numpy(vals["v_cache"], case.dtype)
    rows = [i for i, s in enumerate(case.slot_mapping.tolist())]
    k_new = W.raw_numpy(vals["k_new"], case.dtype)[rows]
    v_new = W.raw_numpy(vals["v_new"], case.dtype)[rows]
    run_store(vals)
    torch.cuda.synchronize()
    k_want, v_want = oracle.store(k_before, v_before, k_new, v_new, case.slot_mapping)
    assert np.array_equal(W.raw_numpy(vals["k_cache"], case.dtype), k_want)
    assert np.array_equal(W.raw_numpy(vals["v_cache"], case.dtype), v_want)
    return host


@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c5s"])
def test_store_bit_exact_small(name):
    case = W.SMALL_CASES[name]()
    print(f"store case={case.name} tokens={case.num_new_tokens}", flush=True)
    _store_and_compare(case, W.materialize(case, DEV))


def test_store_bit_exact_c3_full():
    case = W.c3_prefill()
    print(f"store case={case.name} tokens={case.num_new_tokens}", flush=True)
    _store_and_compare(case, W.materialize(case, DEV))


def test_store_padding_rows_write_nothing():
    case = W.decode_case("pad", 77, lengths=[300, 5, 257], pad_rows=3)
    vals = W.materialize(case, DEV)
    assert (case.slot_mapping[-3:] == -1).all()
    _store_and_compare(case, vals)


def test_store_from_fused_qkv_view():
    """K/V as strided views into one [T, (Hq + 2 Hkv) * d] projection output, the layout
    whose missing strides corrupted the cache in Pico-vLLM dev log #6."""
    case = W.decode_case("fused", 78, lengths=[40, 700, 256, 1])
    vals = W.materialize(case, DEV)
    t, hq, hkv, d = case.num_new_tokens, case.num_q_heads, case.num_kv_heads, case.head_dim
    qkv = torch.empty((t, (hq + 2 * hkv) * d), dtype=torch.bfloat16, device=DEV)
    qkv[:, hq * d:(hq + hkv) * d] = vals["k_new"].reshape(t, -1)
    qkv[:, (hq + hkv) * d:] = vals["v_new"].reshape(t, -1)
    k_view = qkv[:, hq * d:(hq + hkv) * d].view(t, hkv, d)
    v_view = qkv[:, (hq + hkv) * d:].view(t, hkv, d)
    assert not k_view.is_contiguous()
    k_before = W.raw_numpy(vals["k_cache"], case.dtype)
    v_before = W.raw_numpy(vals["v_cache"], case.dtype)
    pa.pa_store_kv(k_view, v_view, vals["k_cache"], vals["v_cache"], vals["slot_mapping"])
    torch.cuda.synchronize()
    k_want, v_want = oracle.store(k_before, v_before, W.raw_numpy(vals["k_new"], "bf16"),
                                  W.raw_numpy(vals["v_new"], "bf16"), case.slot_mapping)
    assert np.array_equal(W.raw_numpy(vals["k_cache"], "bf16"), k_want)
    assert np.array_equal(W.raw_numpy(vals["v_cache"], "bf16"), v_want)


def test_store_misaligned_source_falls_back_to_narrow_words():
    """A source starting one bf16 element past a 16-byte boundary."""
    case = W.decode_case("odd", 79, lengths=[33, 2], hq=4, hkv=2, d=64, bs=16)
    vals = W.materialize(case, DEV)
    t, hkv, d = case.num_new_tokens, case.num_kv_heads, case.head_dim
    buf = torch.empty(t * hkv * d + 1, dtype=torch.bfloat16, device=DEV)
    buf[1:] = vals["k_new"].reshape(-1)
    k_odd = buf[1:].view(t, hkv, d)
    k_before = W.raw_numpy(vals["k_cache"], "bf16")
    v_before = W.raw_numpy(vals["v_cache"], "bf16")
    pa.pa_store_kv(k_odd, vals["v_new"], vals["k_cache"], vals["v_cache"], vals["slot_mapping"])
    torch.cuda.synchronize()
    k_want, v_want = oracle.store(k_before, v_before, W.raw_numpy(vals["k_new"], "bf16"),
                                  W.raw_numpy(vals["v_new"], "bf16"), case.slot_mapping)
    assert np.array_equal(W.raw_numpy(vals["k_cache"], "bf16"), k_want)
    assert np.array_equal(W.raw_numpy(vals["v_cache"], "bf16"), v_want)


@pytest.mark.parametrize("name", ["c4", "c5"])
def test_store_full_size_changes_only_the_new_slots(name):
    """At full size the whole pool is compared on the device: equal to the pool before
    the store everywhere except the new slots, which hold the new rows bit for bit."""
    case = W.FULL_CASES[name]()
    print(f"store case={case.name} tokens={case.num_new_tokens} blocks={case.num_blocks}",
          flush=True)
    vals = W.materialize(case, DEV)
    before = [vals["k_cache"].clone(), vals["v_cache"].clone()]
    run_store(vals)
    torch.cuda.synchronize()
    nb, bs = case.num_blocks, case.block_size
    slots = torch.tensor(case.slot_mapping, dtype=torch.long, device=DEV)
    raw = torch.int16
    for cache, old, new in ((vals["k_cache"], before[0], vals["k_new"]),
                            (vals["v_cache"], before[1], vals["v_new"])):
        c = cache.view(raw).view(nb * bs, -1)
        o = old.view(raw).view(nb * bs, -1)
        changed = torch.nonzero((c != o).any(dim=1)).flatten()
        assert set(changed.tolist()) <= set(case.slot_mapping.tolist())
        assert torch.equal(c.index_select(0, slots), new.view(raw).reshape(len(slots), -1))


@pytest.mark.parametrize("seed", range(8))
def test_store_random_batches(seed):
    """Seeded random batches (kv heads 1 to 8, head_dim 64 or 128, bf16 or fp32, blocks 8 to
    512, ragged lengths with cached prefixes): the pool equals the oracle's store bit for
    bit, every slot outside the step untouched."""
    rng = np.random.default_rng(9400 + seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    bs = int(rng.choice([8, 16, 32, 64, 128, 256, 512]))
    nseq = int(rng.integers(1, 9))
    lengths = rng.integers(1, 1201, size=nseq)
    cached = np.array([int(rng.integers(0, n)) if rng.random() < 0.5 else 0 for n in lengths])
    case = W.prefill_case(f"store_rand_{seed}", 9400 + seed, lengths=lengths, cached=cached,
                          hq=2 * hkv, hkv=hkv, d=d, dtype=dtype, bs=bs)
    print(f"store case={case.name} T={case.num_new_tokens} Hkv={hkv} d={d} {dtype} bs={bs}",
          flush=True)
    _store_and_compare(case, W.materialize(case, DEV))
