"""pa_store_decode (the new rows stored and attended in one launch) against the two-call
path pa_store_kv + pa_decode and against the oracle.

The fused launch must leave the pool bit for bit as the store does and produce the same
split statistics, so the reduced outputs are compared bit for bit with the two-call path;
they are also compared with the oracle within the floating-point bound."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from pa_runner import DEV, HostInputs, assert_close, decode_buffers, default_partition, to_f64

import paged_kv_cache_114_amd as pa

pytestmark = pytest.mark.gpu


def swap_slots_heads(cache):
    return cache.permute(0, 2, 1, 3).contiguous()


def run(case, vals, fused, layout, partition):
    kc, vc = vals["k_cache"].clone(), vals["v_cache"].clone()
    if layout == "bhsd":
        kc, vc = swap_slots_heads(kc), swap_slots_heads(vc)
    ws, out, splits = decode_buffers(case, partition)
    ws.fill_(float("nan"))
    if fused:
        pa.pa_store_decode(vals["k_new"], vals["v_new"], vals["slot_mapping"], vals["q"], kc, vc,
                           vals["block_table"], vals["context_lens"], case.max_context_len,
                           partition, case.scale, ws, layout=layout)
    else:
        pa.pa_store_kv(vals["k_new"], vals["v_new"], kc, vc, vals["slot_mapping"], layout=layout)
        pa.pa_decode(vals["q"], kc, vc, vals["block_table"], vals["context_lens"],
                     case.max_context_len, partition, case.scale, ws, layout=layout)
    pa.pa_decode_reduce(ws, vals["context_lens"], splits, partition, out)
    torch.cuda.synchronize()
    if layout == "bhsd":
        kc, vc = swap_slots_heads(kc), swap_slots_heads(vc)
    return out, kc, vc


def check(case, layout="bshd", partition=None, oracle_seqs=None):
    partition = partition or default_partition(case)
    print(f"store_decode case={case.name} B={case.num_seqs} layout={layout} P={partition}",
          flush=True)
    vals = W.materialize(case, DEV)
    k_before = W.raw_numpy(vals["k_cache"], case.dtype)
    v_before = W.raw_numpy(vals["v_cache"], case.dtype)
    host = HostInputs(case, vals, oracle_seqs)
    out_f, kc_f, vc_f = run(case, vals, True, layout, partition)
    out_s, kc_s, vc_s = run(case, vals, False, layout, partition)
    bits = torch.int16 if case.dtype == "bf16" else torch.int32
    assert torch.equal(out_f.view(bits), out_s.view(bits)), "fused and two-call outputs differ"
    k_want, v_want = oracle.store(k_before, v_before, W.raw_numpy(vals["k_new"], case.dtype),
                                  W.raw_numpy(vals["v_new"], case.dtype), case.slot_mapping)
    assert np.array_equal(W.raw_numpy(kc_f, case.dtype), k_want), "K pool"
    assert np.array_equal(W.raw_numpy(vc_f, case.dtype), v_want), "V pool"
    got = to_f64(out_f, case.dtype)
    assert_close(got[host.seqs], host.decode(), case.dtype, case.name)


@pytest.mark.parametrize("name", ["c1", "c2s", "c4s", "c5s"])
@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_store_decode_small(name, layout):
    check(W.SMALL_CASES[name](), layout)


@pytest.mark.parametrize("partition", [64, 256, 4096])
def test_store_decode_splits(partition):
    """The new token falls in the last of several splits, or in the only one."""
    case = W.decode_case("sd_splits", 5100, lengths=[1, 63, 64, 65, 300, 1000, 2048])
    check(case, partition=partition)


def test_store_decode_padding_rows():
    """Padding rows (slot -1, context 0) store nothing and give zeros."""
    case = W.decode_case("sd_pad", 5200, lengths=[300, 5, 257], pad_rows=3)
    check(case)


def test_store_decode_full_c2():
    check(W.FULL_CASES["c2"]())


@pytest.mark.parametrize("hq,hkv,d,dtype,bs", [
    (8, 8, 128, "bf16", 256),    # group 1
    (16, 4, 128, "bf16", 64),    # group 4
    (16, 2, 128, "bf16", 16),    # group 8
    (16, 8, 64, "bf16", 32),     # head_dim 64
    (4, 2, 128, "f32", 16),      # fp32, head_dim 128
    (24, 3, 128, "bf16", 8),     # odd kv-head count, smallest block
])
def test_store_decode_shapes(hq, hkv, d, dtype, bs):
    """Every GQA group, head_dim and element type the fused launch is built for."""
    case = W.decode_case(f"sdshape_{hq}_{hkv}_{d}_{dtype}_{bs}", 5400 + hq + bs,
                         lengths=[1, 63, 64, 65, 129, 512, 513, 1000], hq=hq, hkv=hkv, d=d,
                         dtype=dtype, bs=bs)
    check(case, partition=64)
    check(case, partition=256, layout="bhsd")


def test_store_decode_large_batch():
    """448 sequences x 8 kv heads in one split each: 3,584 waves, more than the fused
    launch keeps resident on a 256-CU GPU but not more than the plain kernel does, so the
    library stores in a launch of its own first; the bits are the same either way."""
    rng = np.random.default_rng(5600)
    case = W.decode_case("sd_large", 5600, lengths=rng.integers(1, 200, size=448))
    check(case, partition=256, oracle_seqs=list(range(0, 448, 37)))
