"""pa_store_decode_noalloc (the decode step with its split workspace in the
library's fixed device array) against pa_store_decode + pa_decode_reduce with a
caller-owned workspace: outputs and both pools bit for bit, on consecutive calls
that share the fixed array, the later ones smaller."""

import pytest
import torch

import workloads as W
from pa_runner import DEV, decode_buffers, timed_partition

import paged_kv_cache_114_amd as pa

pytestmark = pytest.mark.gpu


def run_both(case, partition):
    print(f"no_alloc case={case.name} B={case.num_seqs} P={partition}", flush=True)
    vals = W.materialize(case, DEV)
    bits = torch.int16 if case.dtype == "bf16" else torch.int32
    kc1, vc1 = vals["k_cache"].clone(), vals["v_cache"].clone()
    kc2, vc2 = vals["k_cache"].clone(), vals["v_cache"].clone()
    ws, ref, splits = decode_buffers(case, partition)
    pa.pa_store_decode(vals["k_new"], vals["v_new"], vals["slot_mapping"], vals["q"], kc1, vc1,
                       vals["block_table"], vals["context_lens"], case.max_context_len, partition,
                       case.scale, ws)
    pa.pa_decode_reduce(ws, vals["context_lens"], splits, partition, ref)
    out = torch.full_like(ref, float("nan"))
    pa.pa_store_decode_noalloc(vals["k_new"], vals["v_new"], vals["slot_mapping"], vals["q"], kc2,
                               vc2, vals["block_table"], vals["context_lens"],
                               case.max_context_len, partition, case.scale, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(bits), ref.view(bits)), "outputs differ"
    assert torch.equal(kc1.view(bits), kc2.view(bits)), "K pools differ"
    assert torch.equal(vc1.view(bits), vc2.view(bits)), "V pools differ"


def test_no_alloc_matches_caller_workspace_on_consecutive_calls():
    big = W.FULL_CASES["c2"]()                  # 64 sequences, 4 splits of 256 tokens
    run_both(big, timed_partition(big))
    small = W.SMALL_CASES["c2s"]()              # 6 sequences
    run_both(small, 128)
    pad = W.decode_case("noalloc_pad", 5300, lengths=[300, 5, 257], pad_rows=2)
    run_both(pad, 64)                           # padding rows: slot -1, context 0
    run_both(W.c1_tiny_decode(), 64)            # fp32, one sequence


def test_no_alloc_refuses_more_than_its_array():
    """A call whose workspace would exceed the fixed 64 MiB is refused before any
    launch, and a later small call still matches."""
    case = W.SMALL_CASES["c2s"]()
    vals = W.materialize(case, DEV)
    out = torch.empty((case.num_seqs, case.num_q_heads, case.head_dim), dtype=torch.bfloat16,
                      device=DEV)
    with pytest.raises(pa.PAError) as e:
        # 64-token splits of a 100,000-token context: 6 x 16 x 1563 x 130 floats > 64 MiB
        pa.pa_store_decode_noalloc(vals["k_new"], vals["v_new"], vals["slot_mapping"], vals["q"],
                                   vals["k_cache"], vals["v_cache"],
                                   torch.zeros((case.num_seqs, 391), dtype=torch.int32,
                                               device=DEV),
                                   vals["context_lens"], 100_000, 64, case.scale, out)
    assert e.value.status == pa.PA_ERR_WORKSPACE
    run_both(case, 128)
