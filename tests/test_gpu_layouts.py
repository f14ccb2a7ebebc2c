"""The head-major pool layout ([num_blocks, num_kv_heads, block_size, head_dim], the
Pico-vLLM pool) and block sizes 32, 64 and 128, through store, decode and prefill.

Each case runs the whole path on caches in the head-major layout and checks:
the store bit for bit against the oracle's store (after transposing the pool
back), the attention output against the oracle, and that output bit for bit
against the same path on the slots-then-heads layout (the arithmetic does not
depend on where a row lives)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from pa_runner import (DEV, HostInputs, assert_close, decode_buffers, default_partition,
                       prefill_workspace, to_f64)

import paged_kv_cache_114_amd as pa

pytestmark = pytest.mark.gpu


def swap_slots_heads(cache):
    """[NB, bs, Hkv, d] <-> [NB, Hkv, bs, d] (the same permutation both ways)."""
    return cache.permute(0, 2, 1, 3).contiguous()


def run_path(case, vals, layout):
    """Store, then decode + reduce or prefill, on caches in ``layout``; returns the
    output and the caches (in that layout)."""
    kc, vc = vals["k_cache"].clone(), vals["v_cache"].clone()
    if layout == "bhsd":
        kc, vc = swap_slots_heads(kc), swap_slots_heads(vc)
    pa.pa_store_kv(vals["k_new"], vals["v_new"], kc, vc, vals["slot_mapping"], layout=layout)
    if case.kind == "decode":
        p = default_partition(case)
        ws, out, splits = decode_buffers(case, p)
        pa.pa_decode(vals["q"], kc, vc, vals["block_table"], vals["context_lens"],
                     case.max_context_len, p, case.scale, ws, layout=layout)
        pa.pa_decode_reduce(ws, vals["context_lens"], splits, p, out)
    else:
        out = torch.empty_like(vals["q"])
        pa.pa_prefill_varlen(vals["q"], kc, vc, vals["cu_seqlens_q"], vals["cu_seqlens_k"],
                             vals["block_table"], case.max_seqlen_q, case.max_context_len,
                             case.scale, out, prefill_workspace(case), layout=layout)
    torch.cuda.synchronize()
    return out, kc, vc


def check_case(case, oracle_seqs=None):
    print(f"layout case={case.name} kind={case.kind} bs={case.block_size} "
          f"T={case.num_new_tokens}", flush=True)
    vals = W.materialize(case, DEV)
    k_before = W.raw_numpy(vals["k_cache"], case.dtype)
    v_before = W.raw_numpy(vals["v_cache"], case.dtype)
    host = HostInputs(case, vals, oracle_seqs)
    out_hm, kc, vc = run_path(case, vals, "bhsd")
    out_sm, _, _ = run_path(case, vals, "bshd")

    k_want, v_want = oracle.store(k_before, v_before, W.raw_numpy(vals["k_new"], case.dtype),
                                  W.raw_numpy(vals["v_new"], case.dtype), case.slot_mapping)
    assert np.array_equal(W.raw_numpy(swap_slots_heads(kc), case.dtype), k_want), "K pool"
    assert np.array_equal(W.raw_numpy(swap_slots_heads(vc), case.dtype), v_want), "V pool"

    bits = torch.int16 if case.dtype == "bf16" else torch.int32
    assert torch.equal(out_hm.view(bits), out_sm.view(bits)), "layouts disagree"
    got = to_f64(out_hm, case.dtype)
    if case.kind == "decode":
        assert_close(got[host.seqs], host.decode(), case.dtype, case.name)
    else:
        assert_close(got[host.token_rows], host.prefill(), case.dtype, case.name)


@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c4s", "c5s", "mixeds"])
def test_head_major_layout_small(name):
    check_case(W.SMALL_CASES[name]())


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_block_sizes_decode(bs):
    case = W.decode_case(f"dec_bs{bs}", 4000 + bs, lengths=[1, bs - 1, bs, bs + 1, 700, 2049],
                         bs=bs)
    check_case(case)


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_block_sizes_prefill(bs):
    case = W.prefill_case(f"pf_bs{bs}", 4100 + bs, lengths=[65, 700, 1500, 33],
                          cached=[0, bs, 3 * bs + 5, 0], bs=bs)
    check_case(case)


def test_head_major_layout_full_c2_c3():
    check_case(W.FULL_CASES["c2"]())
    c3 = W.FULL_CASES["c3"]()
    check_case(c3, oracle_seqs=[0, 3, 7])


def test_head_major_norm_rope_store():
    """The q/k norm + rope + store step writes the same rows into a head-major pool."""
    case = W.SMALL_CASES["c5s"]()
    vals = W.materialize(case, DEV)
    inp = W.projection_inputs(case, DEV)
    t, hq, hkv, d = case.num_new_tokens, case.num_q_heads, case.num_kv_heads, case.head_dim
    outs = {}
    for layout in ("bshd", "bhsd"):
        kc, vc = vals["k_cache"].clone(), vals["v_cache"].clone()
        if layout == "bhsd":
            kc, vc = swap_slots_heads(kc), swap_slots_heads(vc)
        q_out = torch.empty((t, hq, d), dtype=torch.bfloat16, device=DEV)
        pa.pa_qk_norm_rope_store(inp["qkv"], inp["q_norm_weight"], inp["k_norm_weight"],
                                 inp["positions"], inp["slot_mapping"], hq, hkv, 1e-6, 1e6, q_out,
                                 kc, vc, layout=layout)
        torch.cuda.synchronize()
        if layout == "bhsd":
            kc, vc = swap_slots_heads(kc), swap_slots_heads(vc)
        outs[layout] = (q_out, kc, vc)
    for a, b in zip(outs["bshd"], outs["bhsd"]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
