"""pa_prefill_plan + the *_planned prefill calls: the work list built once serves every
layer of a step.

Each planned call must give exactly the bits of the call that builds its own list, on
consecutive calls over different layers (different queries and pools, so a call that
skipped work items would leave wrong rows, not the previous call's), with and without
key-range splits and with the store; the outputs are NaN-filled before every call."""

import pytest
import torch

import workloads as W
from pa_runner import DEV, HostInputs, assert_close, prefill_workspace, to_f64

import paged_kv_cache_114_amd as pa

pytestmark = pytest.mark.gpu

BITS = torch.int16


def layers_of(case, n, seed):
    """n layers: one pool pair and one set of queries and new rows each."""
    base = W.materialize(case, DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    out = []
    for i in range(n):
        lay = {k: v for k, v in base.items()}
        if i:
            for key in ("q", "k_new", "v_new"):
                lay[key] = torch.randn(base[key].shape, generator=gen, device=DEV).to(base[key].dtype)
            for key in ("k_cache", "v_cache"):  # other values, the poison of unused slots kept
                lay[key] = base[key] * (-1.0, 0.5, -0.5)[(i - 1) % 3]
        out.append(lay)
    return out


def call(case, lay, ws, split_keys, store, planned, kc, vc, out):
    args = dict(split_keys=split_keys)
    if store:
        fn = pa.pa_store_prefill_varlen_planned if planned else pa.pa_store_prefill_varlen
        fn(lay["k_new"], lay["v_new"], lay["slot_mapping"], lay["q"], kc, vc, lay["cu_seqlens_q"],
           lay["cu_seqlens_k"], lay["block_table"], case.max_seqlen_q, case.max_context_len,
           case.scale, out, ws, **args)
    else:
        fn = pa.pa_prefill_varlen_planned if planned else pa.pa_prefill_varlen
        fn(lay["q"], kc, vc, lay["cu_seqlens_q"], lay["cu_seqlens_k"], lay["block_table"],
           case.max_seqlen_q, case.max_context_len, case.scale, out, ws, **args)


@pytest.mark.parametrize("name,split_keys,store", [
    ("c3s", 0, False), ("c3s", 0, True), ("mixeds", 0, True), ("c3s", 256, False),
    ("c3s", 256, True), ("c3", 0, True),
])
def test_planned_calls_equal_replanning_calls(name, split_keys, store):
    case = W.SMALL_CASES[name]() if name in W.SMALL_CASES else W.FULL_CASES[name]()
    print(f"plan case={case.name} split_keys={split_keys} store={store}", flush=True)
    layers = layers_of(case, 4, seed=21)
    if not store:  # the pools hold this step's rows already
        for lay in layers:
            pa.pa_store_kv(lay["k_new"], lay["v_new"], lay["k_cache"], lay["v_cache"],
                           lay["slot_mapping"])
    ws_ref = prefill_workspace(case, split_keys)
    ws = prefill_workspace(case, split_keys)
    lay0 = layers[0]
    pa.pa_prefill_plan(lay0["cu_seqlens_q"], lay0["cu_seqlens_k"], case.num_new_tokens,
                       case.num_q_heads, case.num_kv_heads, case.head_dim, case.max_seqlen_q,
                       case.max_context_len, ws, split_keys=split_keys)
    for rep in range(2):  # every layer twice over: the list serves 8 calls in a row
        for i, lay in enumerate(layers):
            results = []
            for planned in (True, False):
                kc, vc = lay["k_cache"].clone(), lay["v_cache"].clone()
                out = torch.full_like(lay["q"], float("nan"))
                call(case, lay, ws if planned else ws_ref, split_keys, store, planned, kc, vc, out)
                torch.cuda.synchronize()
                results.append((out, kc, vc))
            (o_p, k_p, v_p), (o_r, k_r, v_r) = results
            assert torch.equal(o_p.view(BITS), o_r.view(BITS)), (rep, i, "out")
            assert torch.equal(k_p.view(BITS), k_r.view(BITS)), (rep, i, "k cache")
            assert torch.equal(v_p.view(BITS), v_r.view(BITS)), (rep, i, "v cache")
    # and against the oracle, on the last layer
    lay = layers[-1]
    kc, vc = lay["k_cache"].clone(), lay["v_cache"].clone()
    out = torch.full_like(lay["q"], float("nan"))
    call(case, lay, ws, split_keys, store, True, kc, vc, out)
    torch.cuda.synchronize()
    # (when the pool holds the rows already, the oracle's own store rewrites the same bits)
    seqs = list(range(min(case.num_seqs, 4)))
    host = HostInputs(case, lay, seqs)
    got = to_f64(out, case.dtype)
    assert_close(got[host.token_rows], host.prefill(), case.dtype, case.name)


def test_plan_then_replanning_call_then_planned_again():
    """A replanning call on the same workspace leaves a list for the same metadata
    behind, so planned calls after it still match."""
    case = W.SMALL_CASES["mixeds"]()
    layers = layers_of(case, 2, seed=5)
    ws = prefill_workspace(case)
    lay = layers[0]
    pa.pa_prefill_plan(lay["cu_seqlens_q"], lay["cu_seqlens_k"], case.num_new_tokens,
                       case.num_q_heads, case.num_kv_heads, case.head_dim, case.max_seqlen_q,
                       case.max_context_len, ws)
    outs = []
    for planned in (True, False, True):
        out = torch.full_like(lay["q"], float("nan"))
        call(case, layers[1], ws, 0, True, planned, layers[1]["k_cache"].clone(),
             layers[1]["v_cache"].clone(), out)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(BITS), outs[1].view(BITS))
    assert torch.equal(outs[2].view(BITS), outs[1].view(BITS))
