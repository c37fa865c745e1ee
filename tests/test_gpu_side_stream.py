"""Hybrid batches whose span launch runs beside the narrow and group
launches: the narrow and group kernels go to the library's second stream,
forked from the caller's stream after the work queued before the call and
joined back before the merge ("03 -- Engines Papers", section 3: the chunk
and the decodes of a hybrid batch scheduled together). Where the decodes
hold most of the work the plan cuts the span stream for one workgroup per
compute unit. Checked here: the layout reports that count, captured calls
replay to the eager result bit for bit (with eager work between the
replays), and two host threads that enqueue hybrid calls on their own
streams at once both get the single-thread result bit for bit. The outputs
themselves are compared with the oracle by the parity tests, on the same
calls."""
import threading

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_213_amd as pa
from paged_kv_cache_213_amd import workloads as W
from tests import helpers as H
from tests.gpu_common import dev_tensors, out_f64, prepare

pytestmark = pytest.mark.gpu


def _setup(name="c4", small=False):
    wl = W.make_config(name, small=small)
    vals, pre = prepare(wl)
    t = dev_tensors(wl, vals, pre)
    pa.kv_append(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["slots"],
                 k_scale=t["k_scale"], v_scale=t["v_scale"])
    torch.cuda.synchronize()
    return wl, vals, pre, t


def _hybrid(wl, t, stream=None):
    lse = torch.empty(wl.num_tokens, wl.num_q_heads, dtype=torch.float32, device="cuda")
    out = pa.hybrid(t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"], t["qsl"], wl.scale,
                    max_context_len=wl.max_context_len, max_query_len=wl.max_query_len,
                    k_scale=t["k_scale"], v_scale=t["v_scale"], partition_size=0, lse=lse,
                    stream=stream)
    return out, lse


def test_layout_reports_one_span_workgroup_per_compute_unit():
    wl, _, _, t = _setup()
    shape = pa.make_shape(t["q"], t["k_cache"], t["bt"], 0)
    info = pa.workspace_layout(shape, wl.num_seqs, wl.num_tokens, wl.max_context_len,
                               wl.max_query_len, decode=False)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    assert info.span_shared == ncu
    assert info.waves[0] >= 2 * ncu
    # decode layouts have no span stream and never fork
    dec = pa.workspace_layout(shape, wl.num_seqs, wl.num_seqs, wl.max_context_len, 1,
                              decode=True)
    assert dec.span_shared == 0


def test_eager_result_against_the_oracle():
    """The full hybrid batch at the balanced split (span launch beside the
    decodes) against the oracle, every row."""
    wl, vals, pre, t = _setup()
    out, _ = _hybrid(wl, t)
    torch.cuda.synchronize()
    post = H.oracle_append(wl, pre)
    ref, _ = oracle.run_workload(wl, post)
    H.assert_parity(out_f64(out), ref, H.tolerance_key(wl), "c4 full, side stream")


def test_graph_replays_with_the_side_stream():
    wl, _, _, t = _setup()
    ref, ref_lse = _hybrid(wl, t)
    torch.cuda.synchronize()
    shape = pa.make_shape(t["q"], t["k_cache"], t["bt"], 0)
    ws = torch.zeros(pa.workspace_bytes(shape, wl.num_seqs, wl.num_tokens, wl.max_context_len,
                                        wl.max_query_len), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty_like(ref_lse)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pa.plan(shape, t["cl"], ws, query_start_loc=t["qsl"], num_q_tokens=wl.num_tokens,
                max_query_len=wl.max_query_len, max_context_len=wl.max_context_len, stream=s)
        pa.run(shape, t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"], wl.scale, ws,
               query_start_loc=t["qsl"], max_query_len=wl.max_query_len,
               max_context_len=wl.max_context_len, out=out, lse=lse, stream=s)
    for i in range(4):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), f"replay {i}"
        _ = (t["q"].float() * 2).sum().item()  # unrelated eager work between replays


def test_two_host_threads_enqueue_at_once():
    wl, _, _, t = _setup()
    ref, ref_lse = _hybrid(wl, t)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                got = [_hybrid(wl, t, stream=s) for _ in range(4)]
            s.synchronize()
            results[k] = got
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    assert sorted(results) == [0, 1]
    for k, got in results.items():
        for i, (o, l) in enumerate(got):
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"thread {k} call {i}"
            assert torch.equal(l.view(torch.int32), ref_lse.view(torch.int32)), \
                f"thread {k} call {i}"


@pytest.mark.parametrize("seed", range(8))
def test_random_hybrid_batches_at_the_balanced_split(seed):
    """Random chunk/decode mixes (the share rule falls either way) against
    the oracle."""
    from tests.test_gpu_random_batches import _random_batch
    wl = _random_batch(seed)
    vals, pre = prepare(wl)
    t = dev_tensors(wl, vals, pre)
    pa.kv_append(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["slots"],
                 k_scale=t["k_scale"], v_scale=t["v_scale"])
    out, _ = _hybrid(wl, t)
    torch.cuda.synchronize()
    post = H.oracle_append(wl, pre)
    ref, _ = oracle.run_workload(wl, post)
    H.assert_parity(out_f64(out), ref, H.tolerance_key(wl), f"random hybrid {seed}")


@pytest.mark.parametrize("lens,qlens", [([4096], [512]), ([3000, 40, 100], [384, 1, 1]),
                                        ([2048, 2048], [256, 256])])
def test_span_heavy_batches(lens, qlens):
    """Batches whose single-token work is below twice the span work (a
    chunk alone, a chunk beside two short decodes, two chunks): the plan
    keeps the span kernel's whole residency, the side stream still forks
    and joins (its narrow launch has little or nothing to do); every row
    against the oracle."""
    wl = W.custom_workload(lens, qlens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           q_dtype="bf16", kv_dtype="bf16", seed=len(lens) * 7 + qlens[0])
    vals, pre = prepare(wl)
    t = dev_tensors(wl, vals, pre)
    pa.kv_append(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["slots"])
    out, lse = _hybrid(wl, t)
    torch.cuda.synchronize()
    post = H.oracle_append(wl, pre)
    ref, _ = oracle.run_workload(wl, post)
    H.assert_parity(out_f64(out), ref, H.tolerance_key(wl), f"span-heavy {lens} {qlens}")
    assert torch.isfinite(lse).all()
