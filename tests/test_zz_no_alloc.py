"""pa_paged_attn_hybrid_noalloc: the hybrid call on the library's static
per-GPU scratch buffer, for callers that cannot allocate. Two calls in a
row through the C ABI, the second with a smaller batch, each compared with
pa_paged_attn_hybrid on the same inputs (bit for bit: same kernels, same
plan) and with the oracle (the parity tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_213_amd as pa
from paged_kv_cache_213_amd import workloads as W
from tests import helpers as H
from tests.gpu_common import dev_tensors, out_f64, prepare

pytestmark = pytest.mark.gpu


def _call_both(wl):
    vals, pre = prepare(wl)
    post = H.oracle_append(wl, pre)
    t = dev_tensors(wl, vals, pre)
    pa.kv_append(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["slots"],
                 k_scale=t["k_scale"], v_scale=t["v_scale"])
    kw = dict(max_context_len=wl.max_context_len, max_query_len=wl.max_query_len,
              k_scale=t["k_scale"], v_scale=t["v_scale"], partition_size=wl.partition_size)
    out_a = torch.full_like(t["q"], float("nan"))
    lse_a = torch.full((wl.num_tokens, wl.num_q_heads), float("nan"), device="cuda")
    pa.hybrid_noalloc(t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"], t["qsl"], wl.scale,
                      out=out_a, lse=lse_a, **kw)
    out_b = torch.full_like(t["q"], float("nan"))
    lse_b = torch.full((wl.num_tokens, wl.num_q_heads), float("nan"), device="cuda")
    pa.hybrid(t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"], t["qsl"], wl.scale,
              out=out_b, lse=lse_b, **kw)
    torch.cuda.synchronize()
    return out_a, lse_a, out_b, lse_b, post


def _check(wl):
    out_a, lse_a, out_b, lse_b, post = _call_both(wl)
    assert torch.equal(out_a.view(torch.int16) if out_a.dtype == torch.bfloat16 else out_a,
                       out_b.view(torch.int16) if out_b.dtype == torch.bfloat16 else out_b)
    assert torch.equal(lse_a, lse_b)
    ref, ref_lse = oracle.run_workload(wl, post)
    e = H.assert_parity(out_f64(out_a), ref, H.tolerance_key(wl), wl.name)
    le = np.max(np.abs(lse_a.cpu().numpy() - ref_lse) / np.maximum(1.0, np.abs(ref_lse)))
    assert le <= H.TOL[H.tolerance_key(wl)]
    return e


def test_two_calls_in_a_row_second_smaller():
    """A hybrid batch (a 72-token chunked-prefill span among 16 decodes, with
    its 512-token partitions), then a smaller batch of decodes and short
    spans on the same scratch buffer, which still holds the first call's
    records."""
    big = W.make_config("c4", small=True)
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 300, 9)
    ql = np.minimum(rng.integers(1, 6, 9), lens)
    small = W.custom_workload(lens, ql, num_q_heads=32, num_kv_heads=8, head_dim=128,
                              q_dtype="bf16", kv_dtype="bf16", seed=6, name="small-hybrid")
    assert small.num_tokens < big.num_tokens and small.num_seqs < big.num_seqs
    e1 = _check(big)
    e2 = _check(small)
    print(f"no-alloc: {big.name} {e1}; {small.name} {e2}", flush=True)


def test_fp8_and_f32_batches():
    """The other cache kinds go through the same buffer."""
    for name in ("c5", "c1"):
        wl = W.make_config(name, small=True)
        wl_h = W.custom_workload(wl.context_lens, np.ones(wl.num_seqs, np.int32),
                                 num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                                 head_dim=wl.head_dim, q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype,
                                 seed=9, name=name + "-as-hybrid")
        _check(wl_h)


def test_batches_past_the_buffer_are_rejected():
    """A batch whose workspace exceeds the buffer returns PA_ESCRATCH and
    leaves the output untouched."""
    S = 4096
    shape = pa.PaShape(32, 8, 128, 16, 4096, 2048, pa.PA_BF16, pa.PA_BF16, 16, 0, 0)
    need = pa.workspace_bytes(shape, S, S * 64, 32768, 64)
    assert need > pa.PA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(8, 32, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    lib = pa.load_library()
    rc = lib.pa_paged_attn_hybrid_noalloc(
        pa.ctypes.byref(shape), out.data_ptr(), None, q.data_ptr(), q.data_ptr(), q.data_ptr(),
        None, None, q.data_ptr(), q.data_ptr(), q.data_ptr(), S, S * 64, 64, 32768, 0.1,
        torch.cuda.current_stream().cuda_stream)
    assert rc == pa.PA_ESCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


def test_full_workloads_fit_or_are_rejected():
    """Which full-size workloads fit the buffer at this device's wave
    counts (printed), and that the first one fits."""
    sizes = {}
    for name in ("c1", "c2", "c3", "c4", "c5"):
        wl = W.make_config(name)
        shape = pa.PaShape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 16, int(wl.num_blocks),
                           wl.block_tables.shape[1],
                           pa.PA_F32 if wl.q_dtype == "f32" else pa.PA_BF16,
                           {"f32": pa.PA_F32, "bf16": pa.PA_BF16, "fp8": pa.PA_FP8_E4M3FN}[
                               wl.kv_dtype], 0, 0, 0)
        sizes[name] = pa.workspace_bytes(shape, wl.num_seqs, wl.num_tokens, wl.max_context_len,
                                         wl.max_query_len)
    print("workspace bytes at partition_size 0:", sizes, flush=True)
    assert sizes["c2"] <= pa.PA_NOALLOC_SCRATCH_BYTES
