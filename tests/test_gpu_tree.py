"""Tree verification masks on the GPU against the CPU oracle: the spans of
a hybrid batch are candidate trees of draft tokens, each token seeing the
committed context and its own ancestors in the tree ("03 -- Engines
Papers", sections 5 to 7). Spans of more than 64 tokens stay causal."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_213_amd as pa
from paged_kv_cache_213_amd import workloads as W
from tests import helpers as H
from tests.gpu_common import dev_tensors, out_f64, prepare

pytestmark = pytest.mark.gpu


def _tree_step(wl, masks, partition_size=None, seq_subset=None):
    vals, pre = prepare(wl)
    post = H.oracle_append(wl, pre)
    t = dev_tensors(wl, vals, pre)
    pa.kv_append(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["slots"],
                 k_scale=t["k_scale"], v_scale=t["v_scale"])
    P = wl.partition_size if partition_size is None else partition_size
    lse = torch.empty(wl.num_tokens, wl.num_q_heads, dtype=torch.float32, device="cuda")
    tm = torch.from_numpy(masks.view(np.int64)).cuda()
    out = pa.tree(t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"], t["qsl"], wl.scale, tm,
                  max_context_len=wl.max_context_len, max_query_len=wl.max_query_len,
                  k_scale=t["k_scale"], v_scale=t["v_scale"], partition_size=P, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.run_workload(wl, post, seq_subset=seq_subset, tree_mask=masks)
    got, got_lse = out_f64(out), lse.cpu().numpy().astype(np.float64)
    if seq_subset is not None:
        rows = np.concatenate([np.arange(wl.query_start_loc[i], wl.query_start_loc[i + 1])
                               for i in seq_subset])
        got, ref, got_lse, ref_lse = got[rows], ref[rows], got_lse[rows], ref_lse[rows]
    key = H.tolerance_key(wl)
    e = H.assert_parity(got, ref, key, wl.name)
    le = np.max(np.abs(got_lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse)))
    assert le <= H.TOL[key], f"lse error {le}"
    return e, t, out


# spans: one-token decodes, short trees, a tree across a block edge, a full
# 64-token tree, a 65-token span (causal), a long chunk; contexts with a
# ragged committed part, and one span that starts the sequence
_LENS = [300, 41, 16 * 9 + 64, 90, 700, 17, 130, 64 + 5]
_QLENS = [1, 7, 64, 33, 65, 17, 100, 64]


@pytest.mark.parametrize("G,kv,q", [(4, "bf16", "bf16"), (8, "fp8", "bf16"), (2, "f32", "f32"),
                                    (16, "bf16", "bf16")])
@pytest.mark.parametrize("P", [None, 16, 0])
def test_random_trees(G, kv, q, P):
    wl = W.custom_workload(_LENS, _QLENS, num_q_heads=2 * G if G <= 8 else G,
                           num_kv_heads=2 if G <= 8 else 1, head_dim=64 if kv == "f32" else 128,
                           q_dtype=q, kv_dtype=kv, seed=G + 3)
    masks = W.batch_tree_masks(wl.query_lens, seed=G)
    e, _, _ = _tree_step(wl, masks, partition_size=P)
    print(f"G={G} {kv} P={P}: {e}", flush=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_chain_masks_equal_causal_bitwise(kv):
    """A chain in every span is the causal mask: the tree plan must give the
    hybrid path's result bit for bit (same tiles, same order of work)."""
    wl = W.custom_workload(_LENS, _QLENS, num_q_heads=16, num_kv_heads=2, head_dim=128,
                           q_dtype="bf16", kv_dtype=kv, seed=9)
    masks = W.batch_tree_masks(wl.query_lens, seed=0, chain=True)
    _, t, out = _tree_step(wl, masks)
    ref = pa.hybrid(t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"], t["qsl"], wl.scale,
                    max_context_len=wl.max_context_len, max_query_len=wl.max_query_len,
                    k_scale=t["k_scale"], v_scale=t["v_scale"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_plan_reuse_clears_the_tree():
    """A workspace planned with masks and then re-planned with pa_plan runs
    causal spans again (the flag travels with each plan)."""
    wl = W.custom_workload(_LENS, _QLENS, num_q_heads=8, num_kv_heads=2, head_dim=128,
                           q_dtype="bf16", kv_dtype="bf16", seed=2)
    vals, pre = prepare(wl)
    post = H.oracle_append(wl, pre)
    t = dev_tensors(wl, vals, pre)
    pa.kv_append(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["slots"])
    shape = pa.make_shape(t["q"], t["k_cache"], t["bt"])
    nb = pa.workspace_bytes(shape, wl.num_seqs, wl.num_tokens, wl.max_context_len,
                            wl.max_query_len)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    kw = dict(query_start_loc=t["qsl"], num_q_tokens=wl.num_tokens,
              max_query_len=wl.max_query_len, max_context_len=wl.max_context_len)
    masks = W.batch_tree_masks(wl.query_lens, seed=4)
    tm = torch.from_numpy(masks.view(np.int64)).cuda()
    outs = []
    for use_tree in (True, False):
        if use_tree:
            pa.plan_tree(shape, t["cl"], ws, tm, **kw)
        else:
            pa.plan(shape, t["cl"], ws, **kw)
        outs.append(out_f64(pa.run(shape, t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"],
                                   wl.scale, ws, query_start_loc=t["qsl"],
                                   max_query_len=wl.max_query_len,
                                   max_context_len=wl.max_context_len)))
    ref_t, _ = oracle.run_workload(wl, post, tree_mask=masks)
    ref_c, _ = oracle.run_workload(wl, post)
    H.assert_parity(outs[0], ref_t, "bf16", "tree")
    H.assert_parity(outs[1], ref_c, "bf16", "causal")


def test_speculative_verification_batch():
    """A serving-sized verification step: 128 sequences of Llama-3-8B
    shape (32 query heads, 8 KV heads, D 128) with contexts U[128, 4096]
    and candidate trees of 4 to 64 draft tokens; every row."""
    rng = np.random.default_rng(77)
    S = 128
    ql = rng.integers(4, 65, S)
    lens = rng.integers(128, 4097, S) + ql
    wl = W.custom_workload(lens, ql, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           q_dtype="bf16", kv_dtype="bf16", seed=31)
    masks = W.batch_tree_masks(wl.query_lens, seed=31)
    e, _, _ = _tree_step(wl, masks, partition_size=0)
    print(f"spec verify: {e}", flush=True)
