"""GPU-side helpers for the parity tests: run one workload's step (append,
then attention) through the C ABI, with inputs that come from the seeded
generator or from the oracle, never from the GPU path."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_213_amd as pa
from paged_kv_cache_213_amd import workloads as W
from tests import helpers as H


def dev_tensors(wl, vals, pre):
    """Device copies of the pre-append state. fp8 caches come from the
    oracle's encoder (host bytes); others from the generator's tensors."""
    d = torch.device("cuda")
    t = {}
    if wl.kv_dtype == "fp8":
        t["k_cache"] = torch.from_numpy(pre["k_cache"]).to(d)
        t["v_cache"] = torch.from_numpy(pre["v_cache"]).to(d)
        t["k_scale"] = torch.from_numpy(pre["k_scale"]).to(d)
        t["v_scale"] = torch.from_numpy(pre["v_scale"]).to(d)
    else:
        t["k_cache"] = vals.k_cache.to(d).clone()
        t["v_cache"] = vals.v_cache.to(d).clone()
        t["k_scale"] = t["v_scale"] = None
    t["q"] = vals.q.to(d).contiguous()
    t["k_new"] = vals.k_new.to(d).contiguous()
    t["v_new"] = vals.v_new.to(d).contiguous()
    t["bt"] = torch.from_numpy(wl.block_tables).to(d)
    t["cl"] = torch.from_numpy(wl.context_lens).to(d)
    t["qsl"] = torch.from_numpy(wl.query_start_loc).to(d)
    t["slots"] = torch.from_numpy(wl.slot_mapping).to(d)
    return t


def gpu_step(wl, t, *, partition_size=None, hybrid=None, with_lse=True, append=True,
             groups=None, fp8_qk=False):
    """kv_append (in place on t's caches) then attention; returns (out, lse).
    groups: (lists of sequences, shared prefix blocks per list) for cascade
    attention."""
    if append:
        pa.kv_append(t["k_cache"], t["v_cache"], t["k_new"], t["v_new"], t["slots"],
                     k_scale=t["k_scale"], v_scale=t["v_scale"])
    P = wl.partition_size if partition_size is None else partition_size
    lse = torch.empty(wl.num_tokens, wl.num_q_heads, dtype=torch.float32,
                      device="cuda") if with_lse else None
    use_hybrid = (not wl.is_decode) if hybrid is None else hybrid
    if groups is not None:
        pg = pa.PrefixGroups(groups[0], groups[1], "cuda")
        out = pa.cascade(t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"], wl.scale, pg,
                         max_context_len=wl.max_context_len,
                         query_start_loc=t["qsl"] if use_hybrid else None,
                         max_query_len=wl.max_query_len, k_scale=t["k_scale"],
                         v_scale=t["v_scale"], partition_size=P, lse=lse, fp8_qk=fp8_qk)
    elif use_hybrid:
        out = pa.hybrid(t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"], t["qsl"], wl.scale,
                        max_context_len=wl.max_context_len, max_query_len=wl.max_query_len,
                        k_scale=t["k_scale"], v_scale=t["v_scale"], partition_size=P, lse=lse,
                        fp8_qk=fp8_qk)
    else:
        out = pa.decode(t["q"], t["k_cache"], t["v_cache"], t["bt"], t["cl"], wl.scale,
                        max_context_len=wl.max_context_len, k_scale=t["k_scale"],
                        v_scale=t["v_scale"], partition_size=P, lse=lse, fp8_qk=fp8_qk)
    torch.cuda.synchronize()
    return out, lse


def out_f64(out) -> np.ndarray:
    return out.detach().float().cpu().numpy().astype(np.float64)


def prepare(wl, device="cuda"):
    vals = W.materialize(wl, device)
    pre = H.host_pre_append(wl, vals)
    return vals, pre


def check_step(wl, partition_size=None, hybrid=None, seq_subset=None, groups=None,
               fp8_qk=False):
    """One step on the GPU against the oracle on the same inputs: the
    per-element tolerance, the relative-RMS guard and the lse bound.
    Returns (errors, device tensors, post-append host state)."""
    import oracle
    vals, pre = prepare(wl)
    post = H.oracle_append(wl, pre)
    t = dev_tensors(wl, vals, pre)
    out, lse = gpu_step(wl, t, partition_size=partition_size, hybrid=hybrid, groups=groups,
                        fp8_qk=fp8_qk)
    ref, ref_lse = oracle.run_workload(wl, post, seq_subset=seq_subset)
    got = out_f64(out)
    got_lse = lse.cpu().numpy().astype(np.float64)
    key = H.tolerance_key(wl)
    if seq_subset is not None:
        rows = np.concatenate([np.arange(wl.query_start_loc[i], wl.query_start_loc[i + 1])
                               for i in seq_subset])
        got, ref, got_lse, ref_lse = got[rows], ref[rows], got_lse[rows], ref_lse[rows]
    e = H.assert_parity(got, ref, key, wl.name)
    # lse in natural-log units, same tolerance form
    le = np.max(np.abs(got_lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse)))
    assert le <= H.TOL[key], f"lse error {le}"
    return e, t, post
