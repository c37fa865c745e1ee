"""Host logic of bench.py, on the CPU: the one-GPU refusal, the parity
check before timing (it passes on the oracle's own output and fails on a
planted error), and the CPU-baseline fields."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
import oracle
from paged_kv_cache_213_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def _reference(wl, host):
    """The oracle's output for the whole batch from the same host inputs."""
    h = dict(host)
    if wl.kv_dtype == "fp8":
        h["k_cache"] = oracle.fp8_encode_blocks(h.pop("k_src"), h["k_scale"])
        h["v_cache"] = oracle.fp8_encode_blocks(h.pop("v_src"), h["v_scale"])
    else:
        h["k_cache"], h["v_cache"] = h["k_cache"].copy(), h["v_cache"].copy()
    oracle.kv_append(h["k_cache"], h["v_cache"], h["k_new"], h["v_new"], wl.slot_mapping,
                     kv_dtype=wl.kv_dtype, new_dtype=wl.q_dtype, k_scale=h.get("k_scale"),
                     v_scale=h.get("v_scale"), num_kv_heads=wl.num_kv_heads,
                     head_dim=wl.head_dim)
    out, _ = oracle.run_workload(wl, h)
    return out


def test_parity_gate_and_cpu_baseline_on_a_small_batch():
    for name in ("c4", "c5"):
        wl = W.make_config(name, small=True)
        host = bench.host_inputs(wl, W.materialize(wl, "cpu"))
        ref = _reference(wl, host)
        parity, cpu = bench.oracle_leg(wl, host, ref.copy(), budget_s=0.2)
        assert parity["ok"] and parity["max_tol_err"] == 0.0, parity
        assert cpu["unit"] == "GB/s" and cpu["cores"] >= 1 and cpu["value"] > 0
        assert cpu["single_thread"]["value"] > 0 and cpu["cpu_model"]
        # a planted error in one sampled row fails the gate
        bad = ref.copy()
        i = int(bench.parity_sample(wl)[-1])
        bad[wl.query_start_loc[i], 0, 0] += 0.5
        parity_bad, _ = bench.oracle_leg(wl, host, bad, budget_s=0.05)
        assert not parity_bad["ok"]


def test_parity_sample_covers_extremes_and_spans():
    wl = W.make_config("c4", small=True)
    s = bench.parity_sample(wl)
    L = wl.context_lens
    assert int(np.argmin(L)) in s and int(np.argmax(L)) in s
    assert 0 in s and wl.num_seqs - 1 in s
    assert any(wl.query_lens[i] > 1 for i in s)
