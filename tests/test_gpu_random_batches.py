"""Seeded random hybrid batches on the GPU against the CPU oracle.

Each case draws a batch shape the fixed configurations do not pin down: a
mix of single-token decodes and chunked-prefill spans of ragged lengths
(the hybrid batch of "03 -- Engines Papers", section 3), context lengths
from one key to a few thousand, GQA group sizes from 1 to 16, both head
sizes, the three cache kinds and several partition sizes (split-KV pieces
merged by log-sum-exp, section 12). The oracle and the tolerances are those
of every other parity test."""
import numpy as np
import pytest

from paged_kv_cache_213_amd import workloads as W
from tests.gpu_common import check_step

pytestmark = pytest.mark.gpu

KINDS = [("bf16", "bf16"), ("bf16", "fp8"), ("f32", "f32")]


def _random_batch(seed: int):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 25))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2]))
    D = int(rng.choice([64, 128]))
    q_dtype, kv_dtype = KINDS[seed % len(KINDS)]
    P = int(rng.choice([0, 16, 48, 256, 512]))
    # context lengths: short, block-edge and long ones mixed
    pool = np.concatenate([rng.integers(1, 40, S), rng.integers(1, 3000, S),
                           16 * rng.integers(1, 40, S)])
    lens = rng.choice(pool, S).astype(np.int32)
    # most sequences decode one token; some carry a span up to 80 tokens
    span = rng.random(S) < 0.35
    ql = np.where(span, rng.integers(2, 81, S), 1).astype(np.int32)
    ql = np.minimum(ql, lens).astype(np.int32)
    return W.custom_workload(lens, ql, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                             q_dtype=q_dtype, kv_dtype=kv_dtype, partition_size=P,
                             seed=seed, name=f"random-{seed}")


@pytest.mark.parametrize("seed", range(24))
def test_random_hybrid_batch(seed):
    wl = _random_batch(seed)
    e, _, _ = check_step(wl, hybrid=True)
    print(f"seed {seed}: S={wl.num_seqs} T={wl.num_tokens} Hq={wl.num_q_heads} "
          f"Hkv={wl.num_kv_heads} D={wl.head_dim} {wl.q_dtype}/{wl.kv_dtype} "
          f"P={wl.partition_size}: {e}", flush=True)


def _random_sharing_batch(seed: int, decode: bool = False):
    """Random shared-prefix groups (copy-on-write sharing of whole leading
    blocks, "03 -- Engines Papers", section 2) next to unshared sequences;
    members' own tokens lie past their group's prefix. decode: every
    sequence carries one new token and pieces are balanced (no partition
    size), the layout of a parallel-sampling decode step."""
    rng = np.random.default_rng(1000 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2]))
    D = int(rng.choice([64, 128]))
    q_dtype, kv_dtype = KINDS[seed % len(KINDS)]
    P = int(rng.choice([0, 16, 48, 512]))
    ngroups = int(rng.integers(1, 5))
    groups, prefix, lens, ql = [], [], [], []
    for _ in range(ngroups):
        pb = int(rng.integers(1, 41))
        members = []
        for _ in range(int(rng.integers(2, 21))):
            n = 1 if rng.random() < 0.85 else int(rng.integers(2, 40))
            n = 1 if decode else n
            L = 16 * pb + n + int(rng.integers(0, 600))
            members.append(len(lens))
            lens.append(L)
            ql.append(n)
        groups.append(members)
        prefix.append(pb)
    for _ in range(int(rng.integers(0, 8))):  # sequences outside every group
        L = int(rng.integers(1, 2000))
        lens.append(L)
        q1 = 1 if rng.random() < 0.8 else int(rng.integers(1, min(L, 60) + 1))
        ql.append(1 if decode else q1)
    wl = W.custom_workload(np.array(lens, np.int32), np.array(ql, np.int32),
                           num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, q_dtype=q_dtype,
                           kv_dtype=kv_dtype, partition_size=0 if decode else P, seed=seed,
                           name=f"random-sharing-{'decode-' if decode else ''}{seed}")
    for members, pb in zip(groups, prefix):
        lead = wl.block_tables[members[0], :pb].copy()
        for i in members:
            wl.block_tables[i, :pb] = lead
    return wl, (groups, prefix)


@pytest.mark.parametrize("seed", range(64))
def test_random_sharing_batch_cascade(seed):
    wl, groups = _random_sharing_batch(seed)
    e, _, _ = check_step(wl, groups=groups)
    print(f"seed {seed}: S={wl.num_seqs} T={wl.num_tokens} Hq={wl.num_q_heads} "
          f"Hkv={wl.num_kv_heads} D={wl.head_dim} {wl.q_dtype}/{wl.kv_dtype} "
          f"P={wl.partition_size} groups={[len(g) for g in groups[0]]} "
          f"prefix blocks={groups[1]}: {e}", flush=True)


@pytest.mark.parametrize("seed", range(16))
def test_random_sharing_decode_batch_cascade(seed):
    """The sharing batches as decode steps at the balanced split: the group
    and decode pieces share one launch, and the plan charges each group
    segment's start as work when it cuts the group stream."""
    wl, groups = _random_sharing_batch(seed, decode=True)
    assert wl.is_decode
    e, _, _ = check_step(wl, groups=groups)
    print(f"seed {seed}: S={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
          f"D={wl.head_dim} {wl.q_dtype}/{wl.kv_dtype} groups={[len(g) for g in groups[0]]} "
          f"prefix blocks={groups[1]}: {e}", flush=True)


@pytest.mark.parametrize("seed", range(12))
def test_random_tree_batch(seed):
    """Random batches whose spans are candidate trees of draft tokens (one
    ancestor-or-self word per token; spans past 64 tokens stay causal),
    "03 -- Engines Papers", sections 5 to 7."""
    from tests.test_gpu_tree import _tree_step
    wl = _random_batch(100 + seed)
    masks = W.batch_tree_masks(wl.query_lens, seed=seed)
    e, _, _ = _tree_step(wl, masks)
    print(f"seed {seed}: S={wl.num_seqs} T={wl.num_tokens} Hq={wl.num_q_heads} "
          f"{wl.q_dtype}/{wl.kv_dtype} P={wl.partition_size}: {e}", flush=True)
