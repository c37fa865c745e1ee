"""CPU replay of the attention library's work decomposition (plan records,
piece walks, partial slots, cascade buffers and the merge's reads) over
the batches on which builds of the wide kernel once gave wrong rows or
faulted: the small hybrid batch with its sharing group at its 512-token
partition size, the full parallel-sampling batch with its groups, and the
64 random sharing batches of the GPU suite. Each replay asserts that
every index is in range, that no two segments write one slot row, cascade
row or output row, and that every merge read finds the partial the right
segment wrote for the right row (tests/plan_model.py). The resident
counts include the device's (512 span workgroups, 1024 narrow and group
waves) and
odd ones, for the wide, narrow and group streams."""
import numpy as np
import pytest

from paged_kv_cache_213_amd import workloads as W
from tests import plan_model as PM
from tests.test_gpu_random_batches import _random_batch, _random_sharing_batch

WAVES = [(512, 1024, 1024), (1024, 1024, 1024), (37, 13, 29), (8192, 8192, 8192), (512, 256, 64)]


def _groups(wl):
    return (wl.shared_groups, wl.shared_prefix_blocks)


@pytest.mark.parametrize("waves", WAVES)
@pytest.mark.parametrize("P", [None, 16, 0])
@pytest.mark.parametrize("name", ["c4", "c5"])
def test_small_sharing_batches(name, P, waves):
    wl = W.make_config(name, small=True)
    _, _, c = PM.replay_workload(wl, waves=waves, groups=_groups(wl), partition_size=P)
    assert c["cascade_records"] > 0


@pytest.mark.parametrize("waves", WAVES[:3])
def test_full_sampling_batch_with_groups(waves):
    wl = W.make_config("c5")
    _, _, c = PM.replay_workload(wl, waves=waves, groups=_groups(wl), partition_size=0)
    assert c["cascade_records"] == wl.num_seqs * wl.num_kv_heads


def test_full_hybrid_batch_with_groups():
    wl = W.make_config("c4")
    PM.replay_workload(wl, waves=(512, 1024, 1024), groups=_groups(wl), partition_size=0)


@pytest.mark.parametrize("seed", range(64))
def test_random_sharing_batches(seed):
    wl, groups = _random_sharing_batch(seed)
    for waves in ((512, 1024, 1024), (37, 13, 29)):
        PM.replay_workload(wl, waves=waves, groups=groups)


@pytest.mark.parametrize("seed", range(16))
def test_random_sharing_decode_batches(seed):
    """The GPU suite's sharing batches as decode steps: the group stream is
    cut with its segment start cost."""
    wl, groups = _random_sharing_batch(seed, decode=True)
    for waves in ((512, 1024, 1024), (37, 13, 29), (8192, 8192, 8192)):
        _, lay, _ = PM.replay_workload(wl, waves=waves, groups=groups)
        assert lay.part_cost[2] == PM.GROUP_COST_NO_SPANS


@pytest.mark.parametrize("name,P", [("c1", None), ("c2", None), ("c3", None), ("c3", 0),
                                    ("c4", None), ("c4", 0), ("c5", 0)])
def test_full_configs_without_groups(name, P):
    wl = W.make_config(name)
    PM.replay_workload(wl, waves=(512, 1024, 1024), partition_size=P)


@pytest.mark.parametrize("seed", range(24))
def test_random_hybrid_batches(seed):
    wl = _random_batch(seed)
    PM.replay_workload(wl, waves=(512, 1024, 1024))


@pytest.mark.parametrize("seed", range(24))
def test_random_hybrid_batches_with_shared_spans(seed):
    """With the span launch beside the narrow ones (span_shared workgroups),
    the replay's checks still hold; the span stream gets span_shared
    pieces per call exactly where the others hold twice its work."""
    wl = _random_batch(seed)
    plan, lay, _ = PM.replay_workload(wl, waves=(512, 1024, 1024), span_shared=256,
                                      partition_size=0)
    PM.replay_workload(wl, waves=(37, 13, 29), span_shared=11, partition_size=0)
    plan0, _, _ = PM.replay_workload(wl, waves=(512, 1024, 1024), partition_size=0)
    assert len(plan.pieces[1]) == len(plan0.pieces[1])
    assert len(plan.pieces[2]) == len(plan0.pieces[2])
    assert len(plan.pieces[0]) <= len(plan0.pieces[0])


def test_hybrid_batch_shares_the_device_only_when_decodes_dominate():
    """The 512-token chunk beside 128 decodes (decodes hold 8x the span's
    work) is cut for one span workgroup per compute unit; the same chunk
    alone, and the chunk with named 512-token partitions, keep the span
    kernel's whole residency (or the partition size)."""
    wl = W.make_config("c4")
    H = wl.num_kv_heads
    shared, _, _ = PM.replay_workload(wl, waves=(512, 1024, 1024), span_shared=256,
                                      partition_size=0)
    alone, _, _ = PM.replay_workload(wl, waves=(512, 1024, 1024), partition_size=0)
    assert len(shared.pieces[0]) <= 256 < len(alone.pieces[0]) <= 512
    assert len(shared.pieces[0]) % H == 0
    # only the chunk: no single-token work, the span stream keeps 512
    chunk = W.custom_workload([4096], num_q_heads=wl.num_q_heads, num_kv_heads=H,
                              head_dim=wl.head_dim, q_dtype="bf16", kv_dtype="bf16", seed=5,
                              query_lens=[512])
    a, _, _ = PM.replay_workload(chunk, waves=(512, 1024, 1024), span_shared=256,
                                 partition_size=0)
    b, _, _ = PM.replay_workload(chunk, waves=(512, 1024, 1024), partition_size=0)
    assert [p[:4] for p in a.pieces[0]] == [p[:4] for p in b.pieces[0]]
    # fixed partitions: pieces of P / 16 blocks either way
    a, _, _ = PM.replay_workload(wl, waves=(512, 1024, 1024), span_shared=256, partition_size=512)
    b, _, _ = PM.replay_workload(wl, waves=(512, 1024, 1024), partition_size=512)
    assert [p[:4] for p in a.pieces[0]] == [p[:4] for p in b.pieces[0]]


@pytest.mark.parametrize("cost", [(0, 0, 0), (1, 3, 2), (12, 7, 40)])
@pytest.mark.parametrize("seed", range(6))
def test_part_costs(seed, cost):
    """Pieces cut at equal blocks plus a cost per segment started: whatever
    the costs, each head's pieces cover its blocks once, no piece is empty,
    and the splits and merge reads stay consistent."""
    wl, groups = _random_sharing_batch(seed)
    for waves in ((512, 1024, 1024), (37, 13, 29)):
        plan, _, _ = PM.replay_workload(wl, waves=waves, groups=groups, part_cost=cost)
        for st in (0, 1, 2):
            assert all(p[3] > 0 for p in plan.pieces[st])


def test_part_cost_moves_blocks_off_pieces_that_start_many_segments():
    """With a cost per segment, a piece that starts many short segments
    holds fewer blocks than one inside a long segment."""
    wl = W.make_config("c2")
    plan, _, _ = PM.replay_workload(wl, waves=(512, 1024, 1024), part_cost=(0, 8, 0))
    nb = {}
    for (t, kvh, j, n) in plan.pieces[1]:
        nb.setdefault(kvh, []).append(n)
    spread = max(max(v) - min(v) for v in nb.values())
    plan0, _, _ = PM.replay_workload(wl, waves=(512, 1024, 1024), part_cost=(0, 0, 0))
    spread0 = max(max(p[3] for p in plan0.pieces[1][h::wl.num_kv_heads]) -
                  min(p[3] for p in plan0.pieces[1][h::wl.num_kv_heads][:-1])
                  for h in range(wl.num_kv_heads))
    assert spread0 == 0 and spread > 0


def test_model_catches_a_planted_slot_slip():
    """The replay is able to fail: a plan whose merge reads the head slot
    of a segment's first piece (in place of its tail slot) is rejected."""
    wl = W.make_config("c4", small=True)
    lay = PM.make_layout(G=4, Hkv=wl.num_kv_heads, num_seqs=wl.num_seqs,
                         num_tokens=wl.num_tokens, max_context_len=wl.max_context_len,
                         max_query_len=wl.max_query_len, decode=False, partition_size=16,
                         cascade=False, waves=(512, 1024, 1024))
    qsl = np.asarray(wl.query_start_loc)
    plan = PM.build_plan(lay, Hkv=wl.num_kv_heads, context_lens=wl.context_lens, qsl=qsl,
                         num_tokens=wl.num_tokens, max_context_len=wl.max_context_len)
    assert plan.splits
    row0, ntok, kvh, k0, k1, st = plan.splits[0]
    plan.splits[0] = (row0, ntok, kvh, k0 + 1, k1, st)  # drops the first piece
    with pytest.raises(AssertionError):
        PM.check_plan(plan, lay, G=4, Hkv=wl.num_kv_heads, num_seqs=wl.num_seqs,
                      num_tokens=wl.num_tokens, qsl=qsl, group_members=[])


def _lib_layout(wl, groups, P, hybrid):
    import paged_kv_cache_213_amd as pa
    pa.load_library()
    dt = {"f32": pa.PA_F32, "bf16": pa.PA_BF16, "fp8": pa.PA_FP8_E4M3FN}
    shape = pa.PaShape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 16, 1000,
                       wl.block_tables.shape[1], dt[wl.q_dtype], dt[wl.kv_dtype], P,
                       int(groups is not None), 0)
    mq = wl.max_query_len if hybrid else 1
    info = pa.workspace_layout(shape, wl.num_seqs, wl.num_tokens, wl.max_context_len, mq,
                               decode=not hybrid)
    return shape, info


@pytest.mark.parametrize("name,P,grouped", [("c2", 0, False), ("c3", 512, False),
                                            ("c4", 0, True), ("c4", 512, False),
                                            ("c5", 0, True), ("c1", 0, False)])
def test_model_layout_equals_the_librarys(name, P, grouped):
    """The model's workspace bounds are the library's (host-only call; with
    no device to query, both take the 8192-wave bound)."""
    import paged_kv_cache_213_amd as pa
    wl = W.make_config(name)
    groups = _groups(wl) if grouped else None
    hybrid = not wl.is_decode
    shape, info = _lib_layout(wl, groups, P, hybrid)
    lay = PM.make_layout(G=wl.num_q_heads // wl.num_kv_heads, Hkv=wl.num_kv_heads,
                         num_seqs=wl.num_seqs, num_tokens=wl.num_tokens,
                         max_context_len=wl.max_context_len,
                         max_query_len=wl.max_query_len if hybrid else 1, decode=not hybrid,
                         partition_size=P, cascade=grouped, waves=tuple(info.waves),
                         wide_nt=info.wide_row_tiles, f32=wl.kv_dtype == "f32",
                         span_shared=info.span_shared, group_nt=info.group_row_tiles)
    assert (lay.narrow_tokens, lay.wide_tokens, lay.part_blocks, lay.members_per_tile) == (
        info.narrow_tokens, info.wide_tokens, info.part_blocks, info.members_per_tile)
    assert lay.max_tiles == info.max_tiles and lay.max_splits == info.max_splits
    assert lay.max_pieces == tuple(info.max_pieces)
    assert lay.max_cas_recs == info.max_cas_recs
    assert lay.part_cost == tuple(info.part_cost)
    assert lay.span_shared == info.span_shared
    mq = wl.max_query_len if hybrid else 1
    assert info.total <= pa.workspace_bytes(shape, wl.num_seqs, wl.num_tokens,
                                            wl.max_context_len, mq)


def test_group_start_cost_only_without_spans():
    """A decode batch with groups charges each group segment's start eight
    blocks of work, so group pieces that start more segments hold fewer
    blocks; a hybrid batch (spans) charges none."""
    wl = W.make_config("c5")
    plan, lay, _ = PM.replay_workload(wl, waves=(512, 1024, 1024), groups=_groups(wl),
                                      partition_size=0)
    assert lay.part_cost == (6, 0, 8)
    # segments each group piece touches, against its blocks
    segs = {}
    for k, (t, kvh, j, n) in enumerate(plan.pieces[2]):
        tiles = [t]
        left = n - min(n, plan.tiles[t].nb - j)
        while left > 0:
            t += 1
            tiles.append(t)
            left -= min(left, plan.tiles[t].nb)
        segs.setdefault(len(tiles), []).append(n)
    assert len(segs) > 1
    ks = sorted(segs)
    assert max(segs[ks[-1]]) < max(segs[ks[0]])
    hyb = W.make_config("c4")
    _, lay4, _ = PM.replay_workload(hyb, waves=(512, 1024, 1024), groups=_groups(hyb),
                                    partition_size=0)
    assert lay4.part_cost == (6, 0, 0)
