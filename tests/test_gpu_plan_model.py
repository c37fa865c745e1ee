"""The device plan equals the host model of it (tests/plan_model.py), record
for record, on the batches the model's CPU replay checks: the work list a
run streams, the cut segments the merge completes and the cascade records.
With that, the CPU replay's checks (indices in range, one writer per slot
row, cascade row and output row, merge reads matched to their writers)
hold for what the device builds."""
import numpy as np
import pytest
import torch

import paged_kv_cache_213_amd as pa
from paged_kv_cache_213_amd import workloads as W
from tests import plan_model as PM
from tests.test_gpu_random_batches import _random_sharing_batch

pytestmark = pytest.mark.gpu


def _device_plan(wl, groups, P):
    """Run the plan on the device; return (layout info, workspace bytes)."""
    d = torch.device("cuda")
    hybrid = not wl.is_decode
    dt = {"f32": pa.PA_F32, "bf16": pa.PA_BF16, "fp8": pa.PA_FP8_E4M3FN}
    shape = pa.PaShape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 16,
                       int(wl.num_blocks), wl.block_tables.shape[1], dt[wl.q_dtype],
                       dt[wl.kv_dtype], P, int(groups is not None), 0)
    mq = wl.max_query_len if hybrid else 1
    nbytes = pa.workspace_bytes(shape, wl.num_seqs, wl.num_tokens, wl.max_context_len, mq)
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device=d)
    cl = torch.from_numpy(wl.context_lens).to(d)
    qsl = torch.from_numpy(wl.query_start_loc).to(d) if hybrid else None
    if groups is not None:
        pg = pa.PrefixGroups(groups[0], groups[1], d)
        pa.plan_cascade(shape, cl, ws, pg, query_start_loc=qsl, num_q_tokens=wl.num_tokens,
                        max_query_len=mq, max_context_len=wl.max_context_len)
    else:
        pa.plan(shape, cl, ws, query_start_loc=qsl, num_q_tokens=wl.num_tokens,
                max_query_len=mq, max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    info = pa.workspace_layout(shape, wl.num_seqs, wl.num_tokens, wl.max_context_len, mq,
                               decode=not hybrid)
    return info, ws.cpu().numpy()


def _ints(buf, off, count, width):
    return np.frombuffer(buf[off:off + 4 * count * width].tobytes(), np.int32).reshape(count,
                                                                                       width)


def _compare(wl, groups, P):
    info, buf = _device_plan(wl, groups, P)
    hybrid = not wl.is_decode
    G = wl.num_q_heads // wl.num_kv_heads
    lay = PM.make_layout(G=G, Hkv=wl.num_kv_heads, num_seqs=wl.num_seqs,
                         num_tokens=wl.num_tokens, max_context_len=wl.max_context_len,
                         max_query_len=wl.max_query_len if hybrid else 1, decode=not hybrid,
                         partition_size=P, cascade=groups is not None,
                         waves=tuple(info.waves), wide_nt=info.wide_row_tiles,
                         f32=wl.kv_dtype == "f32", part_cost=tuple(info.part_cost),
                         span_shared=info.span_shared, group_nt=info.group_row_tiles)
    qsl = np.asarray(wl.query_start_loc) if hybrid else None
    plan = PM.build_plan(lay, Hkv=wl.num_kv_heads, context_lens=wl.context_lens, qsl=qsl,
                         num_tokens=wl.num_tokens, max_context_len=wl.max_context_len,
                         groups=groups)
    members = [int(i) for g in groups[0] for i in g] if groups is not None else []
    PM.check_plan(plan, lay, G=G, Hkv=wl.num_kv_heads, num_seqs=wl.num_seqs,
                  num_tokens=wl.num_tokens, qsl=qsl, group_members=members)
    hdr = _ints(buf, 0, 1, info.header_words)[0]
    ntiles, nsplit, ncas = int(hdr[0]), int(hdr[1]), int(hdr[2])
    assert ntiles == len(plan.tiles)
    tiles = _ints(buf, info.off_tiles, ntiles, 12)
    want = np.array([[t.seq, t.qtok0, t.ntok, t.nb, t.L, t.qs, t.nspan, t.flags, t.b0]
                     for t in plan.tiles], np.int32).reshape(-1, 9)
    assert np.array_equal(tiles[:, :9], want), "tile records differ"
    for st in (0, 1, 2):
        B, R, V = (int(x) for x in hdr[4 + 4 * st: 7 + 4 * st])
        assert (B, R, V) == (plan.B[st], plan.R[st], len(plan.pieces[st])), f"stream {st}"
        if V:
            ps = _ints(buf, info.off_pieces[st], V, 16)
            assert np.array_equal(ps[:, :4], np.array(plan.pieces[st], np.int32)), \
                f"piece records of stream {st} differ"
            assert np.array_equal(ps[:, 4:13], tiles[ps[:, 0], :9]), "piece tile copies differ"
    assert nsplit == len(plan.splits)
    sp = _ints(buf, info.off_splits, max(nsplit, 1), 8)[:nsplit, :6]
    # the device lists cut segments in any order
    assert sorted(map(tuple, sp.tolist())) == sorted(plan.splits), "cut segments differ"
    if groups is not None:
        S = wl.num_seqs
        cs = _ints(buf, info.off_cas_seq, 6, S)
        assert cs[0].tolist() == plan.cas_prefix
        assert cs[1].tolist() == plan.cas_tile
        assert cs[2].tolist() == plan.cas_gtile
        assert cs[3].tolist() == plan.cas_pos
        assert ncas == len(plan.cas_recs)
        cr = _ints(buf, info.off_cas_recs, max(ncas, 1), 8)[:ncas, :7]
        assert [tuple(r) for r in cr.tolist()] == plan.cas_recs, "cascade records differ"
    return len(plan.tiles), len(plan.splits), len(plan.cas_recs)


@pytest.mark.parametrize("name,P,grouped", [("c4", 512, True), ("c4", 16, True), ("c4", 0, True),
                                            ("c5", 0, True), ("c5", 16, True), ("c2", 0, False),
                                            ("c3", 512, False), ("c1", 0, False)])
def test_small_plans_equal_the_model(name, P, grouped):
    wl = W.make_config(name, small=True)
    groups = (wl.shared_groups, wl.shared_prefix_blocks) if grouped else None
    print(name, P, _compare(wl, groups, P), flush=True)


@pytest.mark.parametrize("name,P,grouped", [("c5", 0, True), ("c4", 0, True), ("c3", 0, False),
                                            ("c2", 0, False)])
def test_full_plans_equal_the_model(name, P, grouped):
    wl = W.make_config(name)
    groups = (wl.shared_groups, wl.shared_prefix_blocks) if grouped else None
    print(name, P, _compare(wl, groups, P), flush=True)


@pytest.mark.parametrize("seed", range(0, 64, 4))
def test_random_sharing_plans_equal_the_model(seed):
    wl, groups = _random_sharing_batch(seed)
    print(seed, _compare(wl, groups, wl.partition_size), flush=True)
