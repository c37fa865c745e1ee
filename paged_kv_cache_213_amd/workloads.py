"""Seeded synthetic inputs for paged attention.

This module only draws data: sequence lengths, physical block pools, block
tables, slot mappings and random values. It holds none of the attention
arithmetic, and it imports neither the HIP binding nor the CPU oracle; both
sides consume what it produces.

The workloads follow the shapes the pages give for paged KV storage:
16-token physical blocks reached through a per-sequence block table
("03 -- Engines Papers", section 2, key trick), continuously batched
sequences with different context lengths (same page, section 1), GQA head
groups ("References", GQA entry), chunked-prefill spans mixed with decodes
(section 3 of the first page) and blocks shared across sequences with a
refcount under copy-on-write (section 2, "What to extract").

Cache layouts produced here (the library's contract):
  K: [num_blocks][Hkv][16][D]   one block-head is 16 token rows of D values
  V: [num_blocks][Hkv][D][16]   one block-head is D rows of 16 token values
Unused slots (tails of last blocks, unused pool blocks, and the slots this
step's new tokens will be appended into) hold NaN, so any read of them shows.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK = 16

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")

CONFIG_TITLES = {
    "c1": "tiny paged decode fp32: 4 seqs {7,16,33,50}, pool 32, GQA 2:1, D=64",
    "c2": "Llama-3-8B-shaped decode bf16: 64 seqs, L~U[128,4096], 32q/8kv, D=128",
    "c3": "long-context split-KV bf16: 256 seqs, L~logU[16,32768], P=512",
    "c4": "hybrid chunked prefill bf16: 512-token chunk at 3584..4095 + 128 decodes",
    "c5": "70B-shaped decode, fp8 e4m3 KV with per-(block,head) scale, G=8",
}


@dataclass
class Workload:
    """Metadata of one synthetic batch (host numpy arrays, int32)."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str  # "f32" | "bf16"  (also the dtype of new K/V rows and of out)
    kv_dtype: str  # "f32" | "bf16" | "fp8"
    context_lens: np.ndarray  # [S] keys each sequence attends over, new tokens included
    query_lens: np.ndarray  # [S] query tokens per sequence (1 for a decode)
    block_tables: np.ndarray  # [S][max_blocks] physical block ids, -1 padded
    num_blocks: int  # size of the physical pool
    partition_size: int  # split-KV partition in tokens (0 = library default)
    seed: int
    shared_groups: list = field(default_factory=list)  # lists of seqs sharing blocks
    shared_prefix_blocks: list = field(default_factory=list)  # per group: shared leading blocks
    # explicit list of slots this step appends (defaults: every query token's slot)
    _slot_mapping: Optional[np.ndarray] = None

    # ---- derived shapes -------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_lens.sum())

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.query_lens == 1))

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def query_start_loc(self) -> np.ndarray:
        qsl = np.zeros(self.num_seqs + 1, dtype=np.int32)
        np.cumsum(self.query_lens, out=qsl[1:])
        return qsl

    @property
    def scale(self) -> float:
        """1/sqrt(D) as the float32 the kernels receive."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def token_positions(self) -> np.ndarray:
        """Position in its sequence of every query token: the last n_i slots."""
        pos = np.empty(self.num_tokens, dtype=np.int64)
        qsl = self.query_start_loc
        for i in range(self.num_seqs):
            n, L = int(self.query_lens[i]), int(self.context_lens[i])
            pos[qsl[i]:qsl[i + 1]] = np.arange(L - n, L)
        return pos

    def token_seq(self) -> np.ndarray:
        return np.repeat(np.arange(self.num_seqs), self.query_lens)

    @property
    def slot_mapping(self) -> np.ndarray:
        """Physical slot (block*16 + offset) of every token appended this step."""
        if self._slot_mapping is not None:
            return self._slot_mapping
        pos = self.token_positions()
        seq = self.token_seq()
        ok = pos >= 0
        blk = self.block_tables[seq, np.where(ok, pos, 0) // BLOCK].astype(np.int64)
        return np.where(ok, blk * BLOCK + pos % BLOCK, -1).astype(np.int32)

    # ---- byte / flop accounting (measurement, not the method) -----------
    @property
    def kv_elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]

    @property
    def q_elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2}[self.q_dtype]

    def kv_bytes_logical(self) -> int:
        """K and V bytes the method must read: each sequence reads its own
        context once per KV head (a shared block counts once per reader).
        This is the KV-cache byte formula of "The LLM inference engine
        playbook", Theme 11 stage 0, for one layer, with heads = KV heads."""
        per_tok = 2 * self.num_kv_heads * self.head_dim * self.kv_elem_bytes
        b = int(self.context_lens.astype(np.int64).sum()) * per_tok
        if self.kv_dtype == "fp8":
            nblk = int(np.sum((self.context_lens.astype(np.int64) + BLOCK - 1) // BLOCK))
            b += nblk * self.num_kv_heads * 2 * 4
        return b

    def kv_bytes_unique(self) -> int:
        """Bytes of distinct physical blocks touched (shared blocks once)."""
        used = set()
        full_tok = 0
        for i in range(self.num_seqs):
            L = int(self.context_lens[i])
            nb = (L + BLOCK - 1) // BLOCK
            for j in range(nb):
                b = int(self.block_tables[i, j])
                if b in used:
                    continue
                used.add(b)
                full_tok += min(BLOCK, L - j * BLOCK)
        per_tok = 2 * self.num_kv_heads * self.head_dim * self.kv_elem_bytes
        extra = len(used) * self.num_kv_heads * 2 * 4 if self.kv_dtype == "fp8" else 0
        return full_tok * per_tok + extra

    def attended_keys(self) -> int:
        """Sum over query tokens of the keys each one attends to (causal)."""
        return int((self.token_positions() + 1).sum())

    def flops(self) -> int:
        """2 flops per multiply-add, QK^T and PV: 4 * Hq * D per (query, key)."""
        return 4 * self.num_q_heads * self.head_dim * self.attended_keys()

    def io_bytes(self) -> int:
        """q in + out written."""
        return self.num_tokens * self.num_q_heads * self.head_dim * 2 * self.q_elem_bytes


# --------------------------------------------------------------------------
# metadata builders
# --------------------------------------------------------------------------

def _blocks_for(L: int) -> int:
    return (L + BLOCK - 1) // BLOCK


def _tables_from_perm(lens, perm) -> np.ndarray:
    """Sequences take consecutive chunks of a shuffled pool, in order."""
    nbs = [_blocks_for(int(L)) for L in lens]
    width = max(1, max(nbs))
    bt = np.full((len(lens), width), -1, dtype=np.int32)
    cur = 0
    for i, nb in enumerate(nbs):
        bt[i, :nb] = perm[cur:cur + nb]
        cur += nb
    return bt


def _pool(rng, needed: int, factor: float = 1.25):
    nblk = max(needed, int(math.ceil(factor * needed)))
    return nblk, rng.permutation(nblk).astype(np.int32)


def _c1(seed: int, small: bool) -> Workload:
    rng = np.random.default_rng(seed)
    lens = np.array([7, 16, 33, 50], dtype=np.int32)
    perm = rng.permutation(32).astype(np.int32)
    bt = _tables_from_perm(lens, perm)
    return Workload("c1", 2, 1, 64, "f32", "f32", lens, np.ones(4, np.int32), bt, 32, 0, seed)


def _plain_decode(name, seed, nseq, lens, hq, hkv, d, part, kv="bf16") -> Workload:
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens(rng), dtype=np.int32) if callable(lens) else np.asarray(lens, np.int32)
    need = int(sum(_blocks_for(int(L)) for L in lens))
    nblk, perm = _pool(rng, need)
    bt = _tables_from_perm(lens, perm)
    return Workload(name, hq, hkv, d, "bf16", kv, lens, np.ones(len(lens), np.int32), bt, nblk, part, seed)


def _c2(seed: int, small: bool) -> Workload:
    n, lo, hi = (8, 128, 1100) if small else (64, 128, 4096)
    return _plain_decode("c2", seed, n, lambda r: r.integers(lo, hi + 1, size=n), 32, 8, 128, 0)


def _loguniform(rng, n, lo, hi):
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def _c3(seed: int, small: bool) -> Workload:
    n, hi = (12, 3000) if small else (256, 32768)
    return _plain_decode("c3", seed, n, lambda r: _loguniform(r, n, 16, hi), 32, 8, 128, 512)


def _c4(seed: int, small: bool) -> Workload:
    """One prefill chunk (the last n_p positions of L_p) plus decodes; half of
    the decodes share the physical blocks of a common prefix."""
    rng = np.random.default_rng(seed)
    if small:
        chunk, Lp, ndec, nshare, prefix, maxL = 72, 600, 16, 8, 128, 900
    else:
        chunk, Lp, ndec, nshare, prefix, maxL = 512, 4096, 128, 64, 1024, 8192
    pb = prefix // BLOCK
    lens = [Lp]
    lens += list(rng.integers(prefix + 1, maxL + 1, size=nshare))  # sharers
    lens += list(rng.integers(1, maxL + 1, size=ndec - nshare))  # private decodes
    lens = np.asarray(lens, dtype=np.int32)
    qlens = np.ones(len(lens), dtype=np.int32)
    qlens[0] = chunk
    need = pb + sum(_blocks_for(int(L)) for L in lens[:1]) \
        + sum(_blocks_for(int(L)) - pb for L in lens[1:1 + nshare]) \
        + sum(_blocks_for(int(L)) for L in lens[1 + nshare:])
    nblk, perm = _pool(rng, need)
    width = max(_blocks_for(int(L)) for L in lens)
    bt = np.full((len(lens), width), -1, dtype=np.int32)
    cur = 0
    shared = perm[cur:cur + pb]
    cur += pb
    for i, L in enumerate(lens):
        nb = _blocks_for(int(L))
        if 1 <= i <= nshare:
            bt[i, :pb] = shared
            bt[i, pb:nb] = perm[cur:cur + nb - pb]
            cur += nb - pb
        else:
            bt[i, :nb] = perm[cur:cur + nb]
            cur += nb
    groups = [list(range(1, 1 + nshare))]
    return Workload("c4", 32, 8, 128, "bf16", "bf16", lens, qlens, bt, nblk, 512, seed,
                    shared_groups=groups, shared_prefix_blocks=[pb])


def _c5(seed: int, small: bool) -> Workload:
    """4-way parallel-sampling groups: all blocks but the last are shared;
    each member owns a private copy of the last (partial) block."""
    rng = np.random.default_rng(seed)
    ngroups, lo, hi = (4, 100, 1500) if small else (32, 1024, 16384)
    glens = rng.integers(lo, hi + 1, size=ngroups)
    need = sum(_blocks_for(int(L)) - 1 + 4 for L in glens)
    nblk, perm = _pool(rng, need)
    width = max(_blocks_for(int(L)) for L in glens)
    lens, groups = [], []
    bt = np.full((4 * ngroups, width), -1, dtype=np.int32)
    cur = 0
    for gi, L in enumerate(glens):
        nb = _blocks_for(int(L))
        shared = perm[cur:cur + nb - 1]
        cur += nb - 1
        members = []
        for m in range(4):
            s = 4 * gi + m
            bt[s, :nb - 1] = shared
            bt[s, nb - 1] = perm[cur]
            cur += 1
            lens.append(int(L))
            members.append(s)
        groups.append(members)
    lens = np.asarray(lens, dtype=np.int32)
    return Workload("c5", 64, 8, 128, "bf16", "fp8", lens, np.ones(len(lens), np.int32), bt,
                    nblk, 0, seed, shared_groups=groups,
                    shared_prefix_blocks=[_blocks_for(int(L)) - 1 for L in glens])


_BUILDERS = {"c1": _c1, "c2": _c2, "c3": _c3, "c4": _c4, "c5": _c5}


def make_config(name: str, seed: Optional[int] = None, small: bool = False) -> Workload:
    """Build one of the five configurations. ``small`` gives a reduced batch
    that still spans several partitions and ragged block tails."""
    if name not in _BUILDERS:
        raise KeyError(f"unknown config {name!r}; expected one of {CONFIG_NAMES}")
    if seed is None:
        seed = 1000 + CONFIG_NAMES.index(name)
    return _BUILDERS[name](seed, small)


def custom_workload(context_lens, query_lens=None, *, num_q_heads=4, num_kv_heads=1,
                    head_dim=64, q_dtype="bf16", kv_dtype="bf16", partition_size=0,
                    seed=0, pool_factor=1.25, block_tables=None, num_blocks=None,
                    name="custom") -> Workload:
    """Arbitrary small batch with a shuffled pool (for edge-case tests)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int32)
    ql = np.ones(len(lens), np.int32) if query_lens is None else np.asarray(query_lens, np.int32)
    if block_tables is None:
        need = int(sum(_blocks_for(int(L)) for L in lens))
        nblk, perm = _pool(rng, max(need, 1), pool_factor)
        bt = _tables_from_perm(lens, perm)
    else:
        bt = np.asarray(block_tables, dtype=np.int32)
        nblk = int(num_blocks)
    return Workload(name, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype, lens, ql,
                    bt, nblk, partition_size, seed)


def random_tree_parents(rng, n: int) -> list:
    """A random candidate tree of n draft tokens in topological order:
    parent[j] < j, -1 for a node hanging off the committed context."""
    return [-1] + [int(rng.integers(-1, j)) for j in range(1, n)]


def tree_masks(parents) -> list:
    """Ancestor-or-self bit masks of a tree given by parent indices: bit k
    of word j is set when node k lies on the path from the context to node
    j (the visibility of a candidate tree, "03 -- Engines Papers",
    sections 5 to 7). A chain (parent j - 1) gives the causal masks."""
    masks = []
    for j, p in enumerate(parents):
        m = 1 << j
        while p >= 0:
            m |= 1 << p
            p = parents[p]
        masks.append(m)
    return masks


def batch_tree_masks(query_lens, seed: int, chain: bool = False) -> np.ndarray:
    """uint64 [sum(query_lens)]: one random tree (or chain) per span of at
    most 64 tokens; longer spans get all-ones words (they stay causal)."""
    rng = np.random.default_rng(seed)
    out = []
    for n in (int(x) for x in query_lens):
        if n > 64:
            out += [(1 << 64) - 1] * n
            continue
        par = [j - 1 for j in range(n)] if chain else random_tree_parents(rng, n)
        out += tree_masks(par)
    return np.array(out, dtype=np.uint64)


# --------------------------------------------------------------------------
# values
# --------------------------------------------------------------------------

@dataclass
class Values:
    """Random tensors for one workload (torch tensors on one device).

    q, k_new, v_new are in the query dtype (float32 or bfloat16).
    For f32/bf16 KV: k_cache/v_cache hold the pre-append cache in its stored
    dtype. For fp8 KV: k_src/v_src hold the float32 source values in cache
    layout (bf16-representable, NaN where unused) with per-(block, KV head)
    scales; turning them into e4m3 bytes is the caller's job (it is the
    append's own arithmetic).
    """

    q: "object"
    k_new: "object"
    v_new: "object"
    k_cache: "object" = None
    v_cache: "object" = None
    k_src: "object" = None
    v_src: "object" = None
    k_scale: "object" = None
    v_scale: "object" = None


def _poison_slots(k, v, blocks, offs):
    """Set slot rows of K ([NB][H][16][D]) and V ([NB][H][D][16]) to NaN."""
    import torch
    if len(blocks) == 0:
        return
    b = torch.as_tensor(np.asarray(blocks, np.int64), device=k.device)
    o = torch.as_tensor(np.asarray(offs, np.int64), device=k.device)
    k.permute(0, 2, 1, 3)[b, o] = float("nan")
    v.permute(0, 3, 1, 2)[b, o] = float("nan")


def materialize(wl: Workload, device="cpu", value_scale: float = 1.0) -> Values:
    """Draw N(0,1) values for q and the whole block pool, with a torch
    generator seeded by the workload seed on ``device``."""
    import torch

    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(wl.seed))
    NB, H, D = wl.num_blocks, wl.num_kv_heads, wl.head_dim
    tdt = torch.float32 if wl.q_dtype == "f32" else torch.bfloat16

    def draw(*shape):
        x = torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)
        if value_scale != 1.0:
            x.mul_(value_scale)
        if wl.q_dtype == "bf16" or wl.kv_dtype != "f32":
            x = x.to(torch.bfloat16).to(torch.float32)  # bf16-representable values
        return x

    k = draw(NB, H, BLOCK, D)
    v = draw(NB, H, D, BLOCK)
    q = draw(wl.num_tokens, wl.num_q_heads, D).to(tdt)

    # copy-on-write images: a member's private last block copies the group's
    # tail slots before its own new token (parallel-sampling layout)
    for grp in wl.shared_groups:
        L0 = int(wl.context_lens[grp[0]])
        last0 = (L0 - 1) // BLOCK
        if all(int(wl.context_lens[s]) == L0 for s in grp):
            src = int(wl.block_tables[grp[0], last0])
            o = (L0 - 1) % BLOCK
            for s in grp[1:]:
                dst = int(wl.block_tables[s, last0])
                if dst != src and o > 0:
                    k[dst, :, :o, :] = k[src, :, :o, :]
                    v[dst, :, :, :o] = v[src, :, :, :o]

    # tails past each context are not data
    tb, to = [], []
    for i in range(wl.num_seqs):
        L = int(wl.context_lens[i])
        if L % BLOCK:
            b = int(wl.block_tables[i, L // BLOCK])
            for o in range(L % BLOCK, BLOCK):
                tb.append(b)
                to.append(o)
    _poison_slots(k, v, tb, to)

    used = np.zeros(NB, dtype=bool)
    for i in range(wl.num_seqs):
        nb = _blocks_for(int(wl.context_lens[i]))
        used[wl.block_tables[i, :nb]] = True
    unused = torch.as_tensor(np.nonzero(~used)[0], device=dev)
    if unused.numel():
        k[unused] = float("nan")
        v[unused] = float("nan")

    # this step's new rows: the values at their slots, then poison the slots
    all_slots = wl.slot_mapping.astype(np.int64)
    has = all_slots >= 0
    slots = all_slots[has]
    k_new = torch.zeros(wl.num_tokens, H, D, device=dev)
    v_new = torch.zeros(wl.num_tokens, H, D, device=dev)
    if slots.size:
        sb = torch.as_tensor(slots // BLOCK, device=dev)
        so = torch.as_tensor(slots % BLOCK, device=dev)
        idx = torch.as_tensor(np.nonzero(has)[0], device=dev)
        k_new[idx] = k.permute(0, 2, 1, 3)[sb, so]  # [T][H][D]
        v_new[idx] = v.permute(0, 3, 1, 2)[sb, so]
    out = Values(q=q, k_new=k_new.to(tdt), v_new=v_new.to(tdt))

    if wl.kv_dtype == "fp8":
        ks = torch.nan_to_num(k.abs(), nan=0.0).amax(dim=(2, 3)) / 448.0
        vs = torch.nan_to_num(v.abs(), nan=0.0).amax(dim=(2, 3)) / 448.0
        out.k_scale = torch.where(ks > 0, ks, torch.ones_like(ks)).to(torch.float32).contiguous()
        out.v_scale = torch.where(vs > 0, vs, torch.ones_like(vs)).to(torch.float32).contiguous()
        _poison_slots(k, v, slots // BLOCK, slots % BLOCK)
        out.k_src, out.v_src = k.contiguous(), v.contiguous()
    else:
        _poison_slots(k, v, slots // BLOCK, slots % BLOCK)
        kdt = torch.float32 if wl.kv_dtype == "f32" else torch.bfloat16
        out.k_cache, out.v_cache = k.to(kdt).contiguous(), v.to(kdt).contiguous()
    return out
