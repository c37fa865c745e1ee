"""MI355X-native paged attention: Python binding of libpagedattn.so.

This module only marshals torch tensors (device memory) and the current
stream into the C ABI declared in include/pagedattn.h; every step of the
computation runs in the library's HIP kernels. If the library is missing
or cannot be loaded, every call raises -- there is no fallback path.

Layouts (see the header for the full contract):
  q, out   [T][Hq][D]           float32 or bfloat16
  k_cache  [num_blocks][Hkv][16][D]
  v_cache  [num_blocks][Hkv][D][16]
  k_scale, v_scale [num_blocks][Hkv] float32 (fp8 caches, stored as uint8)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_F32, PA_BF16, PA_FP8_E4M3FN = 0, 1, 2
PA_OK, PA_EINVAL, PA_EWORKSPACE, PA_EHIP, PA_ENOTSUP = 0, -1, -2, -3, -4
PA_ESCRATCH = -6
PA_NOALLOC_SCRATCH_BYTES = 128 << 20

_lib = None


class PaShape(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("partition_size", ctypes.c_int32),
        ("cascade", ctypes.c_int32),
        ("fp8_qk", ctypes.c_int32),
    ]


class PagedAttentionError(RuntimeError):
    pass


class PaLayoutInfo(ctypes.Structure):
    """Workspace regions of a batch (pa_workspace_layout); streams 0 wide,
    1 narrow, 2 group."""
    _fields_ = [
        ("waves", ctypes.c_int32 * 3),
        ("narrow_tokens", ctypes.c_int32),
        ("wide_tokens", ctypes.c_int32),
        ("part_blocks", ctypes.c_int32),
        ("members_per_tile", ctypes.c_int32),
        ("wide_row_tiles", ctypes.c_int32),
        ("header_words", ctypes.c_int32),
        ("part_cost", ctypes.c_int32 * 3),
        ("span_shared", ctypes.c_int32),
        ("group_row_tiles", ctypes.c_int32),
        ("max_tiles", ctypes.c_int64),
        ("max_pieces", ctypes.c_int64 * 3),
        ("max_splits", ctypes.c_int64),
        ("max_cas_recs", ctypes.c_int64),
        ("off_tiles", ctypes.c_int64),
        ("off_splits", ctypes.c_int64),
        ("off_tree", ctypes.c_int64),
        ("off_cas_seq", ctypes.c_int64),
        ("off_cas_recs", ctypes.c_int64),
        ("off_cas_lse", ctypes.c_int64 * 2),
        ("off_cas_o", ctypes.c_int64 * 2),
        ("off_pieces", ctypes.c_int64 * 3),
        ("off_part_lse", ctypes.c_int64 * 3),
        ("off_part_o", ctypes.c_int64 * 3),
        ("total", ctypes.c_int64),
    ]


def load_library(path: str = LIB_PATH):
    """Load libpagedattn.so (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise PagedAttentionError(
            f"{path} is missing: build it with `python -m paged_kv_cache_213_amd.build`")
    # torch first: the library then binds to the HIP runtime torch already
    # loaded, instead of bringing a second one into the process
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    S = ctypes.POINTER(PaShape)
    lib.pa_workspace_bytes.restype = Z
    lib.pa_workspace_bytes.argtypes = [S, I, I, I, I]
    lib.pa_paged_attn_decode.restype = I
    lib.pa_paged_attn_decode.argtypes = [S, P, P, P, P, P, P, P, P, P, I, I, F, P, Z, P]
    for name in ("pa_paged_attn_run_append", "pa_paged_attn_partial_append",
                 "pa_paged_attn_decode_append"):
        fn = getattr(lib, name)
        fn.restype = I
        fn.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, I, I, F, P, Z, P]
    lib.pa_paged_attn_hybrid.restype = I
    lib.pa_paged_attn_hybrid.argtypes = [S, P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, P, Z, P]
    lib.pa_paged_attn_hybrid_noalloc.restype = I
    lib.pa_paged_attn_hybrid_noalloc.argtypes = [S, P, P, P, P, P, P, P, P, P, P, I, I, I, I, F,
                                                 P]
    lib.pa_plan.restype = I
    lib.pa_plan.argtypes = [S, P, P, I, I, I, I, P, Z, P]
    lib.pa_plan_cascade.restype = I
    lib.pa_plan_cascade.argtypes = [S, P, P, I, I, I, I, I, I, P, P, P, P, Z, P]
    lib.pa_plan_tree.restype = I
    lib.pa_plan_tree.argtypes = [S, P, P, I, I, I, I, P, P, Z, P]
    lib.pa_paged_attn_run.restype = I
    lib.pa_paged_attn_run.argtypes = [S, P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, P, Z, P]
    lib.pa_paged_attn_partial.restype = I
    lib.pa_paged_attn_partial.argtypes = [S, P, P, P, P, P, P, P, P, P, P, I, I, I, I, F, P, Z, P]
    lib.pa_paged_attn_merge.restype = I
    lib.pa_paged_attn_merge.argtypes = [S, P, P, P, P, I, I, I, I, P, Z, P]
    lib.pa_kv_append.restype = I
    lib.pa_kv_append.argtypes = [S, P, P, P, P, P, P, P, I, P]
    lib.pa_fp8_e4m3fn_to_f32.restype = I
    lib.pa_fp8_e4m3fn_to_f32.argtypes = [P, P, I, P]
    lib.pa_workspace_layout.restype = I
    lib.pa_workspace_layout.argtypes = [S, I, I, I, I, I, ctypes.POINTER(PaLayoutInfo)]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [I]
    lib.pa_version.restype = I
    lib.pa_version.argtypes = []
    lib.pa_probe_stream_read.restype = I
    lib.pa_probe_stream_read.argtypes = [P, Z, P, P]
    lib.pa_probe_copy.restype = I
    lib.pa_probe_copy.argtypes = [P, P, Z, P]
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != PA_OK:
        msg = load_library().pa_status_string(rc).decode()
        raise PagedAttentionError(f"{what} failed: {msg} ({rc})")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", None)):
        return PA_FP8_E4M3FN
    raise PagedAttentionError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise PagedAttentionError("all tensors must live in GPU memory")
    if not t.is_contiguous():
        raise PagedAttentionError("all tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def make_shape(q, k_cache, block_tables, partition_size: int = 0,
               cascade: bool = False, fp8_qk: bool = False) -> PaShape:
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if B != 16 or D2 != D:
        raise PagedAttentionError(f"k_cache shape {tuple(k_cache.shape)} does not match q")
    return PaShape(Hq, Hkv, D, 16, NB, block_tables.shape[1], _dtype_code(q),
                   _dtype_code(k_cache), int(partition_size), int(bool(cascade)),
                   int(bool(fp8_qk)))


def workspace_bytes(shape: PaShape, num_seqs: int, num_q_tokens: int, max_context_len: int,
                    max_query_len: int) -> int:
    return int(load_library().pa_workspace_bytes(ctypes.byref(shape), num_seqs, num_q_tokens,
                                                 max_context_len, max_query_len))


def workspace_layout(shape: PaShape, num_seqs: int, num_q_tokens: int, max_context_len: int,
                     max_query_len: int, decode: bool) -> PaLayoutInfo:
    """Bounds and offsets of the workspace regions a plan writes."""
    info = PaLayoutInfo()
    rc = load_library().pa_workspace_layout(ctypes.byref(shape), num_seqs, num_q_tokens,
                                            max_context_len, max_query_len, int(bool(decode)),
                                            ctypes.byref(info))
    _check(rc, "pa_workspace_layout")
    return info


def _workspace(nbytes: int, device, workspace):
    import torch
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise PagedAttentionError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, *,
           max_context_len: int, k_scale=None, v_scale=None, partition_size: int = 0,
           out=None, lse=None, workspace=None, stream=None, fp8_qk: bool = False,
           k_new=None, v_new=None):
    """Paged attention for one query token per sequence.

    q [S][Hq][D]; block_tables [S][max_blocks] int32; context_lens [S] int32
    (including the new token). Returns out [S][Hq][D] in q's dtype (and
    fills ``lse`` [S][Hq] float32 when given). With k_new / v_new
    ([S][Hkv][D], q's dtype) the step's rows are appended at each
    sequence's last position in the same pass (pa_paged_attn_decode_append)."""
    import torch
    lib = load_library()
    shape = make_shape(q, k_cache, block_tables, partition_size, fp8_qk=fp8_qk)
    S = q.shape[0]
    if out is None:
        out = torch.empty_like(q)
    nbytes = workspace_bytes(shape, S, S, max_context_len, 1)
    ws = _workspace(nbytes, q.device, workspace)
    if k_new is not None or v_new is not None:
        rc = lib.pa_paged_attn_decode_append(
            ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_new), _ptr(v_new),
            _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
            _ptr(context_lens), S, int(max_context_len), float(scale), _ptr(ws),
            ws.numel() * ws.element_size(), _stream(stream))
        _check(rc, "pa_paged_attn_decode_append")
        return out
    rc = lib.pa_paged_attn_decode(ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(q),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                  _ptr(block_tables), _ptr(context_lens), S,
                                  int(max_context_len), float(scale), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "pa_paged_attn_decode")
    return out


def hybrid(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale: float, *,
           max_context_len: int, max_query_len: int, k_scale=None, v_scale=None,
           partition_size: int = 0, out=None, lse=None, workspace=None, stream=None,
           fp8_qk: bool = False):
    """Paged attention for a mixed batch of chunked-prefill spans and
    decodes. q [T][Hq][D] with T = query_start_loc[-1]."""
    import torch
    lib = load_library()
    shape = make_shape(q, k_cache, block_tables, partition_size, fp8_qk=fp8_qk)
    T = q.shape[0]
    S = context_lens.shape[0]
    if out is None:
        out = torch.empty_like(q)
    nbytes = workspace_bytes(shape, S, T, max_context_len, max_query_len)
    ws = _workspace(nbytes, q.device, workspace)
    rc = lib.pa_paged_attn_hybrid(ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(q),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                  _ptr(block_tables), _ptr(context_lens), _ptr(query_start_loc),
                                  S, T, int(max_query_len), int(max_context_len), float(scale),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "pa_paged_attn_hybrid")
    return out


def hybrid_noalloc(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                   scale: float, *, max_context_len: int, max_query_len: int, out, lse=None,
                   k_scale=None, v_scale=None, partition_size: int = 0, stream=None,
                   fp8_qk: bool = False):
    """hybrid() without a workspace: the library's static per-GPU scratch
    buffer serves the call, and nothing is allocated (``out`` is the
    caller's). Calls that overlap on one GPU race on that buffer."""
    lib = load_library()
    shape = make_shape(q, k_cache, block_tables, partition_size, fp8_qk=fp8_qk)
    T = q.shape[0]
    S = context_lens.shape[0]
    rc = lib.pa_paged_attn_hybrid_noalloc(ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(q),
                                          _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                          _ptr(v_scale), _ptr(block_tables), _ptr(context_lens),
                                          _ptr(query_start_loc), S, T, int(max_query_len),
                                          int(max_context_len), float(scale), _stream(stream))
    _check(rc, "pa_paged_attn_hybrid_noalloc")
    return out


def cascade(q, k_cache, v_cache, block_tables, context_lens, scale: float, groups, *,
            max_context_len: int, query_start_loc=None, max_query_len: int = 1, k_scale=None,
            v_scale=None, partition_size: int = 0, out=None, lse=None, workspace=None,
            stream=None, fp8_qk: bool = False):
    """Paged attention with shared-prefix groups (``PrefixGroups``): plan
    with the groups, then the attention and merge passes. Same result as
    decode()/hybrid(); each group's prefix is read once for its members."""
    import torch
    shape = make_shape(q, k_cache, block_tables, partition_size, cascade=True, fp8_qk=fp8_qk)
    T = q.shape[0]
    S = context_lens.shape[0]
    mq = max_query_len if query_start_loc is not None else 1
    if out is None:
        out = torch.empty_like(q)
    nbytes = workspace_bytes(shape, S, T, max_context_len, mq)
    ws = _workspace(nbytes, q.device, workspace)
    plan_cascade(shape, context_lens, ws, groups, query_start_loc=query_start_loc,
                 num_q_tokens=T, max_query_len=mq, max_context_len=max_context_len, stream=stream)
    return run(shape, q, k_cache, v_cache, block_tables, context_lens, scale, ws,
               query_start_loc=query_start_loc, max_query_len=mq,
               max_context_len=max_context_len, k_scale=k_scale, v_scale=v_scale, out=out,
               lse=lse, stream=stream)


def tree(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale: float,
         tree_mask, *, max_context_len: int, max_query_len: int, k_scale=None, v_scale=None,
         partition_size: int = 0, out=None, lse=None, workspace=None, stream=None,
         fp8_qk: bool = False):
    """hybrid() whose spans are speculative candidate trees: ``tree_mask``
    [T] int64 (the bits of uint64 words), span token j sees span token
    k <= j where bit k of word j is set (spans of at most 64 tokens)."""
    import torch
    shape = make_shape(q, k_cache, block_tables, partition_size, fp8_qk=fp8_qk)
    T = q.shape[0]
    S = context_lens.shape[0]
    if out is None:
        out = torch.empty_like(q)
    nbytes = workspace_bytes(shape, S, T, max_context_len, max_query_len)
    ws = _workspace(nbytes, q.device, workspace)
    plan_tree(shape, context_lens, ws, tree_mask, query_start_loc=query_start_loc,
              num_q_tokens=T, max_query_len=max_query_len, max_context_len=max_context_len,
              stream=stream)
    return run(shape, q, k_cache, v_cache, block_tables, context_lens, scale, ws,
               query_start_loc=query_start_loc, max_query_len=max_query_len,
               max_context_len=max_context_len, k_scale=k_scale, v_scale=v_scale, out=out,
               lse=lse, stream=stream)


def plan_tree(shape: PaShape, context_lens, workspace, tree_mask, *, query_start_loc,
              num_q_tokens: int, max_query_len: int, max_context_len: int, stream=None):
    """plan() for spans under tree verification masks (``tree_mask`` [T]
    64-bit words on the device, copied into the plan)."""
    lib = load_library()
    if tree_mask.element_size() != 8 or tree_mask.numel() < num_q_tokens:
        raise ValueError("tree_mask needs one 64-bit word per query token")
    S = context_lens.shape[0]
    rc = lib.pa_plan_tree(ctypes.byref(shape), _ptr(context_lens), _ptr(query_start_loc), S,
                          int(num_q_tokens), int(max_query_len), int(max_context_len),
                          _ptr(tree_mask), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "pa_plan_tree")


def plan(shape: PaShape, context_lens, workspace, *, query_start_loc=None, num_q_tokens: int,
         max_query_len: int, max_context_len: int, stream=None):
    """Enqueue the work plan of a batch into ``workspace`` (reusable by every
    run() on the same batch)."""
    lib = load_library()
    S = context_lens.shape[0]
    rc = lib.pa_plan(ctypes.byref(shape), _ptr(context_lens), _ptr(query_start_loc), S,
                     int(num_q_tokens), int(max_query_len), int(max_context_len), _ptr(workspace),
                     workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "pa_plan")


class PrefixGroups:
    """Shared-prefix groups of a batch for cascade attention, as device
    int32 tensors: CSR offsets [G + 1], member sequence indices, and the
    shared leading blocks of each group."""

    def __init__(self, groups, prefix_blocks, device):
        import torch
        offs, mem = [0], []
        for g in groups:
            mem.extend(int(i) for i in g)
            offs.append(len(mem))
        self.num_groups = len(groups)
        self.num_members = len(mem)
        self.offsets = torch.tensor(offs, dtype=torch.int32, device=device)
        self.members = torch.tensor(mem if mem else [0], dtype=torch.int32, device=device)
        self.prefix_blocks = torch.tensor([int(b) for b in prefix_blocks] or [0],
                                          dtype=torch.int32, device=device)


def plan_cascade(shape: PaShape, context_lens, workspace, groups: PrefixGroups, *,
                 query_start_loc=None, num_q_tokens: int, max_query_len: int,
                 max_context_len: int, stream=None):
    """plan() with shared-prefix groups: each group's prefix is read once
    for all its single-token members (shape.cascade must be 1)."""
    lib = load_library()
    S = context_lens.shape[0]
    rc = lib.pa_plan_cascade(ctypes.byref(shape), _ptr(context_lens), _ptr(query_start_loc), S,
                             int(num_q_tokens), int(max_query_len), int(max_context_len),
                             groups.num_groups, groups.num_members, _ptr(groups.offsets),
                             _ptr(groups.members), _ptr(groups.prefix_blocks), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "pa_plan_cascade")


def run(shape: PaShape, q, k_cache, v_cache, block_tables, context_lens, scale: float, workspace,
        *, query_start_loc=None, max_query_len: int, max_context_len: int, k_scale=None,
        v_scale=None, out=None, lse=None, stream=None, passes: str = "both", k_new=None,
        v_new=None):
    """Attention with a plan enqueued earlier by plan(): the attention pass
    and the merge pass ("both"), or only "partial" (pass 1) or "merge".
    With k_new / v_new (decode plans only) the attention pass appends the
    step's rows first (pa_paged_attn_run_append / _partial_append)."""
    import torch
    lib = load_library()
    T = q.shape[0]
    S = context_lens.shape[0]
    if out is None:
        out = torch.empty_like(q)
    wsb = workspace.numel() * workspace.element_size()
    if passes == "merge":
        rc = lib.pa_paged_attn_merge(ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(context_lens),
                                     _ptr(query_start_loc), S, T, int(max_query_len),
                                     int(max_context_len), _ptr(workspace), wsb, _stream(stream))
        _check(rc, "pa_paged_attn_merge")
        return out
    if k_new is not None or v_new is not None:
        if query_start_loc is not None:
            raise ValueError("the fused append goes with decode plans only")
        fn = {"both": lib.pa_paged_attn_run_append,
              "partial": lib.pa_paged_attn_partial_append}[passes]
        rc = fn(ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_new), _ptr(v_new),
                _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                _ptr(context_lens), S, int(max_context_len), float(scale), _ptr(workspace),
                wsb, _stream(stream))
        _check(rc, "pa_paged_attn_" + ("run" if passes == "both" else passes) + "_append")
        return out
    fn = {"both": lib.pa_paged_attn_run, "partial": lib.pa_paged_attn_partial}[passes]
    rc = fn(ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), _ptr(context_lens),
            _ptr(query_start_loc), S, T, int(max_query_len), int(max_context_len), float(scale),
            _ptr(workspace), wsb, _stream(stream))
    _check(rc, "pa_paged_attn_" + ("run" if passes == "both" else passes))
    return out


def kv_append(k_cache, v_cache, k_new, v_new, slot_mapping, *, k_scale=None, v_scale=None,
              block_tables_width: int = 1, stream=None):
    """Write new K/V rows [T][Hkv][D] (q's dtype) into their slots."""
    lib = load_library()
    T, Hkv, D = k_new.shape
    NB = k_cache.shape[0]
    shape = PaShape(Hkv, Hkv, D, 16, NB, max(1, block_tables_width), _dtype_code(k_new),
                    _dtype_code(k_cache), 0)
    rc = lib.pa_kv_append(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                          _ptr(v_scale), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T,
                          _stream(stream))
    _check(rc, "pa_kv_append")


def fp8_to_f32(codes):
    """Decode e4m3fn bytes (uint8 tensor on the GPU) with the device path."""
    import torch
    lib = load_library()
    out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(lib.pa_fp8_e4m3fn_to_f32(_ptr(codes), _ptr(out), codes.numel(), _stream(None)),
           "pa_fp8_e4m3fn_to_f32")
    return out


# ---- measurement probes (include/pagedattn_probe.h) ---------------------

def probe_stream_read(buf, sink, stream=None):
    """Enqueue one streaming read of the whole tensor ``buf``."""
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().pa_probe_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)),
           "pa_probe_stream_read")


def probe_copy(src, dst, stream=None):
    """Enqueue a plain copy of ``src`` into ``dst`` (same byte size)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise PagedAttentionError("copy destination too small")
    _check(load_library().pa_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)),
           "pa_probe_copy")
