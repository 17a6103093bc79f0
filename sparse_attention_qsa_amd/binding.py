"""ctypes binding of libqsa.so.  Argument marshalling only: every step of the path runs in the
library's HIP kernels; torch supplies device memory and the current stream.

The functions carry the C names (qsa_compress, qsa_index_logits_topk, qsa_sparse_gqa, ...).
If libqsa.so has not been built the first call raises -- there is no other code path.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqsa.so")

QSA_OK = 0
DTYPES = {"bf16": 0, "fp8": 1}
AGGS = {"sum": 0, "relu": 1}   # head aggregation of the indexer score

EXPORTED = (
    "qsa_compress", "qsa_index_logits_topk", "qsa_index_logits_topk_workspace_size",
    "qsa_index_logits", "qsa_block_topk",
    "qsa_compress_index_logits_topk", "qsa_compress_index_logits",
    "qsa_compress_index_logits_topk_fused",
    "qsa_sparse_gqa", "qsa_sparse_gqa_workspace_size", "qsa_sparse_gqa_num_splits",
    "qsa_sparse_gqa_merge_kernel",
    "qsa_sparse_gqa_partial", "qsa_sparse_gqa_merge",
    "qsa_sparse_gqa_noalloc", "qsa_sparse_gqa_noalloc_scratch_bytes",
    "qsa_diag_e4m3_decode", "qsa_diag_fp64_sqrt_div", "qsa_diag_read_bandwidth",
    "qsa_status_string", "qsa_abi_version",
)

_P = C.c_void_p
_I32 = C.c_int32
_I64 = C.c_int64


class CompressArgs(C.Structure):
    _fields_ = [
        ("num_tokens", _I32), ("num_requests", _I32),
        ("query_start_loc", _P), ("seq_lens", _P), ("max_query_len", _I32),
        ("q_proj", _P), ("q_proj_row_stride", _I64),
        ("k_proj", _P), ("k_proj_row_stride", _I64),
        ("positions", _P), ("mrope_section", _I32 * 3),
        ("cos_sin", _P), ("max_position", _I32),
        ("q_norm_weight", _P), ("k_norm_weight", _P), ("eps", C.c_float),
        ("ring", _P), ("ring_pos", _P), ("ring_page", _P), ("ring_pages", _I32),
        ("ring_size", _I32),
        ("ckv", _P), ("c_block_table", _P), ("c_block_table_stride", _I32),
        ("c_block_table_width", _I32), ("c_page_size", _I32), ("c_pages", _I32),
        ("num_index_heads", _I32), ("head_dim", _I32), ("rotary_dim", _I32),
        ("compress_ratio", _I32), ("index_dtype", _I32),
        ("q_idx", _P),
        ("main_qkv", _P), ("main_qkv_row_stride", _I64), ("num_q_heads", _I32),
        ("num_kv_heads", _I32), ("main_q_norm_weight", _P), ("main_k_norm_weight", _P),
        ("main_eps", C.c_float), ("main_q", _P), ("main_kv_cache", _P),
        ("main_kv_page_stride", _I64), ("main_kv_head_stride", _I64),
        ("main_kv_token_stride", _I64), ("main_num_pages", _I32), ("main_page_size", _I32),
        ("main_slot_mapping", _P), ("main_kv_dtype", _I32), ("main_k_scale", C.c_float),
        ("main_v_scale", C.c_float),
    ]


class TopkArgs(C.Structure):
    _fields_ = [
        ("num_tokens", _I32), ("num_requests", _I32),
        ("query_start_loc", _P), ("seq_lens", _P),
        ("num_decode_requests", _I32), ("decode_query_len", _I32),
        ("max_query_len", _I32), ("max_seq_len", _I32),
        ("q_idx", _P), ("ckv", _P), ("c_block_table", _P), ("c_block_table_stride", _I32),
        ("c_block_table_width", _I32), ("c_page_size", _I32), ("c_pages", _I32),
        ("num_index_heads", _I32), ("head_dim", _I32), ("compress_ratio", _I32),
        ("budget", _I32), ("index_dtype", _I32),
        ("packed", _P), ("packed_row_stride", _I64), ("index_agg", _I32),
        ("max_logits_bytes", _I64),
    ]


class GqaArgs(C.Structure):
    _fields_ = [
        ("num_tokens", _I32), ("num_requests", _I32), ("num_q_heads", _I32),
        ("num_kv_heads", _I32), ("head_dim", _I32),
        ("q", _P), ("q_row_stride", _I64), ("q_head_stride", _I64),
        ("kv_cache", _P), ("kv_page_stride", _I64), ("kv_head_stride", _I64),
        ("kv_token_stride", _I64), ("num_pages", _I32), ("page_size", _I32),
        ("block_table", _P), ("block_table_stride", _I32), ("block_table_width", _I32),
        ("token_to_req", _P), ("packed", _P), ("packed_row_stride", _I64),
        ("packed_width", _I32),
        ("gate", _P), ("gate_row_stride", _I64), ("gate_head_stride", _I64),
        ("scale", C.c_float), ("num_splits", _I32),
        ("out", _P), ("out_row_stride", _I64), ("out_head_stride", _I64),
        ("kv_dtype", _I32), ("k_scale", C.c_float), ("v_scale", C.c_float),
        ("row_tiles", _I32),
    ]


_lib_handle = None


def lib() -> C.CDLL:
    """The loaded libqsa.so (raises if it was never built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_attention_qsa_amd.build`")
        h = C.CDLL(LIB_PATH)
        h.qsa_compress.argtypes = [C.POINTER(CompressArgs), _P]
        h.qsa_compress.restype = C.c_int
        h.qsa_index_logits_topk_workspace_size.argtypes = [C.POINTER(TopkArgs)]
        h.qsa_index_logits_topk_workspace_size.restype = C.c_size_t
        for f in ("qsa_index_logits_topk", "qsa_index_logits", "qsa_block_topk"):
            getattr(h, f).argtypes = [C.POINTER(TopkArgs), _P, C.c_size_t, _P]
            getattr(h, f).restype = C.c_int
        for f in ("qsa_compress_index_logits_topk", "qsa_compress_index_logits"):
            getattr(h, f).argtypes = [C.POINTER(CompressArgs), C.POINTER(TopkArgs), _P,
                                      C.c_size_t, _P]
            getattr(h, f).restype = C.c_int
        h.qsa_compress_index_logits_topk_fused.argtypes = [C.POINTER(CompressArgs),
                                                           C.POINTER(TopkArgs)]
        h.qsa_compress_index_logits_topk_fused.restype = _I32
        h.qsa_sparse_gqa_workspace_size.argtypes = [C.POINTER(GqaArgs)]
        h.qsa_sparse_gqa_workspace_size.restype = C.c_size_t
        h.qsa_sparse_gqa_num_splits.argtypes = [C.POINTER(GqaArgs)]
        h.qsa_sparse_gqa_num_splits.restype = _I32
        h.qsa_sparse_gqa_merge_kernel.argtypes = [C.POINTER(GqaArgs)]
        h.qsa_sparse_gqa_merge_kernel.restype = _I32
        for f in ("qsa_sparse_gqa", "qsa_sparse_gqa_partial", "qsa_sparse_gqa_merge"):
            getattr(h, f).argtypes = [C.POINTER(GqaArgs), _P, C.c_size_t, _P]
            getattr(h, f).restype = C.c_int
        h.qsa_sparse_gqa_noalloc.argtypes = [C.POINTER(GqaArgs), _P]
        h.qsa_sparse_gqa_noalloc.restype = C.c_int
        h.qsa_sparse_gqa_noalloc_scratch_bytes.argtypes = []
        h.qsa_sparse_gqa_noalloc_scratch_bytes.restype = C.c_size_t
        h.qsa_diag_e4m3_decode.argtypes = [_P, _P]
        h.qsa_diag_e4m3_decode.restype = C.c_int
        h.qsa_diag_fp64_sqrt_div.argtypes = [_P, _P, _I64, _P]
        h.qsa_diag_fp64_sqrt_div.restype = C.c_int
        h.qsa_diag_read_bandwidth.argtypes = [_P, _P, _I64, _I32, _P, _P]
        h.qsa_diag_read_bandwidth.restype = C.c_int
        h.qsa_status_string.argtypes = [C.c_int]
        h.qsa_status_string.restype = C.c_char_p
        h.qsa_abi_version.argtypes = []
        h.qsa_abi_version.restype = _I32
        _lib_handle = h
    return _lib_handle


class QsaError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {lib().qsa_status_string(status).decode()}")


def _check(status: int, call: str) -> None:
    if status != QSA_OK:
        raise QsaError(status, call)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous in its last dimension")


def _shape(t: torch.Tensor, shape: tuple, name: str) -> None:
    """Exact shape check; a None entry matches any extent."""
    if t.dim() != len(shape) or any(w is not None and int(g) != w
                                    for g, w in zip(t.shape, shape)):
        raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")


def _index_codes(t: torch.Tensor, index_dtype: str, name: str) -> None:
    """Indexer storage: bf16 values, or e4m3fn codes held as uint8."""
    if index_dtype not in DTYPES:
        raise ValueError(f"index_dtype must be one of {sorted(DTYPES)}, got {index_dtype!r}")
    _need(t, torch.bfloat16 if index_dtype == "bf16" else torch.uint8, name)


def _q_idx(q_idx: torch.Tensor, T: int, heads: int, index_dtype: str) -> None:
    _index_codes(q_idx, index_dtype, "q_idx")
    _shape(q_idx, (T, heads, 128), "q_idx")
    if not q_idx.is_contiguous():
        raise ValueError("q_idx must be contiguous")


# ------------------------------------------------------------------------------ qsa_compress


def compress_args(*, query_start_loc, seq_lens, max_query_len, q_proj, k_proj, positions,
                  cos_sin, q_norm_weight, k_norm_weight, eps, ring, ring_page, ckv,
                  c_block_table, q_idx, num_index_heads, compress_ratio, index_dtype,
                  ring_pos=None, mrope_section=None, c_block_table_width=None,
                  main=None) -> CompressArgs:
    """`main`, if given, adds the main-attention prepare: a dict with main_qkv [T,
    (2Hq+2Hkv)*128] bf16, num_q_heads, num_kv_heads, main_q_norm_weight, main_k_norm_weight,
    main_eps, main_q [T, Hq, 128] bf16 (out), main_kv_cache [pages, Hkv, P, 256] (bf16, or uint8
    e4m3fn codes), main_slot_mapping [T] int64 and, for an fp8 cache, main_k_scale /
    main_v_scale."""
    _need(q_proj, torch.bfloat16, "q_proj")
    _need(k_proj, torch.bfloat16, "k_proj")
    _need(positions, torch.int64, "positions")
    _need(cos_sin, torch.float32, "cos_sin")
    _need(ring, torch.bfloat16, "ring")
    _need(query_start_loc, torch.int32, "query_start_loc")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(ring_page, torch.int32, "ring_page")
    _need(c_block_table, torch.int32, "c_block_table")
    T = q_proj.shape[0]
    mrope = bool(mrope_section) and any(mrope_section)
    _shape(k_proj, (T, None), "k_proj")
    _shape(positions, (T, 3) if mrope else (T,), "positions")
    for w, name in ((q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight")):
        _need(w, torch.bfloat16, name)
        _shape(w, (128,), name)
    _shape(ring, (None, None, 128), "ring")
    if mrope:
        if ring_pos is None:
            raise ValueError("ring_pos is required with mrope_section")
        _need(ring_pos, torch.int64, "ring_pos")
        _shape(ring_pos, (ring.shape[0], ring.shape[1], 3), "ring_pos")
    _index_codes(ckv, index_dtype, "ckv")
    _shape(ckv, (None, None, 128), "ckv")
    _q_idx(q_idx, T, int(num_index_heads), index_dtype)
    a = CompressArgs()
    a.num_tokens = T
    a.num_requests = seq_lens.shape[0]
    a.query_start_loc = _ptr(query_start_loc)
    a.seq_lens = _ptr(seq_lens)
    a.max_query_len = int(max_query_len)
    a.q_proj = _ptr(q_proj)
    a.q_proj_row_stride = q_proj.stride(0)
    a.k_proj = _ptr(k_proj)
    a.k_proj_row_stride = k_proj.stride(0)
    a.positions = _ptr(positions)
    a.mrope_section = (_I32 * 3)(*(mrope_section or (0, 0, 0)))
    a.cos_sin = _ptr(cos_sin)
    a.max_position = cos_sin.shape[0]
    a.q_norm_weight = _ptr(q_norm_weight)
    a.k_norm_weight = _ptr(k_norm_weight)
    a.eps = float(eps)
    a.ring = _ptr(ring)
    a.ring_pos = _ptr(ring_pos)
    a.ring_page = _ptr(ring_page)
    a.ring_pages = ring.shape[0]
    a.ring_size = ring.shape[1]
    a.ckv = _ptr(ckv)
    a.c_block_table = _ptr(c_block_table)
    a.c_block_table_stride = c_block_table.stride(0)
    a.c_block_table_width = c_block_table.shape[1] if c_block_table_width is None else int(
        c_block_table_width)
    a.c_page_size = ckv.shape[1]
    a.c_pages = ckv.shape[0]
    a.num_index_heads = int(num_index_heads)
    a.head_dim = ring.shape[-1]
    a.rotary_dim = 64
    a.compress_ratio = int(compress_ratio)
    a.index_dtype = DTYPES[index_dtype]
    a.q_idx = _ptr(q_idx)
    if main is not None:
        qkv, cache, slots, mq = (main["main_qkv"], main["main_kv_cache"],
                                 main["main_slot_mapping"], main["main_q"])
        _need(qkv, torch.bfloat16, "main_qkv")
        _need(mq, torch.bfloat16, "main_q")
        _need(slots, torch.int64, "main_slot_mapping")
        fp8 = cache.dtype == torch.uint8
        if not fp8:
            _need(cache, torch.bfloat16, "main_kv_cache")
        a.main_qkv = _ptr(qkv)
        a.main_qkv_row_stride = qkv.stride(0)
        a.num_q_heads = int(main["num_q_heads"])
        a.num_kv_heads = int(main["num_kv_heads"])
        a.main_q_norm_weight = _ptr(main["main_q_norm_weight"])
        a.main_k_norm_weight = _ptr(main["main_k_norm_weight"])
        a.main_eps = float(main["main_eps"])
        a.main_q = _ptr(mq)
        a.main_kv_cache = _ptr(cache)
        a.main_kv_page_stride = cache.stride(0)
        a.main_kv_head_stride = cache.stride(1)
        a.main_kv_token_stride = cache.stride(2)
        a.main_num_pages = cache.shape[0]
        a.main_page_size = cache.shape[2]
        a.main_slot_mapping = _ptr(slots)
        a.main_kv_dtype = DTYPES["fp8" if fp8 else "bf16"]
        a.main_k_scale = float(main.get("main_k_scale", 1.0))
        a.main_v_scale = float(main.get("main_v_scale", 1.0))
    return a


def qsa_compress(stream=None, **kw) -> None:
    a = compress_args(**kw)
    _check(lib().qsa_compress(C.byref(a), _stream(stream)), "qsa_compress")


# ------------------------------------------------------------------------------ qsa_index_logits_topk


def topk_args(*, query_start_loc, seq_lens, q_idx, ckv, c_block_table, packed, num_index_heads,
              compress_ratio, budget, index_dtype, max_query_len, max_seq_len,
              num_decode_requests=0, decode_query_len=0, c_block_table_width=None,
              index_agg="sum", max_logits_bytes=0) -> TopkArgs:
    _need(query_start_loc, torch.int32, "query_start_loc")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(c_block_table, torch.int32, "c_block_table")
    _need(packed, torch.int32, "packed")
    T = q_idx.shape[0]
    _q_idx(q_idx, T, int(num_index_heads), index_dtype)
    _index_codes(ckv, index_dtype, "ckv")
    _shape(ckv, (None, None, 128), "ckv")
    _shape(packed, (T, int(budget) + int(compress_ratio) - 1 + 1), "packed")
    a = TopkArgs()
    a.num_tokens = T
    a.num_requests = seq_lens.shape[0]
    a.query_start_loc = _ptr(query_start_loc)
    a.seq_lens = _ptr(seq_lens)
    a.num_decode_requests = int(num_decode_requests)
    a.decode_query_len = int(decode_query_len)
    a.max_query_len = int(max_query_len)
    a.max_seq_len = int(max_seq_len)
    a.q_idx = _ptr(q_idx)
    a.ckv = _ptr(ckv)
    a.c_block_table = _ptr(c_block_table)
    a.c_block_table_stride = c_block_table.stride(0)
    a.c_block_table_width = c_block_table.shape[1] if c_block_table_width is None else int(
        c_block_table_width)
    a.c_page_size = ckv.shape[1]
    a.c_pages = ckv.shape[0]
    a.num_index_heads = int(num_index_heads)
    a.head_dim = ckv.shape[-1]
    a.compress_ratio = int(compress_ratio)
    a.budget = int(budget)
    a.index_dtype = DTYPES[index_dtype]
    a.packed = _ptr(packed)
    a.packed_row_stride = packed.stride(0)
    a.index_agg = AGGS[index_agg]
    a.max_logits_bytes = int(max_logits_bytes)
    return a


def qsa_index_logits_topk_workspace_size(**kw) -> int:
    a = topk_args(**kw)
    return int(lib().qsa_index_logits_topk_workspace_size(C.byref(a)))


def qsa_index_logits_topk(workspace=None, stream=None, **kw) -> None:
    a = topk_args(**kw)
    need = int(lib().qsa_index_logits_topk_workspace_size(C.byref(a)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=kw["packed"].device)
    _check(lib().qsa_index_logits_topk(C.byref(a), _ptr(workspace), workspace.numel(),
                                       _stream(stream)), "qsa_index_logits_topk")


def qsa_compress_index_logits_topk(compress, topk, workspace=None, stream=None) -> None:
    """qsa_compress(**compress) then qsa_index_logits_topk(**topk) as one call (one launch fewer
    for a batch of one-row decode requests)."""
    ca, ta = compress_args(**compress), topk_args(**topk)
    need = int(lib().qsa_index_logits_topk_workspace_size(C.byref(ta)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=topk["packed"].device)
    _check(lib().qsa_compress_index_logits_topk(C.byref(ca), C.byref(ta), _ptr(workspace),
                                                workspace.numel(), _stream(stream)),
           "qsa_compress_index_logits_topk")


def qsa_compress_index_logits_topk_fused(compress, topk) -> int:
    """1 when qsa_compress_index_logits_topk runs as one scoring launch, 0 when as the two
    calls, -1 for invalid arguments."""
    ca, ta = compress_args(**compress), topk_args(**topk)
    return int(lib().qsa_compress_index_logits_topk_fused(C.byref(ca), C.byref(ta)))


# ------------------------------------------------------------------------------ qsa_sparse_gqa


def gqa_args(*, q, kv_cache, block_table, token_to_req, packed, out, gate=None, scale=0.0,
             num_splits=0, num_requests=None, block_table_width=None, k_scale=1.0,
             v_scale=1.0, row_tiles=False) -> GqaArgs:
    """kv_cache: [pages, Hkv, P, 2*head_dim] bf16 (K then V per token row), or uint8 e4m3fn
    codes with K = code * k_scale and V = code * v_scale."""
    _need(q, torch.bfloat16, "q")
    _need(kv_cache, torch.uint8 if kv_cache.dtype == torch.uint8 else torch.bfloat16,
          "kv_cache")
    _need(block_table, torch.int32, "block_table")
    _need(token_to_req, torch.int32, "token_to_req")
    _need(packed, torch.int32, "packed")
    _need(out, torch.bfloat16, "out")
    T = q.shape[0]
    _shape(q, (T, None, 128), "q")
    _shape(kv_cache, (None, None, None, 256), "kv_cache")
    _shape(token_to_req, (T,), "token_to_req")
    _shape(packed, (T, None), "packed")
    _shape(out, tuple(q.shape), "out")
    if gate is not None:
        _shape(gate, tuple(q.shape), "gate")
    a = GqaArgs()
    a.num_tokens = q.shape[0]
    a.num_requests = block_table.shape[0] if num_requests is None else int(num_requests)
    a.num_q_heads = q.shape[1]
    a.num_kv_heads = kv_cache.shape[1]
    a.head_dim = q.shape[2]
    a.q = _ptr(q)
    a.q_row_stride = q.stride(0)
    a.q_head_stride = q.stride(1)
    a.kv_cache = _ptr(kv_cache)
    a.kv_page_stride = kv_cache.stride(0)
    a.kv_head_stride = kv_cache.stride(1)
    a.kv_token_stride = kv_cache.stride(2)
    a.num_pages = kv_cache.shape[0]
    a.page_size = kv_cache.shape[2]
    a.block_table = _ptr(block_table)
    a.block_table_stride = block_table.stride(0)
    a.block_table_width = block_table.shape[1] if block_table_width is None else int(
        block_table_width)
    a.token_to_req = _ptr(token_to_req)
    a.packed = _ptr(packed)
    a.packed_row_stride = packed.stride(0)
    a.packed_width = packed.shape[1] - 1
    if gate is not None:
        _need(gate, torch.bfloat16, "gate")
        a.gate = _ptr(gate)
        a.gate_row_stride = gate.stride(0)
        a.gate_head_stride = gate.stride(1)
    a.scale = float(scale)
    a.num_splits = int(num_splits)
    a.out = _ptr(out)
    a.out_row_stride = out.stride(0)
    a.out_head_stride = out.stride(1)
    a.row_tiles = 1 if row_tiles else 0
    if kv_cache.dtype == torch.uint8:
        a.kv_dtype = 1
        a.k_scale = float(k_scale)
        a.v_scale = float(v_scale)
    return a


def qsa_sparse_gqa_workspace_size(**kw) -> int:
    a = gqa_args(**kw)
    return int(lib().qsa_sparse_gqa_workspace_size(C.byref(a)))


def qsa_sparse_gqa_num_splits(**kw) -> int:
    a = gqa_args(**kw)
    return int(lib().qsa_sparse_gqa_num_splits(C.byref(a)))


def qsa_sparse_gqa(workspace=None, stream=None, **kw) -> None:
    a = gqa_args(**kw)
    need = int(lib().qsa_sparse_gqa_workspace_size(C.byref(a)))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=kw["out"].device)
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().qsa_sparse_gqa(C.byref(a), _ptr(workspace), nbytes, _stream(stream)),
           "qsa_sparse_gqa")


def qsa_sparse_gqa_noalloc(stream=None, **kw) -> None:
    """qsa_sparse_gqa without a workspace: the split partials live in the library's static
    per-GPU scratch (calls that overlap on one GPU race; serialise them on one stream)."""
    a = gqa_args(**kw)
    _check(lib().qsa_sparse_gqa_noalloc(C.byref(a), _stream(stream)), "qsa_sparse_gqa_noalloc")


# ------------------------------------------------------------------------------ diagnostics


def qsa_diag_e4m3_decode(device="cuda") -> torch.Tensor:
    out = torch.empty(512, dtype=torch.float32, device=device)
    _check(lib().qsa_diag_e4m3_decode(_ptr(out), _stream(None)), "qsa_diag_e4m3_decode")
    return out


def qsa_diag_fp64_sqrt_div(x: torch.Tensor) -> torch.Tensor:
    _need(x, torch.float64, "x")
    out = torch.empty(3 * x.numel(), dtype=torch.float64, device=x.device)
    _check(lib().qsa_diag_fp64_sqrt_div(_ptr(x), _ptr(out), x.numel(), _stream(None)),
           "qsa_diag_fp64_sqrt_div")
    return out


def qsa_diag_read_bandwidth(src: torch.Tensor, chunk_bytes: int, sink: torch.Tensor,
                            chunk_index: torch.Tensor | None = None, stream=None) -> None:
    """Read-bandwidth probe over `src` (a streaming read of every chunk, or a gather of the
    chunks listed in `chunk_index`); see qsa.h."""
    _need(sink, torch.int32, "sink")
    if chunk_index is not None:
        _need(chunk_index, torch.int32, "chunk_index")
        n = chunk_index.numel()
    else:
        n = src.numel() * src.element_size() // int(chunk_bytes)
    _check(lib().qsa_diag_read_bandwidth(_ptr(src), _ptr(chunk_index), n, int(chunk_bytes),
                                         _ptr(sink), _stream(stream)), "qsa_diag_read_bandwidth")
