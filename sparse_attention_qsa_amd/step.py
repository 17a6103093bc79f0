"""One step of the QSA hot path on a workload: qsa_compress -> qsa_index_logits_topk ->
qsa_sparse_gqa, with outputs and workspaces allocated once and the C argument blocks built
once, so that repeated steps cost three C calls.

With `main` (the inputs of the main-attention prepare, see workloads.main_prepare_inputs) the
compress call also prepares the main Q and writes the step's K/V into the main cache, and the
attention then runs on that Q with the output gate read in place from the packed projection."""

from __future__ import annotations

import ctypes as C

import torch

from . import binding as B


class QsaStep:
    def __init__(self, wl, num_splits: int = 0, gate: bool = True, main: dict | None = None,
                 index_agg: str = "sum", max_logits_bytes: int = 0):
        dev = wl.q.device
        T = wl.num_tokens
        idx_dtype = torch.uint8 if wl.index_dtype == "fp8" else torch.bfloat16
        self.wl = wl
        self.q_idx = torch.empty((T, wl.index_heads, 128), dtype=idx_dtype, device=dev)
        self.packed = torch.empty((T, wl.output_width + 1), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, wl.q_heads, 128), dtype=torch.bfloat16, device=dev)
        self.c_args = B.compress_args(
            query_start_loc=wl.query_start_loc, seq_lens=wl.seq_lens,
            max_query_len=wl.max_query_len, q_proj=wl.q_proj, k_proj=wl.k_proj,
            positions=wl.positions, cos_sin=wl.cos_sin, q_norm_weight=wl.q_norm_w,
            k_norm_weight=wl.k_norm_w, eps=wl.eps, ring=wl.ring, ring_page=wl.ring_page,
            ckv=wl.ckv, c_block_table=wl.c_block_table, q_idx=self.q_idx,
            num_index_heads=wl.index_heads, compress_ratio=wl.compress_ratio,
            index_dtype=wl.index_dtype, ring_pos=wl.ring_pos, mrope_section=wl.mrope_section,
            main=main)
        q, g = wl.q, wl.gate
        if main is not None:
            q = main["main_q"]
            g = main["main_qkv"][:, :2 * wl.q_heads * 128].view(T, wl.q_heads, 256)[:, :, 128:]
        self.t_args = B.topk_args(
            query_start_loc=wl.query_start_loc, seq_lens=wl.seq_lens, q_idx=self.q_idx,
            ckv=wl.ckv, c_block_table=wl.c_block_table, packed=self.packed,
            num_index_heads=wl.index_heads, compress_ratio=wl.compress_ratio,
            budget=wl.budget, index_dtype=wl.index_dtype, max_query_len=wl.max_query_len,
            max_seq_len=wl.max_seq_len, num_decode_requests=wl.num_decode_requests,
            decode_query_len=wl.decode_query_len, index_agg=index_agg,
            max_logits_bytes=max_logits_bytes)
        self.g_args = B.gqa_args(
            q=q, kv_cache=wl.kv_cache, block_table=wl.block_table,
            token_to_req=wl.token_to_req, packed=self.packed, out=self.out,
            gate=g if gate else None, num_splits=num_splits,
            k_scale=getattr(wl, "k_scale", 1.0), v_scale=getattr(wl, "v_scale", 1.0))
        L = B.lib()
        t_ws = int(L.qsa_index_logits_topk_workspace_size(C.byref(self.t_args)))
        # Size the attention workspace for the largest split count, so that a caller may
        # later force any num_splits on the same argument block.
        self.g_args.num_splits = 1 << 20
        g_ws = int(L.qsa_sparse_gqa_workspace_size(C.byref(self.g_args)))
        self.g_args.num_splits = num_splits
        self.t_ws = torch.empty(max(t_ws, 256), dtype=torch.uint8, device=dev)
        self.g_ws = torch.empty(max(g_ws, 256), dtype=torch.uint8, device=dev)
        self.num_splits = int(L.qsa_sparse_gqa_num_splits(C.byref(self.g_args)))

    def compress(self, stream=None):
        B._check(B.lib().qsa_compress(C.byref(self.c_args), B._stream(stream)), "qsa_compress")

    def topk(self, stream=None):
        B._check(B.lib().qsa_index_logits_topk(C.byref(self.t_args), self.t_ws.data_ptr(),
                                               self.t_ws.numel(), B._stream(stream)),
                 "qsa_index_logits_topk")

    def gqa(self, stream=None):
        B._check(B.lib().qsa_sparse_gqa(C.byref(self.g_args), self.g_ws.data_ptr(),
                                        self.g_ws.numel(), B._stream(stream)), "qsa_sparse_gqa")

    # qsa_compress + qsa_index_logits_topk as one call (one scoring launch for a batch of
    # one-row requests); `fused` says whether this step's calls qualify.
    @property
    def fused(self) -> bool:
        return int(B.lib().qsa_compress_index_logits_topk_fused(
            C.byref(self.c_args), C.byref(self.t_args))) == 1

    def prep_topk(self, stream=None):
        B._check(B.lib().qsa_compress_index_logits_topk(
            C.byref(self.c_args), C.byref(self.t_args), self.t_ws.data_ptr(), self.t_ws.numel(),
            B._stream(stream)), "qsa_compress_index_logits_topk")

    def prep_logits(self, stream=None):
        B._check(B.lib().qsa_compress_index_logits(
            C.byref(self.c_args), C.byref(self.t_args), self.t_ws.data_ptr(), self.t_ws.numel(),
            B._stream(stream)), "qsa_compress_index_logits")

    # The single kernels of the two-kernel calls (for per-kernel timing).
    def logits(self, stream=None):
        B._check(B.lib().qsa_index_logits(C.byref(self.t_args), self.t_ws.data_ptr(),
                                          self.t_ws.numel(), B._stream(stream)),
                 "qsa_index_logits")

    def block_topk(self, stream=None):
        B._check(B.lib().qsa_block_topk(C.byref(self.t_args), self.t_ws.data_ptr(),
                                        self.t_ws.numel(), B._stream(stream)), "qsa_block_topk")

    def gqa_partial(self, stream=None):
        B._check(B.lib().qsa_sparse_gqa_partial(C.byref(self.g_args), self.g_ws.data_ptr(),
                                                self.g_ws.numel(), B._stream(stream)),
                 "qsa_sparse_gqa_partial")

    def gqa_merge(self, stream=None):
        B._check(B.lib().qsa_sparse_gqa_merge(C.byref(self.g_args), self.g_ws.data_ptr(),
                                              self.g_ws.numel(), B._stream(stream)),
                 "qsa_sparse_gqa_merge")

    def run(self, stream=None, combined=False):
        """One step: the three calls, or (combined) qsa_compress_index_logits_topk and the
        attention."""
        if combined:
            self.prep_topk(stream)
        else:
            self.compress(stream)
            self.topk(stream)
        self.gqa(stream)
        return self.out
