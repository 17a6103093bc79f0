"""Glue between the seeded workloads and the CPU oracle (test infrastructure)."""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

from oracle import qsa as oq


def to_np(t: torch.Tensor | None) -> np.ndarray | None:
    """Device tensor -> numpy; bf16 data comes out as uint16 bit patterns."""
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclasses.dataclass
class OracleStep:
    q_codes: np.ndarray          # [T, Hi, 128]
    state_after: oq.CompressState
    packed: np.ndarray           # [T, W + 1] int32
    out: np.ndarray | None       # [T, Hq, 128] float64


def oracle_compress(wl, requests=None):
    state = oq.CompressState(ring=to_np(wl.ring), ring_pos=to_np(wl.ring_pos), ckv=to_np(wl.ckv))
    q_codes, _ = oq.prepare_index_q(
        to_np(wl.q_proj), to_np(wl.positions), to_np(wl.cos_sin), wl.mrope_section,
        to_np(wl.q_norm_w), wl.eps, wl.index_heads, wl.index_dtype)
    after = oq.compress_step(
        to_np(wl.query_start_loc), to_np(wl.seq_lens), to_np(wl.k_proj), to_np(wl.positions),
        wl.mrope_section, to_np(wl.cos_sin), to_np(wl.k_norm_w), wl.eps, to_np(wl.ring_page),
        to_np(wl.c_block_table), wl.compress_ratio, wl.index_dtype, state, requests=requests)
    return q_codes, after


def oracle_step(wl, rows=None, with_attention=True, agg="sum") -> OracleStep:
    """The whole path on the CPU: prep + compress, logits + top-k + expand, sparse GQA.
    `rows` restricts selection and attention to a subset of rows (their requests are
    compressed; the other rows stay inert)."""
    requests = None
    if rows is not None:
        req = to_np(wl.token_to_req)
        requests = sorted({int(req[i]) for i in rows})
    q_codes, after = oracle_compress(wl, requests)
    packed = oq.index_topk(to_np(wl.query_start_loc), to_np(wl.seq_lens), q_codes, after.ckv,
                           to_np(wl.c_block_table), wl.compress_ratio, wl.budget,
                           wl.index_dtype, rows=rows, agg=agg)
    out = None
    if with_attention:
        out = oq.sparse_gqa(to_np(wl.q), to_np(wl.kv_cache), to_np(wl.block_table),
                            to_np(wl.token_to_req), packed, gate=to_np(wl.gate), rows=rows,
                            kv_dtype=getattr(wl, "kv_dtype", "bf16"),
                            k_scale=getattr(wl, "k_scale", 1.0),
                            v_scale=getattr(wl, "v_scale", 1.0))
    return OracleStep(q_codes=q_codes, state_after=after, packed=packed, out=out)
