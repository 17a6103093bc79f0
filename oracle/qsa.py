"""Plain CPU oracle of the QSA hot path: indexer prep and key compression, indexer scores,
block top-k with expansion into the packed selection buffer, and paged sparse GQA.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this module.  It shares no code with the HIP library and never calls it.

Everything is numpy float64 with the rounding points stated below; loops over requests and
rows are plain Python.  Bit patterns come in and go out as uint16 (bf16) / uint8 (e4m3fn).

Pages cited (by title; quotations are paraphrased, never copied):
  [qsa]      "vllm.models.qwen4_exp.nvidia.qsa" -- the newest revision, class QSAIndexer,
             Qwen4ExpQSAAttention, Qwen4ExpQSAImpl.
  [qsa-old]  "vllm.models.qwen4_exp.nvidia.qsa" on docs.vllm.ai -- the older revision
             (output gate applied outside the kernel).
  [indexer]  "indexer_qsa.py" -- apply_qsa_rope, _supports_fused_pre_indexer, QSAIndexer.
  [fp8kv]    patch "qwen4_exp: FP8 E4M3 KV reader for QSA with a static scale sidecar" --
             the body of _qsa_sparse_paged_gqa_splitk_kernel.
  [ops]      "vllm.models.qwen4_exp.nvidia.ops.qsa" -- _select_config,
             qsa_compress_groups_with_ratio, qsa_sparse_paged_attention, qsa_store_cache_rows.

Canonical arithmetic (the pages compute in float32 with unstated reduction orders, so the
oracle fixes one order; the GPU library reproduces it bit for bit):
  * every prep value is float64; sums of 128 terms use `halving_sum` below; a group mean
    adds its c members first to last, then divides by c;
  * a bf16 result is float64 -> float32 (RNE) -> bf16 (RNE), taken at exactly the points
    where the reference's unfused path holds a bf16 tensor (after pooling, after each
    RMSNorm, after each rotation); the fp8 indexer then casts bf16 -> e4m3fn.
  * products of a bf16/e4m3 value with a float32/float64 value that has at most 45
    significant bits are exact in float64, so a fused multiply-add cannot change a result.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import (
    bf16_bits_to_f64,
    e4m3_bits_to_f64,
    f64_to_bf16_bits,
    f64_to_e4m3_bits,
    round_bf16,
)

HEAD_DIM = 128
ROTARY_DIM = 64
HALF_ROT = ROTARY_DIM // 2


# ----------------------------------------------------------------------------- helpers


def halving_sum(terms: np.ndarray) -> np.ndarray:
    """Canonical float64 sum over the last axis (length a power of two, >= 2).

    First each adjacent pair (2i, 2i+1) is added, then the upper half of the partial sums is
    added onto the lower half until one value is left.  (Reading: the pages use float32
    reductions of unstated order; this order is fixed so that results are reproducible.)
    """
    t = terms[..., 0::2] + terms[..., 1::2]
    while t.shape[-1] > 1:
        h = t.shape[-1] // 2
        t = t[..., :h] + t[..., h:]
    return t[..., 0]


def decode_index_codes(codes: np.ndarray, idx_dtype: str) -> np.ndarray:
    """Indexer storage codes (bf16 uint16 or e4m3fn uint8) -> float64 values."""
    if idx_dtype == "bf16":
        return bf16_bits_to_f64(codes)
    if idx_dtype == "fp8":
        return e4m3_bits_to_f64(codes)
    raise ValueError(idx_dtype)


def encode_index_values(vals: np.ndarray, idx_dtype: str) -> np.ndarray:
    """bf16 values -> indexer storage codes.  fp8: the bf16 value cast to e4m3fn
    ([qsa] QSAIndexer.forward: the prepared bf16 Q is cast with .to(indexer dtype))."""
    if idx_dtype == "bf16":
        return f64_to_bf16_bits(vals)
    if idx_dtype == "fp8":
        return f64_to_e4m3_bits(vals)
    raise ValueError(idx_dtype)


def request_of_rows(query_start_loc: np.ndarray) -> np.ndarray:
    """Request id of every row from the cumulative row offsets [R+1]."""
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    return np.repeat(np.arange(len(qsl) - 1), np.diff(qsl))


def logical_positions(query_start_loc: np.ndarray, seq_lens: np.ndarray) -> np.ndarray:
    """Request-relative position of every row: the n_r rows of request r are the last n_r
    tokens of its seq_lens[r] tokens ([qsa] QSAIndexer metadata `logical_positions`)."""
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    out = np.empty(qsl[-1], dtype=np.int64)
    for r in range(len(lens)):
        n = qsl[r + 1] - qsl[r]
        out[qsl[r]:qsl[r + 1]] = lens[r] - n + np.arange(n)
    return out


# ----------------------------------------------------------------------------- A1: norm


def gemma_rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Per-head Gemma RMSNorm of bf16 rows x [N, 128] with bf16 weight w [128] -> bf16 values.

    y = x / sqrt(mean(x^2) + eps) * (1 + w).  [qsa] QSAIndexer holds q_layernorm and
    k_layernorm as GemmaRMSNorm(head_dim, eps=rms_norm_eps, default 1e-6); the (1 + w) weight
    convention is the Gemma one, written out on the patch page [fp8kv] as
    `normalized * (1.0 + weight)`.
    """
    ss = halving_sum(x * x)                      # x*x is exact in float64
    var = ss / float(HEAD_DIM) + float(np.float32(eps))
    inv = 1.0 / np.sqrt(var)
    y = (x * inv[:, None]) * (1.0 + w)[None, :]
    return round_bf16(y)


# ----------------------------------------------------------------------------- A2/A3: RoPE


def mrope_axis_of_pair(mrope_section) -> np.ndarray:
    """Position axis (0 = T, 1 = H, 2 = W) used by each of the 32 rotary frequencies.

    The pages only constrain interleaved MRoPE: three sections summing to rotary_dim / 2
    ([indexer] _supports_fused_pre_indexer; [qsa] Qwen4ExpQSAAttention.__init__).
    Reading: frequency i uses H when i % 3 == 1 and i < 3*s_H, W when i % 3 == 2 and
    i < 3*s_W, T otherwise.  With equal T/H/W positions any assignment gives 1-D RoPE.
    """
    s_t, s_h, s_w = (int(v) for v in mrope_section)
    if s_t + s_h + s_w != HALF_ROT:
        raise ValueError("mrope_section must sum to rotary_dim / 2")
    axis = np.zeros(HALF_ROT, dtype=np.int64)
    for i in range(HALF_ROT):
        if i % 3 == 1 and i < 3 * s_h:
            axis[i] = 1
        elif i % 3 == 2 and i < 3 * s_w:
            axis[i] = 2
    return axis


def gather_cos_sin(cos_sin: np.ndarray, pos: np.ndarray, mrope_section=None):
    """cos, sin [N, 32] (float32 values as float64) for 1-D positions [N] or triples [N, 3].

    cos_sin [max_pos, 64] holds the cosines in its first 32 columns and the sines in the
    last 32 ([indexer] apply_qsa_rope gathers the cache at the positions and splits it in
    two halves).
    """
    table = np.asarray(cos_sin, dtype=np.float32).astype(np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    if mrope_section is None or not any(mrope_section):
        rows = table[pos]
        return rows[:, :HALF_ROT], rows[:, HALF_ROT:]
    axis = mrope_axis_of_pair(mrope_section)
    sel = pos[:, axis]                            # [N, 32] position per frequency
    cols = np.arange(HALF_ROT)[None, :]
    return table[sel, cols], table[sel, cols + HALF_ROT]


def neox_rope(y: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half (NeoX) rotary embedding of dims 0..63 of bf16 rows y [N, 128]; dims
    64..127 pass through ([indexer] apply_qsa_rope rotates the first rotary_dim dims and
    concatenates the rest; the fused path requires is_neox_style, head_dim 128 and
    rotary_dim 64, _supports_fused_pre_indexer).  Dim i pairs with dim i + 32."""
    out = y.copy()
    a = y[:, :HALF_ROT]
    b = y[:, HALF_ROT:ROTARY_DIM]
    out[:, :HALF_ROT] = a * cos - b * sin       # products exact; one rounding per result
    out[:, HALF_ROT:ROTARY_DIM] = b * cos + a * sin
    return round_bf16(out)


# ----------------------------------------------------------------------------- Q prep


def prepare_index_q(q_proj, rope_pos, cos_sin, mrope_section, q_norm_w, eps, num_heads,
                    idx_dtype):
    """Indexer Q: per-head RMSNorm -> RoPE at the row's position -> indexer dtype.

    [qsa] QSAIndexer.forward, unfused reference path: gemma_rmsnorm, apply_qsa_rope, then
    `.to(self.indexer_dtype)`.  Returns (codes [T, Hi, 128], values [T, Hi, 128]).
    """
    T = q_proj.shape[0]
    x = bf16_bits_to_f64(q_proj[:, :num_heads * HEAD_DIM]).reshape(T * num_heads, HEAD_DIM)
    w = bf16_bits_to_f64(q_norm_w)
    y = gemma_rmsnorm(x, w, eps)
    pos = np.repeat(np.asarray(rope_pos, dtype=np.int64), num_heads, axis=0)
    cos, sin = gather_cos_sin(cos_sin, pos, mrope_section)
    y = neox_rope(y, cos, sin)
    codes = encode_index_values(y, idx_dtype)
    return codes.reshape(T, num_heads, HEAD_DIM), decode_index_codes(codes, idx_dtype).reshape(
        T, num_heads, HEAD_DIM)


# ----------------------------------------------------------------------------- A2: compress


@dataclass
class CompressState:
    """Indexer caches the compress step reads and updates (all arrays are copied)."""
    ring: np.ndarray            # [ring_pages, S, 128] uint16: raw keys, slot = token % S
    ring_pos: np.ndarray | None  # [ring_pages, S, 3] int64 (MRoPE only)
    ckv: np.ndarray             # [c_pages, Pc, 128] uint16 (bf16) or uint8 (e4m3fn)


def compress_step(query_start_loc, seq_lens, k_proj, rope_pos, mrope_section, cos_sin,
                  k_norm_w, eps, ring_page, c_block_table, compress_ratio, idx_dtype,
                  state: CompressState, requests=None) -> CompressState:
    """Pool every group of `compress_ratio` raw keys completed by this step's rows, normalise
    and rotate it, and store it in the compressed-key cache; then update the raw-key ring.

    [ops] qsa_compress_groups_with_ratio: pools completed groups from the compressor-state
    ring and the step's raw rows, returning the pooled bf16 row and the positions of the
    group's first token; [qsa] QSAIndexer.forward then applies k_layernorm and
    apply_qsa_rope at those positions and stores the rows with qsa_store_cache_rows
    (compressed cache first, then the raw ring and its position ring).

    Readings: group g completes at token (g+1)*c - 1 and is the MEAN of its c raw keys
    (sum first to last in float64, divided by c, rounded to bf16); the key is rotated at the
    position of token g*c -- its logical position for 1-D RoPE (the unfused path passes
    logical_positions there), its position triple for MRoPE; the ring keeps token t in slot
    t % S, and after the step it holds the last min(S, seq_len) tokens.

    `requests` optionally restricts the work to a subset of requests (for sampling).
    """
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    c = int(compress_ratio)
    S = state.ring.shape[1]
    Pc = state.ckv.shape[1]
    mrope = mrope_section is not None and any(mrope_section)
    ring = state.ring.copy()
    ring_pos = None if state.ring_pos is None else state.ring_pos.copy()
    ckv = state.ckv.copy()
    w = bf16_bits_to_f64(k_norm_w)
    rope_pos = np.asarray(rope_pos, dtype=np.int64)
    reqs = range(len(lens)) if requests is None else requests

    for r in reqs:
        n = qsl[r + 1] - qsl[r]
        L = lens[r]
        start = L - n                                   # first token of this step
        rp = int(ring_page[r])

        def raw_key(t):
            if t >= start:
                return bf16_bits_to_f64(k_proj[qsl[r] + t - start, :HEAD_DIM])
            return bf16_bits_to_f64(state.ring[rp, t % S])

        def rope_triple(t):
            if t >= start:
                return rope_pos[qsl[r] + t - start]
            return state.ring_pos[rp, t % S]

        groups = [g for g in range(start // c, L // c) if (g + 1) * c - 1 >= start]
        if groups:
            pooled = []
            for g in groups:
                acc = raw_key(g * c).copy()
                for m in range(1, c):
                    acc = acc + raw_key(g * c + m)
                pooled.append(acc / float(c))
            pooled = round_bf16(np.stack(pooled))
            y = gemma_rmsnorm(pooled, w, eps)
            if mrope:
                pos = np.stack([rope_triple(g * c) for g in groups])
            else:
                pos = np.array([g * c for g in groups], dtype=np.int64)
            cos, sin = gather_cos_sin(cos_sin, pos, mrope_section)
            y = neox_rope(y, cos, sin)
            codes = encode_index_values(y, idx_dtype)
            for g, row in zip(groups, codes):
                page = int(c_block_table[r, g // Pc])
                ckv[page, g % Pc] = row
        # Ring update, after every read of this request.
        for t in range(max(start, L - S), L):
            ring[rp, t % S] = k_proj[qsl[r] + t - start, :HEAD_DIM]
            if ring_pos is not None:
                ring_pos[rp, t % S] = rope_pos[qsl[r] + t - start]
    return CompressState(ring=ring, ring_pos=ring_pos, ckv=ckv)


# ----------------------------------------------------------------------------- main prepare


def encode_scaled_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    """e4m3fn codes of x / scale for a main K/V cache with a static per-tensor scale.

    [fp8kv] the cache bytes are written by reshape_and_cache_flash with the layer's scales,
    and that writer clamps to +-448 (it never emits the NaN codes).  Reading: the quotient is
    taken in float32 (correctly rounded), clamped to [-448, 448], then rounded to nearest
    even on the e4m3fn grid.
    """
    q = (np.asarray(x, dtype=np.float64) / float(np.float32(scale))).astype(np.float32)
    return f64_to_e4m3_bits(np.clip(q.astype(np.float64), -448.0, 448.0))


def prepare_main(main_qkv, rope_pos, cos_sin, mrope_section, q_norm_w, k_norm_w, eps,
                 num_q_heads, num_kv_heads, kv_cache, slot_mapping, kv_dtype="bf16",
                 k_scale=1.0, v_scale=1.0):
    """Main-attention prepare: normalised, rotated Q, and the step's K/V in the paged cache.

    [qsa] Qwen4ExpQSAAttention: the q/k/v projection packs a sigmoid output gate next to Q
    (2*Hq heads of 128), then Hkv K heads and Hkv V heads; q_norm and k_norm are
    GemmaRMSNorm(head_dim); the fused qsa_prepare launch takes the main qkv, both norm
    weights, one epsilon, the main cache, the slot mapping and the K/V scales, and returns
    (query, output_gate); the unfused path writes K/V with reshape_and_cache_flash, which
    skips rows whose slot is negative.

    Readings: each Q head's 256 values are its q (first 128) then its gate (last 128); Q and
    K are rotated like the indexer (NeoX on dims 0..63, with the same cos/sin table and the
    row's rotary position: the fused launch receives one table for both); slot s stores at
    page s // P, offset s % P; the gate is returned untouched (the attention reads it in
    place).  The chain is the canonical one of the indexer prep (RMSNorm -> bf16 -> RoPE ->
    bf16); V is stored as given.

    main_qkv: [T, (2*Hq + 2*Hkv)*128] uint16; kv_cache [pages, Hkv, P, 256] uint16 (bf16) or
    uint8 (fp8: K and V as encode_scaled_e4m3 with k_scale / v_scale).  Returns (q bits
    [T, Hq, 128] uint16, a copy of the cache with the step's rows written).
    """
    main_qkv = np.asarray(main_qkv)
    T = main_qkv.shape[0]
    Hq, Hkv, D = int(num_q_heads), int(num_kv_heads), HEAD_DIM
    qg = main_qkv[:, :2 * Hq * D].reshape(T, Hq, 2, D)
    k_bits = main_qkv[:, 2 * Hq * D:(2 * Hq + Hkv) * D].reshape(T, Hkv, D)
    v_bits = main_qkv[:, (2 * Hq + Hkv) * D:(2 * Hq + 2 * Hkv) * D].reshape(T, Hkv, D)
    pos = np.asarray(rope_pos, dtype=np.int64)

    def norm_rope(x_bits, w_bits, heads):
        x = bf16_bits_to_f64(x_bits).reshape(T * heads, D)
        y = gemma_rmsnorm(x, bf16_bits_to_f64(w_bits), eps)
        cos, sin = gather_cos_sin(cos_sin, np.repeat(pos, heads, axis=0), mrope_section)
        return neox_rope(y, cos, sin).reshape(T, heads, D)

    q_out = f64_to_bf16_bits(norm_rope(qg[:, :, 0, :], q_norm_w, Hq)) if T else \
        np.zeros((0, Hq, D), np.uint16)
    cache = np.array(kv_cache, copy=True)
    if T == 0:
        return q_out, cache
    k_vals = norm_rope(k_bits, k_norm_w, Hkv)
    pages, _, P, _ = cache.shape
    for t in range(T):
        slot = int(slot_mapping[t])
        if slot < 0 or slot // P >= pages:
            continue
        page, off = slot // P, slot % P
        for h in range(Hkv):
            if kv_dtype == "fp8":
                cache[page, h, off, :D] = encode_scaled_e4m3(k_vals[t, h], k_scale)
                cache[page, h, off, D:] = encode_scaled_e4m3(bf16_bits_to_f64(v_bits[t, h]),
                                                             v_scale)
            else:
                cache[page, h, off, :D] = f64_to_bf16_bits(k_vals[t, h])
                cache[page, h, off, D:] = v_bits[t, h]
    return q_out, cache


# ----------------------------------------------------------------------------- A3-A5: select


def index_scores(q_vals: np.ndarray, keys: np.ndarray, agg: str = "sum") -> np.ndarray:
    """Indexer score of one row against compressed keys [n, 128]: the sum over the indexer
    heads of the per-head dot products, float64.

    [qsa] QSAIndexer is "weight-free selection"; the decode logits buffer holds one float32
    per (token, compressed column) ([qsa] Qwen4ExpQSAAttention._run_qsa sizes it as
    tokens x columns x 4 bytes), so heads are reduced inside the logits.  Reading: no per-head
    weights, no activation (agg "sum").  The aggregation switch agg "relu" takes max(0, .) of
    each head's product before the sum -- the ReLU-sum of other sparse indexers, kept as an
    alternative should the plain reading prove wrong.  Canonical order: each head's 128
    products by `halving_sum`, then the heads added in order 0, 1, ..., Hi-1.
    """
    if agg not in ("sum", "relu"):
        raise ValueError(f"unknown aggregation {agg!r}")
    s = None
    for h in range(q_vals.shape[0]):
        t = halving_sum(keys * q_vals[h][None, :])
        if agg == "relu":
            t = np.maximum(t, 0.0)
        s = t if s is None else s + t
    return s


def select_blocks(scores: np.ndarray, kb: int) -> np.ndarray:
    """Indices of the kb best blocks, ascending.  Order: higher score first; an exactly
    equal score goes to the lower block index (reading; the pages do not say)."""
    n = len(scores)
    if n <= kb:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -scores))   # primary: -score, secondary: index
    return np.sort(order[:kb])


def expand_row(blocks: np.ndarray, p: int, c: int, budget: int) -> np.ndarray:
    """Packed selection row [W + 1] int32, W = budget + c - 1 ([qsa] QSAIndexer.output_width
    and packed_output_width).

    The chosen blocks' tokens g*c .. g*c+c-1 in ascending order, then the tokens of the
    incomplete group at the row's end (vis*c .. p), then -1 padding, and the count of valid
    entries in the last column ([qsa] QSAIndexer.forward docstring: -1-padded
    request-relative token indices plus a trailing valid-entry count).
    """
    W = budget + c - 1
    vis = (p + 1) // c
    toks = [np.arange(g * c, g * c + c) for g in blocks] + [np.arange(vis * c, p + 1)]
    toks = np.concatenate(toks) if toks else np.zeros(0, np.int64)
    row = np.full(W + 1, -1, dtype=np.int64)
    row[:len(toks)] = toks
    row[W] = len(toks)
    return row.astype(np.int32)


def compressed_keys_of_request(ckv_vals: np.ndarray, c_block_table_row: np.ndarray, n: int):
    """The first n compressed keys of a request, gathered through its block table.  A block
    whose page is outside the cache reads as an all-zero key (reading)."""
    Pc = ckv_vals.shape[1]
    j = np.arange(n)
    col = j // Pc
    page = np.where(col < len(c_block_table_row),
                    c_block_table_row[np.minimum(col, len(c_block_table_row) - 1)], -1)
    ok = (page >= 0) & (page < ckv_vals.shape[0])
    keys = ckv_vals[np.where(ok, page, 0), j % Pc]
    keys[~ok] = 0.0
    return keys


def index_topk(query_start_loc, seq_lens, q_codes, ckv, c_block_table, compress_ratio,
               budget, idx_dtype, rows=None, agg="sum"):
    """Packed selection buffer [T, W + 1] int32 for every row (or only `rows`; the others
    stay -1 with count 0, like the inert rows of [qsa] QSAIndexer.forward).

    Row at position p sees vis = floor((p + 1) / c) completed blocks (reading: a row sees the
    group it completes; W = budget + c - 1 then leaves room for the c - 1 tail tokens).  If
    vis <= budget / c every visible block is taken, otherwise the budget / c best by
    `index_scores` (with aggregation `agg`).
    """
    c = int(compress_ratio)
    kb = budget // c
    W = budget + c - 1
    T = q_codes.shape[0]
    req = request_of_rows(query_start_loc)
    pos = logical_positions(query_start_loc, seq_lens)
    q_vals = decode_index_codes(q_codes, idx_dtype)
    ckv_vals = decode_index_codes(ckv, idx_dtype)
    packed = np.full((T, W + 1), -1, dtype=np.int32)
    packed[:, W] = 0
    rows = range(T) if rows is None else rows
    key_cache = {}
    for i in rows:
        r = int(req[i])
        p = int(pos[i])
        vis = (p + 1) // c
        if vis <= kb:
            blocks = np.arange(vis)
        else:
            if r not in key_cache:
                key_cache = {r: compressed_keys_of_request(
                    ckv_vals, c_block_table[r], int(seq_lens[r]) // c)}
            s = index_scores(q_vals[i], key_cache[r][:vis], agg)
            blocks = select_blocks(s, kb)
        packed[i] = expand_row(blocks, p, c, budget)
    return packed


# ----------------------------------------------------------------------------- A6/A7: GQA


def sparse_gqa(q, kv_cache, block_table, token_to_req, packed, gate=None, scale=None,
               rows=None, kv_dtype="bf16", k_scale=1.0, v_scale=1.0):
    """Sparse GQA over the selected tokens of each row, float64 -> [T, Hq, 128].

    [ops] qsa_sparse_paged_attention / [fp8kv] _qsa_sparse_paged_gqa_splitk_kernel: Q head
    hq uses KV head hq // (Hq / Hkv); entry t of a row maps to page block_table[req,
    t // page_size] and slot t % page_size; entries past the row's count, negative entries
    and pages outside the cache contribute nothing; the result is the softmax-weighted mean
    of V with scale head_dim^-0.5, and a row with no valid entry gives 0.  The optional
    sigmoid output gate multiplies the result ([qsa-old] the gate applied after attention;
    [qsa] fused into the kernel).

    kv_cache: [pages, Hkv, P, 256] uint16, K in the first 128 values of a token's row and V in
    the last 128 ([qsa] Qwen4ExpQSAImpl.forward splits kv_cache.transpose(1, 2) at head_size).
    With kv_dtype "fp8" it holds uint8 e4m3fn codes and static per-tensor scales: K = code *
    k_scale, V = code * v_scale ([fp8kv], e4m3 branch: the kernel folds k_scale into the score
    scale and v_scale into the epilogue, which is the same attention over these values).
    """
    q = bf16_bits_to_f64(q)
    T, Hq, D = q.shape
    pages, Hkv, P, _ = kv_cache.shape
    G = Hq // Hkv
    W = packed.shape[1] - 1
    scale = D ** -0.5 if not scale else float(scale)
    out = np.zeros((T, Hq, D))
    g = None if gate is None else bf16_bits_to_f64(gate)
    rows = range(T) if rows is None else rows
    for i in rows:
        r = int(token_to_req[i])
        count = int(min(max(int(packed[i, W]), 0), W))
        idx = packed[i, :count].astype(np.int64)
        col = idx // P
        ok = (idx >= 0) & (col < block_table.shape[1])
        page = np.where(ok, block_table[r, np.clip(col, 0, block_table.shape[1] - 1)], -1)
        ok &= (page >= 0) & (page < pages)
        idx, page = idx[ok], page[ok]
        if len(idx) == 0:
            continue
        if kv_dtype == "fp8":
            rows_kv = e4m3_bits_to_f64(kv_cache[page, :, idx % P, :])  # [n, Hkv, 256]
            ks, vs = float(k_scale), float(v_scale)
        else:
            rows_kv = bf16_bits_to_f64(kv_cache[page, :, idx % P, :])
            ks = vs = 1.0
        for hq in range(Hq):
            kvh = hq // G
            k = rows_kv[:, kvh, :D] * ks
            v = rows_kv[:, kvh, D:] * vs
            z = (k @ q[i, hq]) * scale
            wgt = np.exp(z - z.max())
            out[i, hq] = (wgt @ v) / wgt.sum()
        if g is not None:
            out[i] = out[i] * (1.0 / (1.0 + np.exp(-g[i])))
    return out
