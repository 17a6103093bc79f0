"""Seeded synthetic inputs for the QSA hot path.

This module only draws random numbers and lays them out; it holds none of the method's
arithmetic.  The tests feed the same tensors to the HIP library and to the CPU oracle, and
the benchmark times the library on them.

The five workloads (sizes as the project's benchmark configurations state them):
  tiny_decode         1 request, 2048 tokens, 4 query rows at its tail; indexer 4 Q heads,
                      c = 4, budget 256, bf16; attention 8 Q / 1 KV heads.
  decode_32k          64 requests x 32768 tokens, 1 row each; indexer 8 heads, c = 4,
                      budget 2048, bf16; attention 16 Q / 2 KV heads.
  fp8_decode          128 requests, lengths uniform in [4096, 65536], 1 row each; fp8
                      indexer, c = 8, budget 2048; attention 16 / 2.
  chunked_prefill     4 requests, each 8192 new rows on top of 8192 cached tokens; indexer 8
                      heads, c = 4, budget 2048, bf16; attention 16 / 2.
  spec_verify_mrope   256 requests, lengths log-uniform in [1024, 131072], 4 verify rows
                      each, interleaved MRoPE positions [rows, 3] with section (12, 10, 10),
                      c = 8, budget 4096, fp8 indexer; fragmented page tables.
  decode_32k_fp8kv    decode_32k with the main KV cache in e4m3fn codes and static scales
                      (k_scale 0.0167, v_scale 0.0161).

Recipe: activations N(0, 1) float32 rounded to bf16; norm weights N(0, 0.1^2) -> bf16; the
rotary table cos/sin(pos * 10000^(-2i/64)) in float64 rounded to float32; the indexer
pre-state (the raw-key ring holding the S tokens before the step, and the compressed rows of
every group completed before the step) is drawn N(0, 1) -> bf16 (-> e4m3fn for the fp8
indexer); main K/V N(0, 1) bf16 for every token; page tables are seeded random permutations
of a page pool (1.25x the pages needed for the fragmented workload); unused cache rows are
filled with NaN so that a read of one shows up in the output.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEAD_DIM = 128
ROTARY_DIM = 64
PAGE_SIZE = 16          # main KV page (tokens)
C_PAGE_SIZE = 16        # compressed-key cache page (compressed rows)
RING_SIZE = 16          # raw-key ring slots per request

CONFIGS = {
    "tiny_decode": dict(num_requests=1, lengths=("fixed", 2048), rows=4, index_heads=4,
                        compress_ratio=4, budget=256, index_dtype="bf16", q_heads=8,
                        kv_heads=1, mrope_section=None, pool_factor=1.0),
    "decode_32k": dict(num_requests=64, lengths=("fixed", 32768), rows=1, index_heads=8,
                       compress_ratio=4, budget=2048, index_dtype="bf16", q_heads=16,
                       kv_heads=2, mrope_section=None, pool_factor=1.0),
    "fp8_decode": dict(num_requests=128, lengths=("uniform", 4096, 65536), rows=1,
                       index_heads=8, compress_ratio=8, budget=2048, index_dtype="fp8",
                       q_heads=16, kv_heads=2, mrope_section=None, pool_factor=1.0),
    "chunked_prefill": dict(num_requests=4, lengths=("fixed", 16384), rows=8192,
                            index_heads=8, compress_ratio=4, budget=2048, index_dtype="bf16",
                            q_heads=16, kv_heads=2, mrope_section=None, pool_factor=1.0),
    "spec_verify_mrope": dict(num_requests=256, lengths=("loguniform", 1024, 131072), rows=4,
                              index_heads=8, compress_ratio=8, budget=4096,
                              index_dtype="fp8", q_heads=16, kv_heads=2,
                              mrope_section=(12, 10, 10), pool_factor=1.25),
    # decode_32k with an fp8 e4m3 main KV cache and static per-tensor scales (the FP8 KV
    # reader patch page); the scales are arbitrary non-powers of two that keep N(0, 1) values
    # far inside the e4m3 range.
    "decode_32k_fp8kv": dict(num_requests=64, lengths=("fixed", 32768), rows=1, index_heads=8,
                             compress_ratio=4, budget=2048, index_dtype="bf16", q_heads=16,
                             kv_heads=2, mrope_section=None, pool_factor=1.0,
                             kv_dtype="fp8", k_scale=0.0167, v_scale=0.0161),
    # chunked_prefill with the fp8 e4m3 indexer (its logits on the fp8 matrix cores).
    "chunked_prefill_fp8": dict(num_requests=4, lengths=("fixed", 16384), rows=8192,
                                index_heads=8, compress_ratio=4, budget=2048,
                                index_dtype="fp8", q_heads=16, kv_heads=2, mrope_section=None,
                                pool_factor=1.0),
}

CONFIG_SEEDS = {"decode_32k_fp8kv": 1006, "tiny_decode": 1001, "decode_32k": 1002, "fp8_decode": 1003,
                "chunked_prefill": 1004, "spec_verify_mrope": 1005, "chunked_prefill_fp8": 1007}


@dataclasses.dataclass
class Workload:
    """All inputs of one step (device tensors; bf16 data as torch.bfloat16, e4m3fn data as
    torch.uint8)."""
    name: str
    num_requests: int
    num_tokens: int
    index_heads: int
    compress_ratio: int
    budget: int
    index_dtype: str
    q_heads: int
    kv_heads: int
    mrope_section: tuple | None
    eps: float
    seq_lens_host: np.ndarray          # [R] int64 (host copy of seq_lens)
    rows_host: np.ndarray              # [R] int64 rows per request
    max_query_len: int
    max_seq_len: int
    query_start_loc: torch.Tensor      # [R+1] int32
    seq_lens: torch.Tensor             # [R] int32
    token_to_req: torch.Tensor         # [T] int32
    positions: torch.Tensor            # [T] or [T, 3] int64 rotary positions
    q_proj: torch.Tensor               # [T, Hi*128] bf16
    k_proj: torch.Tensor               # [T, 128] bf16
    cos_sin: torch.Tensor              # [max_pos, 64] float32
    q_norm_w: torch.Tensor             # [128] bf16
    k_norm_w: torch.Tensor             # [128] bf16
    ring: torch.Tensor                 # [ring_pages, S, 128] bf16
    ring_pos: torch.Tensor | None      # [ring_pages, S, 3] int64 (MRoPE only)
    ring_page: torch.Tensor            # [R] int32
    ckv: torch.Tensor                  # [c_pages, Pc, 128] bf16 or uint8 (e4m3fn)
    c_block_table: torch.Tensor        # [R, cw] int32
    q: torch.Tensor                    # [T, Hq, 128] bf16
    kv_cache: torch.Tensor             # [pages, Hkv, P, 256] bf16, or uint8 e4m3fn codes
    block_table: torch.Tensor          # [R, bw] int32
    gate: torch.Tensor                 # [T, Hq, 128] bf16
    kv_dtype: str = "bf16"             # "bf16" or "fp8" (K = code * k_scale, V = code * v_scale)
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def output_width(self) -> int:
        return self.budget + self.compress_ratio - 1

    @property
    def num_decode_requests(self) -> int:
        """Leading requests whose rows form a uniform decode batch: the run of requests at the
        front with the first request's row count, when that count is small (all of them for a
        uniform decode batch; none when the batch starts with a prefill request)."""
        n0 = int(self.rows_host[0])
        if n0 > DECODE_MAX_ROWS:
            return 0
        k = 0
        while k < self.num_requests and int(self.rows_host[k]) == n0:
            k += 1
        return k

    @property
    def decode_query_len(self) -> int:
        return int(self.rows_host[0]) if self.num_decode_requests else 0


DECODE_MAX_ROWS = 16


def _torch_gen(device, seed: int, field: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1009 + field)
    return g


def _normal_bf16(shape, device, seed, field, std=1.0):
    g = _torch_gen(device, seed, field)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16)


def rotary_table(max_pos: int, base: float = 10000.0) -> torch.Tensor:
    """cos/sin table [max_pos, 64]: columns 0..31 cos(pos * base^(-2i/64)), 32..63 sin."""
    i = np.arange(ROTARY_DIM // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / ROTARY_DIM)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32))


def _lengths(spec, R, rng):
    kind = spec[0]
    if kind == "fixed":
        return np.full(R, spec[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(spec[1], spec[2] + 1, size=R).astype(np.int64)
    if kind == "loguniform":
        lo, hi = math.log(spec[1]), math.log(spec[2])
        return np.floor(np.exp(rng.uniform(lo, hi, size=R))).astype(np.int64)
    raise ValueError(kind)


def _page_table(needed: np.ndarray, pool_factor: float, rng):
    """Random page assignment: a table [R, max(needed)] of distinct pages from a pool of
    ceil(pool_factor * sum(needed)) pages (-1 past each request's need)."""
    total = int(needed.sum())
    pool = max(1, int(math.ceil(total * pool_factor)))
    perm = rng.permutation(pool)[:total].astype(np.int32)
    width = max(1, int(needed.max()))
    table = np.full((len(needed), width), -1, dtype=np.int32)
    off = 0
    for r, n in enumerate(needed):
        table[r, :n] = perm[off:off + n]
        off += n
    return table, pool


def make_workload(name: str, device="cpu", seed: int | None = None, **overrides) -> Workload:
    """Build the named workload.  `overrides` replace entries of its configuration (e.g.
    num_requests=4, lengths=("fixed", 600), rows=3) for scaled-down parity cases.  `rows` may
    also be a sequence (rows of each request: decode requests first, then prefill requests, as
    one mixed batch), and page_size, c_page_size and ring_size replace the main page (16), the
    compressed page (16) and the raw-key ring width (16)."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    seed = CONFIG_SEEDS.get(name, 1000) if seed is None else seed
    rng = np.random.default_rng(seed)
    R = int(cfg["num_requests"])
    lens = _lengths(cfg["lengths"], R, rng)
    if np.ndim(cfg["rows"]) == 0:
        rows = np.full(R, int(cfg["rows"]), dtype=np.int64)
    else:
        rows = np.asarray(cfg["rows"], dtype=np.int64)
        if rows.shape != (R,):
            raise ValueError("rows must give one count per request")
    rows = np.minimum(rows, lens)
    T = int(rows.sum())
    c = int(cfg["compress_ratio"])
    Hi = int(cfg["index_heads"])
    Hq, Hkv = int(cfg["q_heads"]), int(cfg["kv_heads"])
    mrope = cfg["mrope_section"]
    idt = cfg["index_dtype"]
    S = int(cfg.get("ring_size", RING_SIZE))
    Pc = int(cfg.get("c_page_size", C_PAGE_SIZE))
    P = int(cfg.get("page_size", PAGE_SIZE))

    qsl = np.zeros(R + 1, dtype=np.int64)
    qsl[1:] = np.cumsum(rows)
    tok_req = np.repeat(np.arange(R), rows).astype(np.int32)
    logical = np.concatenate([np.arange(L - n, L) for L, n in zip(lens, rows)]).astype(np.int64)

    # Rotary positions: 1-D logical positions, or interleaved MRoPE triples (t, t+dh, t+dw)
    # with per-token offsets in 0..63.
    max_pos = int(lens.max()) + 128
    if mrope:
        off_rng = np.random.default_rng(seed + 77)

        def triples(t):
            d = off_rng.integers(0, 64, size=(len(t), 2))
            return np.stack([t, t + d[:, 0], t + d[:, 1]], 1).astype(np.int64)
        positions = triples(logical)
    else:
        positions = logical.copy()

    # Ring pre-state: one page per request (a seeded permutation), raw keys of the S tokens
    # before the step in slots t % S.
    ring_page = rng.permutation(R).astype(np.int32)
    ring = _normal_bf16((R, S, HEAD_DIM), device, seed, 1)
    ring_pos = None
    if mrope:
        rp = np.zeros((R, S, 3), dtype=np.int64)
        for r in range(R):
            start = lens[r] - rows[r]
            t = np.arange(max(0, start - S), start)
            if len(t):
                rp[ring_page[r], t % S] = triples(t)
        ring_pos = torch.from_numpy(rp).to(device)

    # Compressed-key cache: rows of groups completed before the step are random
    # (N(0,1) -> bf16 [-> e4m3fn]); every other row is NaN.
    vis_max = lens // c
    c_need = (vis_max + Pc - 1) // Pc
    c_table, c_pages = _page_table(c_need, cfg["pool_factor"], rng)
    ckv_vals = _normal_bf16((c_pages, Pc, HEAD_DIM), device, seed, 2)
    valid = torch.zeros((c_pages, Pc), dtype=torch.bool)
    for r in range(R):
        done = int((lens[r] - rows[r]) // c)
        g = np.arange(done)
        if done:
            pg = torch.from_numpy(c_table[r, g // Pc].astype(np.int64))
            valid[pg, torch.from_numpy(g % Pc)] = True
    valid = valid.to(device)
    if idt == "fp8":
        ckv = ckv_vals.to(torch.float8_e4m3fn).view(torch.uint8)
        ckv = torch.where(valid[..., None], ckv, torch.full_like(ckv, 0x7F))
    else:
        ckv = torch.where(valid[..., None], ckv_vals,
                          torch.full_like(ckv_vals, float("nan")))

    # Main paged K/V: every token of every request holds N(0,1) K and V; other slots NaN.
    need = (lens + P - 1) // P
    table, pages = _page_table(need, cfg["pool_factor"], rng)
    kv = _normal_bf16((pages, Hkv, P, 2 * HEAD_DIM), device, seed, 3)
    used = torch.zeros((pages, P), dtype=torch.bool)
    for r in range(R):
        n_full, rem = divmod(int(lens[r]), P)
        pg = torch.from_numpy(table[r, :need[r]].astype(np.int64))
        used[pg[:n_full]] = True
        if rem:
            used[pg[n_full], :rem] = True
    kv = torch.where(used.to(device)[:, None, :, None], kv, torch.full_like(kv, float("nan")))
    kv_dtype = cfg.get("kv_dtype", "bf16")
    k_scale = float(cfg.get("k_scale", 1.0))
    v_scale = float(cfg.get("v_scale", 1.0))
    if kv_dtype == "fp8":
        # e4m3fn codes of value / scale (clamped inside the finite range); unused slots keep
        # the NaN code 0x7F.
        sc = torch.cat([torch.full((HEAD_DIM,), k_scale), torch.full((HEAD_DIM,), v_scale)])
        x = kv.float() / sc.to(device)
        x = torch.where(torch.isnan(x), x, x.clamp(-440.0, 440.0))
        kv = x.to(torch.float8_e4m3fn).view(torch.uint8)
        kv = torch.where(used.to(device)[:, None, :, None], kv, torch.full_like(kv, 0x7F))

    def dev(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.to(dtype) if dtype is not None else t).to(device)

    return Workload(
        name=name, num_requests=R, num_tokens=T, index_heads=Hi, compress_ratio=c,
        budget=int(cfg["budget"]), index_dtype=idt, q_heads=Hq, kv_heads=Hkv,
        mrope_section=tuple(mrope) if mrope else None, eps=1e-6,
        seq_lens_host=lens, rows_host=rows, max_query_len=int(rows.max()),
        max_seq_len=int(lens.max()),
        query_start_loc=dev(qsl, torch.int32), seq_lens=dev(lens, torch.int32),
        token_to_req=dev(tok_req), positions=dev(positions),
        q_proj=_normal_bf16((T, Hi * HEAD_DIM), device, seed, 4),
        k_proj=_normal_bf16((T, HEAD_DIM), device, seed, 5),
        cos_sin=rotary_table(max_pos).to(device),
        q_norm_w=_normal_bf16((HEAD_DIM,), device, seed, 6, std=0.1),
        k_norm_w=_normal_bf16((HEAD_DIM,), device, seed, 7, std=0.1),
        ring=ring, ring_pos=ring_pos, ring_page=dev(ring_page), ckv=ckv,
        c_block_table=dev(c_table), q=_normal_bf16((T, Hq, HEAD_DIM), device, seed, 8),
        kv_cache=kv, block_table=dev(table),
        gate=_normal_bf16((T, Hq, HEAD_DIM), device, seed, 9),
        kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale,
    )


def main_prepare_inputs(wl: Workload, seed: int | None = None) -> dict:
    """Inputs of the main-attention prepare for a workload's rows (the keyword block of the
    binding's `main` argument): the packed main projection [T, (2Hq + 2Hkv)*128] ~ N(0, 1)
    (per Q head its q then its gate, then the K and V heads), norm weights ~ N(0, 0.1^2), and
    the slot of each row's token in the workload's main cache (page from its block table,
    offset p % P).  Draws numbers only; the output buffer main_q is allocated here."""
    seed = CONFIG_SEEDS.get(wl.name, 1000) if seed is None else seed
    device = wl.q_proj.device
    T, Hq, Hkv = wl.num_tokens, wl.q_heads, wl.kv_heads
    P = wl.kv_cache.shape[2]
    qsl = wl.query_start_loc.cpu().numpy().astype(np.int64)
    table = wl.block_table.cpu().numpy().astype(np.int64)
    slots = np.empty(T, dtype=np.int64)
    for r in range(wl.num_requests):
        n = qsl[r + 1] - qsl[r]
        p = np.arange(wl.seq_lens_host[r] - n, wl.seq_lens_host[r])
        slots[qsl[r]:qsl[r + 1]] = table[r, p // P] * P + p % P
    out = dict(
        main_qkv=_normal_bf16((T, (2 * Hq + 2 * Hkv) * HEAD_DIM), device, seed, 10),
        num_q_heads=Hq, num_kv_heads=Hkv,
        main_q_norm_weight=_normal_bf16((HEAD_DIM,), device, seed, 11, std=0.1),
        main_k_norm_weight=_normal_bf16((HEAD_DIM,), device, seed, 12, std=0.1),
        main_eps=1e-6,
        main_q=torch.empty((T, Hq, HEAD_DIM), dtype=torch.bfloat16, device=device),
        main_kv_cache=wl.kv_cache,
        main_slot_mapping=torch.from_numpy(slots).to(device),
    )
    if wl.kv_dtype == "fp8":
        out.update(main_k_scale=wl.k_scale, main_v_scale=wl.v_scale)
    return out
