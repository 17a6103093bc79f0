"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: prepared Q, compressed-cache and ring bytes bit-exact; packed selection int-exact;
attention output within max-abs 2e-2 (bf16 indexer) or 6e-2 (fp8 indexer) of the float64
oracle.
"""

import numpy as np
import pytest
import torch

from oracle import qsa as oq
from oracle.numerics import bf16_bits_to_f64, e4m3_bits_to_f64
from sparse_attention_qsa_amd import binding as B
from sparse_attention_qsa_amd.step import QsaStep
from tests.gpu_util import (SCALED, TOL, gpu_out_f64, log, max_abs, oracle_step, run_gpu,
                            to_np, workload)
from tests.oracle_io import oracle_compress

pytestmark = pytest.mark.gpu

NAMES = list(SCALED)


# ----------------------------------------------------------------------------- device arithmetic


def test_device_e4m3_decoders_match_the_definition():
    log("diag: e4m3 decode of all 256 codes")
    out = B.qsa_diag_e4m3_decode().cpu().numpy().astype(np.float64)
    ref = e4m3_bits_to_f64(np.arange(256, dtype=np.uint32).astype(np.uint8))
    assert np.array_equal(out[:256], ref, equal_nan=True), "hardware e4m3 converter"
    assert np.array_equal(out[256:], ref, equal_nan=True), "definitional e4m3 decoder"


def test_device_fp64_sqrt_and_divide_are_correctly_rounded():
    log("diag: fp64 sqrt / divide on 2M inputs")
    rng = np.random.default_rng(7)
    x = np.concatenate([
        np.exp(rng.uniform(-40, 40, 1_000_000)),
        rng.uniform(1e-6, 300.0, 1_000_000),          # the range RMSNorm variances live in
    ])
    got = B.qsa_diag_fp64_sqrt_div(torch.from_numpy(x).cuda()).cpu().numpy().reshape(-1, 3)
    r = np.sqrt(x)
    assert np.array_equal(got[:, 0], r)
    assert np.array_equal(got[:, 1], 1.0 / x)
    assert np.array_equal(got[:, 2], 1.0 / r)


# ----------------------------------------------------------------------------- the three calls


@pytest.mark.parametrize("name", NAMES)
def test_compress_bytes_match_oracle(name):
    wl = workload(name)
    log(f"compress parity {name}: T={wl.num_tokens} R={wl.num_requests}")
    ref = oracle_step(wl, with_attention=False)        # reads the pre-state first
    st = run_gpu(wl)
    assert np.array_equal(to_np(st.q_idx).view(np.uint8), ref.q_codes.view(np.uint8))
    assert np.array_equal(to_np(wl.ckv).view(np.uint8), ref.state_after.ckv.view(np.uint8))
    assert np.array_equal(to_np(wl.ring), ref.state_after.ring)
    if wl.ring_pos is not None:
        assert np.array_equal(to_np(wl.ring_pos), ref.state_after.ring_pos)


@pytest.mark.parametrize("name", NAMES)
def test_selection_is_exact_and_attention_within_tolerance(name):
    wl = workload(name)
    log(f"step parity {name}: T={wl.num_tokens} R={wl.num_requests}")
    ref = oracle_step(wl)
    st = run_gpu(wl)
    packed = to_np(st.packed)
    assert np.array_equal(packed, ref.packed), (
        f"{int((packed != ref.packed).any(axis=1).sum())} rows differ")
    err = max_abs(gpu_out_f64(st), ref.out)
    log(f"  max-abs {err:.3e}")
    assert err <= TOL[wl.index_dtype]


@pytest.mark.parametrize("name", ["tiny_decode", "decode_32k", "spec_verify_mrope",
                                  "decode_32k_fp8kv"])
def test_attention_alone_on_oracle_indices_and_split_invariance(name):
    wl = workload(name)
    log(f"gqa parity {name}")
    ref = oracle_step(wl)
    st = run_gpu(wl)
    st.packed.copy_(torch.from_numpy(ref.packed).cuda())
    outs = []
    for splits in (1, 0, 4, 1000):
        st.g_args.num_splits = splits
        st.gqa()
        torch.cuda.synchronize()
        o = gpu_out_f64(st)
        assert max_abs(o, ref.out) <= TOL[wl.index_dtype]
        outs.append(o)
    # Split count changes only float32 summation order and one bf16 rounding.
    for o in outs[1:]:
        assert max_abs(outs[0], o) <= 2 ** -6


def test_full_size_decode_32k_on_sampled_rows():
    wl = workload("decode_32k", num_requests=64, lengths=("fixed", 32768))
    rows = [0, 17, 42, 63]
    log(f"full-size decode_32k, sampled rows {rows}")
    ref = oracle_step(wl, rows=rows)
    st = run_gpu(wl)
    packed = to_np(st.packed)
    assert np.array_equal(packed[rows], ref.packed[rows])
    err = max_abs(gpu_out_f64(st)[rows], ref.out[rows])
    log(f"  max-abs {err:.3e}")
    assert err <= TOL["bf16"]
    # Every row: count, ascending indices, -1 padding (properties that hold at any size).
    W = wl.output_width
    assert np.all(packed[:, W] == 2048)
    assert np.all(np.diff(packed[:, :2048], axis=1) > 0)
    assert np.all(packed[:, 2048:W] == -1)


def test_full_size_decode_32k_fp8_kv_on_sampled_rows():
    """The fp8 main-KV attention at the size bench.py times for it, in that launch
    configuration, on sampled rows."""
    wl = workload("decode_32k_fp8kv", num_requests=64, lengths=("fixed", 32768))
    rows = [1, 30, 62]
    log(f"full-size decode_32k_fp8kv, sampled rows {rows}")
    ref = oracle_step(wl, rows=rows)
    st = run_gpu(wl)
    assert np.array_equal(to_np(st.packed)[rows], ref.packed[rows])
    err = max_abs(gpu_out_f64(st)[rows], ref.out[rows])
    log(f"  max-abs {err:.3e}")
    assert err <= TOL["bf16"]


def test_full_size_fp8_decode_on_sampled_rows():
    """The fp8-indexer decode workload at the size bench.py times (128 requests of 4096..65536
    tokens), in that launch configuration: its logits grid does not fit the chip in one round,
    so the persistent work-list kernel scores it."""
    wl = workload("fp8_decode", num_requests=128, lengths=("uniform", 4096, 65536))
    L = wl.seq_lens_host
    rows = sorted({0, 63, 127, int(np.argmax(L)), int(np.argmin(L))})
    log(f"full-size fp8_decode, sampled rows {rows}")
    ref = oracle_step(wl, rows=rows)
    st = run_gpu(wl)
    packed = to_np(st.packed)
    assert np.array_equal(packed[rows], ref.packed[rows])
    err = max_abs(gpu_out_f64(st)[rows], ref.out[rows])
    log(f"  max-abs {err:.3e}")
    assert err <= TOL["fp8"]
    # Every row (one per request, p = L - 1, at least 512 visible blocks): kb*c plus the tail.
    W, c = wl.output_width, wl.compress_ratio
    assert np.array_equal(packed[:, W], 2048 + L % c)
    for i in range(wl.num_tokens):
        n = packed[i, W]
        assert np.all(np.diff(packed[i, :n]) > 0) and packed[i, 0] >= 0
        assert packed[i, n - 1] <= L[i] - 1 and np.all(packed[i, n:W] == -1)


def test_full_size_spec_verify_on_sampled_rows():
    """The speculative-verify workload at the size bench.py times (256 requests of 1024..131072
    tokens, 4 MRoPE rows each, fp8 indexer), on rows of the longest, the shortest and a few
    other requests."""
    wl = workload("spec_verify_mrope", num_requests=256, lengths=("loguniform", 1024, 131072))
    L = wl.seq_lens_host
    reqs = sorted({0, 100, 255, int(np.argmax(L)), int(np.argmin(L))})
    rows = [4 * r + i for r in reqs for i in (0, 3)]
    log(f"full-size spec_verify_mrope, requests {reqs}")
    ref = oracle_step(wl, rows=rows)
    st = run_gpu(wl)
    packed = to_np(st.packed)
    assert np.array_equal(packed[rows], ref.packed[rows])
    err = max_abs(gpu_out_f64(st)[rows], ref.out[rows])
    log(f"  max-abs {err:.3e}")
    assert err <= TOL["fp8"]


@pytest.mark.parametrize("case", ["bf16_1row", "bf16_2rows", "bf16_3rows", "fp8_2rows", "relu"])
def test_work_list_kernel_on_many_short_requests(case):
    """Batches whose one-item-per-workgroup logits grid would not fit the chip in one round are
    scored by the persistent work-list kernel: many requests of uneven length, each compared
    row by row (bf16 indexer with one, two and three rows per request, e4m3 with two, and the
    ReLU-sum switch)."""
    rows = {"bf16_2rows": 2, "bf16_3rows": 3, "fp8_2rows": 2}.get(case, 1)
    R = 300 if rows == 3 else 600
    base = "fp8_decode" if case.startswith("fp8") else "decode_32k"
    wl = workload(base, num_requests=R, lengths=("uniform", 2100, 6000), rows=rows)
    agg = "relu" if case == "relu" else "sum"
    log(f"work-list logits {case}: R={R} T={wl.num_tokens}")
    ref = oracle_step(wl, with_attention=False, agg=agg)
    st = QsaStep(wl, index_agg=agg)
    st.compress()
    st.topk()
    torch.cuda.synchronize()
    packed = to_np(st.packed)
    assert np.array_equal(packed, ref.packed), (
        f"{int((packed != ref.packed).any(axis=1).sum())} rows differ")


@pytest.mark.parametrize("name", ["chunked_prefill", "chunked_prefill_fp8"])
def test_work_list_kernel_with_matrix_core_requests(name):
    """Many prefill requests (17 rows each, scored on the matrix cores) in a call whose max |k|
    pass needs the work-list kernel, bf16 and e4m3 indexer; sampled rows compared."""
    wl = workload(name, num_requests=270, lengths=("uniform", 2100, 4000), rows=17)
    rows = [0, 16, 17 * 100 + 5, 17 * 269 + 16]
    log(f"work-list max|k| pass with MFMA requests: T={wl.num_tokens}")
    ref = oracle_step(wl, rows=rows, with_attention=False)
    st = QsaStep(wl)
    st.compress()
    st.topk()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(st.packed)[rows], ref.packed[rows])


def _cap_for_rows(wl, rows: int) -> int:
    """A logits cap (bytes) that makes windows of `rows` rows."""
    cols = max(1, wl.max_seq_len // wl.compress_ratio)
    return rows * ((cols + 63) // 64 * 64) * 4


@pytest.mark.parametrize("name,rows,kw", [
    ("chunked_prefill", 100, {}),                  # windows cut 128-row matrix-core blocks
    ("chunked_prefill", 1100, dict(rows=640)),     # a window of 1100 rows: prefill top-k
    ("decode_32k", 2, {}),
    ("spec_verify_mrope", 7, {}),                  # windows cut a request's verify rows
    ("fp8_decode", 3, {}),
    ("decode_32k", 150, dict(num_requests=600, lengths=("uniform", 2100, 6000))),  # work list
    ("decode_32k", 3, dict(rows=2)),               # two and three rows per request, windowed
    ("decode_32k", 4, dict(rows=3)),
    ("fp8_decode", 3, dict(rows=2)),
    ("chunked_prefill_fp8", 100, {}),              # e4m3 max |k| pass in windows
    # Decode and prefill requests in one call under a cap: windows that hold only decode rows,
    # windows that start inside a prefill request (past its first 128-row block too), and
    # windows holding the end of one prefill request and the start of the next.
    ("decode_32k", 3, dict(num_requests=6, rows=(1, 1, 1, 1, 40, 24))),
    ("decode_32k", 200, dict(num_requests=5, rows=(1, 1, 300, 1, 260))),
])
def test_logits_cap_runs_in_windows_with_the_same_selection(name, rows, kw):
    """With a logits memory cap the call scores and selects window by window, reusing a
    workspace sized for one window; the packed rows equal the oracle's, bit for bit."""
    wl = workload(name, **kw)
    cap = _cap_for_rows(wl, rows)
    log(f"logits cap {name}: T={wl.num_tokens}, windows of {rows} rows")
    ref = oracle_step(wl, with_attention=False)
    st = QsaStep(wl, max_logits_bytes=cap)
    full = B.lib().qsa_index_logits_topk_workspace_size(
        B.C.byref(QsaStep(workload(name, **kw)).t_args))
    assert st.t_ws.numel() < full or rows >= wl.num_tokens
    st.compress()
    st.topk()
    torch.cuda.synchronize()
    packed = to_np(st.packed)
    assert np.array_equal(packed, ref.packed), (
        f"{int((packed != ref.packed).any(axis=1).sum())} rows differ")


def test_logits_cap_with_relu_sum():
    wl = workload("decode_32k", num_requests=40, lengths=("uniform", 2100, 6000), rows=3)
    q_codes, after = oracle_compress(wl)
    ref = oq.index_topk(to_np(wl.query_start_loc), to_np(wl.seq_lens), q_codes, after.ckv,
                        to_np(wl.c_block_table), wl.compress_ratio, wl.budget, wl.index_dtype,
                        agg="relu")
    st = QsaStep(wl, index_agg="relu", max_logits_bytes=_cap_for_rows(wl, 10))
    st.compress()
    st.topk()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(st.packed), ref)


def test_prefill_row_counts_select_exactly():
    """Calls with many rows take the prefill top-k configuration (three 8-bit radix passes,
    256 threads): 1280 rows here, every one compared."""
    wl = workload("chunked_prefill", rows=640)
    assert wl.num_tokens >= 1024
    log(f"prefill top-k parity: T={wl.num_tokens}")
    ref = oracle_step(wl, with_attention=False)
    st = run_gpu(wl)
    packed = to_np(st.packed)
    assert np.array_equal(packed, ref.packed), (
        f"{int((packed != ref.packed).any(axis=1).sum())} rows differ")


def test_full_size_chunked_prefill_on_sampled_rows():
    """The whole chunked_prefill step (4 x 8192 rows on 8192 cached tokens: MFMA logits,
    prefill top-k, attention) at full size, on sampled rows."""
    wl = workload("chunked_prefill", num_requests=4, lengths=("fixed", 16384), rows=8192)
    rows = [0, 4097, 8191, 8192 + 777, 3 * 8192 + 8191]
    log(f"full-size chunked_prefill, sampled rows {rows}")
    ref = oracle_step(wl, rows=rows, with_attention=False)
    st = QsaStep(wl)
    st.compress()
    st.topk()
    torch.cuda.synchronize()
    packed = to_np(st.packed)
    assert np.array_equal(packed[rows], ref.packed[rows])
    # Every row: the count is kb*c plus the uncompressed tail (p+1) mod c, p = 8192 + i.
    W, c = wl.output_width, wl.compress_ratio
    p = 8192 + np.tile(np.arange(8192), 4)
    assert np.array_equal(packed[:, W], 2048 + (p + 1) % c)
    # The attention over the 32,768 rows (one split each, the launch bench.py times), on the
    # sampled rows, from the oracle's own selection.
    st.gqa()
    torch.cuda.synchronize()
    ref_out = oq.sparse_gqa(to_np(wl.q), to_np(wl.kv_cache), to_np(wl.block_table),
                            to_np(wl.token_to_req), ref.packed, gate=to_np(wl.gate), rows=rows)
    err = max_abs(gpu_out_f64(st)[rows], ref_out[rows])
    log(f"  attention max-abs {err:.3e}")
    assert err <= TOL["bf16"]


def test_full_size_chunked_prefill_fp8_indexer_on_sampled_rows():
    """The fp8-indexer prefill (e4m3 logits on the matrix cores) at full size, sampled rows,
    selection and attention."""
    wl = workload("chunked_prefill_fp8", num_requests=4, lengths=("fixed", 16384), rows=8192)
    rows = [3, 4096 + 5, 8192 + 8191, 2 * 8192 + 128, 3 * 8192 + 4000]
    log(f"full-size chunked_prefill_fp8, sampled rows {rows}")
    ref = oracle_step(wl, rows=rows)
    st = run_gpu(wl)
    packed = to_np(st.packed)
    assert np.array_equal(packed[rows], ref.packed[rows])
    err = max_abs(gpu_out_f64(st)[rows], ref.out[rows])
    log(f"  max-abs {err:.3e}")
    assert err <= TOL["fp8"]


def test_fp8_kv_scales_act_on_scores_and_output():
    """Doubling v_scale doubles the output; a k_scale change equals the same change of the
    softmax scale (both within the float32 / bf16 rounding of the kernel)."""
    wl = workload("decode_32k_fp8kv")
    st = run_gpu(wl)
    base = gpu_out_f64(st)
    st.g_args.v_scale = 2.0 * wl.v_scale
    st.gqa()
    torch.cuda.synchronize()
    assert max_abs(gpu_out_f64(st), 2.0 * base) <= 2 ** -7 * (np.abs(base).max() + 1.0)
    st.g_args.v_scale = wl.v_scale
    st.g_args.k_scale = 1.5 * wl.k_scale
    st.gqa()
    torch.cuda.synchronize()
    a = gpu_out_f64(st)
    st.g_args.k_scale = wl.k_scale
    st.g_args.scale = 1.5 * 128 ** -0.5
    st.gqa()
    torch.cuda.synchronize()
    assert max_abs(a, gpu_out_f64(st)) <= 2 ** -6


# ----------------------------------------------------------------------------- edge cases


def test_budget_at_least_context_gives_every_token():
    wl = workload("tiny_decode", budget=4096)
    ref = oracle_step(wl)
    st = run_gpu(wl)
    assert np.array_equal(to_np(st.packed), ref.packed)
    assert max_abs(gpu_out_f64(st), ref.out) <= TOL["bf16"]


def test_exact_ties_go_to_the_lower_block():
    # Every compressed row of the pre-state is the same key: all visible blocks tie exactly
    # (except the ones this step writes), so the selection is decided by block index alone.
    wl = workload("decode_32k", num_requests=3, lengths=("fixed", 5000))
    row = wl.ckv[wl.c_block_table[0, 0], 0].clone()
    wl.ckv[:] = row
    ref = oracle_step(wl, with_attention=False)
    st = run_gpu(wl)
    assert np.array_equal(to_np(st.packed), ref.packed)


@pytest.mark.parametrize("base,kw", [
    ("decode_32k", dict(num_requests=3, lengths=("fixed", 5000))),
    ("chunked_prefill", dict(num_requests=2, lengths=("fixed", 3000), rows=600)),
])
def test_all_zero_keys_tie_whatever_the_sign_of_zero(base, kw):
    """An all-zero compressed cache (the step's own groups aside): the canonical scores of
    the visible blocks are +0 or -0 (a product with a negative query element is -0), which
    tie exactly, so the lower blocks win.  The band is every visible block, which the top-k
    ranks by a radix select over (score, block) rather than by pairwise comparison."""
    wl = workload(base, **kw)
    wl.ckv.zero_()
    log(f"all-zero keys: {base} T={wl.num_tokens}")
    ref = oracle_step(wl, with_attention=False)
    st = run_gpu(wl)
    packed = to_np(st.packed)
    assert np.array_equal(packed, ref.packed), (
        f"{int((packed != ref.packed).any(axis=1).sum())} rows differ")


def test_exact_ties_on_matrix_core_rows():
    """Rows scored on the matrix cores (stored as fp16, certified with the rounding bound):
    every compressed row of the pre-state is the same key, so the visible blocks tie exactly
    and the lower block index decides; one call takes the decode top-k configuration (fewer
    than 1024 rows), the other the prefill one."""
    for rows in (100, 600):
        wl = workload("chunked_prefill", num_requests=2, lengths=("fixed", 3000), rows=rows)
        row = wl.ckv[wl.c_block_table[0, 0], 0].clone()
        wl.ckv[:] = row
        log(f"matrix-core ties: T={wl.num_tokens}")
        ref = oracle_step(wl, with_attention=False)
        st = run_gpu(wl)
        packed = to_np(st.packed)
        assert np.array_equal(packed, ref.packed), (
            f"{int((packed != ref.packed).any(axis=1).sum())} rows differ")


def test_exact_ties_on_fp8_matrix_core_rows():
    wl = workload("chunked_prefill_fp8", num_requests=2, lengths=("fixed", 3000), rows=100)
    row = wl.ckv[wl.c_block_table[0, 0], 0].clone()
    wl.ckv[:] = row
    ref = oracle_step(wl, with_attention=False)
    st = run_gpu(wl)
    assert np.array_equal(to_np(st.packed), ref.packed)


@pytest.mark.parametrize("w", [1023.0, 65535.0])
def test_matrix_core_rows_with_scaled_fp16_logits(w):
    """Matrix-core logits are stored as fp16 scaled by 2^-e per row (e from kappa * A).
    Indexer norm weights of w make the scores far exceed the fp16 range (|q . k| ~ 1e4 .. 1e9;
    e = 7 and more), and the selection must still be the oracle's, in the decode (fewer than
    1024 rows) and the prefill top-k configurations."""
    for rows in (100, 600):
        wl = workload("chunked_prefill", num_requests=2, lengths=("fixed", 3000), rows=rows)
        wl.q_norm_w.fill_(w)
        wl.k_norm_w.fill_(w)
        log(f"scaled fp16 logits: w={w} T={wl.num_tokens}")
        ref = oracle_step(wl, with_attention=False)
        st = run_gpu(wl)
        packed = to_np(st.packed)
        assert np.array_equal(packed, ref.packed), (
            f"{int((packed != ref.packed).any(axis=1).sum())} rows differ")


@pytest.mark.parametrize("splits", [0, 4, 1000])
def test_inert_rows_invalid_entries_and_empty_requests(splits):
    """A row with count 0, a negative entry and an entry past the block table, with the
    automatic plan, four splits merged in the workgroup and the most splits (merge kernel)."""
    wl = workload("tiny_decode")
    ref = oracle_step(wl)
    st = run_gpu(wl)
    st.g_args.num_splits = splits
    W = wl.output_width
    packed = ref.packed.copy()
    packed[0, W] = 0                              # count 0 -> zero output
    packed[1, 5] = -1                             # a masked entry
    packed[2, 7] = 10 ** 6                        # past the block table -> masked
    st.packed.copy_(torch.from_numpy(packed).cuda())
    st.gqa()
    torch.cuda.synchronize()
    ref_out = oq.sparse_gqa(to_np(wl.q), to_np(wl.kv_cache), to_np(wl.block_table),
                            to_np(wl.token_to_req), packed, gate=to_np(wl.gate))
    out = gpu_out_f64(st)
    assert np.all(out[0] == 0.0)
    assert max_abs(out, ref_out) <= TOL["bf16"]


def test_zero_rows_is_a_no_op():
    wl = workload("tiny_decode")
    st = run_gpu(wl)
    before = st.out.clone()
    a = B.gqa_args(q=wl.q[:0], kv_cache=wl.kv_cache, block_table=wl.block_table,
                   token_to_req=wl.token_to_req[:0], packed=st.packed[:0], out=st.out[:0])
    assert B.lib().qsa_sparse_gqa(B.C.byref(a), None, 0, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(before, st.out)


@pytest.mark.parametrize("name,splits", [("decode_32k", 0), ("decode_32k", 4),
                                         ("chunked_prefill", 0), ("fp8_decode", 0)])
def test_single_kernel_calls_equal_the_combined_calls(name, splits):
    """qsa_index_logits + qsa_block_topk and qsa_sparse_gqa_partial + qsa_sparse_gqa_merge
    (the per-kernel calls the benchmark times) give the combined calls' results bit for bit;
    with splits merged in the workgroup the merge call has nothing to do."""
    wl = workload(name)
    twin = workload(name)
    log(f"single-kernel calls {name}: T={wl.num_tokens}, num_splits={splits}")
    a = QsaStep(wl, num_splits=splits)
    a.run()
    b = QsaStep(twin, num_splits=splits)
    b.compress()
    b.logits()
    b.block_topk()
    b.gqa_partial()
    b.gqa_merge()
    torch.cuda.synchronize()
    assert a.num_splits == b.num_splits
    assert np.array_equal(to_np(a.packed), to_np(b.packed))
    assert np.array_equal(to_np(a.out), to_np(b.out))



@pytest.mark.parametrize("name", ["tiny_decode", "decode_32k", "fp8_decode", "chunked_prefill"])
def test_relu_sum_selection_is_exact(name):
    """The ReLU-sum aggregation switch: the selection equals the oracle's on the same workload
    (bit for bit), and differs from the plain-sum selection somewhere."""
    wl = workload(name)
    log(f"relu-sum selection {name}: T={wl.num_tokens}")
    q_codes, after = oracle_compress(wl)
    args = (to_np(wl.query_start_loc), to_np(wl.seq_lens), q_codes, after.ckv,
            to_np(wl.c_block_table), wl.compress_ratio, wl.budget, wl.index_dtype)
    ref = oq.index_topk(*args, agg="relu")
    st = QsaStep(wl, index_agg="relu")
    st.compress()
    st.topk()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(st.packed), ref)
    if name != "tiny_decode":
        assert not np.array_equal(ref, oq.index_topk(*args, agg="sum"))


def test_relu_sum_with_sixteen_heads():
    """ReLU-sum with 16 indexer heads (every operand column of the matrix-core kernel a head)."""
    wl = workload("decode_32k", index_heads=16)
    q_codes, after = oracle_compress(wl)
    ref = oq.index_topk(to_np(wl.query_start_loc), to_np(wl.seq_lens), q_codes, after.ckv,
                        to_np(wl.c_block_table), wl.compress_ratio, wl.budget, wl.index_dtype,
                        agg="relu")
    st = QsaStep(wl, index_agg="relu")
    st.compress()
    st.topk()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(st.packed), ref)


def _advance(wl, seed):
    """The next decode step of `wl` (one row per request): each request one token longer, its
    row at the next position with fresh projections; the caches are shared with `wl`."""
    import copy
    nxt = copy.copy(wl)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    nxt.seq_lens_host = wl.seq_lens_host + wl.rows_host
    nxt.seq_lens = wl.seq_lens + torch.from_numpy(wl.rows_host).to(torch.int32).cuda()
    nxt.max_seq_len = int(nxt.seq_lens_host.max())
    nxt.positions = wl.positions + 1
    for name in ("q_proj", "k_proj", "q", "gate"):
        t = getattr(wl, name)
        setattr(nxt, name, torch.randn(t.shape, generator=g, device="cuda").to(t.dtype))
    return nxt


def test_speculative_step_reuses_selection_and_rollback_rewrites_the_caches():
    """Later speculative steps reuse step 0's selection (the pages' skip_topk: the caches are
    still updated, the top-k is skipped, the attention reads the step-0 packed rows); a rejected
    token is rolled back by running the next step at the same position again, which leaves the
    caches exactly as if the rejected token had never been written (the ring is wider than a
    group, so no slot a pooled group needs is overwritten)."""
    wl = workload("decode_32k")
    log(f"speculative reuse and rollback: R={wl.num_requests}")
    st0 = QsaStep(wl)
    st0.run()
    torch.cuda.synchronize()
    packed0 = st0.packed.clone()
    pre = (wl.ring.clone(), wl.ckv.clone())            # caches after step 0
    # Step 1 (a speculative token X): compress, no top-k, attention on the step-0 rows.
    x = _advance(wl, 11)
    q_codes, after = oracle_compress(x)                 # oracle from the post-step-0 caches
    st1 = QsaStep(x)
    st1.compress()
    st1.packed.copy_(packed0)
    st1.gqa()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(wl.ckv).view(np.uint8), after.ckv.view(np.uint8))
    assert np.array_equal(to_np(wl.ring), after.ring)
    ref = oq.sparse_gqa(to_np(x.q), to_np(x.kv_cache), to_np(x.block_table),
                        to_np(x.token_to_req), to_np(packed0), gate=to_np(x.gate))
    assert max_abs(gpu_out_f64(st1), ref) <= TOL[wl.index_dtype]
    # Rollback: token X rejected, the step runs again at the same position with token Y.
    y = _advance(wl, 12)
    QsaStep(y).compress()
    torch.cuda.synchronize()
    after_xy = (wl.ring.clone(), wl.ckv.clone())
    wl.ring.copy_(pre[0])
    wl.ckv.copy_(pre[1])
    QsaStep(y).compress()                               # Y alone, from the step-0 caches
    torch.cuda.synchronize()
    assert torch.equal(after_xy[0], wl.ring)
    assert torch.equal(after_xy[1].view(torch.uint8), wl.ckv.view(torch.uint8))


@pytest.mark.parametrize("name", ["decode_32k", "spec_verify_mrope", "chunked_prefill"])
def test_step_captured_in_a_graph_replays_the_eager_results(name):
    """The three calls make no host synchronisation, allocation or memset, so a caller can
    capture a whole step in a HIP graph (decode loops in serving engines do).  Every replay,
    with eager work on the same buffers in between, gives the eager step's results bit for
    bit (this also covers the work-list kernel, which clears its own counter on the device)."""
    wl = workload(name)
    log(f"graph replay {name}: T={wl.num_tokens}")
    st = QsaStep(wl)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run(side)                       # eager, on a side stream, before the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_packed, ref_out = st.packed.clone(), st.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()
    for rep in range(3):
        st.packed.fill_(-7)                # eager work between the replays
        st.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"  replay {rep}")
        assert torch.equal(st.packed, ref_packed)
        assert torch.equal(st.out.view(torch.int16), ref_out.view(torch.int16))
        st.run()                           # an eager step between replays too
        torch.cuda.synchronize()
        assert torch.equal(st.packed, ref_packed)
    del g


def test_row_tiled_prefill_attention_every_row_and_adversarial_entries():
    """With row_tiles set, calls of 2048+ rows with 8 query heads per KV head take the
    row-tiled kernel for every 32-row tile of one request (the tile that straddles the two requests, and the rows past the
    last full tile, go to the per-row kernel).  Every row is compared with the oracle, with the
    top-k's selection and then with rows holding a duplicated entry (its tile falls back to the
    per-row kernel, which counts the token twice as the oracle does), negative entries and
    entries past the block table."""
    wl = workload("chunked_prefill", num_requests=2, rows=1100, lengths=("fixed", 3300))
    assert wl.num_tokens >= 2048
    log(f"row-tiled attention: T={wl.num_tokens}")
    ref = oracle_step(wl)
    st = run_gpu(wl)
    assert np.array_equal(to_np(st.packed), ref.packed)
    per_row = gpu_out_f64(st)
    st.g_args.row_tiles = 1
    st.gqa()
    torch.cuda.synchronize()
    err = max_abs(gpu_out_f64(st), ref.out)
    log(f"  max-abs (selection) {err:.3e}; against the per-row path {max_abs(gpu_out_f64(st), per_row):.3e}")
    assert max_abs(gpu_out_f64(st), per_row) <= 2 ** -6
    assert err <= TOL["bf16"]
    W = wl.output_width
    adv = ref.packed.copy()
    r_dup, r_neg, r_big = 5, 40, 1500
    c = adv[r_dup, W]
    adv[r_dup, c] = adv[r_dup, 7]            # token listed twice
    adv[r_dup, W] = c + 1
    adv[r_neg, 3] = -1
    adv[r_neg, 10] = -77
    adv[r_big, 0] = 10 ** 7                  # past the block table
    st.packed.copy_(torch.from_numpy(adv).cuda())
    st.gqa()
    torch.cuda.synchronize()
    want = oq.sparse_gqa(to_np(wl.q), to_np(wl.kv_cache), to_np(wl.block_table),
                         to_np(wl.token_to_req), adv, gate=to_np(wl.gate))
    err = max_abs(gpu_out_f64(st), want)
    log(f"  max-abs (adversarial entries) {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("chunk_bytes", [1024, 2048, 3072, 4096])
def test_read_bandwidth_probe_reads_every_chunk_once(chunk_bytes):
    """The bench's read probe folds the XOR of every 32-bit word it reads into one word: a
    streaming read gives the XOR of the whole buffer, a gather the XOR of the listed chunks
    (a chunk listed twice cancels out)."""
    g = torch.Generator().manual_seed(chunk_bytes)
    n_chunks = 3001
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_chunks * chunk_bytes // 4,), generator=g,
                          dtype=torch.int64).to(torch.int32)
    src = words.cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.qsa_diag_read_bandwidth(src, chunk_bytes, sink)
    torch.cuda.synchronize()
    per_chunk = np.bitwise_xor.reduce(words.numpy().view(np.uint32).reshape(n_chunks, -1), axis=1)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(per_chunk))
    idx = torch.randint(0, n_chunks, (5000,), generator=g, dtype=torch.int32)
    sink.zero_()
    B.qsa_diag_read_bandwidth(src, chunk_bytes, sink, chunk_index=idx.cuda())
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(per_chunk[idx.numpy()])
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(expect)
