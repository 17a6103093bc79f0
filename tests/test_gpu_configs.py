"""GPU parity on every configuration the C ABI accepts beyond the five workloads' own shapes:
decode and prefill requests mixed in one call, GQA group sizes 1, 2, 4 and 16, compress
ratios 2, 16, 32 and 64, main pages of 32 and 48 tokens, compressed pages of 5, 8 and 32 rows,
and 1, 3, 12 and 16 indexer heads.

Bars as in the workload parity tests: prepared Q, compressed-cache and ring bytes bit-exact;
packed selection int-exact; attention output within max-abs 2e-2 (bf16 indexer) or 6e-2 (fp8
indexer) of the float64 oracle.  Every case runs the whole step through the C ABI.
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import TOL, gpu_out_f64, log, max_abs, oracle_step, run_gpu, to_np, workload

pytestmark = pytest.mark.gpu

# name -> (base workload, overrides of its scaled-down configuration)
CASES = {
    # [qsa] QSAIndexer.forward: decode requests lead the batch, prefill requests follow.  Rows
    # of one-row requests are scored on the vector units, requests of more than 16 rows on
    # the matrix cores, in the same call.
    "mixed_bf16": ("decode_32k", dict(num_requests=6, rows=(1, 1, 1, 1, 40, 24))),
    "mixed_fp8": ("fp8_decode", dict(num_requests=6, rows=(1, 1, 1, 150, 33, 2))),
    # 1,102 rows in the call: the prefill configuration of the top-k next to decode rows.
    "mixed_topk_prefill": ("decode_32k", dict(num_requests=3, rows=(1, 1, 1100),
                                              lengths=("fixed", 2200))),
    # Contexts up to the largest the top-k holds in registers (32,768 compressed columns): the
    # 1,024-thread configuration, beyond the 16,384 columns of the workloads' own shapes.
    # Two rows per request (speculative decoding with one draft token): the two-row instance
    # of the vector-unit logits.
    "two_rows": ("decode_32k", dict(rows=2)),
    "long_context": ("decode_32k", dict(num_requests=3, lengths=("uniform", 70000, 131072))),
    # One-row batches that fill the chip with 2048-key logits workgroups (the wide instance of
    # the vector-unit logits), bf16 and e4m3 indexer.
    "wide_bf16": ("decode_32k", dict(num_requests=256, compress_ratio=2, lengths=("fixed", 4096))),
    "wide_fp8": ("fp8_decode", dict(num_requests=256, compress_ratio=2, lengths=("fixed", 4096))),
    "wide_ragged": ("decode_32k", dict(num_requests=128, lengths=("uniform", 10000, 14000))),
    "max_context": ("decode_32k", dict(num_requests=2, lengths=("fixed", 131072))),
    # GQA group sizes ([ops] qsa_sparse_paged_attention pads the group to a power of two).
    "G1": ("decode_32k", dict(q_heads=2, kv_heads=2)),
    "G2": ("decode_32k", dict(q_heads=4, kv_heads=2)),
    "G4": ("spec_verify_mrope", dict(q_heads=8, kv_heads=2)),
    "G16": ("chunked_prefill", dict(q_heads=16, kv_heads=1, rows=96)),
    "G16_fp8kv": ("decode_32k_fp8kv", dict(q_heads=16, kv_heads=1)),
    "G1_fp8kv": ("decode_32k_fp8kv", dict(q_heads=4, kv_heads=4)),
    "G2_fp8kv": ("decode_32k_fp8kv", dict(q_heads=4, kv_heads=2)),
    "G4_fp8kv": ("decode_32k_fp8kv", dict(q_heads=8, kv_heads=2)),
    # Compress ratios: any power of two > 1 ([indexer] _supports_fused_pre_indexer); the ring
    # is at least one group wide.
    "c2": ("decode_32k", dict(compress_ratio=2, rows=3)),
    "c2_prefill": ("chunked_prefill", dict(compress_ratio=2, num_requests=1, rows=1100,
                                           lengths=("fixed", 2600))),
    "c16": ("spec_verify_mrope", dict(compress_ratio=16, ring_size=32)),
    "c32": ("chunked_prefill", dict(compress_ratio=32, ring_size=32, rows=96)),
    "c64": ("fp8_decode", dict(compress_ratio=64, ring_size=64, rows=2)),
    # Main KV pages: any multiple of 16 tokens ([qsa] Qwen4ExpQSABackend's kernel block sizes).
    "P32": ("decode_32k", dict(page_size=32)),
    "P48_fp8kv": ("decode_32k_fp8kv", dict(page_size=48)),
    # Compressed-key pages of other sizes, a non-power of two among them.
    "Pc8": ("decode_32k", dict(c_page_size=8)),
    "Pc32": ("chunked_prefill", dict(c_page_size=32, rows=96)),
    "Pc5": ("fp8_decode", dict(c_page_size=5)),
    # Indexer head counts: the matrix-core logits hold up to 8 heads; 9..16 go to the vector
    # units for prefill too.
    "Hi16_prefill": ("chunked_prefill", dict(index_heads=16, rows=96)),
    "Hi3_prefill_fp8": ("chunked_prefill_fp8", dict(index_heads=3, rows=96)),
    "Hi12_decode": ("decode_32k", dict(index_heads=12)),
    "Hi1_decode_fp8": ("fp8_decode", dict(index_heads=1)),
}


def _case(name):
    base, over = CASES[name]
    return workload(base, **over)


@pytest.mark.parametrize("name", list(CASES))
def test_step_parity_on_accepted_configuration(name):
    wl = _case(name)
    log(f"config {name}: T={wl.num_tokens} R={wl.num_requests} rows={wl.rows_host.tolist()[:8]} "
        f"Hq/Hkv={wl.q_heads}/{wl.kv_heads} c={wl.compress_ratio} Hi={wl.index_heads} "
        f"P={wl.kv_cache.shape[2]} Pc={wl.ckv.shape[1]} S={wl.ring.shape[1]} "
        f"decode_requests={wl.num_decode_requests}")
    ref = oracle_step(wl)                    # reads the pre-state before the GPU updates it
    st = run_gpu(wl)
    assert np.array_equal(to_np(st.q_idx).view(np.uint8), ref.q_codes.view(np.uint8))
    assert np.array_equal(to_np(wl.ckv).view(np.uint8), ref.state_after.ckv.view(np.uint8))
    assert np.array_equal(to_np(wl.ring), ref.state_after.ring)
    if wl.ring_pos is not None:
        assert np.array_equal(to_np(wl.ring_pos), ref.state_after.ring_pos)
    packed = to_np(st.packed)
    assert np.array_equal(packed, ref.packed), (
        f"{int((packed != ref.packed).any(axis=1).sum())} rows differ")
    err = max_abs(gpu_out_f64(st), ref.out)
    log(f"  max-abs {err:.3e}")
    assert err <= TOL[wl.index_dtype]


@pytest.mark.parametrize("name", ["G1", "G2", "G4", "G16", "G16_fp8kv", "G1_fp8kv", "P32",
                                  "P48_fp8kv"])
def test_attention_split_invariance_on_accepted_configuration(name):
    """The attention alone on the oracle's selection, with one split, the automatic plan and
    the maximum (every split merged by log-sum-exp)."""
    wl = _case(name)
    log(f"config gqa {name}")
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
    for o in outs[1:]:
        assert max_abs(outs[0], o) <= 2 ** -6
