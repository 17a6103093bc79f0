"""GPU parity of the main-attention prepare (fused into qsa_compress) against the oracle,
through the C ABI: main Q bits and the whole main cache bit-exact, the indexer results
unchanged, and the attention on the prepared Q with the gate read in place within the
attention tolerance."""

import numpy as np
import pytest
import torch

from oracle import qsa as oq
from oracle.numerics import bf16_bits_to_f64
from sparse_attention_qsa_amd.step import QsaStep
from sparse_attention_qsa_amd.workloads import main_prepare_inputs
from tests.gpu_util import TOL, log, max_abs, to_np, workload
from tests.oracle_io import oracle_compress

pytestmark = pytest.mark.gpu

NAMES = ["tiny_decode", "decode_32k", "spec_verify_mrope", "chunked_prefill", "decode_32k_fp8kv"]


def _oracle_main(wl, m, cache_before, slots=None):
    return oq.prepare_main(
        to_np(m["main_qkv"]), to_np(wl.positions), to_np(wl.cos_sin), wl.mrope_section,
        to_np(m["main_q_norm_weight"]), to_np(m["main_k_norm_weight"]), m["main_eps"],
        wl.q_heads, wl.kv_heads, cache_before,
        to_np(m["main_slot_mapping"]) if slots is None else slots, kv_dtype=wl.kv_dtype,
        k_scale=m.get("main_k_scale", 1.0), v_scale=m.get("main_v_scale", 1.0))


@pytest.mark.parametrize("name", NAMES)
def test_main_prepare_bytes_match_oracle(name):
    wl = workload(name)
    m = main_prepare_inputs(wl)
    log(f"main prepare parity {name}: T={wl.num_tokens} Hq={wl.q_heads} Hkv={wl.kv_heads} "
        f"kv={wl.kv_dtype}")
    cache_before = to_np(wl.kv_cache).copy()
    q_codes, after = oracle_compress(wl)
    ref_q, ref_cache = _oracle_main(wl, m, cache_before)
    st = QsaStep(wl, main=m)
    st.compress()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(m["main_q"]), ref_q)
    assert np.array_equal(to_np(wl.kv_cache).view(np.uint8), ref_cache.view(np.uint8))
    # The indexer's results do not change with the main prepare in the same launch.
    assert np.array_equal(to_np(st.q_idx).view(np.uint8), q_codes.view(np.uint8))
    assert np.array_equal(to_np(wl.ckv).view(np.uint8), after.ckv.view(np.uint8))
    assert np.array_equal(to_np(wl.ring), after.ring)


def test_negative_and_out_of_range_slots_write_nothing():
    wl = workload("decode_32k")
    m = main_prepare_inputs(wl)
    slots = to_np(m["main_slot_mapping"]).copy()
    slots[::2] = -1
    slots[1] = wl.kv_cache.shape[0] * wl.kv_cache.shape[2] + 5   # page past the cache
    m["main_slot_mapping"] = torch.from_numpy(slots).cuda()
    log(f"main prepare slot masking: T={wl.num_tokens}")
    cache_before = to_np(wl.kv_cache).copy()
    _, ref_cache = _oracle_main(wl, m, cache_before, slots=slots)
    st = QsaStep(wl, main=m)
    st.compress()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(wl.kv_cache), ref_cache)


@pytest.mark.parametrize("name", ["decode_32k", "decode_32k_fp8kv", "spec_verify_mrope"])
def test_attention_on_prepared_q_with_gate_in_place(name):
    wl = workload(name)
    m = main_prepare_inputs(wl)
    log(f"main prepare + step {name}: T={wl.num_tokens}")
    cache_before = to_np(wl.kv_cache).copy()
    q_codes, after = oracle_compress(wl)
    ref_q, ref_cache = _oracle_main(wl, m, cache_before)
    st = QsaStep(wl, main=m)
    st.run()
    torch.cuda.synchronize()
    packed = to_np(st.packed)
    ref_packed = oq.index_topk(to_np(wl.query_start_loc), to_np(wl.seq_lens), q_codes, after.ckv,
                               to_np(wl.c_block_table), wl.compress_ratio, wl.budget,
                               wl.index_dtype)
    assert np.array_equal(packed, ref_packed)
    Hq = wl.q_heads
    gate = to_np(m["main_qkv"])[:, :2 * Hq * 128].reshape(-1, Hq, 2, 128)[:, :, 1, :]
    ref = oq.sparse_gqa(ref_q, ref_cache, to_np(wl.block_table), to_np(wl.token_to_req),
                        ref_packed, gate=np.ascontiguousarray(gate), kv_dtype=wl.kv_dtype,
                        k_scale=wl.k_scale, v_scale=wl.v_scale)
    got = st.out.float().cpu().numpy().astype(np.float64)
    err = max_abs(got, ref)
    log(f"  max abs {err:.3e}")
    assert err <= TOL[wl.index_dtype]
    assert np.all(np.isfinite(got))
