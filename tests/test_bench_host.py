"""CPU tests of bench.py's host logic: the one-GPU guard, the algorithmic byte and FLOP counts the
roofline divides by, and the parsing of rocprofv3 counter files into per-launch traffic.  No GPU
is touched."""

import json
import os
import subprocess
import sys

import torch

import bench
from sparse_attention_qsa_amd.workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _packed(wl, picks):
    """A packed selection: row t lists picks[t] (token positions) and its count at column W."""
    W = wl.output_width
    pk = torch.full((wl.num_tokens, W + 1), -1, dtype=torch.int32)
    for t, sel in enumerate(picks):
        pk[t, :len(sel)] = torch.tensor(sel, dtype=torch.int32)
        pk[t, W] = len(sel)
    return pk


def test_algorithmic_bytes_count_each_selected_token_once_per_request():
    # 3 requests of 2 rows; the rows of one request overlap, so K/V count the union.
    wl = make_workload("decode_32k", num_requests=3, lengths=("fixed", 96), rows=2)
    assert wl.num_tokens == 6
    picks = [[0, 1, 2], [2, 3],          # request 0: union {0,1,2,3}
             [5], [5],                   # request 1: union {5}
             [], [7, 8, 9, 10, 11]]      # request 2: union {7..11}
    per_call, per_kernel, kv_tokens = bench.algorithmic_bytes(wl, _packed(wl, picks))
    assert kv_tokens == 4 + 1 + 5
    T, Hi, Hq, Hkv, W = 6, 8, 16, 2, wl.output_width
    assert (wl.index_heads, wl.q_heads, wl.kv_heads, wl.compress_ratio) == (Hi, Hq, Hkv, 4)
    # Every request sees 96 // 4 = 24 compressed keys; bf16 codes, 128 wide.
    assert per_call["qsa_index_logits_topk"] == (3 * 24 * 128 * 2 + T * Hi * 128 * 2
                                                 + T * (W + 1) * 4)
    assert per_call["qsa_sparse_gqa"] == (kv_tokens * Hkv * 512 + T * Hq * 128 * 2 * 3
                                          + T * (W + 1) * 4)
    # Rows 94 and 95 of each request complete the group 92..95 only: one compressed row each.
    ring = int(sum(min(int(wl.ring.shape[1]), 2) for _ in range(3)))
    assert per_call["qsa_compress"] == (T * Hi * 128 * 2 + T * 128 * 2 + T * Hi * 128 * 2
                                        + 3 * 128 * 2 + ring * 128 * 2)
    # The per-kernel split adds up to the calls that launch the kernels.
    assert per_kernel["prep_compress_kernel"] == per_call["qsa_compress"]
    assert (per_kernel["logits_valu_kernel"] + per_kernel["topk_kernel"]
            == per_call["qsa_index_logits_topk"])
    assert (per_kernel["gqa_partial_kernel"] + per_kernel["gqa_merge_kernel"]
            == per_call["qsa_sparse_gqa"])


def test_combined_call_moves_the_bytes_of_the_two_calls_it_replaces():
    wl = make_workload("decode_32k", num_requests=3, lengths=("fixed", 96), rows=1)
    pk = _packed(wl, [[0, 1], [4], [8, 9, 10]])
    sep, sep_k, _ = bench.algorithmic_bytes(wl, pk)
    comb, comb_k, _ = bench.algorithmic_bytes(wl, pk, combined=True)
    assert set(comb) == {"qsa_compress_index_logits_topk", "qsa_sparse_gqa"}
    assert (comb["qsa_compress_index_logits_topk"]
            == sep["qsa_compress"] + sep["qsa_index_logits_topk"])
    assert comb["qsa_sparse_gqa"] == sep["qsa_sparse_gqa"]
    # The fused scoring kernel computes q_idx instead of reading it; the top-k reads it.
    q_idx = wl.num_tokens * wl.index_heads * 128 * 2
    assert comb_k["prep_logits_kernel"] == (sep_k["prep_compress_kernel"]
                                            + sep_k["logits_valu_kernel"] - q_idx)
    assert comb_k["topk_kernel"] == sep_k["topk_kernel"] + q_idx
    assert sum(comb_k.values()) == sum(comb.values())
    assert set(comb_k) == {"prep_logits_kernel", "topk_kernel", "gqa_partial_kernel",
                           "gqa_merge_kernel"}


def test_algorithmic_bytes_use_one_byte_codes_for_fp8():
    wl8 = make_workload("decode_32k_fp8kv", num_requests=2, lengths=("fixed", 64), rows=1)
    picks = [[1, 2, 3], [4]]
    per8, _, kv8 = bench.algorithmic_bytes(wl8, _packed(wl8, picks))
    assert kv8 == 4
    T, Hq, W = wl8.num_tokens, wl8.q_heads, wl8.output_width
    assert wl8.kv_dtype == "fp8"
    assert per8["qsa_sparse_gqa"] == kv8 * wl8.kv_heads * 256 + T * Hq * 128 * 6 + T * (W + 1) * 4


def test_matrix_core_logits_flop_count_the_causal_visible_blocks():
    wl = make_workload("chunked_prefill", num_requests=2, lengths=("fixed", 64), rows=32)
    # Rows at positions 32..63, compress ratio 4: a row at x sees (x + 1) // 4 blocks.
    pairs = 2 * sum((x + 1) // 4 for x in range(32, 64))
    executed, per_head = bench.mfma_logits_flop(wl, "sum")
    assert executed == pairs * 2 * 3 * 128
    assert per_head == pairs * 2 * wl.index_heads * 128
    assert bench.mfma_logits_flop(wl, "relu") == (0, 0)
    # Requests of at most MFMA_MIN_ROWS rows stay on the vector path.
    small = make_workload("chunked_prefill", num_requests=1, lengths=("fixed", 64),
                          rows=bench.MFMA_MIN_ROWS)
    assert bench.mfma_logits_flop(small, "sum") == (0, 0)


def _write_counter_csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w") as f:
        f.write(",".join(cols) + "\n")
        for r in rows:
            f.write(",".join(f'"{v}"' if "," in str(v) else str(v) for v in r) + "\n")


def test_counter_files_give_per_dispatch_means_summed_over_instances(tmp_path):
    sub = tmp_path / "host" / "pid"
    sub.mkdir(parents=True)
    k1 = "void qsa::(anonymous namespace)::topk_kernel<8>(qsa::TopkParams)"
    k2 = "void qsa::(anonymous namespace)::gqa_partial_kernel<8, false, 1>(qsa::GqaParams)"
    _write_counter_csv(sub / "x_counter_collection.csv", [
        (1, k1, "FETCH_SIZE", 10.0), (1, k1, "FETCH_SIZE", 30.0),     # two instances: 40
        (2, k1, "FETCH_SIZE", 60.0),                                 # 60
        (2, k1, "WRITE_SIZE", 5.0),
        (3, k2, "FETCH_SIZE", 7.0),
    ])
    rows = bench._counter_rows(str(tmp_path))
    fetch = bench._per_dispatch(rows, "FETCH_SIZE")
    assert fetch[k1] == (50.0, 2)
    assert fetch[k2] == (7.0, 1)
    assert bench._per_dispatch(rows, "WRITE_SIZE") == {k1: (5.0, 1)}
    assert bench._short(k1) == "topk_kernel<8>"
    assert bench._call_of(k1) == "topk_kernel"
    assert bench._call_of(k2) == "gqa_partial_kernel"
    assert bench._call_of("void other_kernel(int)") is None


def test_traffic_record_applies_only_to_its_workload_and_current_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "sparse_attention_qsa_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNELS["topk_kernel"][1]:
        (csrc / f).write_text(f"// {f}\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_record("topk_kernel", "decode_32k") is None     # no record file
    rec = {"workloads": {"decode_32k": {"topk_kernel": {
        "bytes_per_launch": 1234, "source_sha256": bench._source_hash("topk_kernel")}}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.traffic_record("topk_kernel", "decode_32k") == 1234
    assert bench.traffic_record("topk_kernel", "fp8_decode") is None
    assert bench.traffic_record("gqa_merge_kernel", "decode_32k") is None
    (csrc / "topk.hip").write_text("// changed\n")                       # stale record
    assert bench.traffic_record("topk_kernel", "decode_32k") is None


def test_committed_traffic_records_name_known_kernels_and_workloads():
    path = os.path.join(ROOT, "profiles", "traffic.json")
    recs = json.load(open(path))["workloads"]
    from sparse_attention_qsa_amd.workloads import CONFIGS
    for wl, per in recs.items():
        assert wl in CONFIGS
        cal = per.pop("_calibration")
        assert cal["FETCH_SIZE"] > 0 and cal["WRITE_SIZE"] > 0     # copy-kernel scale factors
        for kernel, rec in per.items():
            assert kernel in bench.KERNELS
            assert rec["bytes_per_launch"] > 0 and len(rec["source_sha256"]) == 64
