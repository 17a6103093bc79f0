"""Host-side checks of libqsa.so that need no GPU: the library loads, exports every symbol the
header declares, its argument blocks have the C layout, and invalid calls are rejected before any
launch (so they run on a CPU-only machine)."""

import ctypes as C
import os
import re
import subprocess
import tempfile

import pytest
import torch

from sparse_attention_qsa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libqsa.so not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const\s+)?[a-z_0-9]+[\s\*]+(qsa_[a-z_0-9]+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"qsa_compress", "qsa_index_logits_topk", "qsa_sparse_gqa"} <= set(names)
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTED)
    assert lib.qsa_abi_version() == 9
    assert lib.qsa_status_string(3) == b"QSA_ERR_WORKSPACE_TOO_SMALL"


STRUCTS = {"qsa_compress_args": B.CompressArgs, "qsa_topk_args": B.TopkArgs,
           "qsa_gqa_args": B.GqaArgs}


def test_argument_blocks_have_the_c_layout():
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(){"]
    for cname, cls in STRUCTS.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", src, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    got = dict(line.rsplit(" ", 1) for line in out.strip().splitlines())
    for cname, cls in STRUCTS.items():
        assert int(got[cname]) == C.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(cls, f).offset, f"{cname}.{f}"


FAKE = 1 << 20   # a non-null, 256-byte-aligned stand-in pointer; never dereferenced here


def _gqa(**over):
    a = B.GqaArgs(num_tokens=64, num_requests=64, num_q_heads=16, num_kv_heads=2, head_dim=128,
                  q=FAKE, q_row_stride=16 * 128, q_head_stride=128, kv_cache=FAKE,
                  kv_page_stride=2 * 16 * 256, kv_head_stride=16 * 256, kv_token_stride=256,
                  num_pages=131072, page_size=16, block_table=FAKE, block_table_stride=2048,
                  block_table_width=2048, token_to_req=FAKE, packed=FAKE,
                  packed_row_stride=2052, packed_width=2051, out=FAKE,
                  out_row_stride=16 * 128, out_head_stride=128)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _topk(**over):
    a = B.TopkArgs(num_tokens=64, num_requests=64, query_start_loc=FAKE, seq_lens=FAKE,
                   num_decode_requests=64, decode_query_len=1, max_query_len=1,
                   max_seq_len=32768, q_idx=FAKE, ckv=FAKE, c_block_table=FAKE,
                   c_block_table_stride=512, c_block_table_width=512, c_page_size=16,
                   c_pages=32768, num_index_heads=8, head_dim=128, compress_ratio=4,
                   budget=2048, index_dtype=0, packed=FAKE, packed_row_stride=2052)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_split_plan_and_workspace_sizes():
    lib = B.lib()
    a = _gqa()
    # 65 tiles of 32 tokens; 128 (row, KV head) units of bf16 K/V: one workgroup of 8 waves per
    # unit, 8 splits of 9 tiles merged in the workgroup (no partials, no merge kernel).
    assert lib.qsa_sparse_gqa_num_splits(C.byref(a)) == 8
    assert lib.qsa_sparse_gqa_merge_kernel(C.byref(a)) == 0
    assert lib.qsa_sparse_gqa_workspace_size(C.byref(a)) == 0
    # 64 units: 768 / 64 = 12 splits wanted -> 6 tiles each -> 11 splits, merged by the merge
    # kernel from partials in the workspace.
    half = _gqa(num_tokens=32)
    assert lib.qsa_sparse_gqa_num_splits(C.byref(half)) == 11
    assert lib.qsa_sparse_gqa_merge_kernel(C.byref(half)) == 1
    assert lib.qsa_sparse_gqa_workspace_size(C.byref(half)) >= 11 * 32 * 16 * 128 * 4
    # 384 units: 2 splits, two kernels; a forced 4 splits are merged in the workgroup.
    assert lib.qsa_sparse_gqa_num_splits(C.byref(_gqa(num_tokens=192))) == 2
    assert lib.qsa_sparse_gqa_merge_kernel(C.byref(_gqa(num_tokens=192))) == 1
    assert lib.qsa_sparse_gqa_merge_kernel(C.byref(_gqa(num_tokens=192, num_splits=4))) == 0
    assert lib.qsa_sparse_gqa_merge_kernel(C.byref(_gqa(num_splits=9))) == 1
    assert lib.qsa_sparse_gqa_merge_kernel(C.byref(_gqa(head_dim=64))) == -1
    # fp8 K/V: 2048 / 128 = 16 splits wanted -> 5 tiles each -> 13 splits.
    f8 = _gqa(kv_dtype=1, kv_page_stride=2 * 16 * 256, kv_head_stride=16 * 256,
              kv_token_stride=256)
    assert lib.qsa_sparse_gqa_num_splits(C.byref(f8)) == 13
    assert lib.qsa_sparse_gqa_merge_kernel(C.byref(f8)) == 1
    one = _gqa(num_splits=1)
    assert lib.qsa_sparse_gqa_num_splits(C.byref(one)) == 1
    assert lib.qsa_sparse_gqa_workspace_size(C.byref(one)) == 0
    assert lib.qsa_sparse_gqa_merge_kernel(C.byref(one)) == 0
    big = _gqa(num_tokens=4096)
    assert lib.qsa_sparse_gqa_num_splits(C.byref(big)) == 1
    t = _topk()
    ws = lib.qsa_index_logits_topk_workspace_size(C.byref(t))
    assert ws >= 64 * 8192 * (4 + 4 + 8)    # logits + band index + band score per column
    # A logits cap of 10 rows' logits: the per-row arrays are sized for 10 rows, not 64.
    capped = _topk(max_logits_bytes=10 * 8192 * 4)
    wc = lib.qsa_index_logits_topk_workspace_size(C.byref(capped))
    assert 10 * 8192 * 16 <= wc < 11 * 8192 * 16 + 64 * 64 * 4 + 4096
    # A cap below one row still runs one row per window.
    tiny = _topk(max_logits_bytes=1)
    assert lib.qsa_index_logits_topk_workspace_size(C.byref(tiny)) >= 8192 * 16
    assert lib.qsa_index_logits_topk_workspace_size(C.byref(_topk(max_logits_bytes=-1))) == 0


def test_invalid_calls_are_rejected_before_any_launch():
    lib = B.lib()
    INVAL, NOTSUP, SMALL = 1, 2, 3
    # The split top-k calls hand the workspace over between them: not under a multi-window cap.
    capped = _topk(max_logits_bytes=10 * 8192 * 4)
    ws = lib.qsa_index_logits_topk_workspace_size(C.byref(capped))
    assert lib.qsa_index_logits(C.byref(capped), FAKE, ws, None) == NOTSUP
    assert lib.qsa_block_topk(C.byref(capped), FAKE, ws, None) == NOTSUP
    assert lib.qsa_index_logits_topk(C.byref(_topk(max_logits_bytes=-5)), FAKE, ws, None) == INVAL
    # ReLU-sum takes up to 16 heads (one per matrix-core operand column), like the plain sum.
    assert lib.qsa_index_logits_topk_workspace_size(C.byref(_topk(index_agg=1,
                                                                    num_index_heads=16))) > 0
    assert lib.qsa_index_logits_topk_workspace_size(C.byref(_topk(index_agg=1,
                                                                    num_index_heads=17))) == 0
    assert lib.qsa_sparse_gqa(C.byref(_gqa(head_dim=64)), None, 0, None) == NOTSUP
    assert lib.qsa_sparse_gqa(C.byref(_gqa(num_q_heads=12)), None, 0, None) == NOTSUP
    assert lib.qsa_sparse_gqa(C.byref(_gqa(page_size=8)), None, 0, None) == NOTSUP
    assert lib.qsa_sparse_gqa(C.byref(_gqa(q=None)), None, 0, None) == INVAL
    assert lib.qsa_sparse_gqa(C.byref(_gqa(kv_token_stride=100)), None, 0, None) == INVAL
    assert lib.qsa_sparse_gqa(C.byref(_gqa(packed_row_stride=2051)), None, 0, None) == INVAL
    assert lib.qsa_sparse_gqa(C.byref(_gqa(num_tokens=32)), None, 0, None) == SMALL  # partials
    assert lib.qsa_sparse_gqa(C.byref(_gqa(num_tokens=0)), None, 0, None) == 0
    # fp8 main KV: a known dtype, finite non-negative scales, 16-byte strides in bytes.
    assert lib.qsa_sparse_gqa(C.byref(_gqa(kv_dtype=5)), None, 0, None) == NOTSUP
    assert lib.qsa_sparse_gqa(C.byref(_gqa(kv_dtype=1, k_scale=-1.0)), None, 0, None) == INVAL
    assert lib.qsa_sparse_gqa(C.byref(_gqa(kv_dtype=1, v_scale=float("nan"))), None, 0,
                              None) == INVAL
    assert lib.qsa_sparse_gqa(C.byref(_gqa(kv_dtype=1, kv_token_stride=264)), None, 0,
                              None) == INVAL
    assert lib.qsa_sparse_gqa(C.byref(_gqa(kv_dtype=1)), None, 0, None) == SMALL
    assert lib.qsa_index_logits_topk(C.byref(_topk(budget=2047)), None, 0, None) == INVAL
    # Compressed cache rows are numbered in 32 bits.
    assert lib.qsa_index_logits_topk(C.byref(_topk(c_pages=1 << 27, c_page_size=16)), None, 0,
                                     None) == NOTSUP
    # The top-k holds a row's scores in registers: at most 32,768 compressed columns.
    assert lib.qsa_index_logits_topk_workspace_size(C.byref(_topk(max_seq_len=4 * 32768))) > 0
    assert lib.qsa_index_logits_topk(C.byref(_topk(max_seq_len=4 * 32768 + 4)), None, 0,
                                     None) == NOTSUP
    assert lib.qsa_index_logits_topk(C.byref(_topk(compress_ratio=3)), None, 0, None) == NOTSUP
    assert lib.qsa_index_logits_topk(C.byref(_topk(index_dtype=7)), None, 0, None) == NOTSUP
    assert lib.qsa_index_logits_topk(C.byref(_topk(index_agg=2)), None, 0, None) == NOTSUP
    # ReLU-sum with more than 16 heads: as for the plain sum.
    assert lib.qsa_index_logits_topk(C.byref(_topk(index_agg=1, num_index_heads=17)), None, 0,
                                     None) == NOTSUP
    assert lib.qsa_index_logits_topk(C.byref(_topk(index_agg=1)), None, 0, None) == SMALL
    assert lib.qsa_index_logits_topk(C.byref(_topk()), None, 0, None) == SMALL
    assert lib.qsa_index_logits_topk(C.byref(_topk(num_tokens=0)), None, 0, None) == 0
    assert lib.qsa_index_logits_topk_workspace_size(C.byref(_topk(head_dim=64))) == 0
    # The single-kernel halves validate exactly as the calls they split.
    assert lib.qsa_index_logits(C.byref(_topk(budget=2047)), None, 0, None) == INVAL
    assert lib.qsa_block_topk(C.byref(_topk(compress_ratio=3)), None, 0, None) == NOTSUP
    assert lib.qsa_block_topk(C.byref(_topk()), None, 0, None) == SMALL
    assert lib.qsa_index_logits(C.byref(_topk(num_tokens=0)), None, 0, None) == 0
    assert lib.qsa_sparse_gqa_partial(C.byref(_gqa(head_dim=64)), None, 0, None) == NOTSUP
    assert lib.qsa_sparse_gqa_merge(C.byref(_gqa(q=None)), None, 0, None) == INVAL
    assert lib.qsa_sparse_gqa_merge(C.byref(_gqa(num_tokens=32)), None, 0, None) == SMALL
    assert lib.qsa_sparse_gqa_partial(C.byref(_gqa(num_tokens=0)), None, 0, None) == 0
    c = B.CompressArgs()
    assert lib.qsa_compress(C.byref(c), None) == 0           # zero rows: a no-op
    c.num_tokens, c.num_requests = 1, 1
    assert lib.qsa_compress(C.byref(c), None) == NOTSUP      # head_dim 0
    c.head_dim, c.rotary_dim, c.num_index_heads, c.compress_ratio = 128, 64, 8, 4
    assert lib.qsa_compress(C.byref(c), None) == INVAL       # NULL tensors
    assert lib.qsa_compress(None, None) == INVAL


def _compress(**over):
    a = B.CompressArgs(num_tokens=64, num_requests=64, query_start_loc=FAKE, seq_lens=FAKE,
                       max_query_len=1, q_proj=FAKE, q_proj_row_stride=8 * 128, k_proj=FAKE,
                       k_proj_row_stride=128, positions=FAKE, cos_sin=FAKE, max_position=40000,
                       q_norm_weight=FAKE, k_norm_weight=FAKE, eps=1e-6, ring=FAKE,
                       ring_page=FAKE, ring_pages=64, ring_size=16, ckv=FAKE,
                       c_block_table=FAKE, c_block_table_stride=512, c_block_table_width=512,
                       c_page_size=16, c_pages=32768, num_index_heads=8, head_dim=128,
                       rotary_dim=64, compress_ratio=4, index_dtype=0, q_idx=FAKE,
                       main_qkv=FAKE, main_qkv_row_stride=(2 * 16 + 2 * 2) * 128,
                       num_q_heads=16, num_kv_heads=2, main_q_norm_weight=FAKE,
                       main_k_norm_weight=FAKE, main_eps=1e-6, main_q=FAKE,
                       main_kv_cache=FAKE, main_kv_page_stride=2 * 16 * 256,
                       main_kv_head_stride=16 * 256, main_kv_token_stride=256,
                       main_num_pages=8192, main_page_size=16, main_slot_mapping=FAKE,
                       main_kv_dtype=0, main_k_scale=1.0, main_v_scale=1.0)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_combined_prepare_and_selection_plan_and_invalid_calls():
    """qsa_compress_index_logits_topk fuses the indexer prepare into the scoring launch only for
    one-row batches on the wide scoring layout whose two argument blocks describe the same
    requests and caches; anything invalid is rejected before any launch (no GPU here)."""
    lib = B.lib()
    INVAL, NOTSUP, SMALL = 1, 2, 3
    fused = lambda c, t: lib.qsa_compress_index_logits_topk_fused(C.byref(c), C.byref(t))  # noqa
    c, t = _compress(main_qkv=None), _topk()     # 64 one-row requests of 32k tokens
    assert fused(c, t) == 1
    many = dict(num_tokens=256, num_requests=256)
    assert fused(_compress(main_qkv=None, **many),
                 _topk(num_decode_requests=256, max_seq_len=8192, **many)) == 1
    assert fused(_compress(), t) == 0                            # main-attention prepare
    assert fused(c, _topk(index_agg=1)) == 0                     # ReLU-sum
    assert fused(c, _topk(max_logits_bytes=8192 * 4)) == 0       # logits windows
    assert fused(_compress(main_qkv=None, max_query_len=2), _topk(max_query_len=2)) == 0
    assert fused(c, _topk(q_idx=FAKE + 256)) == 0                # the blocks disagree
    assert fused(c, _topk(c_block_table_width=256)) == 0
    # 1024-key workgroups at one per CU: 64 x 2 and 32 x 8 fit the chip, 100 x 4 does not (and
    # its 2048-key workgroups would not fill it).
    assert fused(c, _topk(max_seq_len=8192)) == 1
    half = dict(num_tokens=32, num_requests=32)
    assert fused(_compress(main_qkv=None, **half), _topk(num_decode_requests=32, **half)) == 1
    odd = dict(num_tokens=100, num_requests=100)
    assert fused(_compress(main_qkv=None, **odd),
                 _topk(num_decode_requests=100, max_seq_len=16384, **odd)) == 0
    assert fused(_compress(main_qkv=None, head_dim=64), t) == -1
    assert fused(c, _topk(budget=3)) == -1
    call = lambda c, t, n=1 << 40, f=lib.qsa_compress_index_logits_topk: f(  # noqa: E731
        C.byref(c) if c is not None else None, C.byref(t), FAKE, n, None)
    assert call(_compress(main_qkv=None, head_dim=64), t) == NOTSUP
    assert call(c, _topk(budget=3)) == INVAL
    assert call(None, t) == INVAL
    assert call(c, t, 16) == SMALL
    assert call(c, _topk(max_logits_bytes=8192 * 4), f=lib.qsa_compress_index_logits) == NOTSUP


def test_invalid_main_prepare_arguments_are_rejected_before_any_launch():
    lib = B.lib()
    INVAL, NOTSUP = 1, 2
    call = lambda **o: lib.qsa_compress(C.byref(_compress(**o)), None)  # noqa: E731
    assert call(num_q_heads=0) == NOTSUP
    assert call(num_kv_heads=65) == NOTSUP
    assert call(main_kv_dtype=5) == NOTSUP
    assert call(main_q=None) == INVAL
    assert call(main_slot_mapping=None) == INVAL
    assert call(main_qkv_row_stride=(2 * 16 + 2 * 2) * 128 - 2) == INVAL
    assert call(main_qkv_row_stride=(2 * 16 + 2 * 2) * 128 + 1) == INVAL
    assert call(main_kv_token_stride=200) == INVAL
    assert call(main_kv_token_stride=260) == INVAL           # 520 bytes: not a 16-byte multiple
    assert call(main_page_size=0) == INVAL
    assert call(main_kv_dtype=1, main_k_scale=0.0) == INVAL
    assert call(main_kv_dtype=1, main_v_scale=float("nan")) == INVAL
    assert call(main_kv_dtype=1, main_kv_token_stride=264) == INVAL
    assert call(main_slot_mapping=FAKE + 4) == INVAL
    assert call(main_kv_cache=FAKE + 8) == INVAL


def test_binding_rejects_tensors_that_do_not_match_the_call():
    """The Python binding refuses, before any C call, tensors whose dtype or shape does not fit
    the sizes it derives the argument blocks from (an e4m3 q_idx with a bf16 indexer would
    make the kernels read and write past the buffers)."""
    from sparse_attention_qsa_amd.workloads import make_workload
    wl = make_workload("tiny_decode", device="cpu")
    T, Hi = wl.num_tokens, wl.index_heads
    q_idx = torch.empty((T, Hi, 128), dtype=torch.bfloat16)
    packed = torch.empty((T, wl.output_width + 1), dtype=torch.int32)
    out = torch.empty((T, wl.q_heads, 128), dtype=torch.bfloat16)
    comp = dict(query_start_loc=wl.query_start_loc, seq_lens=wl.seq_lens,
                max_query_len=wl.max_query_len, q_proj=wl.q_proj, k_proj=wl.k_proj,
                positions=wl.positions, cos_sin=wl.cos_sin, q_norm_weight=wl.q_norm_w,
                k_norm_weight=wl.k_norm_w, eps=wl.eps, ring=wl.ring, ring_page=wl.ring_page,
                ckv=wl.ckv, c_block_table=wl.c_block_table, q_idx=q_idx, num_index_heads=Hi,
                compress_ratio=wl.compress_ratio, index_dtype="bf16")
    B.compress_args(**comp)                                           # the good call builds
    bad = [
        dict(q_idx=q_idx.view(torch.uint8)[..., :128]),               # e4m3 buffer, bf16 call
        dict(q_idx=torch.empty((T, Hi - 1, 128), dtype=torch.bfloat16)),
        dict(ckv=wl.ckv.view(torch.uint8)),                           # cache dtype mismatch
        dict(index_dtype="fp8"),                                      # q_idx and ckv are bf16
        dict(k_proj=wl.k_proj[:T - 1]),
        dict(positions=torch.stack([wl.positions] * 3, 1)),           # triples without MRoPE
        dict(mrope_section=(12, 10, 10)),                             # 1-D positions, no ring_pos
        dict(q_norm_weight=wl.q_norm_w.float()),
        dict(k_norm_weight=wl.k_norm_w[:64]),
    ]
    for over in bad:
        with pytest.raises(ValueError):
            B.compress_args(**{**comp, **over})
    sel = dict(query_start_loc=wl.query_start_loc, seq_lens=wl.seq_lens, q_idx=q_idx,
               ckv=wl.ckv, c_block_table=wl.c_block_table, packed=packed,
               num_index_heads=Hi, compress_ratio=wl.compress_ratio, budget=wl.budget,
               index_dtype="bf16", max_query_len=wl.max_query_len,
               max_seq_len=wl.max_seq_len)
    B.topk_args(**sel)
    for over in (dict(index_dtype="fp8"), dict(num_index_heads=Hi + 1),
                 dict(packed=packed[:, :-1]), dict(budget=wl.budget * 2),
                 dict(ckv=wl.ckv.view(torch.uint8))):
        with pytest.raises(ValueError):
            B.topk_args(**{**sel, **over})
    att = dict(q=wl.q, kv_cache=wl.kv_cache, block_table=wl.block_table,
               token_to_req=wl.token_to_req, packed=packed, out=out, gate=wl.gate)
    B.gqa_args(**att)
    for over in (dict(out=out[:, :1]), dict(token_to_req=wl.token_to_req[:1]),
                 dict(packed=packed[:1]), dict(gate=wl.gate[:, :, :64]),
                 dict(kv_cache=wl.kv_cache[..., :128])):
        with pytest.raises(ValueError):
            B.gqa_args(**{**att, **over})


def test_no_alloc_attention_rejects_before_any_launch():
    """qsa_sparse_gqa_noalloc validates like qsa_sparse_gqa, and refuses a plan whose partials
    exceed its static scratch (here 64 forced splits of 1024 rows x 16 heads) before touching a
    device."""
    lib = B.lib()
    INVAL, NOTSUP, SMALL = 1, 2, 3
    limit = lib.qsa_sparse_gqa_noalloc_scratch_bytes()
    assert limit == 40 << 20
    assert lib.qsa_sparse_gqa_noalloc(None, None) == INVAL
    assert lib.qsa_sparse_gqa_noalloc(C.byref(_gqa(num_tokens=0)), None) == 0
    assert lib.qsa_sparse_gqa_noalloc(C.byref(_gqa(head_dim=64)), None) == NOTSUP
    assert lib.qsa_sparse_gqa_noalloc(C.byref(_gqa(q=None)), None) == INVAL
    big = _gqa(num_tokens=1024, num_splits=64)
    assert lib.qsa_sparse_gqa_workspace_size(C.byref(big)) > limit
    assert lib.qsa_sparse_gqa_noalloc(C.byref(big), None) == SMALL
    # Every automatic split plan fits the scratch, whatever the rows, heads and K/V dtype.
    for T in (1, 2, 3, 5, 17, 64, 100, 255, 383, 767, 1023, 2047, 4096, 65536):
        for hkv in (1, 2, 4, 8):
            for G in (1, 2, 4, 8, 16):
                for kv_dtype in (0, 1):
                    a = _gqa(num_tokens=T, num_kv_heads=hkv, num_q_heads=hkv * G,
                             q_row_stride=hkv * G * 128, out_row_stride=hkv * G * 128,
                             kv_head_stride=16 * 256, kv_page_stride=hkv * 16 * 256,
                             num_pages=1024, kv_dtype=kv_dtype)
                    need = lib.qsa_sparse_gqa_workspace_size(C.byref(a))
                    assert (0 < need) == (lib.qsa_sparse_gqa_merge_kernel(C.byref(a)) == 1)
                    assert need <= limit, (T, hkv, G, kv_dtype, need)


def test_read_bandwidth_probe_rejects_bad_arguments():
    lib = B.lib()
    INVAL = 1
    assert lib.qsa_diag_read_bandwidth(None, None, 4, 2048, FAKE, None) == INVAL
    assert lib.qsa_diag_read_bandwidth(FAKE, None, 4, 2048, None, None) == INVAL
    assert lib.qsa_diag_read_bandwidth(FAKE, None, 4, 1000, FAKE, None) == INVAL
    assert lib.qsa_diag_read_bandwidth(FAKE, None, 4, 8192, FAKE, None) == INVAL
    assert lib.qsa_diag_read_bandwidth(FAKE + 8, None, 4, 2048, FAKE, None) == INVAL
    assert lib.qsa_diag_read_bandwidth(FAKE, None, -1, 2048, FAKE, None) == INVAL
    assert lib.qsa_diag_read_bandwidth(FAKE, None, 0, 2048, FAKE, None) == 0
