"""The allocation-free attention call (qsa_sparse_gqa_noalloc) against qsa_sparse_gqa with a
caller workspace, through the C ABI: two calls in a row, the second on a smaller input."""

import ctypes as C

import numpy as np
import pytest
import torch

from sparse_attention_qsa_amd import binding as B
from tests.gpu_util import TOL, gpu_out_f64, log, max_abs, oracle_step, run_gpu, workload

pytestmark = pytest.mark.gpu


def _both(wl, ref):
    """qsa_sparse_gqa (workspace) and qsa_sparse_gqa_noalloc on the same arguments."""
    st = run_gpu(wl)
    st.packed.copy_(torch.from_numpy(ref.packed).cuda())
    st.gqa()
    torch.cuda.synchronize()
    with_ws = st.out.clone()
    st.out.fill_(float("nan"))
    splits = B.lib().qsa_sparse_gqa_num_splits(C.byref(st.g_args))
    rc = B.lib().qsa_sparse_gqa_noalloc(C.byref(st.g_args), B._stream(None))
    assert rc == 0, B.lib().qsa_status_string(rc)
    torch.cuda.synchronize()
    return st, with_ws, splits


def test_no_alloc_attention_equals_the_workspace_call_twice_then_smaller():
    big = workload("decode_32k")                 # 6 requests, several splits per row
    small = workload("tiny_decode")              # 4 rows of one request, one KV head
    for wl in (big, small):
        log(f"no-alloc attention {wl.name}: T={wl.num_tokens} Hq/Hkv={wl.q_heads}/{wl.kv_heads}")
        ref = oracle_step(wl)
        st, with_ws, splits = _both(wl, ref)
        assert splits > 1                        # the partials really go through the scratch
        assert torch.equal(st.out.view(torch.int16), with_ws.view(torch.int16))
        err = max_abs(gpu_out_f64(st), ref.out)
        log(f"  splits {splits}, max-abs vs oracle {err:.3e}")
        assert err <= TOL[wl.index_dtype]


def test_no_alloc_attention_forced_splits_and_fp8_kv():
    """A forced split count (the maximum the plan allows) and the fp8 K/V instance, each
    compared with the workspace call, bit for bit."""
    for name, splits in (("decode_32k", 1000), ("decode_32k_fp8kv", 0)):
        wl = workload(name)
        log(f"no-alloc attention {name}, num_splits={splits}")
        ref = oracle_step(wl)
        st = run_gpu(wl)
        st.packed.copy_(torch.from_numpy(ref.packed).cuda())
        st.g_args.num_splits = splits
        st.gqa()
        torch.cuda.synchronize()
        with_ws = st.out.clone()
        st.out.fill_(float("nan"))
        rc = B.lib().qsa_sparse_gqa_noalloc(C.byref(st.g_args), B._stream(None))
        assert rc == 0, B.lib().qsa_status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(st.out.view(torch.int16), with_ws.view(torch.int16))
        assert max_abs(gpu_out_f64(st), ref.out) <= TOL[wl.index_dtype]
