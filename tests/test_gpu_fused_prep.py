"""GPU parity of qsa_compress_index_logits_topk, the prepare + selection call.  On a batch of
one-row requests that fills the chip it runs as one scoring launch (the indexer prepare done
inside the logits kernel); its outputs must equal the oracle's and, bit for bit, those of
qsa_compress followed by qsa_index_logits_topk on the same inputs.  Other batches run as the two
calls."""

import numpy as np
import pytest
import torch

from sparse_attention_qsa_amd.step import QsaStep
from sparse_attention_qsa_amd.workloads import make_workload
from tests.gpu_util import SCALED, log, oracle_step, to_np

pytestmark = pytest.mark.gpu

# One-row batches the combined call fuses: 256 requests of at most 2,048 compressed keys (one
# 2048-key workgroup each), 64 of 8,192 (four each, the decode_32k step itself), and batches
# whose 1024-key workgroups fit the chip at one per CU (the small cases).
FUSED = {
    "bf16_small": ("decode_32k", dict(num_requests=64, lengths=("uniform", 5000, 8192))),
    "fp8_small": ("fp8_decode", dict(num_requests=32, lengths=("uniform", 4096, 32768))),
    "bf16": ("decode_32k", dict(num_requests=256, lengths=("fixed", 8192))),
    # Lengths that are not multiples of c: some rows complete no group.
    "bf16_ragged": ("decode_32k", dict(num_requests=256, lengths=("uniform", 5000, 8192))),
    "fp8_indexer": ("fp8_decode", dict(num_requests=256, lengths=("uniform", 9000, 16384))),
    "mrope": ("spec_verify_mrope",
              dict(num_requests=256, rows=1, lengths=("loguniform", 1024, 16384))),
    "decode_32k": ("decode_32k", dict(num_requests=64, lengths=("fixed", 32768))),
}


def _pair(name, seed=None, **kw):
    """Two copies of one workload (same seed), each with its step."""
    wa = make_workload(name, device="cuda", seed=seed, **kw)
    wb = make_workload(name, device="cuda", seed=seed, **kw)
    return (wa, QsaStep(wa)), (wb, QsaStep(wb))


def _assert_same_state(wa, sa, wb, sb):
    assert np.array_equal(to_np(sa.q_idx).view(np.uint8), to_np(sb.q_idx).view(np.uint8))
    assert np.array_equal(to_np(wa.ckv).view(np.uint8), to_np(wb.ckv).view(np.uint8))
    assert np.array_equal(to_np(wa.ring), to_np(wb.ring))
    if wa.ring_pos is not None:
        assert np.array_equal(to_np(wa.ring_pos), to_np(wb.ring_pos))
    pa, pb = to_np(sa.packed), to_np(sb.packed)
    assert np.array_equal(pa, pb), f"{int((pa != pb).any(axis=1).sum())} rows differ"


@pytest.mark.parametrize("case", sorted(FUSED))
def test_fused_prepare_equals_the_two_calls(case):
    name, kw = FUSED[case]
    (wa, sa), (wb, sb) = _pair(name, **kw)
    log(f"fused prepare {case}: R={wa.num_requests}")
    assert sb.fused and sa.fused
    sa.compress()
    sa.topk()
    sb.prep_topk()
    torch.cuda.synchronize()
    _assert_same_state(wa, sa, wb, sb)


@pytest.mark.parametrize("case", ["bf16", "bf16_ragged", "fp8_indexer", "mrope", "bf16_small",
                                  "fp8_small"])
def test_fused_prepare_matches_the_oracle(case):
    name, kw = FUSED[case]
    wl = make_workload(name, device="cuda", **kw)
    st = QsaStep(wl)
    assert st.fused
    log(f"fused prepare vs oracle {case}: R={wl.num_requests}")
    ref = oracle_step(wl, with_attention=False)  # reads the pre-state first
    st.prep_topk()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(st.q_idx).view(np.uint8), ref.q_codes.view(np.uint8))
    assert np.array_equal(to_np(wl.ckv).view(np.uint8), ref.state_after.ckv.view(np.uint8))
    assert np.array_equal(to_np(wl.ring), ref.state_after.ring)
    if wl.ring_pos is not None:
        assert np.array_equal(to_np(wl.ring_pos), ref.state_after.ring_pos)
    packed = to_np(st.packed)
    assert np.array_equal(packed, ref.packed), (
        f"{int((packed != ref.packed).any(axis=1).sum())} rows differ")


def test_fused_prepare_on_the_full_decode_step_sampled_rows():
    name, kw = FUSED["decode_32k"]
    wl = make_workload(name, device="cuda", **kw)
    st = QsaStep(wl)
    rows = [0, 21, 40, 63]
    log(f"fused prepare, full-size decode_32k, sampled rows {rows}")
    ref = oracle_step(wl, rows=rows)
    st.run(combined=True)
    torch.cuda.synchronize()
    packed = to_np(st.packed)
    assert np.array_equal(packed[rows], ref.packed[rows])
    out = st.out.float().cpu().numpy().astype(np.float64)
    assert float(np.max(np.abs(out[rows] - ref.out[rows]))) <= 2e-2


def test_fused_prepare_edge_rows():
    """A request whose ring page is out of range (its ring reads as zero and is not written), a
    request whose completed group's page column is past its block table (the group is not
    stored and its key is not scored), and one whose group page is out of the cache."""
    name, kw = FUSED["bf16"]
    (wa, sa), (wb, sb) = _pair(name, **kw)
    for wl in (wa, wb):
        wl.ring_page[3] = -1
        wl.ring_page[7] = wl.ring.shape[0] + 5
        g_col = (8192 // 4 - 1) // wl.ckv.shape[1]
        wl.c_block_table[11, g_col] = wl.ckv.shape[0]     # page out of the cache
        wl.c_block_table[12, g_col] = -1
    torch.cuda.synchronize()
    assert sb.fused
    sa.compress()
    sa.topk()
    sb.prep_topk()
    torch.cuda.synchronize()
    _assert_same_state(wa, sa, wb, sb)


def test_split_prepare_then_block_topk_equals_the_combined_call():
    name, kw = FUSED["bf16_ragged"]
    (wa, sa), (wb, sb) = _pair(name, **kw)
    sa.prep_topk()
    sb.prep_logits()
    sb.block_topk()
    torch.cuda.synchronize()
    _assert_same_state(wa, sa, wb, sb)


@pytest.mark.parametrize("name, kw", [("decode_32k", dict(rows=2)), ("spec_verify_mrope", {}),
                                      ("chunked_prefill", {}),
                                      ("decode_32k", dict(num_requests=300))])
def test_combined_call_runs_the_two_calls_when_not_fused(name, kw):
    (wa, sa), (wb, sb) = _pair(name, **{**SCALED[name], **kw})
    log(f"combined call, unfused {name}")
    assert not sb.fused
    sa.compress()
    sa.topk()
    sb.prep_topk()
    torch.cuda.synchronize()
    _assert_same_state(wa, sa, wb, sb)


def test_combined_step_captured_in_a_graph_replays_the_eager_results():
    """The fused launch makes no host synchronisation, allocation or memset either: a step with
    the combined call, captured in a HIP graph, replays the eager results bit for bit, with
    eager work on the same buffers in between."""
    name, kw = FUSED["bf16"]
    wl = make_workload(name, device="cuda", **kw)
    st = QsaStep(wl)
    assert st.fused
    log(f"graph replay of the combined step: R={wl.num_requests}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run(side, combined=True)        # eager, on a side stream, before the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (st.packed, st.out, st.q_idx, wl.ckv, wl.ring)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(combined=True)
    torch.cuda.synchronize()
    for rep in range(3):
        st.packed.fill_(-7)                # eager work between the replays
        st.out.fill_(float("nan"))
        st.q_idx.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"  replay {rep}")
        for a, b in zip((st.packed, st.out, st.q_idx, wl.ckv, wl.ring), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
        st.run(combined=True)              # an eager step between replays too
        torch.cuda.synchronize()
        assert torch.equal(st.packed, ref[0])
    del g
