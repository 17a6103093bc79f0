"""Helpers of the GPU parity tests (test infrastructure)."""

from __future__ import annotations

import sys

import numpy as np
import torch

from sparse_attention_qsa_amd.step import QsaStep
from sparse_attention_qsa_amd.workloads import make_workload
from tests.oracle_io import oracle_step, to_np

# Scaled-down versions of the five workloads: same head counts, ratios, budgets and dtypes,
# lengths chosen so that the oracle finishes in seconds while rows still select among many
# more blocks than the budget keeps, span several key tiles and end in ragged tails.
SCALED = {
    "tiny_decode": dict(),
    "decode_32k": dict(num_requests=6, lengths=("uniform", 3000, 9000)),
    "fp8_decode": dict(num_requests=8, lengths=("uniform", 2500, 14000)),
    "chunked_prefill": dict(num_requests=2, lengths=("uniform", 3000, 4100), rows=384),
    "spec_verify_mrope": dict(num_requests=10, lengths=("loguniform", 1024, 24000)),
    "decode_32k_fp8kv": dict(num_requests=6, lengths=("uniform", 3000, 9000)),
    "chunked_prefill_fp8": dict(num_requests=2, lengths=("uniform", 3000, 4100), rows=384),
}

TOL = {"bf16": 2e-2, "fp8": 6e-2}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def workload(name: str, seed=None, **kw):
    args = dict(SCALED[name])
    args.update(kw)
    return make_workload(name, device="cuda", seed=seed, **args)


def run_gpu(wl, num_splits: int = 0) -> QsaStep:
    st = QsaStep(wl, num_splits=num_splits)
    st.run()
    torch.cuda.synchronize()
    return st


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def gpu_out_f64(st: QsaStep) -> np.ndarray:
    return st.out.float().cpu().numpy().astype(np.float64)


__all__ = ["SCALED", "TOL", "log", "workload", "run_gpu", "max_abs", "gpu_out_f64",
           "oracle_step", "to_np"]
