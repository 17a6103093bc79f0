"""MI355X (gfx950) implementation of the QSA sparse-attention hot path.

The work runs in libqsa.so (HIP kernels behind a C ABI, include/qsa.h); `binding` marshals torch
tensors into its calls, `step.QsaStep` chains the three calls of one step, `workloads` builds
seeded synthetic inputs.  Nothing here computes the method on the CPU.
"""

from .binding import (LIB_PATH, QsaError, lib, qsa_compress, qsa_diag_e4m3_decode,  # noqa: F401
                      qsa_diag_fp64_sqrt_div, qsa_index_logits_topk,
                      qsa_index_logits_topk_workspace_size, qsa_sparse_gqa,
                      qsa_sparse_gqa_num_splits, qsa_sparse_gqa_workspace_size)
