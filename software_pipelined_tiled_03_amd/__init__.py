"""MI355X-native software-pipelined tiled half-precision GEMM.

The compute path is the HIP library built from csrc/ (C-ABI in
include/pipegemm.h); this package is its binding, the tuning front end
(tuning.py) and the seeded synthetic input generator (inputs.py).  Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""
from .binding import (GEMM_BF16, GEMM_F16, GEMM_NN, GEMM_NT, AlignmentError, GemmArgumentError, GemmError,
                      attention, attn_check, attn_default_config, attn_fwd_raw, attn_lds_bytes,
                      GemmHipError, LdsBudgetError, UnsupportedConfigError, gemm_check, gemm_lds_budget,
                      gemm_lds_bytes, gemm_nn, gemm_nn_raw, gemm_nn_relu_raw, gemm_nt, gemm_nt_raw, gemm_nt_relu_raw,
                      gemm_stamped, gemm_stamped_raw, last_error, load)
from . import tuning
from .tuning import (RANKED_OUT, TuneResult, TuningSpaceError, built_configs, default_config, matmul, model_costs, plan,
                     prune, rank, tune)

__all__ = ["GEMM_BF16", "GEMM_F16", "GEMM_NN", "GEMM_NT", "AlignmentError", "GemmArgumentError", "GemmError",
           "GemmHipError", "LdsBudgetError", "UnsupportedConfigError", "gemm_check", "gemm_lds_budget",
           "gemm_lds_bytes", "gemm_nn", "gemm_nn_raw", "gemm_nn_relu_raw", "gemm_nt", "gemm_nt_raw",
           "gemm_nt_relu_raw", "gemm_stamped", "gemm_stamped_raw", "last_error", "load",
           "attention", "attn_check", "attn_default_config", "attn_fwd_raw", "attn_lds_bytes",
           "RANKED_OUT", "TuneResult", "TuningSpaceError", "built_configs", "default_config", "matmul",
           "model_costs", "plan", "prune", "rank", "tune"]
