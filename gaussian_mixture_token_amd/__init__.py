"""MI355X-native (gfx950) forward and backward passes of Gaussian Mixture Attention (GMA).

The computation lives in libgma.so (hand-written HIP kernels behind the C ABI of
include/gma.h); this package only builds it, loads it and passes PyTorch tensors to it.
"""
from .api import (GmaError, backward, decode_prepare, decode_step, forward, forward_bidir,  # noqa: F401
                  forward_causal, forward_causal_noalloc, problem, responsibilities, responsibility_stats,
                  workspace_size)
from .workloads import WORKLOADS, Workload, make_dout, make_inputs, make_params, workload  # noqa: F401
