"""KOSMOS-style self-scheduling persistent kernels for MI355X (gfx950).

Collectives fused into their GEMMs, one persistent launch each, run on one
GPU's share with the other ranks emulated:

* :func:`ag_gemm`      -- all-gather + GEMM (movers become builders)
* :func:`gemm_rs`      -- GEMM + reduce-scatter (builders become reducers)
* :func:`moe_dispatch` -- expert layer, router -> permutation -> token movement
* :func:`moe_combine`  -- grouped SwiGLU experts, push results back, fold
* :func:`moe_layer`    -- the whole expert layer, forward, in one launch
* :func:`moe_layer_bwd` -- its backward direction (data and router
  gradients) in one launch

The compute is in ``libkos.so`` (hand-written HIP, C ABI in
``include/kos.h``); this package only marshals torch tensors into pointers.
"""
from ._binding import (KOS_BF16, KOS_F32, MODE_FIXED, MODE_FUSED, MODE_UNFUSED, RS_BAND,  # noqa: F401
                       RS_ROW, EXPORTS, KosError, MoeShape, Opts, lib, opts)
from .api import (Workspace, ag_gemm, ag_gemm_mx, ag_gemm_noalloc, gemm_rs, gemm_rs_mx, moe_combine,  # noqa: F401
                  moe_dispatch, moe_layer, moe_layer_bwd)
