"""MI355X (gfx950) library for Interleaved Head Attention: the layer's forward pass, its
gradients, the attention step alone (forward and backward) and the Nexus inner attention.

The compute path is libiha.so (HIP kernels behind the C ABI of include/iha.h); this
package is its thin Python binding plus the seeded synthetic workloads used by the
tests and the benchmark.
"""
from ._binding import (IHA_BF16, IHA_F32, IHA_FLAG_CHECK, IHA_FLAG_FUSED_COLLAPSE, IHA_MASK_CAUSAL, IHA_MASK_NONE,
                       IHA_MASK_WINDOW, IHA_PLAN_MIX_FUSED, IHAError, LIB_PATH, STATIC_WORKSPACE_BYTES,
                       TIMED_EVENTS, iha_attention, iha_attention_backward, iha_backward,
                       iha_backward_workspace_bytes, iha_forward, iha_forward_static, iha_nexus_inner,
                       iha_plan, iha_status_str, iha_workspace_bytes, load_library, make_problem)

__all__ = ["iha_forward", "iha_backward", "iha_backward_workspace_bytes", "iha_nexus_inner",
           "iha_forward_static", "STATIC_WORKSPACE_BYTES", "iha_attention", "iha_attention_backward",
           "iha_plan", "iha_workspace_bytes", "iha_status_str", "IHAError", "make_problem",
           "load_library", "LIB_PATH", "IHA_MASK_NONE", "IHA_MASK_CAUSAL", "IHA_MASK_WINDOW",
           "IHA_F32", "IHA_BF16", "IHA_FLAG_CHECK", "IHA_FLAG_FUSED_COLLAPSE", "IHA_PLAN_MIX_FUSED",
           "TIMED_EVENTS"]
