"""MI355X-native (gfx950) Mamba-2 SSD chunked forward pass.

The compute path is libssd.so (hand-written HIP kernels behind the C ABI of
include/ssd.h); :mod:`.binding` marshals torch tensors into it.  Importing this
package does not load the library; the first call does, and raises if it is
missing.
"""
from .binding import (FORWARD_EVENTS, SSD_BF16, SSD_F32, ForwardPlan, SsdError, SsdProblem, StepPlan, make_problem,
                      plan_candidates, problem_of, ssd_chunk_cumsum, ssd_chunk_out, ssd_forward,
                      ssd_forward_noalloc, ssd_plan, ssd_state_pass, ssd_step, ssd_status_string,
                      ssd_validate, ssd_workspace_bytes, ssd_workspace_bytes_planned,
                      ssd_workspace_layout, workspace_for, workspace_views)
from .tune import autotune

__all__ = ["FORWARD_EVENTS", "SSD_BF16", "SSD_F32", "ForwardPlan", "SsdError", "SsdProblem", "StepPlan", "autotune",
           "make_problem", "plan_candidates", "problem_of", "ssd_workspace_bytes_planned",
           "ssd_chunk_cumsum", "ssd_chunk_out", "ssd_forward", "ssd_forward_noalloc", "ssd_plan", "ssd_state_pass", "ssd_step",
           "ssd_status_string", "ssd_validate", "ssd_workspace_bytes", "ssd_workspace_layout",
           "workspace_for", "workspace_views"]
