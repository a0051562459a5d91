"""MI355X (gfx950) library for the per-denoising-step unmask decision of
masked diffusion language models.

The computation runs in hand-written HIP kernels behind the C ABI of
``include/dlm.h`` (``libdlm.so`` in this directory); :mod:`.api` is the thin
torch binding and :mod:`.synth` the seeded synthetic-input generators.
"""
from ._lib import DLMError  # noqa: F401
from .api import (DEFAULTS, cap_select, dapd_select, dapd_step, decide_step,  # noqa: F401
                  dapd_workspace_bytes, depcap_boundary, factor_select, fastdllm_select,
                  fixed_block_eligible, step_stats, topk_select)
