"""Jamba's Mamba-1 mixer (conv1d + SiLU, x_proj, dt/B/C RMSNorms, dt_proj + softplus, selective scan, D skip,
SiLU(z) gate) as hand-written HIP kernels for AMD MI355X (gfx950), behind the C ABI of include/jm_mixer.h.

``Mixer`` wraps the two entry points (``jm_mixer_prefill``, ``jm_mixer_decode_step``) on torch tensors (``prefill``
and ``decode_step`` are the same calls as plain functions of a weight dict);
``Layer`` the whole Mamba layer around the mixer (include/jm_layer.h: pre-norm, in_proj, mixer, out_proj,
residual).
"""

from ._lib import (JM_BF16, JM_DISC_EULER, JM_DISC_ZOH, JM_F32, JMError, Mixer, Dims, Weights, WorkspaceLayout, call_decode_step,  # noqa: F401
                   call_prefill, decode_workspace_size, lib, make_dims, pack_weights, prefill_workspace_size,
                   status_string, workspace_layout)
from ._lib import Layer, LayerDims, LayerWeights, call_layer, layer_workspace_size, make_layer_dims  # noqa: F401
from ._lib import call_decode_step_slots, call_prefill_varlen, varlen_workspace_size  # noqa: F401
from ._lib import call_decode_step_noalloc, call_decode_step_single_kernel, noalloc_scratch_limit  # noqa: F401
from ._lib import decode_step, mixer_for, prefill  # noqa: F401
from ._lib import (ScanDims, scan_backward, scan_dims, scan_forward, scan_saved_states_size,  # noqa: F401
                   scan_workspace_size)
