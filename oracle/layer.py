"""Plain fp64 CPU oracle of the whole Jamba Mamba layer around the mixer (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import it; the HIP library
never calls it and shares no code with it.

The layer is the mixer's pre-norm residual block, in the order the Jamba pages give its parts:

  1. RMSNorm of the residual stream (width d_model)   (the neurarch "Jamba" page: its Structure table puts an
     RMSNorm of normalizedShape 4096 before each Mamba block, and its Exported PyTorch listing an
     nn.RMSNorm(4096) before each mixer; llm-architectures-explained, "Jamba v0.1", Facts: norm type RMSNorm,
     placement pre; TransformerLens, architecture overview: pre-norm, mixer, residual);
  2. in_proj (d_model -> 2 d_inner, no bias), split into the mixer's x | z
                                                      (TransformerLens "supported_architectures.jamba",
                                                       architecture overview: in_proj ... out_proj);
  3. the mixer (oracle.mixer);
  4. out_proj (d_inner -> d_model, no bias)          (same overview);
  5. the residual add: out = x_res + out_proj(y).

Reading taken where the pages leave it open: in_proj's rows hold x first and z second (Mamba's convention,
the same order the library's strided x / z views assume); neither projection has a bias; the layer norm is
the mixer's own rms_norm definition with its own weight and eps.  No page prints that eps (the listing
leaves nn.RMSNorm at its default): the value 1e-6 of the selective-parameter norms is used.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .mixer import mixer_prefill, rms_norm

__all__ = ["layer_prefill", "layer_decode_step"]


def layer_prefill(x_res: np.ndarray, lw: Dict[str, np.ndarray], w: Dict[str, np.ndarray], dt_rank: int,
                  d_state: int, eps: float = 1e-6, layer_eps: float = 1e-6,
                  conv_state: Optional[np.ndarray] = None, ssm_state: Optional[np.ndarray] = None,
                  return_intermediates: bool = False, zoh: bool = False):
    """The layer from the residual stream x_res [B, L, d_model] to x_res + out_proj(mixer(...)).

    ``lw`` holds norm_w [d_model], in_proj_w [2 C, d_model], out_proj_w [d_model, C]; ``w`` the mixer's
    weights; ``zoh`` selects the mixer's exact zero-order-hold variant.  Returns (out, conv_state_out,
    ssm_state_out[, intermediates]).
    """
    C = w["D"].shape[0]
    hn = rms_norm(x_res, lw["norm_w"], layer_eps)
    xz = hn @ lw["in_proj_w"].T
    x, z = xz[..., :C], xz[..., C:]
    y, conv_out, h = mixer_prefill(x, z, w, dt_rank, d_state, eps, conv_state, ssm_state, zoh=zoh)
    out = x_res + y @ lw["out_proj_w"].T
    if not return_intermediates:
        return out, conv_out, h
    return out, conv_out, h, {"hn": hn, "x": x, "z": z, "y": y}


def layer_decode_step(x_t: np.ndarray, lw: Dict[str, np.ndarray], w: Dict[str, np.ndarray], dt_rank: int,
                      d_state: int, conv_state: np.ndarray, ssm_state: np.ndarray, eps: float = 1e-6,
                      layer_eps: float = 1e-6):
    """One decode step of the layer: the prefill definition with L = 1.  x_t is [B, d_model]."""
    out, conv_out, h = layer_prefill(x_t[:, None, :], lw, w, dt_rank, d_state, eps, layer_eps, conv_state,
                                     ssm_state)
    return out[:, 0, :], conv_out, h
