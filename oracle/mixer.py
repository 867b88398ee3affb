"""Plain, slow fp64 CPU oracle of the Jamba Mamba-1 mixer (test infrastructure only).

This module is the reference the HIP library is checked against.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the library never calls it and shares no code with it.

Every step is the plain definition, written out in float64 numpy, in the order the mixer applies them:

  1. causal depthwise conv1d (kernel 4) + bias, then SiLU
        - Jamba (neurarch), "Exported PyTorch": Mamba(d_conv=4, expand=2);
        - TransformerLens "supported_architectures.jamba", architecture overview: in_proj / conv1d / x_proj /
          dt_proj / out_proj;
  2. x_proj to the selective parameters, split dt | B | C      (same overview; the toy SimpleMambaSSM of the
     Jamba Guide's "Hands-On Implementation" projects B, C and dt from the input the same way);
  3. Jamba's RMSNorms on the dt, B and C slices                 (same overview: dt/b/c layernorms);
  4. dt_proj + bias + softplus                                  (Jamba Guide, SimpleMambaSSM: softplus of a
     biased dt projection);
  5. discretisation  Abar = exp(dt * A),  Bbar = dt * B,  A = -exp(A_log)
                                                                (Jamba Guide, "Inside the Mamba State-Space
     Layers", S6 forward flow and the discretisation equations; A_log convention from SimpleMambaSSM);
  6. recurrence  h_t = Abar_t * h_{t-1} + Bbar_t * x_t,  y_t = C_t . h_t  (+ D * x_t skip)
                                                                (same section, recurrent state update);
  7. gate  out = y * SiLU(z).

Readings where the pages leave a step open (each is listed with its reason in the design notes): the D skip,
the conv bias and the SiLU after the conv, and the z gate are not on the pages and follow the mixer's
conventional form; B is discretised as dt*B (the pages' own approximation) by default, with the exact ZOH
form the pages print beside it as an option; the norms apply
to the dt slice before dt_proj; rms_norm(v) = v / sqrt(mean(v^2) + eps) * w; the conv state holds the last
K-1 raw inputs, oldest first; the SSM state is fp32 on the device and fp64 here.

Arrays are numpy float64.  Activations are [B, L, C]; the conv state is [B, C, K-1]; the SSM state is
[B, C, N]; weights use PyTorch [out, in] layouts.
"""

from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "causal_conv1d_silu", "x_proj", "split_dbc", "rms_norm", "softplus", "dt_proj_softplus",
    "selective_scan", "silu", "mixer_prefill", "mixer_decode_step", "mixer_prefill_slabs",
]


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v * sigmoid(v) = v / (1 + e^-v)."""
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def causal_conv1d_silu(x: np.ndarray, conv_w: np.ndarray, conv_b: Optional[np.ndarray],
                       conv_state: Optional[np.ndarray]):
    """Depthwise causal conv1d + bias, then SiLU.

    x [B, L, C]; conv_w [C, K]; conv_b [C] or None (zero); conv_state [B, C, K-1] or None (zeros),
    holding the K-1 raw inputs that precede x[:, 0], oldest first.

    The extended input is xe[tau] = conv_state[tau + K - 1] for tau < 0 and x[tau] for tau >= 0.  Output
    u[t, c] = b[c] + sum_j conv_w[c, j] * xe[t - (K-1) + j, c]: tap K-1 multiplies the current token, as a
    PyTorch Conv1d with groups=C and left padding K-1 does.  Returns (SiLU(u) [B, L, C],
    new conv state [B, C, K-1] = the last K-1 entries of xe).
    """
    B, L, C = x.shape
    K = conv_w.shape[1]
    if conv_state is None:
        conv_state = np.zeros((B, C, K - 1))
    xe = np.concatenate([np.transpose(conv_state, (0, 2, 1)), x], axis=1)      # [B, K-1+L, C]
    u = np.zeros((B, L, C)) if conv_b is None else np.broadcast_to(conv_b, (B, L, C)).copy()
    for j in range(K):
        # xe index of token t - (K-1) + j is t + j
        u += conv_w[:, j] * xe[:, j:j + L, :]
    new_state = np.transpose(xe[:, L:L + K - 1, :], (0, 2, 1)).copy()
    return silu(u), new_state


def x_proj(xc: np.ndarray, x_proj_w: np.ndarray) -> np.ndarray:
    """dbc[b, t, k] = sum_c x_proj_w[k, c] * xc[b, t, c]."""
    return xc @ x_proj_w.T


def split_dbc(dbc: np.ndarray, dt_rank: int, d_state: int):
    """Split the x_proj output into the dt slice [.., R], the B slice [.., N] and the C slice [.., N]."""
    R, N = dt_rank, d_state
    return dbc[..., :R], dbc[..., R:R + N], dbc[..., R + N:R + 2 * N]


def rms_norm(v: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) * w over the last axis."""
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * w


def softplus(v: np.ndarray) -> np.ndarray:
    """log(1 + e^v), evaluated without overflow."""
    return np.logaddexp(0.0, v)


def dt_proj_softplus(dln: np.ndarray, dt_proj_w: np.ndarray, dt_proj_b: np.ndarray) -> np.ndarray:
    """delta[b, t, c] = softplus(sum_r dt_proj_w[c, r] * dln[b, t, r] + dt_proj_b[c])."""
    return softplus(dln @ dt_proj_w.T + dt_proj_b)


def selective_scan(xc: np.ndarray, delta: np.ndarray, A_log: np.ndarray, Bn: np.ndarray, Cn: np.ndarray,
                   D: np.ndarray, h0: Optional[np.ndarray], zoh: bool = False):
    """The selective scan, one token at a time.

    xc, delta [B, L, C]; A_log [C, N]; Bn, Cn [B, L, N] (shared by all channels); D [C];
    h0 [B, C, N] or None (zeros).  With A = -exp(A_log), for t = 0 .. L-1:
        h[b, c, n] <- exp(delta[b,t,c] * A[c,n]) * h[b, c, n] + Bbar[b,t,c,n] * xc[b,t,c]
        y[b, t, c]  = sum_n Cn[b,t,n] * h[b, c, n] + D[c] * xc[b,t,c]
    where Bbar = delta * Bn (the pages' approximation, the default) or, with ``zoh``, the exact zero-order
    hold of the same section's discretisation equation, (delta A)^-1 (exp(delta A) - 1) delta Bn, which for
    the diagonal A is expm1(delta * A) / A * Bn; where A = 0 (A_log = -inf) that expression is 0 / 0 and
    its value is its limit as A -> 0, delta * Bn.
    Returns (y [B, L, C], h after the last token [B, C, N]).
    """
    B, L, C = xc.shape
    N = A_log.shape[1]
    A = -np.exp(A_log)
    h = np.zeros((B, C, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    y = np.empty((B, L, C))
    for t in range(L):
        dt = delta[:, t, :]                                    # [B, C]
        abar = np.exp(dt[:, :, None] * A[None, :, :])          # [B, C, N]
        if zoh:
            dA = dt[:, :, None] * A[None, :, :]
            with np.errstate(invalid="ignore", divide="ignore"):
                coef = np.where(A[None] == 0.0, dt[:, :, None], np.expm1(dA) / A[None, :, :])
            bbar = coef * Bn[:, t, None, :]
            bbar_x = bbar * xc[:, t, :, None]
        else:
            bbar_x = (dt * xc[:, t, :])[:, :, None] * Bn[:, t, None, :]
        h = abar * h + bbar_x
        y[:, t, :] = np.sum(h * Cn[:, t, None, :], axis=-1) + D * xc[:, t, :]
    return y, h


def mixer_prefill(x: np.ndarray, z: np.ndarray, w: Dict[str, np.ndarray], dt_rank: int, d_state: int,
                  eps: float = 1e-6, conv_state: Optional[np.ndarray] = None,
                  ssm_state: Optional[np.ndarray] = None, channels: Optional[Sequence[int]] = None,
                  return_intermediates: bool = False, zoh: bool = False):
    """The mixer from x, z to the gated output, plus the final conv and SSM states.

    ``w`` holds conv_w, conv_b, x_proj_w, dt_norm_w, b_norm_w, c_norm_w, dt_proj_w, dt_proj_b, A_log, D.
    With ``channels`` given, steps 4-7 (dt_proj, scan, gate) are evaluated for those channels only; steps
    1-3 always cover every channel because x_proj contracts over all of them.  ``ssm_state`` then holds the
    selected channels only ([B, len(channels), N]), and so does the returned SSM state; the conv state is
    always full.  ``zoh`` selects the exact zero-order-hold input matrix in the scan (see selective_scan).
    Returns (out, conv_state_out, ssm_state_out[, intermediates]).
    """
    xc, conv_out = causal_conv1d_silu(x, w["conv_w"], w.get("conv_b"), conv_state)
    dbc = x_proj(xc, w["x_proj_w"])
    dl, bv, cv = split_dbc(dbc, dt_rank, d_state)
    dln = rms_norm(dl, w["dt_norm_w"], eps)
    bn = rms_norm(bv, w["b_norm_w"], eps)
    cn = rms_norm(cv, w["c_norm_w"], eps)
    sel = slice(None) if channels is None else np.asarray(channels)
    delta = dt_proj_softplus(dln, w["dt_proj_w"][sel], w["dt_proj_b"][sel])
    y, h = selective_scan(xc[..., sel], delta, w["A_log"][sel], bn, cn, w["D"][sel], ssm_state, zoh)
    out = y * silu(z[..., sel])
    if not return_intermediates:
        return out, conv_out, h
    inter = {"xc": xc, "dbc": dbc, "dln": dln, "Bn": bn, "Cn": cn, "delta": delta, "y": y}
    return out, conv_out, h, inter


def mixer_decode_step(x_t: np.ndarray, z_t: np.ndarray, w: Dict[str, np.ndarray], dt_rank: int, d_state: int,
                      conv_state: np.ndarray, ssm_state: np.ndarray, eps: float = 1e-6, zoh: bool = False):
    """One decode step: the prefill definition with L = 1.  x_t, z_t are [B, C]."""
    out, conv_out, h = mixer_prefill(x_t[:, None, :], z_t[:, None, :], w, dt_rank, d_state, eps,
                                     conv_state, ssm_state, zoh=zoh)
    return out[:, 0, :], conv_out, h


def mixer_prefill_slabs(get_slab, n_tokens: int, slab: int, w: Dict[str, np.ndarray], dt_rank: int,
                        d_state: int, eps: float = 1e-6, conv_state: Optional[np.ndarray] = None,
                        ssm_state: Optional[np.ndarray] = None, channels: Optional[Sequence[int]] = None,
                        keep=None):
    """A long prefill run as consecutive prefills that hand the conv and SSM states on.

    ``get_slab(t0, t1)`` returns (x, z) float64 for tokens [t0, t1).  ``keep(t0, out)`` receives each slab's
    output (to retain a sample of it).  Returns (conv_state_out, ssm_state_out).
    """
    for t0 in range(0, n_tokens, slab):
        t1 = min(n_tokens, t0 + slab)
        xs, zs = get_slab(t0, t1)
        out, conv_state, ssm_state = mixer_prefill(xs, zs, w, dt_rank, d_state, eps, conv_state, ssm_state,
                                                   channels)
        if keep is not None:
            keep(t0, out)
    return conv_state, ssm_state
