"""Plain fp64 CPU oracle of the selective scan's backward pass (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import it; the HIP library
never calls it and shares no code with it.

The forward it differentiates is the scan with the D skip and the SiLU(z) gate (Jamba Guide, aifetchly
blog, "Inside the Mamba State-Space Layers: Mathematical Mechanics": discretisation equations and recurrent
state update; the same section notes that training computes the scan over whole sequences at once):

    A = -exp(A_log),  a_t = exp(delta_t * A),  h_t = a_t * h_{t-1} + delta_t * B_t * x_t,
    y_t = C_t . h_t + D * x_t,  out_t = y_t * SiLU(z_t).

The pages print no backward; it is the chain rule applied to these lines in reverse time, written out below
without reordering.  With dy_t = dout_t * SiLU(z_t) and G_t the gradient that reaches h_t from later tokens
(dh_final at the last token), the total gradient of h_t is g_t = G_t + C_t * dy_t, and
    G_{t-1} = a_t * g_t                         (the state's own path)
    d delta_t  = sum_n g_t * (h_{t-1} * a_t * A + B_t * x_t)
    d x_t      = sum_n g_t * delta_t * B_t + D * dy_t
    d B_t      = sum_c g_t * delta_t * x_t      (B_t is shared by every channel)
    d C_t      = sum_c dy_t * h_t               (C_t likewise)
    d A        = sum_t g_t * h_{t-1} * a_t * delta_t,   d A_log = d A * A   (dA/dA_log = -exp(A_log) = A)
    d D        = sum_t dy_t * x_t
    d z_t      = dout_t * y_t * SiLU'(z_t),  SiLU'(z) = s * (1 + z * (1 - s)),  s = sigmoid(z)
    d h0       = G_{-1} = a_0 * g_0.
Sums over the batch are taken for the parameters A_log and D.  Arrays are numpy float64.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

__all__ = ["selective_scan_backward", "scan_forward_gated"]


def _sigmoid(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def scan_forward_gated(xc: np.ndarray, delta: np.ndarray, A_log: np.ndarray, Bn: np.ndarray, Cn: np.ndarray,
                       D: np.ndarray, z: np.ndarray, h0: Optional[np.ndarray] = None):
    """The forward the backward differentiates: returns (out [B, L, C], y [B, L, C], h_L [B, C, N]).

    xc, delta, z [B, L, C]; Bn, Cn [B, L, N]; A_log [C, N]; D [C]; h0 [B, C, N] or None (zeros)."""
    Bb, L, C = xc.shape
    N = A_log.shape[1]
    A = -np.exp(A_log)
    h = np.zeros((Bb, C, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    y = np.empty((Bb, L, C))
    for t in range(L):
        a = np.exp(delta[:, t, :, None] * A[None])
        h = a * h + (delta[:, t, :] * xc[:, t, :])[:, :, None] * Bn[:, t, None, :]
        y[:, t, :] = np.sum(h * Cn[:, t, None, :], axis=-1) + D * xc[:, t, :]
    return y * (z * _sigmoid(z)), y, h


def selective_scan_backward(xc: np.ndarray, delta: np.ndarray, A_log: np.ndarray, Bn: np.ndarray, Cn: np.ndarray,
                            D: np.ndarray, z: np.ndarray, dout: np.ndarray, h0: Optional[np.ndarray] = None,
                            dh_final: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of  sum(dout * out) + sum(dh_final * h_L)  with respect to every input of the gated scan.

    Shapes as in scan_forward_gated; dout [B, L, C]; dh_final [B, C, N] or None (zero).  Channels are
    independent except through dB and dC, which sum over them: given the arrays of a subset of channels, the
    function returns that subset's gradients and its contributions to dB / dC.
    Returns dxc, ddelta, dz [B, L, C]; dB, dC [B, L, N]; dA_log [C, N]; dD [C]; dh0 [B, C, N].
    """
    Bb, L, C = xc.shape
    N = A_log.shape[1]
    A = -np.exp(A_log)
    # forward, keeping every state (h_hist[t] = h after token t)
    h = np.zeros((Bb, C, N)) if h0 is None else np.array(h0, dtype=np.float64, copy=True)
    h_init = h.copy()
    h_hist = np.empty((L, Bb, C, N))
    y = np.empty((Bb, L, C))
    for t in range(L):
        a = np.exp(delta[:, t, :, None] * A[None])
        h = a * h + (delta[:, t, :] * xc[:, t, :])[:, :, None] * Bn[:, t, None, :]
        h_hist[t] = h
        y[:, t, :] = np.sum(h * Cn[:, t, None, :], axis=-1) + D * xc[:, t, :]
    s = _sigmoid(z)
    dy = dout * (z * s)
    dz = dout * y * (s * (1.0 + z * (1.0 - s)))

    dxc = np.empty_like(xc, dtype=np.float64)
    ddelta = np.empty_like(delta, dtype=np.float64)
    dB = np.empty((Bb, L, N))
    dC = np.empty((Bb, L, N))
    dA = np.zeros((Bb, C, N))
    G = np.zeros((Bb, C, N)) if dh_final is None else np.array(dh_final, dtype=np.float64, copy=True)
    for t in range(L - 1, -1, -1):
        g = G + Cn[:, t, None, :] * dy[:, t, :, None]                  # [B, C, N]
        h_prev = h_hist[t - 1] if t > 0 else h_init
        a = np.exp(delta[:, t, :, None] * A[None])
        dt = delta[:, t, :, None]
        xt = xc[:, t, :, None]
        ddelta[:, t, :] = np.sum(g * (h_prev * a * A[None] + Bn[:, t, None, :] * xt), axis=-1)
        dxc[:, t, :] = np.sum(g * dt * Bn[:, t, None, :], axis=-1) + D * dy[:, t, :]
        dB[:, t, :] = np.sum(g * dt * xt, axis=1)
        dC[:, t, :] = np.sum(dy[:, t, :, None] * h_hist[t], axis=1)
        dA += g * h_prev * a * dt
        G = a * g
    return {
        "dxc": dxc, "ddelta": ddelta, "dz": dz, "dB": dB, "dC": dC,
        "dA_log": np.sum(dA, axis=0) * A, "dD": np.sum(dy * xc, axis=(0, 1)), "dh0": G,
    }
