"""Plain fp64 CPU oracle of the serving-style calls (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import it; the HIP library
never calls it and shares no code with it.

A server that batches whichever requests are active (continuous batching: Jamba Guide, aifetchly blog,
"Production Engineering: Serving & Hardware Best Practices") needs two things from the mixer:

  - prefill of several prompts of different lengths in one call, packed one after another with no padding,
    delimited by offsets cu_seqlens (sequence s is packed tokens [cu[s], cu[s+1]));
  - per-sequence conv / recurrent states kept in pools, addressed by a slot index per sequence
    (TransformerLens "supported_architectures.jamba": generation carries the Mamba conv and recurrent
    states in a cache).

Neither changes what is computed for a sequence: each one is exactly the mixer (or layer) of oracle.mixer /
oracle.layer run on its own tokens from its own states, which is how this module writes them — a loop over
the sequences.  Reading taken where the pages are silent: a slot outside [0, pool) (a padding entry) runs
from zero states and its final states are dropped; an empty sequence leaves its states unchanged.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .layer import layer_prefill
from .mixer import mixer_prefill

__all__ = ["mixer_prefill_varlen", "layer_prefill_varlen", "mixer_decode_step_slots", "layer_decode_step_slots",
           "gather_rows", "scatter_rows"]


def gather_rows(states: Optional[np.ndarray], rows: Sequence[int], shape) -> np.ndarray:
    """The initial states of a batch: states[rows[i]] per sequence, zeros for a row outside the tensor or
    a missing tensor.  ``shape`` is the shape of one row."""
    out = np.zeros((len(rows),) + tuple(shape))
    if states is not None:
        for i, r in enumerate(rows):
            if 0 <= r < states.shape[0]:
                out[i] = states[r]
    return out


def scatter_rows(states: np.ndarray, rows: Sequence[int], values: np.ndarray) -> np.ndarray:
    """A copy of ``states`` with row rows[i] replaced by values[i]; rows outside the tensor are dropped."""
    out = np.array(states, dtype=np.float64, copy=True)
    for i, r in enumerate(rows):
        if 0 <= r < out.shape[0]:
            out[r] = values[i]
    return out


def _rows(nseq: int, slots: Optional[Sequence[int]]) -> List[int]:
    return list(range(nseq)) if slots is None else [int(s) for s in slots]


def mixer_prefill_varlen(x: np.ndarray, z: np.ndarray, cu_seqlens: Sequence[int], w: Dict[str, np.ndarray],
                         dt_rank: int, d_state: int, eps: float = 1e-6, conv_state: Optional[np.ndarray] = None,
                         ssm_state: Optional[np.ndarray] = None, slots: Optional[Sequence[int]] = None,
                         zoh: bool = False):
    """The mixer over a packed batch (``zoh``: the exact zero-order-hold input matrix, see oracle.mixer).

    x, z [T, C] hold the sequences back to back; sequence s is rows [cu[s], cu[s+1]).  The state tensors
    conv_state [R, C, K-1] / ssm_state [R, C, N] (None: zeros) give sequence s the initial states of row s,
    or of row slots[s] when ``slots`` is given (a row outside [0, R): zeros).  Returns (out [T, C],
    conv_state_out, ssm_state_out): the state tensors after the call, i.e. the inputs with each sequence's
    final states written to its row (a missing input reads as zeros of nseq rows without slots, else of as
    many rows as the other state tensor, or the largest slot + 1).
    """
    cu = [int(v) for v in cu_seqlens]
    nseq = len(cu) - 1
    C = x.shape[1]
    K = w["conv_w"].shape[1]
    rows = _rows(nseq, slots)
    n_rows = nseq if slots is None else (conv_state.shape[0] if conv_state is not None else
                                         ssm_state.shape[0] if ssm_state is not None else max(rows) + 1)
    conv_out = np.zeros((n_rows, C, K - 1)) if conv_state is None else np.array(conv_state, dtype=np.float64)
    ssm_out = np.zeros((n_rows, C, d_state)) if ssm_state is None else np.array(ssm_state, dtype=np.float64)
    out = np.zeros_like(x, dtype=np.float64)
    for s in range(nseq):
        c0 = gather_rows(conv_state, [rows[s]], (C, K - 1))
        h0 = gather_rows(ssm_state, [rows[s]], (C, d_state))
        if cu[s + 1] > cu[s]:
            o, cf, hf = mixer_prefill(x[None, cu[s]:cu[s + 1]], z[None, cu[s]:cu[s + 1]], w, dt_rank, d_state, eps,
                                      c0, h0, zoh=zoh)
            out[cu[s]:cu[s + 1]] = o[0]
        else:
            cf, hf = c0, h0
        conv_out = scatter_rows(conv_out, [rows[s]], cf)
        ssm_out = scatter_rows(ssm_out, [rows[s]], hf)
    return out, conv_out, ssm_out


def layer_prefill_varlen(x_res: np.ndarray, cu_seqlens: Sequence[int], lw: Dict[str, np.ndarray],
                         w: Dict[str, np.ndarray], dt_rank: int, d_state: int, eps: float = 1e-6,
                         layer_eps: float = 1e-6, conv_state: Optional[np.ndarray] = None,
                         ssm_state: Optional[np.ndarray] = None, slots: Optional[Sequence[int]] = None):
    """The whole layer over a packed batch x_res [T, d_model]; states as in mixer_prefill_varlen."""
    cu = [int(v) for v in cu_seqlens]
    nseq = len(cu) - 1
    C = w["D"].shape[0]
    K = w["conv_w"].shape[1]
    rows = _rows(nseq, slots)
    n_rows = nseq if slots is None else (conv_state.shape[0] if conv_state is not None else
                                         ssm_state.shape[0] if ssm_state is not None else max(rows) + 1)
    conv_out = np.zeros((n_rows, C, K - 1)) if conv_state is None else np.array(conv_state, dtype=np.float64)
    ssm_out = np.zeros((n_rows, C, d_state)) if ssm_state is None else np.array(ssm_state, dtype=np.float64)
    out = np.array(x_res, dtype=np.float64, copy=True)
    for s in range(nseq):
        c0 = gather_rows(conv_state, [rows[s]], (C, K - 1))
        h0 = gather_rows(ssm_state, [rows[s]], (C, d_state))
        if cu[s + 1] > cu[s]:
            o, cf, hf = layer_prefill(x_res[None, cu[s]:cu[s + 1]], lw, w, dt_rank, d_state, eps, layer_eps, c0, h0)
            out[cu[s]:cu[s + 1]] = o[0]
        else:
            cf, hf = c0, h0
        conv_out = scatter_rows(conv_out, [rows[s]], cf)
        ssm_out = scatter_rows(ssm_out, [rows[s]], hf)
    return out, conv_out, ssm_out


def mixer_decode_step_slots(x_t: np.ndarray, z_t: np.ndarray, w: Dict[str, np.ndarray], dt_rank: int,
                            d_state: int, conv_pool: np.ndarray, ssm_pool: np.ndarray, slots: Sequence[int],
                            eps: float = 1e-6):
    """One decode step of a batch whose states live in pools: sequence b at row slots[b].

    Returns (out [B, C], conv_pool_out, ssm_pool_out)."""
    cu = list(range(x_t.shape[0] + 1))     # one token per sequence
    return mixer_prefill_varlen(x_t, z_t, cu, w, dt_rank, d_state, eps, conv_pool, ssm_pool, slots)


def layer_decode_step_slots(x_t: np.ndarray, lw: Dict[str, np.ndarray], w: Dict[str, np.ndarray], dt_rank: int,
                            d_state: int, conv_pool: np.ndarray, ssm_pool: np.ndarray, slots: Sequence[int],
                            eps: float = 1e-6, layer_eps: float = 1e-6):
    """One decode step of the whole layer with pooled states.  Returns (out [B, d_model], pools...)."""
    cu = list(range(x_t.shape[0] + 1))
    return layer_prefill_varlen(x_t, cu, lw, w, dt_rank, d_state, eps, layer_eps, conv_pool, ssm_pool, slots)
