"""ctypes binding of libjm_mixer.so (the C ABI in include/jm_mixer.h, include/jm_layer.h and include/jm_scan.h).

The functions here only marshal arguments: torch tensors provide device memory and the stream, their
data pointers go to the library, and every step of the mixer runs in the library's HIP kernels.  If the
library is missing, loading fails loudly; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libjm_mixer.so")

JM_OK, JM_ERR_INVALID_ARG, JM_ERR_UNSUPPORTED, JM_ERR_ALIGNMENT, JM_ERR_WORKSPACE, JM_ERR_HIP = 0, -1, -2, -3, -4, -5
JM_ERR_SCRATCH_LIMIT = -6
JM_F32, JM_BF16 = 0, 1
JM_DISC_EULER, JM_DISC_ZOH = 0, 1

WEIGHT_NAMES = ("conv_w", "conv_b", "x_proj_w", "dt_norm_w", "b_norm_w", "c_norm_w", "dt_proj_w", "dt_proj_b",
                "A_log", "D")


class JMError(RuntimeError):
    """A nonzero status from the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("d_inner", ctypes.c_int32),
                ("d_state", ctypes.c_int32), ("dt_rank", ctypes.c_int32), ("d_conv", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("x_row_stride", ctypes.c_int64), ("z_row_stride", ctypes.c_int64),
                ("discretization", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [("xc", ctypes.c_int64), ("dbc", ctypes.c_int64), ("dln", ctypes.c_int64), ("bc", ctypes.c_int64),
                ("delta", ctypes.c_int64), ("carries", ctypes.c_int64), ("dbc_splits", ctypes.c_int32),
                ("scan_chunks", ctypes.c_int32), ("total_bytes", ctypes.c_int64), ("xproj_path", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class LayerDims(ctypes.Structure):
    _fields_ = [("mixer", Dims), ("d_model", ctypes.c_int32), ("layer_norm_eps", ctypes.c_float)]


LAYER_WEIGHT_NAMES = ("norm_w", "in_proj_w", "out_proj_w")


class ScanDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("d_inner", ctypes.c_int32),
                ("d_state", ctypes.c_int32), ("io_dtype", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHT_NAMES] + [("mixer", Weights)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (built by ``python -m mamba_selective_scan_05_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mamba_selective_scan_05_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, V, I, S = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        for name in ("jm_mixer_prefill", "jm_mixer_decode_step"):
            f = getattr(L, name)
            f.argtypes = [P(Dims), P(Weights), V, V, V, V, V, V, V, V, S, V]
            f.restype = I
        for name in ("jm_mixer_prefill_workspace_size", "jm_mixer_decode_workspace_size"):
            f = getattr(L, name)
            f.argtypes = [P(Dims)]
            f.restype = S
        L.jm_status_string.argtypes = [I]
        L.jm_status_string.restype = ctypes.c_char_p
        L.jm_mixer_prefill_workspace_layout.argtypes = [P(Dims), P(WorkspaceLayout)]
        L.jm_mixer_prefill_workspace_layout.restype = I
        for name in ("jm_mixer_prefill_profiled", "jm_mixer_decode_step_profiled"):
            f = getattr(L, name)
            f.argtypes = [P(Dims), P(Weights), V, V, V, V, V, V, V, V, S, V, P(V), I]
            f.restype = I
        L.jm_stage_name.argtypes = [I]
        L.jm_stage_name.restype = ctypes.c_char_p
        for name in ("jm_layer_prefill", "jm_layer_decode_step"):
            f = getattr(L, name)
            f.argtypes = [P(LayerDims), P(LayerWeights), V, V, V, V, V, V, V, S, V]
            f.restype = I
        L.jm_mixer_decode_step_noalloc.argtypes = [P(Dims), P(Weights), V, V, V, V, V, V, V, V]
        L.jm_mixer_decode_step_noalloc.restype = I
        L.jm_mixer_decode_noalloc_scratch_limit.argtypes = []
        L.jm_mixer_decode_noalloc_scratch_limit.restype = S
        L.jm_mixer_decode_step_slots.argtypes = [P(Dims), P(Weights), V, V, V, V, V, ctypes.c_int32, V, V, S, V]
        L.jm_mixer_decode_step_slots.restype = I
        L.jm_mixer_decode_step_single_kernel.argtypes = [P(Dims), P(Weights), V, V, V, V, V, V, V, ctypes.c_int32, V,
                                                         V, S, V]
        L.jm_mixer_decode_step_single_kernel.restype = I
        L.jm_layer_decode_step_slots.argtypes = [P(LayerDims), P(LayerWeights), V, V, V, V, ctypes.c_int32, V, V,
                                                 S, V]
        L.jm_layer_decode_step_slots.restype = I
        L.jm_mixer_prefill_varlen.argtypes = [P(Dims), P(Weights), V, V, V, V, V, V, V, V, V, ctypes.c_int32, V, S,
                                              V]
        L.jm_mixer_prefill_varlen.restype = I
        L.jm_layer_prefill_varlen.argtypes = [P(LayerDims), P(LayerWeights), V, V, V, V, V, V, V, V,
                                              ctypes.c_int32, V, S, V]
        L.jm_layer_prefill_varlen.restype = I
        L.jm_mixer_prefill_varlen_workspace_size.argtypes = [P(Dims)]
        L.jm_mixer_prefill_varlen_workspace_size.restype = S
        L.jm_layer_prefill_varlen_workspace_size.argtypes = [P(LayerDims)]
        L.jm_layer_prefill_varlen_workspace_size.restype = S
        L.jm_scan_forward.argtypes = [P(ScanDims)] + [V] * 10 + [S, V]
        L.jm_scan_forward.restype = I
        L.jm_scan_forward_train.argtypes = [P(ScanDims)] + [V] * 11 + [S, V]
        L.jm_scan_forward_train.restype = I
        L.jm_scan_backward.argtypes = [P(ScanDims)] + [V] * 18 + [S, V]
        L.jm_scan_backward.restype = I
        for name in ("jm_scan_forward_workspace_size", "jm_scan_backward_workspace_size",
                     "jm_scan_saved_states_size"):
            f = getattr(L, name)
            f.argtypes = [P(ScanDims)]
            f.restype = S
        for name in ("jm_layer_prefill_workspace_size", "jm_layer_decode_workspace_size"):
            f = getattr(L, name)
            f.argtypes = [P(LayerDims)]
            f.restype = S
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().jm_status_string(status).decode()


def make_dims(batch: int, seqlen: int, d_inner: int, dt_rank: int, io_dtype: int, d_state: int = 16,
              d_conv: int = 4, norm_eps: float = 1e-6, x_row_stride: int = 0, z_row_stride: int = 0,
              discretization: int = 0) -> Dims:
    """discretization: JM_DISC_EULER (0, dt * B) or JM_DISC_ZOH (1, the exact zero-order hold)."""
    return Dims(batch, seqlen, d_inner, d_state, dt_rank, d_conv, io_dtype, norm_eps, x_row_stride, z_row_stride,
                discretization, 0)


def prefill_workspace_size(dims: Dims) -> int:
    return int(lib().jm_mixer_prefill_workspace_size(ctypes.byref(dims)))


def decode_workspace_size(dims: Dims) -> int:
    return int(lib().jm_mixer_decode_workspace_size(ctypes.byref(dims)))


def workspace_layout(dims: Dims) -> WorkspaceLayout:
    lay = WorkspaceLayout()
    s = lib().jm_mixer_prefill_workspace_layout(ctypes.byref(dims), ctypes.byref(lay))
    if s != JM_OK:
        raise JMError(s, "jm_mixer_prefill_workspace_layout")
    return lay


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def pack_weights(w: Dict[str, torch.Tensor]) -> Weights:
    return Weights(*[_ptr(w.get(n)) for n in WEIGHT_NAMES])


def _ref(s):
    return None if s is None else ctypes.byref(s)


def call_prefill(dims: Dims, weights: Weights, x, z, out, conv_in, conv_out, h_in, h_out, ws, ws_bytes: int,
                 stream: int) -> int:
    """The raw entry point on integer device pointers (None for NULL)."""
    return lib().jm_mixer_prefill(_ref(dims), _ref(weights), x, z, out, conv_in, conv_out, h_in, h_out, ws,
                                  ws_bytes, stream)


def call_decode_step(dims: Dims, weights: Weights, x, z, out, conv_in, conv_out, h_in, h_out, ws, ws_bytes: int,
                     stream: int) -> int:
    return lib().jm_mixer_decode_step(_ref(dims), _ref(weights), x, z, out, conv_in, conv_out, h_in, h_out, ws,
                                      ws_bytes, stream)


def call_decode_step_noalloc(dims: Dims, weights: Weights, x, z, out, conv_in, conv_out, h_in, h_out,
                             stream: int) -> int:
    """jm_mixer_decode_step_noalloc: the decode step with the library's own device scratch (no workspace)."""
    return lib().jm_mixer_decode_step_noalloc(_ref(dims), _ref(weights), x, z, out, conv_in, conv_out, h_in, h_out,
                                              stream)


def call_decode_step_single_kernel(dims: Dims, weights: Weights, x, z, out, conv_in, conv_out, h_in, h_out,
                                   pool_size: int, slots, ws, ws_bytes: int, stream: int) -> int:
    """jm_mixer_decode_step_single_kernel on integer device pointers (slots None: a plain batch)."""
    return lib().jm_mixer_decode_step_single_kernel(_ref(dims), _ref(weights), x, z, out, conv_in, conv_out, h_in,
                                                    h_out, pool_size, slots, ws, ws_bytes, stream)


def noalloc_scratch_limit() -> int:
    return int(lib().jm_mixer_decode_noalloc_scratch_limit())


def call_decode_step_slots(dims: Dims, weights: Weights, x, z, out, conv_pool, ssm_pool, pool_size: int, slots,
                           ws, ws_bytes: int, stream: int) -> int:
    """The raw state-pool decode entry point on integer device pointers (None for NULL)."""
    return lib().jm_mixer_decode_step_slots(_ref(dims), _ref(weights), x, z, out, conv_pool, ssm_pool, pool_size,
                                            slots, ws, ws_bytes, stream)


def call_prefill_varlen(dims: Dims, weights: Weights, x, z, out, cu_seqlens, conv_in, conv_out, h_in, h_out,
                       slots, pool_size: int, ws, ws_bytes: int, stream: int) -> int:
    """The raw packed-batch prefill entry point on integer device pointers (None for NULL)."""
    return lib().jm_mixer_prefill_varlen(_ref(dims), _ref(weights), x, z, out, cu_seqlens, conv_in, conv_out, h_in,
                                         h_out, slots, pool_size, ws, ws_bytes, stream)


def varlen_workspace_size(dims: Dims) -> int:
    return int(lib().jm_mixer_prefill_varlen_workspace_size(ctypes.byref(dims)))


def _check_cu(cu_seqlens: torch.Tensor) -> int:
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 2 or \
            not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector of n_seq + 1 offsets")
    return int(cu_seqlens.shape[0]) - 1


def _check_pools(conv_pool: torch.Tensor, ssm_pool: torch.Tensor, slots: torch.Tensor, batch: int) -> int:
    if slots.dtype != torch.int32 or slots.dim() != 1 or slots.shape[0] != batch or not slots.is_contiguous():
        raise ValueError(f"slots must be a contiguous int32 vector of length {batch}")
    if conv_pool.shape[0] != ssm_pool.shape[0]:
        raise ValueError("conv and SSM state pools differ in rows")
    _check_contiguous(conv_pool=conv_pool, ssm_pool=ssm_pool)
    return int(conv_pool.shape[0])


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return JM_F32
    if t.dtype == torch.bfloat16:
        return JM_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _row_stride(t: torch.Tensor, rows_per_batch: int) -> int:
    """Row stride of a [B, L, C] (or [B, C]) view whose channel dim is contiguous and whose rows are evenly
    spaced across the batch."""
    if t.stride(-1) != 1:
        raise ValueError("the channel dimension must be contiguous")
    rs = t.stride(-2) if t.dim() == 3 else t.stride(0)
    if t.numel() == 0:
        return int(t.shape[-1])
    if t.dim() == 3 and t.shape[0] > 1 and t.stride(0) != rows_per_batch * rs:
        raise ValueError("rows must be evenly spaced across the batch")
    return int(rs)


def _check_contiguous(**tensors) -> None:
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Mixer:
    """Holds the weights (device tensors in the I/O dtype) and a reusable workspace."""

    def __init__(self, weights: Dict[str, torch.Tensor], dt_rank: int, d_state: int = 16, d_conv: int = 4,
                 norm_eps: float = 1e-6, zoh: bool = False):
        self.zoh = zoh
        self.w = {k: v.contiguous() for k, v in weights.items()}
        self.packed = pack_weights(self.w)
        self.dt_rank, self.d_state, self.d_conv, self.eps = dt_rank, d_state, d_conv, norm_eps
        self.d_inner = self.w["conv_w"].shape[0]
        self.device = self.w["conv_w"].device
        self.dtype = self.w["conv_w"].dtype
        self._ws = None

    def dims(self, batch: int, seqlen: int, x_row_stride: int = 0, z_row_stride: int = 0) -> Dims:
        return make_dims(batch, seqlen, self.d_inner, self.dt_rank, _io_dtype(self.w["conv_w"]), self.d_state,
                         self.d_conv, self.eps, x_row_stride, z_row_stride, JM_DISC_ZOH if self.zoh else JM_DISC_EULER)

    def workspace(self, nbytes: int) -> torch.Tensor:
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def prefill(self, x: torch.Tensor, z: torch.Tensor, conv_state: Optional[torch.Tensor] = None,
                ssm_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                conv_state_out: Optional[torch.Tensor] = None, ssm_state_out: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        B, L, C = x.shape
        dims = self.dims(B, L, _row_stride(x, L), _row_stride(z, L))
        nbytes = prefill_workspace_size(dims)
        if nbytes == 0:
            raise JMError(JM_ERR_INVALID_ARG, "jm_mixer_prefill_workspace_size")
        ws = self.workspace(nbytes)
        if out is None:
            out = torch.empty((B, L, C), dtype=self.dtype, device=self.device)
        if conv_state_out is None:
            conv_state_out = torch.empty((B, C, self.d_conv - 1), dtype=self.dtype, device=self.device)
        if ssm_state_out is None:
            ssm_state_out = torch.empty((B, C, self.d_state), dtype=torch.float32, device=self.device)
        _check_contiguous(out=out, conv_state=conv_state, conv_state_out=conv_state_out, ssm_state=ssm_state,
                          ssm_state_out=ssm_state_out)
        s = call_prefill(dims, self.packed, _ptr(x), _ptr(z), _ptr(out), _ptr(conv_state), _ptr(conv_state_out),
                         _ptr(ssm_state), _ptr(ssm_state_out), _ptr(ws), ws.numel(), _stream(self.device))
        if s != JM_OK:
            raise JMError(s, "jm_mixer_prefill")
        return out, conv_state_out, ssm_state_out

    def decode_step(self, x: torch.Tensor, z: torch.Tensor, conv_state: torch.Tensor, ssm_state: torch.Tensor,
                    out: Optional[torch.Tensor] = None, conv_state_out: Optional[torch.Tensor] = None,
                    ssm_state_out: Optional[torch.Tensor] = None, in_place: bool = False,
                    single_kernel: bool = False) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """One token per sequence: x, z are [B, C].  With in_place=True the states are updated in place;
        single_kernel=True runs jm_mixer_decode_step_single_kernel instead of jm_mixer_decode_step."""
        B, C = x.shape
        dims = self.dims(B, 1, _row_stride(x, 1), _row_stride(z, 1))
        nbytes = decode_workspace_size(dims)
        if nbytes == 0:
            raise JMError(JM_ERR_INVALID_ARG, "jm_mixer_decode_workspace_size")
        ws = self.workspace(nbytes)
        if out is None:
            out = torch.empty((B, C), dtype=self.dtype, device=self.device)
        if in_place:
            conv_state_out, ssm_state_out = conv_state, ssm_state
        if conv_state_out is None:
            conv_state_out = torch.empty_like(conv_state)
        if ssm_state_out is None:
            ssm_state_out = torch.empty_like(ssm_state)
        _check_contiguous(out=out, conv_state=conv_state, conv_state_out=conv_state_out, ssm_state=ssm_state,
                          ssm_state_out=ssm_state_out)
        if single_kernel:
            s = call_decode_step_single_kernel(dims, self.packed, _ptr(x), _ptr(z), _ptr(out), _ptr(conv_state),
                                               _ptr(conv_state_out), _ptr(ssm_state), _ptr(ssm_state_out), 0, None,
                                               _ptr(ws), ws.numel(), _stream(self.device))
            if s != JM_OK:
                raise JMError(s, "jm_mixer_decode_step_single_kernel")
            return out, conv_state_out, ssm_state_out
        s = call_decode_step(dims, self.packed, _ptr(x), _ptr(z), _ptr(out), _ptr(conv_state), _ptr(conv_state_out),
                             _ptr(ssm_state), _ptr(ssm_state_out), _ptr(ws), ws.numel(), _stream(self.device))
        if s != JM_OK:
            raise JMError(s, "jm_mixer_decode_step")
        return out, conv_state_out, ssm_state_out

    def prefill_varlen(self, x: torch.Tensor, z: torch.Tensor, cu_seqlens: torch.Tensor,
                       conv_state: Optional[torch.Tensor] = None, ssm_state: Optional[torch.Tensor] = None,
                       slots: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       conv_state_out: Optional[torch.Tensor] = None, ssm_state_out: Optional[torch.Tensor] = None,
                       in_place: bool = False) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """A packed batch: x, z [T, C] hold the sequences back to back, cu_seqlens (device int32 [n + 1])
        delimits them.  States have one row per sequence, or are pools indexed by ``slots`` (device int32
        [n]); with in_place=True the input states are updated in place."""
        T, C = x.shape
        nseq = _check_cu(cu_seqlens)
        dims = self.dims(nseq, T, _row_stride(x, T), _row_stride(z, T))
        nbytes = varlen_workspace_size(dims)
        if nbytes == 0:
            raise JMError(JM_ERR_INVALID_ARG, "jm_mixer_prefill_varlen_workspace_size")
        ws = self.workspace(nbytes)
        rows = nseq
        pool = 0
        if slots is not None:
            if slots.dtype != torch.int32 or slots.shape != (nseq,) or not slots.is_contiguous():
                raise ValueError(f"slots must be a contiguous int32 vector of length {nseq}")
            ref = conv_state if conv_state is not None else conv_state_out
            if ref is None:
                raise ValueError("a state pool needs the conv state tensor (input or output) to size it")
            rows = pool = int(ref.shape[0])
        if out is None:
            out = torch.empty((T, C), dtype=self.dtype, device=self.device)
        if in_place:
            conv_state_out, ssm_state_out = conv_state, ssm_state
        if conv_state_out is None:
            conv_state_out = torch.empty((rows, C, self.d_conv - 1), dtype=self.dtype, device=self.device)
        if ssm_state_out is None:
            ssm_state_out = torch.empty((rows, C, self.d_state), dtype=torch.float32, device=self.device)
        _check_contiguous(out=out, conv_state=conv_state, conv_state_out=conv_state_out, ssm_state=ssm_state,
                          ssm_state_out=ssm_state_out)
        s = call_prefill_varlen(dims, self.packed, _ptr(x), _ptr(z), _ptr(out), _ptr(cu_seqlens), _ptr(conv_state),
                                _ptr(conv_state_out), _ptr(ssm_state), _ptr(ssm_state_out), _ptr(slots), pool,
                                _ptr(ws), ws.numel(), _stream(self.device))
        if s != JM_OK:
            raise JMError(s, "jm_mixer_prefill_varlen")
        return out, conv_state_out, ssm_state_out

    def decode_step_slots(self, x: torch.Tensor, z: torch.Tensor, conv_pool: torch.Tensor, ssm_pool: torch.Tensor,
                          slots: torch.Tensor, out: Optional[torch.Tensor] = None,
                          single_kernel: bool = False) -> torch.Tensor:
        """One token per sequence with the states in pools ([P, C, K-1] and [P, C, N]) updated in place at
        rows slots[b] (a device int32 [B]; an entry outside [0, P) runs from zero states and stores none).
        single_kernel=True runs jm_mixer_decode_step_single_kernel instead of jm_mixer_decode_step_slots."""
        B, C = x.shape
        pool = _check_pools(conv_pool, ssm_pool, slots, B)
        dims = self.dims(B, 1, _row_stride(x, 1), _row_stride(z, 1))
        nbytes = decode_workspace_size(dims)
        if nbytes == 0:
            raise JMError(JM_ERR_INVALID_ARG, "jm_mixer_decode_workspace_size")
        ws = self.workspace(nbytes)
        if out is None:
            out = torch.empty((B, C), dtype=self.dtype, device=self.device)
        _check_contiguous(out=out)
        if single_kernel:
            s = call_decode_step_single_kernel(dims, self.packed, _ptr(x), _ptr(z), _ptr(out), _ptr(conv_pool),
                                               _ptr(conv_pool), _ptr(ssm_pool), _ptr(ssm_pool), pool, _ptr(slots),
                                               _ptr(ws), ws.numel(), _stream(self.device))
            if s != JM_OK:
                raise JMError(s, "jm_mixer_decode_step_single_kernel")
            return out
        s = call_decode_step_slots(dims, self.packed, _ptr(x), _ptr(z), _ptr(out), _ptr(conv_pool), _ptr(ssm_pool),
                                   pool, _ptr(slots), _ptr(ws), ws.numel(), _stream(self.device))
        if s != JM_OK:
            raise JMError(s, "jm_mixer_decode_step_slots")
        return out


def make_layer_dims(batch: int, seqlen: int, d_inner: int, dt_rank: int, io_dtype: int, d_model: int,
                    d_state: int = 16, d_conv: int = 4, norm_eps: float = 1e-6,
                    layer_norm_eps: float = 1e-6, discretization: int = 0) -> LayerDims:
    return LayerDims(make_dims(batch, seqlen, d_inner, dt_rank, io_dtype, d_state, d_conv, norm_eps,
                               discretization=discretization), d_model, layer_norm_eps)


def layer_workspace_size(dims: LayerDims, decode: bool = False) -> int:
    f = lib().jm_layer_decode_workspace_size if decode else lib().jm_layer_prefill_workspace_size
    return int(f(ctypes.byref(dims)))


def call_layer(dims: LayerDims, weights: LayerWeights, x_res, out, conv_in, conv_out, h_in, h_out, ws,
               ws_bytes: int, stream: int, decode: bool = False) -> int:
    """The raw layer entry point on integer device pointers (None for NULL)."""
    f = lib().jm_layer_decode_step if decode else lib().jm_layer_prefill
    return f(_ref(dims), _ref(weights), x_res, out, conv_in, conv_out, h_in, h_out, ws, ws_bytes, stream)


class Layer:
    """The whole Mamba layer (pre-norm, in_proj, mixer, out_proj, residual): holds the layer's and the mixer's
    weights (device tensors in the I/O dtype) and a reusable workspace."""

    def __init__(self, layer_weights: Dict[str, torch.Tensor], mixer_weights: Dict[str, torch.Tensor], dt_rank: int,
                 d_state: int = 16, d_conv: int = 4, norm_eps: float = 1e-6, layer_norm_eps: float = 1e-6,
                 zoh: bool = False):
        self.mixer = Mixer(mixer_weights, dt_rank, d_state, d_conv, norm_eps, zoh)
        self.lw = {k: v.contiguous() for k, v in layer_weights.items()}
        self.packed = LayerWeights(*[_ptr(self.lw[n]) for n in LAYER_WEIGHT_NAMES], self.mixer.packed)
        self.d_model = self.lw["norm_w"].shape[0]
        self.layer_eps = layer_norm_eps
        self.device, self.dtype = self.mixer.device, self.mixer.dtype
        self._ws = None

    def dims(self, batch: int, seqlen: int) -> LayerDims:
        m = self.mixer
        return make_layer_dims(batch, seqlen, m.d_inner, m.dt_rank, _io_dtype(m.w["conv_w"]), self.d_model,
                               m.d_state, m.d_conv, m.eps, self.layer_eps, JM_DISC_ZOH if m.zoh else JM_DISC_EULER)

    def workspace(self, nbytes: int) -> torch.Tensor:
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def _run(self, x_res, conv_state, ssm_state, out, conv_state_out, ssm_state_out, decode: bool):
        B = x_res.shape[0]
        L = 1 if decode else x_res.shape[1]
        C = self.mixer.d_inner
        dims = self.dims(B, L)
        nbytes = layer_workspace_size(dims, decode)
        if nbytes == 0:
            raise JMError(JM_ERR_INVALID_ARG, "jm_layer_*_workspace_size")
        ws = self.workspace(nbytes)
        if out is None:
            out = torch.empty_like(x_res)
        if conv_state_out is None:
            conv_state_out = torch.empty((B, C, self.mixer.d_conv - 1), dtype=self.dtype, device=self.device)
        if ssm_state_out is None:
            ssm_state_out = torch.empty((B, C, self.mixer.d_state), dtype=torch.float32, device=self.device)
        _check_contiguous(x_res=x_res, out=out, conv_state=conv_state, conv_state_out=conv_state_out,
                          ssm_state=ssm_state, ssm_state_out=ssm_state_out)
        s = call_layer(dims, self.packed, _ptr(x_res), _ptr(out), _ptr(conv_state), _ptr(conv_state_out),
                       _ptr(ssm_state), _ptr(ssm_state_out), _ptr(ws), ws.numel(), _stream(self.device), decode)
        if s != JM_OK:
            raise JMError(s, "jm_layer_decode_step" if decode else "jm_layer_prefill")
        return out, conv_state_out, ssm_state_out

    def prefill(self, x_res: torch.Tensor, conv_state: Optional[torch.Tensor] = None,
                ssm_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                conv_state_out: Optional[torch.Tensor] = None, ssm_state_out: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """x_res [B, L, d_model] -> (out, conv_state_out, ssm_state_out); out may be x_res itself."""
        return self._run(x_res, conv_state, ssm_state, out, conv_state_out, ssm_state_out, False)

    def decode_step(self, x_res: torch.Tensor, conv_state: torch.Tensor, ssm_state: torch.Tensor,
                    out: Optional[torch.Tensor] = None, in_place: bool = False
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """x_res [B, d_model]; with in_place=True the states are updated in place."""
        co, so = (conv_state, ssm_state) if in_place else (None, None)
        return self._run(x_res, conv_state, ssm_state, out, co, so, True)

    def prefill_varlen(self, x_res: torch.Tensor, cu_seqlens: torch.Tensor, conv_state: Optional[torch.Tensor] = None,
                       ssm_state: Optional[torch.Tensor] = None, slots: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, in_place: bool = False
                       ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """A packed batch x_res [T, d_model] split by cu_seqlens (device int32 [n + 1]); states per sequence or
        in pools through ``slots``; with in_place=True the input states are updated in place."""
        T = x_res.shape[0]
        nseq = _check_cu(cu_seqlens)
        m = self.mixer
        C = m.d_inner
        dims = self.dims(nseq, T)
        nbytes = int(lib().jm_layer_prefill_varlen_workspace_size(ctypes.byref(dims)))
        if nbytes == 0:
            raise JMError(JM_ERR_INVALID_ARG, "jm_layer_prefill_varlen_workspace_size")
        ws = self.workspace(nbytes)
        rows, pool = nseq, 0
        if slots is not None:
            if slots.dtype != torch.int32 or slots.shape != (nseq,) or not slots.is_contiguous():
                raise ValueError(f"slots must be a contiguous int32 vector of length {nseq}")
            if conv_state is None:
                raise ValueError("a state pool needs the conv state tensor to size it")
            rows = pool = int(conv_state.shape[0])
        if out is None:
            out = torch.empty_like(x_res)
        if in_place:
            co, so = conv_state, ssm_state
        else:
            co = torch.empty((rows, C, m.d_conv - 1), dtype=self.dtype, device=self.device)
            so = torch.empty((rows, C, m.d_state), dtype=torch.float32, device=self.device)
        _check_contiguous(x_res=x_res, out=out, conv_state=conv_state, ssm_state=ssm_state, co=co, so=so)
        s = lib().jm_layer_prefill_varlen(_ref(dims), _ref(self.packed), _ptr(x_res), _ptr(out), _ptr(cu_seqlens),
                                          _ptr(conv_state), _ptr(co), _ptr(ssm_state), _ptr(so), _ptr(slots), pool,
                                          _ptr(ws), ws.numel(), _stream(self.device))
        if s != JM_OK:
            raise JMError(s, "jm_layer_prefill_varlen")
        return out, co, so

    def decode_step_slots(self, x_res: torch.Tensor, conv_pool: torch.Tensor, ssm_pool: torch.Tensor,
                          slots: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """x_res [B, d_model]; the states live in pools updated in place at rows slots[b] (device int32 [B])."""
        B = x_res.shape[0]
        pool = _check_pools(conv_pool, ssm_pool, slots, B)
        dims = self.dims(B, 1)
        nbytes = layer_workspace_size(dims, True)
        if nbytes == 0:
            raise JMError(JM_ERR_INVALID_ARG, "jm_layer_decode_workspace_size")
        ws = self.workspace(nbytes)
        if out is None:
            out = torch.empty_like(x_res)
        _check_contiguous(x_res=x_res, out=out)
        s = lib().jm_layer_decode_step_slots(_ref(dims), _ref(self.packed), _ptr(x_res), _ptr(out), _ptr(conv_pool),
                                             _ptr(ssm_pool), pool, _ptr(slots), _ptr(ws), ws.numel(),
                                             _stream(self.device))
        if s != JM_OK:
            raise JMError(s, "jm_layer_decode_step_slots")
        return out


def mixer_for(weights: Dict[str, torch.Tensor], norm_eps: float = 1e-6, zoh: bool = False) -> "Mixer":
    """A Mixer for a weight dict, with dt_rank, d_state and d_conv read from the weight shapes."""
    return Mixer(weights, weights["dt_proj_w"].shape[1], weights["A_log"].shape[1], weights["conv_w"].shape[-1],
                 norm_eps, zoh)


def prefill(x: torch.Tensor, z: torch.Tensor, weights: Dict[str, torch.Tensor],
            conv_state: Optional[torch.Tensor] = None, ssm_state: Optional[torch.Tensor] = None,
            norm_eps: float = 1e-6, zoh: bool = False) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """jm_mixer_prefill on torch tensors: x, z [B, L, C] (row strides may exceed C), states [B, C, K-1] and
    [B, C, N] fp32 or None (zeros); returns (out, conv_state_out, ssm_state_out).  Each call allocates its
    workspace; a Mixer reuses one across calls."""
    return mixer_for(weights, norm_eps, zoh).prefill(x, z, conv_state, ssm_state)


def decode_step(x: torch.Tensor, z: torch.Tensor, weights: Dict[str, torch.Tensor], conv_state: torch.Tensor,
                ssm_state: torch.Tensor, norm_eps: float = 1e-6, zoh: bool = False, in_place: bool = False
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """jm_mixer_decode_step on torch tensors: one token per sequence, x, z [B, C]; with in_place=True the
    states are updated in place.  Returns (out, conv_state_out, ssm_state_out)."""
    return mixer_for(weights, norm_eps, zoh).decode_step(x, z, conv_state, ssm_state, in_place=in_place)


# ----------------------------------------------------------------------------- the gated scan alone (training)

def scan_dims(batch: int, seqlen: int, d_inner: int, io_dtype: int, d_state: int = 16) -> ScanDims:
    return ScanDims(batch, seqlen, d_inner, d_state, io_dtype)


def scan_workspace_size(dims: ScanDims, backward: bool = False) -> int:
    f = lib().jm_scan_backward_workspace_size if backward else lib().jm_scan_forward_workspace_size
    return int(f(ctypes.byref(dims)))


def _scan_ws(dims: ScanDims, backward: bool, device) -> torch.Tensor:
    n = scan_workspace_size(dims, backward)
    if n == 0:
        raise JMError(JM_ERR_INVALID_ARG, "jm_scan_*_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def scan_saved_states_size(dims: ScanDims) -> int:
    return int(lib().jm_scan_saved_states_size(ctypes.byref(dims)))


def scan_forward(x: torch.Tensor, delta: torch.Tensor, z: torch.Tensor, bc: torch.Tensor, A_log: torch.Tensor,
                 D: torch.Tensor, h0: Optional[torch.Tensor] = None, save: bool = False):
    """The gated scan forward (jm_scan_forward): x, delta, z [B, L, C] in the I/O dtype, bc [B*L, 2N] fp32,
    A_log [C, N], D [C]; returns (out [B, L, C], h_out [B, C, N] fp32).  With save (jm_scan_forward_train),
    also the saved states [B, ceil(L / 32), N, C] fp32 for scan_backward, as a third result."""
    B, L, C = x.shape
    N = A_log.shape[1]
    _check_contiguous(x=x, delta=delta, z=z, bc=bc, A_log=A_log, D=D, h0=h0)
    dims = scan_dims(B, L, C, _io_dtype(x), N)
    ws = _scan_ws(dims, False, x.device)
    out = torch.empty_like(x)
    h_out = torch.empty((B, C, N), dtype=torch.float32, device=x.device)
    if not save:
        s = lib().jm_scan_forward(ctypes.byref(dims), _ptr(x), _ptr(delta), _ptr(z), _ptr(bc), _ptr(A_log),
                                  _ptr(D), _ptr(h0), _ptr(out), _ptr(h_out), _ptr(ws), ws.numel(),
                                  _stream(x.device))
        if s != JM_OK:
            raise JMError(s, "jm_scan_forward")
        return out, h_out
    saved = torch.empty((B, (L + 31) // 32, N, C), dtype=torch.float32, device=x.device)
    if saved.numel() * 4 != scan_saved_states_size(dims):
        raise JMError(JM_ERR_INVALID_ARG, "jm_scan_saved_states_size")
    s = lib().jm_scan_forward_train(ctypes.byref(dims), _ptr(x), _ptr(delta), _ptr(z), _ptr(bc), _ptr(A_log),
                                    _ptr(D), _ptr(h0), _ptr(out), _ptr(h_out), _ptr(saved), _ptr(ws), ws.numel(),
                                    _stream(x.device))
    if s != JM_OK:
        raise JMError(s, "jm_scan_forward_train")
    return out, h_out, saved


def scan_backward(x: torch.Tensor, delta: torch.Tensor, z: torch.Tensor, bc: torch.Tensor, A_log: torch.Tensor,
                  D: torch.Tensor, dout: torch.Tensor, h0: Optional[torch.Tensor] = None,
                  dh_final: Optional[torch.Tensor] = None, need_dh0: bool = True,
                  saved_states: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Gradients of sum(dout * out) + sum(dh_final * h_L) (jm_scan_backward): returns dx, ddelta, dz (I/O
    dtype), dbc [B*L, 2N], dA_log [C, N], dD [C] and dh0 [B, C, N] (fp32).  saved_states: the third result
    of scan_forward(..., save=True) on the same inputs, or None (recomputed)."""
    B, L, C = x.shape
    N = A_log.shape[1]
    _check_contiguous(x=x, delta=delta, z=z, bc=bc, A_log=A_log, D=D, dout=dout, h0=h0, dh_final=dh_final,
                      saved_states=saved_states)
    dims = scan_dims(B, L, C, _io_dtype(x), N)
    ws = _scan_ws(dims, True, x.device)
    dev = x.device
    g = {"dx": torch.empty_like(x), "ddelta": torch.empty_like(x), "dz": torch.empty_like(x),
         "dbc": torch.empty((B * L, 2 * N), dtype=torch.float32, device=dev),
         "dA_log": torch.empty((C, N), dtype=torch.float32, device=dev),
         "dD": torch.empty((C,), dtype=torch.float32, device=dev),
         "dh0": torch.empty((B, C, N), dtype=torch.float32, device=dev) if need_dh0 else None}
    s = lib().jm_scan_backward(ctypes.byref(dims), _ptr(x), _ptr(delta), _ptr(z), _ptr(bc), _ptr(A_log), _ptr(D),
                               _ptr(h0), _ptr(dout), _ptr(dh_final), _ptr(saved_states), _ptr(g["dx"]),
                               _ptr(g["ddelta"]), _ptr(g["dz"]),
                               _ptr(g["dbc"]), _ptr(g["dA_log"]), _ptr(g["dD"]), _ptr(g["dh0"]), _ptr(ws), ws.numel(),
                               _stream(dev))
    if s != JM_OK:
        raise JMError(s, "jm_scan_backward")
    return g
