"""Seeded synthetic inputs for the Jamba Mamba-1 mixer, shared by the oracle side and the HIP side.

This module holds the workload recipes (shapes, value distributions, seeds) and nothing of the method's
arithmetic: no convolution, projection, normalisation, discretisation or scan is computed here.  The
shapes follow the Jamba v0.1 architecture fields (llm-architectures-explained, "Jamba v0.1", table
"Every architecture field": d_inner 8192, state 16, conv kernel 4, dt_rank 256) and the Mamba-1 mixer's
parameter list (TransformerLens, "supported_architectures.jamba", architecture overview).

Distributions (the second argument of N is a variance):
    x, z            ~ N(0, 1)
    conv_w          ~ U(-0.5, 0.5), conv_b = 0
    x_proj_w        ~ N(0, 1/d_inner)        rows ordered dt | B | C
    dt_proj_w       ~ N(0, 1/dt_rank)
    dt_proj_b       = log(expm1(u)), u ~ U(1e-3, 0.1)   (so the bias alone puts dt in [1e-3, 0.1])
    A_log[c, n]     = log(n + 1)
    D               = 1
    dt/B/C norm w   = 1, eps = 1e-6
    decode h0       ~ N(0, 0.1) fp32, conv0 ~ N(0, 1) in the I/O dtype

The whole Mamba layer around the mixer (pre-norm, in_proj, mixer, out_proj, residual) adds, with d_model
the residual width (4096 in Jamba v0.1):
    x_res           ~ N(0, 1)                 [B, L, d_model]
    layer norm w    ~ 1 + U(-0.5, 0.5)        [d_model], eps = 1e-6
    in_proj_w       ~ N(0, 1/d_model)         [2 d_inner, d_model], rows ordered x | z
    out_proj_w      ~ N(0, 1/d_inner)         [d_model, d_inner]

Serving workloads (continuous batching) add:
    packed lengths  nseq - 1 distinct cut points drawn uniformly from 1 .. T-1 (numpy default_rng(seed)),
                    so the prompts of one packed batch vary widely in length
    pool slots      distinct pool rows drawn uniformly without replacement (numpy default_rng(seed))

The gated scan on its own (the training forward and backward) takes delta ~ U(1e-3, 0.2) directly,
B and C ~ N(0, 1) as the RMSNorms leave them, dout ~ N(0, 1), h0 and dh_final ~ N(0, 0.1).

Every tensor draws from its own torch generator whose seed is a child of numpy's SeedSequence(1000 + cfg),
spawned in a fixed order, so a tensor's values do not depend on which other tensors were generated.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

# Fixed spawn order of the per-tensor child seeds; appending new names at the end keeps old values stable.
_TENSOR_ORDER = (
    "x", "z", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D",
    "dt_norm_w", "b_norm_w", "c_norm_w", "conv_state", "ssm_state", "x_steps", "z_steps",
    "layer_norm_w", "in_proj_w", "out_proj_w", "x_res", "x_res_steps",
    "scan_delta", "scan_bc", "scan_dout", "scan_dh_final",
)


@dataclasses.dataclass(frozen=True)
class MixerConfig:
    """One workload: the mixer's dimensions, I/O dtype and sequence shape."""

    name: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int = 16
    dt_rank: int = 256
    d_conv: int = 4
    io_dtype: str = "bf16"          # "f32" or "bf16"; the SSM state is always fp32
    norm_eps: float = 1e-6
    decode_steps: int = 0           # > 0: a decode workload of this many single-token steps
    with_state: bool = False        # draw an initial conv / SSM state (decode workloads always do)
    seed: int = 1000
    d_model: int = 0                # residual width of the whole layer (0: the mixer alone)

    @property
    def width(self) -> int:
        """Columns of the x_proj output: dt_rank + 2 * d_state."""
        return self.dt_rank + 2 * self.d_state

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.io_dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "MixerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny fp32 mixer, Jamba-v0.1 prefill at 4K, batched prefill, 256K context, decode.
CONFIGS = (
    MixerConfig("tiny_f32_B1_L64_C64", batch=1, seqlen=64, d_inner=64, dt_rank=8, io_dtype="f32", seed=1000),
    MixerConfig("jamba_prefill_B1_L4096", batch=1, seqlen=4096, d_inner=8192, seed=1001),
    MixerConfig("jamba_prefill_B8_L4096", batch=8, seqlen=4096, d_inner=8192, seed=1002),
    MixerConfig("jamba_prefill_B1_L262144", batch=1, seqlen=262144, d_inner=8192, seed=1003),
    MixerConfig("jamba_decode_B256_x128", batch=256, seqlen=1, d_inner=8192, decode_steps=128,
                with_state=True, seed=1004),
)


# Serving-style workloads at Jamba v0.1's widths: 4096 tokens of 8 prompts of mixed lengths prefilled as one
# packed batch into rows of a 64-row state pool; decode of 256 sequences whose states sit in a 1024-row pool.
SERVING_CONFIGS = (
    CONFIGS[1].replace(name="jamba_varlen_prefill_T4096_n8_pool64", batch=8, with_state=True, seed=1201),
    CONFIGS[4].replace(name="jamba_decode_slots_B256_pool1024", seed=1202),
)
SERVING_POOL_ROWS = (64, 1024)


def packed_lengths(total: int, nseq: int, seed: int) -> List[int]:
    """Lengths of nseq prompts packed into ``total`` tokens (each >= 1): nseq - 1 distinct cut points drawn
    uniformly from 1 .. total - 1."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, total), nseq - 1, replace=False))
    return [int(v) for v in np.diff(np.concatenate([[0], cuts, [total]]))]


def pool_slots(n: int, pool: int, seed: int) -> List[int]:
    """n distinct rows of a pool of ``pool`` rows, drawn uniformly without replacement."""
    rng = np.random.default_rng(seed)
    return [int(v) for v in rng.choice(pool, n, replace=False)]


def _child_seeds(seed: int) -> Dict[str, int]:
    kids = np.random.SeedSequence(seed).spawn(len(_TENSOR_ORDER))
    return {name: int(k.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
            for name, k in zip(_TENSOR_ORDER, kids)}


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std: float, seed: int, device: str) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return t.mul_(std) if std != 1.0 else t


def _uniform(shape, lo: float, hi: float, seed: int, device: str) -> torch.Tensor:
    t = torch.rand(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def make_weights(cfg: MixerConfig, device: str = "cpu") -> Dict[str, torch.Tensor]:
    """All mixer weights in the config's I/O dtype (PyTorch [out, in] layouts, contiguous).

    Weights are always drawn on the CPU generator so that they are identical whatever the device.
    """
    s = _child_seeds(cfg.seed)
    C, N, R, K, W = cfg.d_inner, cfg.d_state, cfg.dt_rank, cfg.d_conv, cfg.width
    u = _uniform((C,), 1e-3, 0.1, s["dt_proj_b"], "cpu").double()
    w = {
        "conv_w": _uniform((C, K), -0.5, 0.5, s["conv_w"], "cpu"),
        "conv_b": torch.zeros(C),
        "x_proj_w": _normal((W, C), math.sqrt(1.0 / C), s["x_proj_w"], "cpu"),
        "dt_proj_w": _normal((C, R), math.sqrt(1.0 / R), s["dt_proj_w"], "cpu"),
        # inverse of log(1 + e^v) at u, in fp64 before rounding: the bias alone gives dt = u
        "dt_proj_b": torch.log(torch.expm1(u)).float(),
        "A_log": torch.log(torch.arange(1, N + 1, dtype=torch.float64)).float().repeat(C, 1),
        "D": torch.ones(C),
        "dt_norm_w": torch.ones(R),
        "b_norm_w": torch.ones(N),
        "c_norm_w": torch.ones(N),
    }
    return {k: v.to(cfg.torch_dtype).contiguous().to(device) for k, v in w.items()}


def make_activations(cfg: MixerConfig, device: str = "cpu", seqlen: Optional[int] = None,
                     row_stride: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """x and z of shape [B, L, C] in the I/O dtype.

    With ``row_stride`` > C, x and z are the two halves of one [B, L, row_stride] buffer laid out as
    [x | z | pad], the way an in_proj output would hold them, so both are strided views.
    """
    s = _child_seeds(cfg.seed)
    B, C = cfg.batch, cfg.d_inner
    L = cfg.seqlen if seqlen is None else seqlen
    x = _normal((B, L, C), 1.0, s["x"], device).to(cfg.torch_dtype)
    z = _normal((B, L, C), 1.0, s["z"], device).to(cfg.torch_dtype)
    if row_stride is None or row_stride == C:
        return {"x": x, "z": z}
    assert row_stride >= 2 * C
    buf = torch.zeros((B, L, row_stride), dtype=cfg.torch_dtype, device=device)
    buf[..., :C] = x
    buf[..., C:2 * C] = z
    return {"x": buf[..., :C], "z": buf[..., C:2 * C], "buffer": buf}


def make_state(cfg: MixerConfig, device: str = "cpu") -> Dict[str, torch.Tensor]:
    """Initial conv state [B, C, K-1] (I/O dtype, oldest first) and SSM state [B, C, N] (fp32)."""
    s = _child_seeds(cfg.seed)
    B, C, N, K = cfg.batch, cfg.d_inner, cfg.d_state, cfg.d_conv
    conv = _normal((B, C, K - 1), 1.0, s["conv_state"], device).to(cfg.torch_dtype)
    h = _normal((B, C, N), math.sqrt(0.1), s["ssm_state"], device)
    return {"conv_state": conv, "ssm_state": h}


def make_decode_tokens(cfg: MixerConfig, device: str = "cpu") -> Dict[str, torch.Tensor]:
    """The decode workload's tokens: x and z of shape [B, steps, C] (step t is [:, t, :])."""
    s = _child_seeds(cfg.seed)
    B, C, T = cfg.batch, cfg.d_inner, cfg.decode_steps
    x = _normal((B, T, C), 1.0, s["x_steps"], device).to(cfg.torch_dtype)
    z = _normal((B, T, C), 1.0, s["z_steps"], device).to(cfg.torch_dtype)
    return {"x": x, "z": z}


# The whole Mamba layer at Jamba v0.1's widths (d_model 4096 around d_inner 8192): 4K prefill and decode.
LAYER_CONFIGS = (
    CONFIGS[1].replace(name="jamba_layer_prefill_B1_L4096", d_model=4096, seed=1101),
    CONFIGS[4].replace(name="jamba_layer_decode_B256", d_model=4096, seed=1104),
)


def make_layer_weights(cfg: MixerConfig, device: str = "cpu") -> Dict[str, torch.Tensor]:
    """The layer's own weights (pre-norm, in_proj, out_proj) in the I/O dtype; the mixer's come from
    make_weights.  Drawn on the CPU generator, like the mixer's."""
    assert cfg.d_model > 0
    s = _child_seeds(cfg.seed)
    C, Dm = cfg.d_inner, cfg.d_model
    w = {
        "norm_w": _uniform((Dm,), 0.5, 1.5, s["layer_norm_w"], "cpu"),
        "in_proj_w": _normal((2 * C, Dm), math.sqrt(1.0 / Dm), s["in_proj_w"], "cpu"),
        "out_proj_w": _normal((Dm, C), math.sqrt(1.0 / C), s["out_proj_w"], "cpu"),
    }
    return {k: v.to(cfg.torch_dtype).contiguous().to(device) for k, v in w.items()}


def make_layer_input(cfg: MixerConfig, device: str = "cpu", steps: int = 0) -> torch.Tensor:
    """The residual stream entering the layer: [B, L, d_model], or [B, steps, d_model] decode tokens."""
    assert cfg.d_model > 0
    s = _child_seeds(cfg.seed)
    if steps:
        return _normal((cfg.batch, steps, cfg.d_model), 1.0, s["x_res_steps"], device).to(cfg.torch_dtype)
    return _normal((cfg.batch, cfg.seqlen, cfg.d_model), 1.0, s["x_res"], device).to(cfg.torch_dtype)


def make_scan_problem(cfg: MixerConfig, device: str = "cpu", with_state: bool = True) -> Dict[str, torch.Tensor]:
    """Inputs of the gated scan alone and of its backward (training): x = xc, z ~ N(0, 1) and delta ~
    U(1e-3, 0.2) [B, L, C] in the I/O dtype; bc ~ N(0, 1) [B*L, 2N] fp32 (B then C, as the RMSNorms leave
    them); A_log and D as the mixer's; dout ~ N(0, 1) [B, L, C]; h0 and dh_final ~ N(0, 0.1) fp32."""
    s = _child_seeds(cfg.seed)
    B, L, C, N = cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state
    w = make_weights(cfg, device)
    a = make_activations(cfg, device)
    p = {
        "x": a["x"].contiguous(), "z": a["z"].contiguous(),
        "delta": _uniform((B, L, C), 1e-3, 0.2, s["scan_delta"], device).to(cfg.torch_dtype),
        "bc": _normal((B * L, 2 * N), 1.0, s["scan_bc"], device),
        "A_log": w["A_log"], "D": w["D"],
        "dout": _normal((B, L, C), 1.0, s["scan_dout"], device).to(cfg.torch_dtype),
        "h0": None, "dh_final": None,
    }
    if with_state:
        p["h0"] = make_state(cfg, device)["ssm_state"]
        p["dh_final"] = _normal((B, C, N), math.sqrt(0.1), s["scan_dh_final"], device)
    return p


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of an fp32 / bf16 tensor (any device) to a float64 numpy array."""
    return t.detach().to("cpu").double().numpy()
