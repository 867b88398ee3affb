"""GPU parity at exactly the shapes and launch configurations the benchmark times, through the C ABI, against
the fp64 oracle (the mixer's own five workloads are in test_gpu_parity.py):

  - the whole Mamba layer at Jamba v0.1's widths (d_model 4096, d_inner 8192): the 4K-token prefill, compared
    in full, and decode steps of 256 sequences (the decode GEMMs take other kernels than at small sizes);
  - the gated scan's training calls at B = 1, L = 4096, d_inner 8192: the forward, the training forward that
    saves the piece states, the backward that recomputes them and the backward from the saved states;
  - the serving calls: a packed batch of 8 prompts of mixed lengths (4096 tokens) in place into a 64-row
    state pool, and 256-sequence decode steps over a 1024-row pool with the slot sets the benchmark rotates.

Tolerances are the mixer's (parity_util); the backward's gradients are compared relative to their largest
magnitude, as in test_gpu_backward.py.
"""

import numpy as np
import pytest
import torch

import oracle
from jm_inputs import CONFIGS, LAYER_CONFIGS, SERVING_CONFIGS, SERVING_POOL_ROWS, make_activations, \
    make_layer_input, make_layer_weights, make_scan_problem, make_state, make_weights, packed_lengths, pool_slots, \
    to_f64
from parity_util import assert_bitwise, assert_close, log, weights_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


def _layer(cfg, w, lw):
    import mamba_selective_scan_05_amd as jm
    return jm.Layer(lw, w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps, 1e-6)


def test_layer_prefill_jamba_4k_full():
    cfg = LAYER_CONFIGS[0]
    w, lw = make_weights(cfg, DEV), make_layer_weights(cfg, DEV)
    x_res = make_layer_input(cfg, DEV)
    log(f"[{cfg.name}] B={cfg.batch} L={cfg.seqlen} d_model={cfg.d_model} C={cfg.d_inner}")
    out, cs, hs = _layer(cfg, w, lw).prefill(x_res)
    torch.cuda.synchronize()
    log("  layer oracle over every channel ...")
    ro, rc, rh = oracle.layer_prefill(to_f64(x_res), weights_f64(lw), weights_f64(w), cfg.dt_rank, cfg.d_state,
                                      cfg.norm_eps, 1e-6)
    assert_close("out", out, ro, "bf16")
    # in bf16 the residual's rounding dominates the output; the increment alone is checked as well
    assert_close("increment", to_f64(out) - to_f64(x_res), ro - to_f64(x_res), "bf16")
    assert_close("h_final", hs, rh, "bf16")
    assert_close("conv_state", cs, rc, "bf16")


def test_layer_decode_jamba_B256_steps():
    cfg = LAYER_CONFIGS[1]
    w, lw = make_weights(cfg, DEV), make_layer_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    xs = make_layer_input(cfg, DEV, steps=3)
    log(f"[{cfg.name}] B={cfg.batch} d_model={cfg.d_model} C={cfg.d_inner}, 3 steps in place")
    layer = _layer(cfg, w, lw)
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    c64, h64 = to_f64(st["conv_state"]), to_f64(st["ssm_state"])
    w64, lw64 = weights_f64(w), weights_f64(lw)
    for t in range(xs.shape[1]):
        x = xs[:, t].contiguous()
        out, _, _ = layer.decode_step(x, cs, hs, in_place=True)
        torch.cuda.synchronize()
        ro, c64, h64 = oracle.layer_decode_step(to_f64(x), lw64, w64, cfg.dt_rank, cfg.d_state, c64, h64,
                                                cfg.norm_eps, 1e-6)
        assert_close(f"out[{t}]", out, ro, "bf16")
        assert_close(f"increment[{t}]", to_f64(out) - to_f64(x), ro - to_f64(x), "bf16")
    assert_close("h_final", hs, h64, "bf16")
    assert_close("conv_state", cs, c64, "bf16")


def test_scan_training_calls_jamba_4k():
    import mamba_selective_scan_05_amd as jm
    # the benchmark's training problem
    cfg = CONFIGS[1].replace(name="jamba_scan_train_B1_L4096", seed=1301)
    p = make_scan_problem(cfg, DEV)
    B, L, C, N = cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state
    log(f"[{cfg.name}] B={B} L={L} C={C} bf16")
    args = (p["x"], p["delta"], p["z"], p["bc"], p["A_log"], p["D"], p["h0"])
    out, h = jm.scan_forward(*args)
    out2, h2, saved = jm.scan_forward(*args, save=True)
    g = jm.scan_backward(*args[:6], p["dout"], p["h0"], p["dh_final"])
    gs = jm.scan_backward(*args[:6], p["dout"], p["h0"], p["dh_final"], saved_states=saved)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(h, h2)
    bc = to_f64(p["bc"]).reshape(B, L, 2 * N)
    f = {k: to_f64(p[k]) for k in ("x", "delta", "z", "A_log", "D", "dout", "h0", "dh_final")}
    ro, _, rh = oracle.scan_forward_gated(f["x"], f["delta"], f["A_log"], bc[..., :N], bc[..., N:], f["D"], f["z"],
                                          f["h0"])
    assert_close("forward out", out, ro, "bf16")
    assert_close("forward h_out", h, rh, "bf16")
    log("  backward oracle over every channel ...")
    r = oracle.selective_scan_backward(f["x"], f["delta"], f["A_log"], bc[..., :N], bc[..., N:], f["D"], f["z"],
                                       f["dout"], f["h0"], f["dh_final"])
    for label, gg in (("recomputed", g), ("saved", gs)):
        for mine, ref in (("dx", "dxc"), ("ddelta", "ddelta"), ("dz", "dz"), ("dA_log", "dA_log"), ("dD", "dD"),
                          ("dh0", "dh0")):
            assert_close(f"{label} {mine}", gg[mine], r[ref], "bf16")
        dbc = gg["dbc"].reshape(B, L, 2 * N)
        assert_close(f"{label} dB", dbc[..., :N], r["dB"], "bf16")
        assert_close(f"{label} dC", dbc[..., N:], r["dC"], "bf16")


def test_serving_packed_prefill_as_benched():
    import mamba_selective_scan_05_amd as jm
    cfg, rows = SERVING_CONFIGS[0], SERVING_POOL_ROWS[0]
    w = make_weights(cfg, DEV)
    T, C = cfg.seqlen, cfg.d_inner
    a = make_activations(cfg.replace(batch=1), DEV)
    x, z = a["x"][0].contiguous(), a["z"][0].contiguous()
    lens = packed_lengths(T, cfg.batch, cfg.seed)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    slots = pool_slots(cfg.batch, rows, cfg.seed)
    st = make_state(cfg.replace(batch=rows), DEV)
    cp, hp = st["conv_state"].clone(), st["ssm_state"].clone()
    log(f"[{cfg.name}] lengths {lens} slots {slots} pool {rows}, in place")
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    out, _, _ = m.prefill_varlen(x, z, cu, cp, hp, slots=torch.tensor(slots, dtype=torch.int32, device=DEV),
                                 in_place=True)
    torch.cuda.synchronize()
    ro, rc, rh = oracle.mixer_prefill_varlen(to_f64(x), to_f64(z), cu.cpu().numpy(), weights_f64(w), cfg.dt_rank,
                                             cfg.d_state, cfg.norm_eps, to_f64(st["conv_state"]),
                                             to_f64(st["ssm_state"]), slots)
    assert_close("out", out, ro, "bf16")
    idx = torch.tensor(slots, device=DEV, dtype=torch.long)
    assert_close("ssm_state[slots]", hp[idx], rh[slots], "bf16")
    assert_bitwise("conv_state[slots]", cp[idx], torch.from_numpy(rc[slots]).to(cfg.torch_dtype))
    rest = torch.tensor(sorted(set(range(rows)) - set(slots)), device=DEV, dtype=torch.long)
    assert torch.equal(cp[rest], st["conv_state"][rest]) and torch.equal(hp[rest], st["ssm_state"][rest])


def test_serving_decode_pool_1024_as_benched():
    import mamba_selective_scan_05_amd as jm
    cfg, rows = SERVING_CONFIGS[1], SERVING_POOL_ROWS[1]
    B, C = cfg.batch, cfg.d_inner
    w = make_weights(cfg, DEV)
    st = make_state(cfg.replace(batch=rows), DEV)
    cp, hp = st["conv_state"].clone(), st["ssm_state"].clone()
    perm = pool_slots(rows, rows, cfg.seed)
    sets = [perm[k * B:(k + 1) * B] for k in range(rows // B)]
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    xs = torch.randn((3, B, C), generator=g, device=DEV).to(cfg.torch_dtype)
    zs = torch.randn((3, B, C), generator=g, device=DEV).to(cfg.torch_dtype)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    c64, h64 = to_f64(st["conv_state"]), to_f64(st["ssm_state"])
    w64 = weights_f64(w)
    # steps over slot sets 0, 1, 0: the third step continues rows the first one updated
    for step, k in enumerate((0, 1, 0)):
        sl = sets[k]
        log(f"[{cfg.name}] step {step}: B={B} over a {rows}-row pool, slot set {k}")
        out = m.decode_step_slots(xs[step], zs[step], cp, hp, torch.tensor(sl, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        ro, rc, rh = oracle.mixer_decode_step(to_f64(xs[step]), to_f64(zs[step]), w64, cfg.dt_rank, cfg.d_state,
                                              c64[sl], h64[sl], cfg.norm_eps)
        c64[sl], h64[sl] = rc, rh
        assert_close(f"out[{step}]", out, ro, "bf16")
    touched = sorted(set(sets[0]) | set(sets[1]))
    idx = torch.tensor(touched, device=DEV, dtype=torch.long)
    assert_close("ssm pool (touched rows)", hp[idx], h64[touched], "bf16")
    assert_bitwise("conv pool (touched rows)", cp[idx], torch.from_numpy(c64[touched]).to(cfg.torch_dtype))
    rest = torch.tensor(sorted(set(range(rows)) - set(touched)), device=DEV, dtype=torch.long)
    assert torch.equal(cp[rest], st["conv_state"][rest]) and torch.equal(hp[rest], st["ssm_state"][rest])
