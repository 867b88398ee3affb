"""GPU parity of jm_mixer_decode_step_single_kernel (bf16, d_inner a multiple of 256, dt_rank a multiple of 32 up
to 256, at most 1024 sequences) against the fp64 oracle, through the C ABI.

The step runs as one cooperative kernel: conv + x_proj partial sums per unit of 32 sequences x 256 channels, a
grid-wide barrier, the norms per sequence, a second barrier, then dt_proj and the state update per unit.  The
cases cover ragged last units (B not a multiple of 32), channel slice counts that are and are not a multiple
of 8 (the two unit-to-workgroup mappings), more units than resident workgroups (units loop, xc through HBM),
more sequences than workgroups (the norm phase loops), the exact zero-order hold, strided x / z, a state pool
with slots outside it, repeated calls through one workspace (the barrier flags are keyed to each launch), a
workspace poisoned with all bits set (determinism: two runs bit for bit), and the Jamba decode shape against
the default (multi-kernel) decode step.
"""

import pytest
import torch

import oracle
from jm_inputs import MixerConfig, make_activations, make_state, make_weights, to_f64
from parity_util import assert_bitwise, assert_close, log, weights_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


CASES = [
    # name, batch, d_inner, dt_rank, zoh, x/z row stride
    ("ragged_B37_C512", 37, 512, 64, False, None),
    ("zoh_B70_C768", 70, 768, 96, True, None),          # 3 channel slices: not a multiple of 8
    ("strided_B33_C1024", 33, 1024, 256, False, 2080),
    ("more_units_than_groups_B300", 300, 8192, 256, False, None),
    ("many_sequences_B1024_C2048", 1024, 2048, 128, False, None),
    ("one_sequence_C256_R32", 1, 256, 32, False, None),
]


@pytest.mark.parametrize("name,B,C,R,zoh,stride", CASES, ids=[c[0] for c in CASES])
def test_single_kernel_step_matches_oracle(name, B, C, R, zoh, stride):
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig(f"dk_{name}", batch=B, seqlen=1, d_inner=C, dt_rank=R, io_dtype="bf16", seed=300 + B,
                      with_state=True)
    log(f"[{cfg.name}] B={B} C={C} R={R} zoh={zoh} stride={stride}")
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV, row_stride=stride)
    st = make_state(cfg, DEV)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps, zoh=zoh)
    x, z = a["x"][:, 0], a["z"][:, 0]
    out, cs, hs = m.decode_step(x, z, st["conv_state"], st["ssm_state"], single_kernel=True)
    torch.cuda.synchronize()
    ro, rc, rh = oracle.mixer_decode_step(to_f64(x), to_f64(z), weights_f64(w), R, cfg.d_state,
                                          to_f64(st["conv_state"]), to_f64(st["ssm_state"]), cfg.norm_eps, zoh=zoh)
    assert_close("out", out, ro, "bf16")
    assert_close("ssm_state", hs, rh, "bf16")
    assert_bitwise("conv_state", cs, torch.from_numpy(rc).to(cfg.torch_dtype))


def test_single_kernel_step_repeated_calls_share_a_workspace():
    # successive steps through one workspace (each launch keys its barrier flags to its own id, so the flags
    # an earlier call left behind never count), the states updated in place, against the oracle stepped
    # alongside
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig("dk_repeat", batch=64, seqlen=1, d_inner=1024, dt_rank=64, io_dtype="bf16", seed=331,
                      with_state=True)
    w = make_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    w64 = weights_f64(w)
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    c64, h64 = to_f64(cs), to_f64(hs)
    g = torch.Generator(device=DEV)
    g.manual_seed(332)
    for t in range(4):
        x = torch.randn((cfg.batch, cfg.d_inner), generator=g, device=DEV).to(cfg.torch_dtype)
        z = torch.randn((cfg.batch, cfg.d_inner), generator=g, device=DEV).to(cfg.torch_dtype)
        out, _, _ = m.decode_step(x, z, cs, hs, in_place=True, single_kernel=True)
        torch.cuda.synchronize()
        ro, c64, h64 = oracle.mixer_decode_step(to_f64(x), to_f64(z), w64, cfg.dt_rank, cfg.d_state, c64, h64,
                                                cfg.norm_eps)
        assert_close(f"step {t} out", out, ro, "bf16")
    assert_close("ssm_state after 4 steps", hs, h64, "bf16")


def test_single_kernel_step_matches_the_default_step_at_jamba_widths():
    # B = 256, d_inner 8192: both decode entry points against each other over every element, in place
    import mamba_selective_scan_05_amd as jm
    from jm_inputs import CONFIGS, make_decode_tokens
    cfg = CONFIGS[4]
    w = make_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    tok = make_decode_tokens(cfg.replace(decode_steps=2), DEV)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    c1, h1 = st["conv_state"].clone(), st["ssm_state"].clone()
    c2, h2 = st["conv_state"].clone(), st["ssm_state"].clone()
    for t in range(2):
        x, z = tok["x"][:, t], tok["z"][:, t]
        o1, _, _ = m.decode_step(x, z, c1, h1, in_place=True, single_kernel=True)
        o2, _, _ = m.decode_step(x, z, c2, h2, in_place=True)
        torch.cuda.synchronize()
        assert_close(f"step {t} out vs default step", o1, o2.double().cpu().numpy(), "bf16")
    assert_close("ssm_state vs default step", h1, h2.double().cpu().numpy(), "bf16")
    assert_bitwise("conv_state vs default step", c1, c2)


def test_single_kernel_step_over_a_pool():
    import mamba_selective_scan_05_amd as jm
    P, C, R = 9, 512, 32
    slots = [5, 1, -1, 3, 9, 0, 8]      # -1 and 9 (== pool size) are outside the pool
    B = len(slots)
    pcfg = MixerConfig("dk_pool", batch=P, seqlen=1, d_inner=C, dt_rank=R, io_dtype="bf16", seed=334,
                       with_state=True)
    w = make_weights(pcfg, DEV)
    st = make_state(pcfg, DEV)
    a = make_activations(pcfg.replace(batch=B), DEV)
    x, z = a["x"][:, 0].contiguous(), a["z"][:, 0].contiguous()
    m = jm.Mixer(w, R, pcfg.d_state, pcfg.d_conv, pcfg.norm_eps)
    conv_pool, ssm_pool = st["conv_state"].clone(), st["ssm_state"].clone()
    sl = torch.tensor(slots, dtype=torch.int32, device=DEV)
    out = m.decode_step_slots(x, z, conv_pool, ssm_pool, sl, single_kernel=True)
    torch.cuda.synchronize()
    ro, rc, rh = oracle.mixer_decode_step_slots(to_f64(x), to_f64(z), weights_f64(w), R, pcfg.d_state,
                                                to_f64(st["conv_state"]), to_f64(st["ssm_state"]), slots,
                                                pcfg.norm_eps)
    assert_close("out", out, ro, "bf16")
    touched = sorted(s for s in slots if 0 <= s < P)
    rest = [r for r in range(P) if r not in touched]
    idx = torch.as_tensor(touched, device=DEV)
    assert_close("ssm pool (touched rows)", ssm_pool[idx], rh[touched], "bf16")
    assert_bitwise("conv pool (touched rows)", conv_pool[idx], torch.from_numpy(rc[touched]).to(pcfg.torch_dtype))
    r_ = torch.as_tensor(rest, device=DEV)
    assert torch.equal(conv_pool[r_], st["conv_state"][r_]) and torch.equal(ssm_pool[r_], st["ssm_state"][r_])


def test_single_kernel_step_deterministic_over_a_poisoned_workspace():
    # the grid barriers' flags live in the workspace: whatever it holds (here all bits set) must not let a
    # workgroup pass early, and two runs must agree bit for bit
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig("dk_poison", batch=96, seqlen=1, d_inner=2048, dt_rank=128, io_dtype="bf16", seed=335,
                      with_state=True)
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    x, z = a["x"][:, 0], a["z"][:, 0]
    ws = m.workspace(jm.decode_workspace_size(m.dims(cfg.batch, 1)))
    runs = []
    for _ in range(2):
        ws.fill_(0xFF)
        runs.append(m.decode_step(x, z, st["conv_state"], st["ssm_state"], single_kernel=True))
        torch.cuda.synchronize()
    for i, name in enumerate(("out", "conv_state", "ssm_state")):
        assert torch.isfinite(runs[0][i].float()).all(), name
        assert torch.equal(runs[0][i], runs[1][i]), name
    ro, rc, rh = oracle.mixer_decode_step(to_f64(x), to_f64(z), weights_f64(w), cfg.dt_rank, cfg.d_state,
                                          to_f64(st["conv_state"]), to_f64(st["ssm_state"]), cfg.norm_eps)
    assert_close("out", runs[1][0], ro, "bf16")
