"""GPU check that the one-token step agrees bit for bit with a one-token prefill (bf16).

The step runs its own conv kernel (it also shifts the conv state) and the scan's one-token path; a prefill of
one token runs the general conv, the same x_proj, norm and dt_proj, and the scan.  The arithmetic is the same
in the same order, so the output, SSM state and conv state must match bit for bit, over tile counts with
ragged last tiles, channel blocks that are and are not a multiple of 8, dt_ranks below 256, strided x / z,
the zero-order hold, and in place.  Against the fp64 oracle the decode paths are covered by the parity,
serving and ZOH suites.
"""

import pytest
import torch

from jm_inputs import MixerConfig, make_activations, make_state, make_weights
from parity_util import assert_bitwise, log

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
    ("jamba_B256", 256, 8192, 256, False, None),
    ("tiny_ragged", 3, 128, 64, False, None),
    ("ragged_tiles_rank8_zoh", 130, 256, 8, True, None),
    ("blocks_not_mult_of_8", 200, 192, 256, False, None),
    ("one_sequence", 1, 64, 256, False, None),
    ("strided_xz", 77, 512, 128, False, 1040),
    ("many_sequences", 40001, 64, 16, False, None),
    ("jamba_B64_zoh", 64, 8192, 256, True, None),
]


@pytest.mark.parametrize("name,B,C,R,zoh,stride", CASES, ids=[c[0] for c in CASES])
def test_decode_step_bitwise_equals_one_token_prefill(name, B, C, R, zoh, stride):
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig(f"step_{name}", batch=B, seqlen=1, d_inner=C, dt_rank=R, io_dtype="bf16", seed=90)
    log(f"[{cfg.name}] B={B} C={C} R={R} zoh={zoh} stride={stride}")
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV, row_stride=stride)
    st = make_state(cfg, DEV)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps, zoh=zoh)
    po, pc, ph = m.prefill(a["x"], a["z"], st["conv_state"], st["ssm_state"])
    do, dc, dh = m.decode_step(a["x"][:, 0], a["z"][:, 0], st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    assert_bitwise("out", do, po[:, 0])
    assert_bitwise("ssm_state", dh, ph)
    assert_bitwise("conv_state", dc, pc)
    # in place: the same results
    cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
    io, _, _ = m.decode_step(a["x"][:, 0], a["z"][:, 0], cs, hs, in_place=True)
    torch.cuda.synchronize()
    assert_bitwise("out in place", io, do)
    assert_bitwise("ssm_state in place", hs, dh)
    assert_bitwise("conv_state in place", cs, dc)


def test_module_level_calls_match_the_mixer():
    # jm.prefill / jm.decode_step (dims read from the weight shapes) are the Mixer's calls
    import mamba_selective_scan_05_amd as jm
    cfg = MixerConfig("module_calls", batch=2, seqlen=70, d_inner=128, dt_rank=16, io_dtype="bf16", seed=91)
    w = make_weights(cfg, DEV)
    a = make_activations(cfg, DEV)
    st = make_state(cfg, DEV)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    ref = m.prefill(a["x"], a["z"], st["conv_state"], st["ssm_state"])
    got = jm.prefill(a["x"], a["z"], w, st["conv_state"], st["ssm_state"], norm_eps=cfg.norm_eps)
    dref = m.decode_step(a["x"][:, 0], a["z"][:, 0], st["conv_state"], st["ssm_state"])
    dgot = jm.decode_step(a["x"][:, 0], a["z"][:, 0], w, st["conv_state"], st["ssm_state"], norm_eps=cfg.norm_eps)
    torch.cuda.synchronize()
    for name, g, r in zip(("out", "conv_state", "ssm_state") * 2, got + dgot, ref + dref):
        assert_bitwise(name, g, r)
