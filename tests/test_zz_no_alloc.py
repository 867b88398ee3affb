"""GPU: the allocation-free decode step (jm_mixer_decode_step_noalloc) against the decode step with a caller
workspace (jm_mixer_decode_step), through the C ABI.  Both run the same kernels on the same inputs, so the
outputs and the updated states must be bitwise equal; two calls in a row, the second on a smaller batch, show
that the shared device scratch carries nothing from one call into the next."""

import pytest
import torch

from jm_inputs import CONFIGS, make_decode_tokens, make_state, make_weights
from parity_util import log

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


def _step_both(cfg, seed_step):
    import mamba_selective_scan_05_amd as jm
    w = make_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    tok = make_decode_tokens(cfg.replace(decode_steps=seed_step + 1), DEV)
    x, z = tok["x"][:, seed_step].contiguous(), tok["z"][:, seed_step].contiguous()
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    dims = m.dims(cfg.batch, 1)
    stream = torch.cuda.current_stream().cuda_stream
    # reference: the entry point with a caller workspace (poisoned: nothing may depend on its contents)
    ws = torch.full((jm.decode_workspace_size(dims),), 0xFF, dtype=torch.uint8, device=DEV)
    outs = {}
    for name in ("workspace", "noalloc"):
        cs, hs = st["conv_state"].clone(), st["ssm_state"].clone()
        out = torch.full((cfg.batch, cfg.d_inner), float("nan"), dtype=cfg.torch_dtype, device=DEV)
        if name == "workspace":
            s = jm.call_decode_step(dims, m.packed, x.data_ptr(), z.data_ptr(), out.data_ptr(), cs.data_ptr(),
                                    cs.data_ptr(), hs.data_ptr(), hs.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        else:
            s = jm.call_decode_step_noalloc(dims, m.packed, x.data_ptr(), z.data_ptr(), out.data_ptr(),
                                            cs.data_ptr(), cs.data_ptr(), hs.data_ptr(), hs.data_ptr(), stream)
        assert s == 0, jm.status_string(s)
        outs[name] = (out, cs, hs)
    torch.cuda.synchronize()
    return outs


def test_noalloc_decode_matches_workspace_decode_twice():
    # B = 256 at Jamba's widths, then a smaller batch (B = 7) at another d_inner, through the same scratch
    for cfg, step in ((CONFIGS[4], 0), (CONFIGS[4].replace(name="noalloc_small", batch=7, d_inner=1024, seed=81), 1)):
        log(f"[{cfg.name}] B={cfg.batch} C={cfg.d_inner}: noalloc vs workspace decode step")
        r = _step_both(cfg, step)
        for i, name in enumerate(("out", "conv_state", "ssm_state")):
            a, b = r["workspace"][i], r["noalloc"][i]
            assert torch.isfinite(a.float()).all(), name
            assert torch.equal(a, b), f"{name}: noalloc differs from the workspace entry point"
