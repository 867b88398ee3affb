"""Host-side bookkeeping of bench.py (no GPU): the algorithmic byte counts per stage and how the stage times
are grouped, which the bench's GB/s, HBM fractions and roofline line are computed from."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_fused_conv_x_proj_bytes_drop_only_the_xc_read():
    # conv + x_proj as one kernel moves x in, xc out, the partial sums out and the weights once: exactly the two
    # separate stages' bytes without x_proj's read of xc
    B, L, C, N, R, esize = 1, 262144, 8192, 16, 256, 2
    alg = bench.algorithmic_bytes(B, L, C, N, R, esize)
    assert alg["conv_silu_x_proj"] == alg["conv_silu"] + alg["x_proj"] - B * L * C * esize
    # per token at d_inner 8192, bf16: conv x 2C + xc 2C, x_proj xc 2C + dbc 4 (R + 2N), scan xc/delta/z/out 8C
    T = B * L
    assert (alg["conv_silu"] - C * 5 * esize) // T == 4 * C
    assert (alg["x_proj"] - (R + 2 * N) * C * esize) // T == 2 * C + 4 * (R + 2 * N)


def test_stage_groups_cover_every_stage_once():
    stage_ms = {"conv_silu": 0.005, "x_proj": 2.5, "norm": 0.13, "dt_proj": 1.4, "scan_local": 4.6,
                "scan_carry": 0.02, "scan_full": 6.3}
    total = sum(stage_ms.values())
    for fused in (False, True):
        g = bench.stage_groups(stage_ms, fused)
        assert abs(sum(g.values()) - total) < 1e-12
        assert ("conv_silu_x_proj" in g) == fused and ("x_proj" in g) != fused
        # every group has algorithmic bytes, so the mixer's GB/s sums each byte once
        alg = bench.algorithmic_bytes(1, 4096, 8192, 16, 256, 2)
        assert all(k in alg for k in g)
