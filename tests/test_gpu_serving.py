"""GPU parity of the serving-style entry points, through the C ABI: decode over pools of per-sequence states
(jm_mixer_decode_step_slots, jm_layer_decode_step_slots) and prefill of packed variable-length batches
(jm_mixer_prefill_varlen, jm_layer_prefill_varlen) against the fp64 oracle.

A serving engine batches whichever sequences are generating and keeps their conv / SSM states in pools;
the step reads and writes row slots[b] in place.  Checked here, over several steps with the pool carried
between them:
  - out and the updated rows against the fp64 oracle run on the gathered states (zeros for an entry
    outside the pool), to the mixer's tolerances; the conv state rows bit for bit (mixer level);
  - the same step through the plain decode entry point on gathered copies of the states gives bitwise the
    same out and states (the two share their kernels);
  - rows no valid slot names, and every row an out-of-range entry would have touched, stay bitwise
    unchanged.
"""

import numpy as np
import pytest
import torch

import oracle
from jm_inputs import MixerConfig, make_activations, make_decode_tokens, make_layer_input, make_layer_weights, \
    make_state, make_weights, to_f64
from parity_util import assert_bitwise, assert_close, log, weights_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mamba_selective_scan_05_amd as jm
    jm.lib()


def _pool_cfg(name, pool, C, R, io, seed, d_model=0):
    # the pool's states come from make_state with batch = pool rows
    return MixerConfig(name, batch=pool, seqlen=1, d_inner=C, dt_rank=R, io_dtype=io, seed=seed, with_state=True,
                       d_model=d_model, decode_steps=3)


def _gather(pool64, slots, P):
    rows = [pool64[s] if 0 <= s < P else np.zeros_like(pool64[0]) for s in slots]
    return np.stack(rows)


def _scatter(pool64, slots, P, rows):
    for i, s in enumerate(slots):
        if 0 <= s < P:
            pool64[s] = rows[i]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_mixer_decode_slots(io):
    import mamba_selective_scan_05_amd as jm
    P, C, R = 7, 256, 16
    slots = [5, 1, -1, 3, 7]          # -1 and 7 (== pool size) are outside the pool
    B = len(slots)
    pcfg = _pool_cfg(f"slots_{io}", P, C, R, io, 41)
    tcfg = pcfg.replace(batch=B)
    w = make_weights(pcfg, DEV)
    st = make_state(pcfg, DEV)
    tok = make_decode_tokens(tcfg, DEV)
    m = jm.Mixer(w, R, pcfg.d_state, pcfg.d_conv, pcfg.norm_eps)
    conv_pool, ssm_pool = st["conv_state"].clone(), st["ssm_state"].clone()
    conv0, ssm0 = conv_pool.clone(), ssm_pool.clone()
    sl = torch.tensor(slots, dtype=torch.int32, device=DEV)
    c64, h64 = to_f64(conv_pool), to_f64(ssm_pool)
    w64 = weights_f64(w)
    log(f"[slots_{io}] pool={P} slots={slots} C={C} R={R} steps={tcfg.decode_steps}")
    for t in range(tcfg.decode_steps):
        x, z = tok["x"][:, t].contiguous(), tok["z"][:, t].contiguous()
        # the plain entry point on gathered copies of the states (zero states for the out-of-range entries)
        idx = torch.tensor([s if 0 <= s < P else 0 for s in slots], device=DEV)
        valid = torch.tensor([0 <= s < P for s in slots], device=DEV)
        gc = torch.where(valid[:, None, None], conv_pool[idx], torch.zeros_like(conv_pool[idx]))
        gh = torch.where(valid[:, None, None], ssm_pool[idx], torch.zeros_like(ssm_pool[idx]))
        ref_out, ref_c, ref_h = m.decode_step(x, z, gc, gh)
        out = m.decode_step_slots(x, z, conv_pool, ssm_pool, sl)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"step {t}: out differs from the plain decode step"
        for i, s in enumerate(slots):
            if 0 <= s < P:
                assert torch.equal(conv_pool[s], ref_c[i]) and torch.equal(ssm_pool[s], ref_h[i]), (t, s)
        ro, rc, rh = oracle.mixer_decode_step(to_f64(x), to_f64(z), w64, R, pcfg.d_state, _gather(c64, slots, P),
                                              _gather(h64, slots, P), pcfg.norm_eps)
        _scatter(c64, slots, P, rc)
        _scatter(h64, slots, P, rh)
        assert_close(f"out[{t}]", out, ro, io)
    assert_close("ssm pool", ssm_pool, h64, io)
    assert_bitwise("conv pool", conv_pool, torch.from_numpy(c64).to(pcfg.torch_dtype))
    for r in (0, 2, 4, 6):            # rows no valid slot names
        assert torch.equal(conv_pool[r], conv0[r]) and torch.equal(ssm_pool[r], ssm0[r]), r


def test_mixer_decode_slots_permuted_full_pool_matches_plain():
    # every row used, in a scrambled order, at a decode-sized batch (the 32-column x_proj groups)
    import mamba_selective_scan_05_amd as jm
    P, C, R = 64, 512, 32
    cfg = _pool_cfg("slots_perm", P, C, R, "bf16", 42)
    w = make_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    tok = make_decode_tokens(cfg, DEV)
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(42))
    sl = perm.to(torch.int32).to(DEV)
    m = jm.Mixer(w, R, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    conv_pool, ssm_pool = st["conv_state"].clone(), st["ssm_state"].clone()
    cs, hs = st["conv_state"][perm.to(DEV)].clone(), st["ssm_state"][perm.to(DEV)].clone()
    log(f"[slots_perm] pool={P} C={C} R={R}")
    for t in range(cfg.decode_steps):
        x, z = tok["x"][:, t].contiguous(), tok["z"][:, t].contiguous()
        o1 = m.decode_step_slots(x, z, conv_pool, ssm_pool, sl)
        o2, _, _ = m.decode_step(x, z, cs, hs, in_place=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), t
    inv = torch.argsort(perm).to(DEV)
    assert torch.equal(conv_pool, cs[inv]) and torch.equal(ssm_pool, hs[inv])


def test_layer_decode_slots():
    import mamba_selective_scan_05_amd as jm
    P, C, R, Dm = 6, 128, 16, 64
    slots = [4, -1, 0, 2]
    B = len(slots)
    pcfg = _pool_cfg("layer_slots", P, C, R, "bf16", 43, d_model=Dm)
    tcfg = pcfg.replace(batch=B)
    w = make_weights(pcfg, DEV)
    lw = make_layer_weights(pcfg, DEV)
    st = make_state(pcfg, DEV)
    xs = make_layer_input(tcfg, DEV, steps=3)
    layer = jm.Layer(lw, w, R, pcfg.d_state, pcfg.d_conv, pcfg.norm_eps, 1e-6)
    conv_pool, ssm_pool = st["conv_state"].clone(), st["ssm_state"].clone()
    conv0, ssm0 = conv_pool.clone(), ssm_pool.clone()
    sl = torch.tensor(slots, dtype=torch.int32, device=DEV)
    c64, h64 = to_f64(conv_pool), to_f64(ssm_pool)
    w64, lw64 = weights_f64(w), weights_f64(lw)
    log(f"[layer_slots] pool={P} slots={slots} C={C} d_model={Dm}")
    for t in range(xs.shape[1]):
        x = xs[:, t].contiguous()
        idx = torch.tensor([s if s >= 0 else 0 for s in slots], device=DEV)
        valid = torch.tensor([s >= 0 for s in slots], device=DEV)
        gc = torch.where(valid[:, None, None], conv_pool[idx], torch.zeros_like(conv_pool[idx]))
        gh = torch.where(valid[:, None, None], ssm_pool[idx], torch.zeros_like(ssm_pool[idx]))
        ref_out, ref_c, ref_h = layer.decode_step(x, gc, gh)
        out = layer.decode_step_slots(x, conv_pool, ssm_pool, sl)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), t
        for i, s in enumerate(slots):
            if s >= 0:
                assert torch.equal(conv_pool[s], ref_c[i]) and torch.equal(ssm_pool[s], ref_h[i]), (t, s)
        ro, rc, rh = oracle.layer_decode_step(to_f64(x), lw64, w64, R, pcfg.d_state, _gather(c64, slots, P),
                                              _gather(h64, slots, P), pcfg.norm_eps, 1e-6)
        _scatter(c64, slots, P, rc)
        _scatter(h64, slots, P, rh)
        assert_close(f"out[{t}]", out, ro, "bf16")
    assert_close("ssm pool", ssm_pool, h64, "bf16")
    assert_close("conv pool", conv_pool, c64, "bf16")
    for r in (1, 3, 5):
        assert torch.equal(conv_pool[r], conv0[r]) and torch.equal(ssm_pool[r], ssm0[r]), r


# ----------------------------------------------------------------------------- packed variable-length prefill

# lengths chosen against the scan's 128-token pieces at d_inner 256 (checked below): sequences that span
# pieces, one that starts exactly at a piece start, sequences starting inside a piece and running past it,
# empty sequences, sequences shorter than the conv window, and a last sequence inside the last piece
VARLEN_LENS = [200, 0, 56, 1, 2, 300, 129, 70, 0]


def _packed(cfg, lens, seed_cfg):
    T = sum(lens)
    a = make_activations(seed_cfg.replace(batch=1, seqlen=T), DEV)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    return a["x"][0].contiguous(), a["z"][0].contiguous(), cu


def _check_varlen(io, with_state, slots=None, pool=None, seed=44, lens=VARLEN_LENS, C=256, R=16, in_place=False):
    import mamba_selective_scan_05_amd as jm
    nseq = len(lens)
    rows = nseq if slots is None else pool
    cfg = MixerConfig(f"varlen_{io}", batch=rows, seqlen=1, d_inner=C, dt_rank=R, io_dtype=io, seed=seed,
                      with_state=True)
    w = make_weights(cfg, DEV)
    x, z, cu = _packed(cfg, lens, cfg)
    T = x.shape[0]
    st = make_state(cfg, DEV) if with_state else {"conv_state": None, "ssm_state": None}
    m = jm.Mixer(w, R, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    lay = jm.workspace_layout(jm.make_dims(1, T, C, R, jm.JM_BF16 if io == "bf16" else jm.JM_F32))
    short = lambda v: v if v is None or len(v) <= 12 else f"{len(v)} entries, first {v[:6]}"
    log(f"[varlen_{io}] lens={short(lens)} T={T} C={C} pieces={lay.scan_chunks} state={with_state} "
        f"slots={short(slots)} in_place={in_place}")
    sl = None if slots is None else torch.tensor(slots, dtype=torch.int32, device=DEV)
    # outputs start as copies of the inputs (or NaN), so rows the call must not touch are checkable
    if with_state:
        cs_in, hs_in = st["conv_state"].clone(), st["ssm_state"].clone()
        co, so = (cs_in, hs_in) if in_place else (cs_in.clone(), hs_in.clone())
    else:
        cs_in = hs_in = None
        co = torch.full((rows, C, 3), float("nan"), dtype=cfg.torch_dtype, device=DEV)
        so = torch.full((rows, C, 16), float("nan"), device=DEV)
    before_c, before_h = co.clone(), so.clone()
    out, co, so = m.prefill_varlen(x, z, cu, cs_in, hs_in, slots=sl, conv_state_out=co, ssm_state_out=so)
    torch.cuda.synchronize()
    c64 = None if not with_state else to_f64(st["conv_state"])
    h64 = None if not with_state else to_f64(st["ssm_state"])
    ro, rc, rh = oracle.mixer_prefill_varlen(to_f64(x), to_f64(z), cu.cpu().numpy(), weights_f64(w), R,
                                             cfg.d_state, cfg.norm_eps, c64, h64, slots)
    assert_close("out", out, ro, io)
    named = sorted({r for r in (range(nseq) if slots is None else slots) if 0 <= r < rows})
    idx = torch.tensor(named, device=DEV, dtype=torch.long)
    assert_close(f"ssm_state[{len(named)} rows]", so[idx], rh[named], io)
    assert_bitwise(f"conv_state[{len(named)} rows]", co[idx], torch.from_numpy(rc[named]).to(cfg.torch_dtype))
    rest = torch.tensor(sorted(set(range(rows)) - set(named)), device=DEV, dtype=torch.long)
    if rest.numel():   # rows no sequence names keep their bytes
        assert torch.equal(co[rest].view(torch.uint8), before_c[rest].view(torch.uint8))
        assert torch.equal(so[rest].view(torch.uint8), before_h[rest].view(torch.uint8))
    return lay


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("with_state", [True, False])
def test_prefill_varlen_small(io, with_state):
    lay = _check_varlen(io, with_state)
    assert lay.scan_chunks == 6     # 758 tokens in pieces of 128: the boundaries above fall as intended


def test_prefill_varlen_pool_in_place():
    # sequences read and write pool rows in place; a padding entry (-1) and an out-of-range entry (9) run
    # from zero states and store nothing; the pool rows no sequence names stay untouched
    slots = [6, 2, -1, 0, 4, 9, 1, 7, 3]
    _check_varlen("bf16", True, slots=slots, pool=9, seed=45, in_place=True)


def test_prefill_varlen_single_piece_and_all_empty():
    import mamba_selective_scan_05_amd as jm
    _check_varlen("bf16", True, lens=[5, 0, 40, 3], seed=46)         # one scan piece, no carries
    # no tokens at all: every sequence is empty and keeps its states
    cfg = MixerConfig("varlen_empty", batch=3, seqlen=1, d_inner=128, dt_rank=16, io_dtype="bf16", seed=47,
                      with_state=True)
    w = make_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    m = jm.Mixer(w, 16)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    x = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    out, co, so = m.prefill_varlen(x, x, cu, st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    assert out.shape == (0, 128)
    assert torch.equal(co, st["conv_state"]) and torch.equal(so, st["ssm_state"])


def test_prefill_varlen_jamba_widths_4k_tokens():
    # Jamba v0.1's widths (d_inner 8192, dt_rank 256) with 4096 packed tokens of mixed lengths, the
    # token count of the 4K prefill workload
    _check_varlen("bf16", True, lens=[1000, 37, 2048, 0, 500, 511], C=8192, R=256, seed=48)


def test_layer_prefill_varlen():
    import mamba_selective_scan_05_amd as jm
    lens = [150, 0, 3, 300, 60]
    C, R, Dm = 128, 16, 64
    nseq, T = len(lens), sum(lens)
    cfg = MixerConfig("layer_varlen", batch=nseq, seqlen=1, d_inner=C, dt_rank=R, io_dtype="bf16", seed=49,
                      with_state=True, d_model=Dm)
    w = make_weights(cfg, DEV)
    lw = make_layer_weights(cfg, DEV)
    st = make_state(cfg, DEV)
    xr = make_layer_input(cfg.replace(batch=1, seqlen=T), DEV)[0].contiguous()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    layer = jm.Layer(lw, w, R, cfg.d_state, cfg.d_conv, cfg.norm_eps, 1e-6)
    log(f"[layer_varlen] lens={lens} C={C} d_model={Dm}")
    out, co, so = layer.prefill_varlen(xr, cu, st["conv_state"], st["ssm_state"])
    torch.cuda.synchronize()
    ro, rc, rh = oracle.layer_prefill_varlen(to_f64(xr), cu.cpu().numpy(), weights_f64(lw), weights_f64(w), R,
                                             cfg.d_state, cfg.norm_eps, 1e-6, to_f64(st["conv_state"]),
                                             to_f64(st["ssm_state"]))
    assert_close("out", out, ro, "bf16")
    assert_close("ssm_state", so, rh, "bf16")
    assert_close("conv_state", co, rc, "bf16")


def test_prefill_varlen_many_tiny_sequences():
    # 1500 sequences of 0..9 tokens (about 30 sequence starts per 128-token scan piece, many inside the conv
    # window of the previous one), in place into a 4000-row pool through scattered slots
    rng = np.random.default_rng(50)
    lens = [int(v) for v in rng.integers(0, 10, 1500)]
    slots = [int(v) for v in rng.choice(4000, 1500, replace=False)]
    _check_varlen("bf16", True, slots=slots, pool=4000, seed=51, lens=lens, C=128, R=16, in_place=True)
