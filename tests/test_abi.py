"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects bad arguments on the
host before anything is enqueued (no GPU is touched by these tests)."""

import ctypes
import os
import re

import pytest

import mamba_selective_scan_05_amd as jm
from mamba_selective_scan_05_amd import _lib

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))

FAKE = 0x10000          # 16-byte aligned stand-in pointer; never dereferenced because validation fails first
WS_BIG = 1 << 40


def declared_functions():
    src = "\n".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(jm_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"jm_mixer_prefill", "jm_mixer_decode_step", "jm_mixer_prefill_workspace_size",
            "jm_mixer_decode_workspace_size", "jm_status_string", "jm_layer_prefill", "jm_layer_decode_step",
            "jm_layer_prefill_workspace_size", "jm_layer_decode_workspace_size"} <= set(names)
    L = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def _dims(**kw):
    d = dict(batch=1, seqlen=64, d_inner=64, dt_rank=8, io_dtype=jm.JM_F32)
    d.update(kw)
    return jm.make_dims(**d)


def _weights(**override):
    w = {n: FAKE for n in _lib.WEIGHT_NAMES}
    w.update(override)
    return jm.Weights(*[w[n] for n in _lib.WEIGHT_NAMES])


def _call(dims, weights=None, decode=False, **ptr):
    p = dict(x=FAKE, z=FAKE, out=FAKE, conv_in=FAKE, conv_out=FAKE, h_in=FAKE, h_out=FAKE, ws=FAKE, ws_bytes=WS_BIG)
    p.update(ptr)
    f = jm.call_decode_step if decode else jm.call_prefill
    return f(dims, weights or _weights(), p["x"], p["z"], p["out"], p["conv_in"], p["conv_out"], p["h_in"],
             p["h_out"], p["ws"], p["ws_bytes"], 0)


@pytest.mark.parametrize("decode", [False, True])
def test_validation_rejects_bad_arguments_before_launch(decode):
    E = _lib
    assert _call(_dims(d_state=8), decode=decode) == E.JM_ERR_UNSUPPORTED
    assert _call(_dims(d_conv=3), decode=decode) == E.JM_ERR_UNSUPPORTED
    assert _call(_dims(d_inner=96), decode=decode) == E.JM_ERR_UNSUPPORTED
    assert _call(_dims(dt_rank=12), decode=decode) == E.JM_ERR_UNSUPPORTED
    assert _call(_dims(dt_rank=520), decode=decode) == E.JM_ERR_UNSUPPORTED
    assert _call(_dims(io_dtype=7), decode=decode) == E.JM_ERR_UNSUPPORTED
    assert _call(_dims(batch=0), decode=decode) == E.JM_ERR_INVALID_ARG
    assert _call(_dims(norm_eps=-1.0), decode=decode) == E.JM_ERR_INVALID_ARG
    assert _call(_dims(x_row_stride=32), decode=decode) == E.JM_ERR_INVALID_ARG
    assert _call(_dims(z_row_stride=68), decode=decode) == E.JM_ERR_ALIGNMENT
    assert _call(_dims(), _weights(A_log=None), decode=decode) == E.JM_ERR_INVALID_ARG
    assert _call(_dims(), _weights(D=FAKE + 4), decode=decode) == E.JM_ERR_ALIGNMENT
    assert _call(_dims(), _weights(conv_b=FAKE + 8), decode=decode) == E.JM_ERR_ALIGNMENT
    assert _call(_dims(), x=FAKE + 2, decode=decode) == E.JM_ERR_ALIGNMENT
    assert _call(_dims(), h_out=None, decode=decode) == E.JM_ERR_INVALID_ARG
    assert _call(_dims(), conv_out=None, decode=decode) == E.JM_ERR_INVALID_ARG
    assert _call(_dims(), ws=None, decode=decode) == E.JM_ERR_WORKSPACE
    assert _call(_dims(), ws_bytes=1024, decode=decode) == E.JM_ERR_WORKSPACE
    assert _call(_dims(), x=None, decode=decode) == E.JM_ERR_INVALID_ARG
    assert _call(None, decode=decode) == E.JM_ERR_INVALID_ARG


def test_decode_requires_input_states_prefill_does_not():
    assert _call(_dims(), decode=True, conv_in=None) == _lib.JM_ERR_INVALID_ARG
    assert _call(_dims(), decode=True, h_in=None) == _lib.JM_ERR_INVALID_ARG
    # prefill with NULL states only fails on the (too small) workspace, i.e. the states were accepted
    assert _call(_dims(), conv_in=None, h_in=None, ws_bytes=16) == _lib.JM_ERR_WORKSPACE


def test_prefill_with_empty_sequence_needs_no_activations():
    # seqlen 0: x, z, out may be NULL; the call only fails here on the workspace size
    assert _call(_dims(seqlen=0), x=None, z=None, out=None, ws_bytes=0) == _lib.JM_ERR_WORKSPACE
    assert _call(_dims(seqlen=-1)) == _lib.JM_ERR_INVALID_ARG


def test_workspace_sizes_and_layout():
    assert jm.prefill_workspace_size(_dims(d_state=8)) == 0
    assert jm.decode_workspace_size(_dims(d_inner=100)) == 0
    d = jm.make_dims(1, 4096, 8192, 256, jm.JM_BF16)
    n = jm.prefill_workspace_size(d)
    lay = jm.workspace_layout(d)
    assert lay.total_bytes == n
    T, C, W = 4096, 8192, 288
    assert lay.dbc_splits >= 1 and lay.scan_chunks >= 1
    assert lay.xproj_path == 0                                  # the 4K bf16 prefill: 288-column tiles
    assert jm.workspace_layout(jm.make_dims(256, 1, 8192, 256, jm.JM_BF16)).xproj_path == 1   # decode-sized
    assert jm.workspace_layout(jm.make_dims(1, 4096, 8192, 256, jm.JM_F32)).xproj_path == 2
    # 32768 tokens or more: 256-token tiles with the conv inside x_proj (the 256K prefill, B = 8 x 4096)
    assert jm.workspace_layout(jm.make_dims(1, 262144, 8192, 256, jm.JM_BF16)).xproj_path == 4
    assert jm.workspace_layout(jm.make_dims(8, 4096, 8192, 256, jm.JM_BF16)).xproj_path == 4
    assert n >= T * C * 2 * 2 + lay.dbc_splits * T * W * 4 + T * 256 * 2 + T * 32 * 4
    offs = sorted([lay.xc, lay.dbc, lay.dln, lay.bc, lay.delta])
    assert offs[0] == 0 and all(o % 256 == 0 for o in offs) and offs[-1] < n
    # decode needs a workspace sized for one token per sequence, independent of seqlen, with room for the
    # single-kernel step's wider x_proj partial sums (32 slices of 256 channels)
    dd = jm.make_dims(256, 9999, 8192, 256, jm.JM_BF16)
    d1 = jm.make_dims(256, 1, 8192, 256, jm.JM_BF16)
    assert jm.decode_workspace_size(dd) == jm.decode_workspace_size(d1)
    assert jm.decode_workspace_size(d1) >= jm.prefill_workspace_size(d1)
    assert jm.decode_workspace_size(d1) >= 32 * 256 * 288 * 4 + 256 * 8192 * 2
    with pytest.raises(jm.JMError):
        jm.workspace_layout(_dims(d_state=4))


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert len(jm.status_string(s)) >= 2
    assert jm.status_string(-99) == "unknown status"


def test_layer_validation_before_launch():
    # the whole-layer entry points check everything (their own dims and pointers and the mixer's) before
    # anything is enqueued; with stand-in pointers they must return an error without touching a GPU
    d = jm.make_layer_dims(2, 64, 128, 16, jm.JM_BF16, 64)
    n = jm.layer_workspace_size(d)
    assert n > 0 and jm.layer_workspace_size(d, decode=True) > 0
    assert jm.layer_workspace_size(jm.make_layer_dims(2, 64, 128, 16, jm.JM_BF16, 60)) == 0      # d_model % 8
    assert jm.layer_workspace_size(jm.make_layer_dims(2, 64, 96, 16, jm.JM_BF16, 64)) == 0       # d_inner % 64
    mixer_w = jm.Weights(*([FAKE] * 10))
    lw = jm.LayerWeights(FAKE, FAKE, FAKE, mixer_w)
    call = lambda dims, w, x, out, ci, co, hi, ho, ws, nbytes, decode=False: jm.call_layer(
        dims, w, x, out, ci, co, hi, ho, ws, nbytes, 0, decode)
    assert call(d, lw, FAKE, FAKE, None, None, None, None, FAKE, WS_BIG) == _lib.JM_ERR_INVALID_ARG   # no outputs
    assert call(d, lw, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, n - 1) == _lib.JM_ERR_WORKSPACE
    assert call(d, lw, FAKE + 4, FAKE, None, FAKE, None, FAKE, FAKE, WS_BIG) == _lib.JM_ERR_ALIGNMENT
    assert call(d, jm.LayerWeights(None, FAKE, FAKE, mixer_w), FAKE, FAKE, None, FAKE, None, FAKE, FAKE,
                WS_BIG) == _lib.JM_ERR_INVALID_ARG
    bad_mixer = jm.Weights(*([FAKE] * 9 + [None]))          # D missing: the mixer's own check, still first
    assert call(d, jm.LayerWeights(FAKE, FAKE, FAKE, bad_mixer), FAKE, FAKE, None, FAKE, None, FAKE, FAKE,
                WS_BIG) == _lib.JM_ERR_INVALID_ARG
    assert call(d, lw, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, WS_BIG, decode=True) == _lib.JM_ERR_INVALID_ARG


def test_state_pool_decode_validation_before_launch():
    # the state-pool decode entry points check their slot arguments on the host before anything is enqueued
    d = _dims(batch=3)
    w = _weights()
    call = lambda pool, slots, ws_bytes=WS_BIG: jm.call_decode_step_slots(d, w, FAKE, FAKE, FAKE, FAKE, FAKE, pool,
                                                                          slots, FAKE, ws_bytes, 0)
    assert call(4, None) == _lib.JM_ERR_INVALID_ARG            # no slot vector
    assert call(0, FAKE) == _lib.JM_ERR_INVALID_ARG            # empty pool
    assert call(-3, FAKE) == _lib.JM_ERR_INVALID_ARG
    assert call(4, FAKE + 2) == _lib.JM_ERR_ALIGNMENT          # int32 indices need 4-byte alignment
    assert call(4, FAKE, ws_bytes=16) == _lib.JM_ERR_WORKSPACE  # the slot arguments were accepted
    assert jm.call_decode_step_slots(d, w, FAKE, FAKE, FAKE, None, FAKE, 4, FAKE, FAKE, WS_BIG, 0) == \
        _lib.JM_ERR_INVALID_ARG                                  # no conv state pool
    mixer_w = jm.Weights(*([FAKE] * 10))
    lw = jm.LayerWeights(FAKE, FAKE, FAKE, mixer_w)
    ld = jm.make_layer_dims(3, 1, 128, 16, jm.JM_BF16, 64)
    L = _lib.lib()
    lcall = lambda pool, slots, ws_bytes=WS_BIG: L.jm_layer_decode_step_slots(
        ctypes.byref(ld), ctypes.byref(lw), FAKE, FAKE, FAKE, FAKE, pool, slots, FAKE, ws_bytes, None)
    assert lcall(4, None) == _lib.JM_ERR_INVALID_ARG
    assert lcall(0, FAKE) == _lib.JM_ERR_INVALID_ARG
    assert lcall(4, FAKE + 2) == _lib.JM_ERR_ALIGNMENT
    assert lcall(4, FAKE, ws_bytes=16) == _lib.JM_ERR_WORKSPACE


def test_varlen_prefill_validation_before_launch():
    d = _dims(batch=3, seqlen=64)
    w = _weights()
    call = lambda cu=FAKE, slots=None, pool=0, ws_bytes=WS_BIG, dims=d: jm.call_prefill_varlen(
        dims, w, FAKE, FAKE, FAKE, cu, FAKE, FAKE, FAKE, FAKE, slots, pool, FAKE, ws_bytes, 0)
    assert call(cu=None) == _lib.JM_ERR_INVALID_ARG             # no offsets
    assert call(cu=FAKE + 2) == _lib.JM_ERR_ALIGNMENT           # int32 offsets need 4-byte alignment
    assert call(slots=FAKE, pool=0) == _lib.JM_ERR_INVALID_ARG  # a pool needs rows
    assert call(slots=FAKE + 1, pool=4) == _lib.JM_ERR_ALIGNMENT
    assert call(ws_bytes=16) == _lib.JM_ERR_WORKSPACE           # everything else was accepted
    assert call(slots=FAKE, pool=4, ws_bytes=16) == _lib.JM_ERR_WORKSPACE
    too_long = _dims(batch=3, seqlen=(1 << 21) + 1)
    assert jm.varlen_workspace_size(too_long) == 0
    assert call(dims=too_long) == _lib.JM_ERR_UNSUPPORTED
    # the workspace of a packed batch depends on the total length, not on how it is split
    n1 = jm.varlen_workspace_size(jm.make_dims(1, 4096, 8192, 256, jm.JM_BF16))
    n8 = jm.varlen_workspace_size(jm.make_dims(8, 4096, 8192, 256, jm.JM_BF16))
    assert n1 > 0 and n8 == n1
    # zero tokens: x, z, out may be NULL
    assert jm.call_prefill_varlen(_dims(batch=2, seqlen=0), w, None, None, None, FAKE, None, FAKE, None, FAKE,
                                  None, 0, FAKE, 0, 0) == _lib.JM_ERR_WORKSPACE
    mixer_w = jm.Weights(*([FAKE] * 10))
    lw = jm.LayerWeights(FAKE, FAKE, FAKE, mixer_w)
    ld = jm.make_layer_dims(3, 64, 128, 16, jm.JM_BF16, 64)
    L = _lib.lib()
    assert L.jm_layer_prefill_varlen_workspace_size(ctypes.byref(ld)) > 0
    lcall = lambda cu=FAKE, ws_bytes=WS_BIG: L.jm_layer_prefill_varlen(
        ctypes.byref(ld), ctypes.byref(lw), FAKE, FAKE, cu, None, FAKE, None, FAKE, None, 0, FAKE, ws_bytes, None)
    assert lcall(cu=None) == _lib.JM_ERR_INVALID_ARG
    assert lcall(cu=FAKE + 2) == _lib.JM_ERR_ALIGNMENT
    assert lcall(ws_bytes=16) == _lib.JM_ERR_WORKSPACE


def test_scan_train_validation_before_launch():
    d = jm.scan_dims(2, 64, 128, jm.JM_BF16)
    L = _lib.lib()
    nf, nb = jm.scan_workspace_size(d), jm.scan_workspace_size(d, True)
    assert nf > 0 and nb > 0
    assert jm.scan_workspace_size(jm.scan_dims(2, 64, 96, jm.JM_BF16)) == 0                 # d_inner % 64
    assert jm.scan_workspace_size(jm.scan_dims(2, 64, 128, jm.JM_BF16, d_state=8), True) == 0
    assert jm.scan_workspace_size(jm.scan_dims(2, (1 << 21) + 1, 128, jm.JM_BF16)) == 0
    fwd = lambda dims, ws_bytes=WS_BIG, x=FAKE, h_out=FAKE: L.jm_scan_forward(
        ctypes.byref(dims), x, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, h_out, FAKE, ws_bytes, None)
    assert fwd(d, x=None) == _lib.JM_ERR_INVALID_ARG
    assert fwd(d, h_out=None) == _lib.JM_ERR_INVALID_ARG
    assert fwd(d, x=FAKE + 4) == _lib.JM_ERR_ALIGNMENT
    assert fwd(d, ws_bytes=nf - 1) == _lib.JM_ERR_WORKSPACE
    assert fwd(jm.scan_dims(0, 64, 128, jm.JM_BF16)) == _lib.JM_ERR_INVALID_ARG
    bwd = lambda dims, ws_bytes=WS_BIG, dx=FAKE, dA=FAKE, dout=FAKE, saved=None: L.jm_scan_backward(
        ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, dout, None, saved, dx, FAKE, FAKE, FAKE, dA,
        FAKE, None, FAKE, ws_bytes, None)
    assert bwd(d, dx=None) == _lib.JM_ERR_INVALID_ARG
    assert bwd(d, dA=None) == _lib.JM_ERR_INVALID_ARG
    assert bwd(d, dout=FAKE + 8) == _lib.JM_ERR_ALIGNMENT
    assert bwd(d, saved=FAKE + 4) == _lib.JM_ERR_ALIGNMENT
    assert bwd(d, ws_bytes=nb - 1) == _lib.JM_ERR_WORKSPACE
    # no tokens: the activations may be NULL; only the parameter gradients are required
    e = jm.scan_dims(2, 0, 128, jm.JM_BF16)
    assert L.jm_scan_backward(ctypes.byref(e), None, None, None, None, FAKE, FAKE, None, None, None, None, None,
                              None, None, None, FAKE, FAKE, None, FAKE, 0, None) == _lib.JM_ERR_WORKSPACE
    # the training forward: saved states of B * ceil(L / 32) * N * C floats, required when there are tokens
    assert jm.scan_saved_states_size(d) == 2 * 2 * 16 * 128 * 4
    assert jm.scan_saved_states_size(jm.scan_dims(1, 33, 64, jm.JM_F32)) == 2 * 16 * 64 * 4
    assert jm.scan_saved_states_size(jm.scan_dims(2, 64, 96, jm.JM_BF16)) == 0
    ftr = lambda dims, saved=FAKE, ws_bytes=WS_BIG: L.jm_scan_forward_train(
        ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, saved, FAKE, ws_bytes, None)
    assert ftr(d, saved=None) == _lib.JM_ERR_INVALID_ARG
    assert ftr(d, saved=FAKE + 4) == _lib.JM_ERR_ALIGNMENT
    assert ftr(d, ws_bytes=nf - 1) == _lib.JM_ERR_WORKSPACE
    assert ftr(jm.scan_dims(2, 64, 96, jm.JM_BF16)) == _lib.JM_ERR_UNSUPPORTED


def test_discretization_field():
    assert _call(_dims(discretization=2)) == _lib.JM_ERR_UNSUPPORTED
    d = _dims(discretization=jm.JM_DISC_ZOH)
    assert _call(d, ws_bytes=16) == _lib.JM_ERR_WORKSPACE          # the variant is accepted
    d.reserved = 1
    assert _call(d) == _lib.JM_ERR_INVALID_ARG
    assert ctypes.sizeof(jm.Dims) == 56


def test_batch_limit():
    assert _call(_dims(batch=(1 << 16) + 1)) == _lib.JM_ERR_UNSUPPORTED
    assert _call(_dims(batch=1 << 16), ws_bytes=16) == _lib.JM_ERR_WORKSPACE
    assert jm.scan_workspace_size(jm.scan_dims((1 << 16) + 1, 64, 128, jm.JM_BF16)) == 0


def test_module_level_mixer_reads_dims_from_weight_shapes():
    # host only: the weight dict's shapes give dt_rank, d_state and d_conv; nothing is launched
    from jm_inputs import MixerConfig, make_weights
    cfg = MixerConfig("shapes", batch=1, seqlen=8, d_inner=128, dt_rank=24, io_dtype="bf16", seed=5)
    m = jm.mixer_for(make_weights(cfg), norm_eps=1e-5, zoh=True)
    assert (m.d_inner, m.dt_rank, m.d_state, m.d_conv, m.eps, m.zoh) == (128, 24, 16, 4, 1e-5, True)
    d = m.dims(3, 9)
    assert (d.batch, d.seqlen, d.d_inner, d.dt_rank, d.discretization) == (3, 9, 128, 24, jm.JM_DISC_ZOH)


def test_noalloc_decode_rejects_calls_beyond_its_scratch_before_launch():
    # a decode batch whose workspace exceeds the static scratch: rejected before any HIP call
    limit = jm.noalloc_scratch_limit()
    assert limit == 32 << 20
    small = _dims(batch=256, seqlen=1, d_inner=8192, dt_rank=256, io_dtype=jm.JM_BF16)
    big = _dims(batch=4096, seqlen=1, d_inner=8192, dt_rank=256, io_dtype=jm.JM_BF16)
    assert jm.decode_workspace_size(small) <= limit < jm.decode_workspace_size(big)
    args = [FAKE] * 7 + [0]
    assert jm.call_decode_step_noalloc(big, _weights(), *args) == _lib.JM_ERR_SCRATCH_LIMIT
    assert "32 MiB" in jm.status_string(_lib.JM_ERR_SCRATCH_LIMIT)
    # dims errors come first, as in jm_mixer_decode_step
    assert jm.call_decode_step_noalloc(_dims(d_state=8), _weights(), *args) == _lib.JM_ERR_UNSUPPORTED


def test_single_kernel_decode_checks_before_launch():
    # shapes and devices the single-kernel step does not take are refused with nothing enqueued (no fallback)
    w = _weights()
    args = lambda d, pool=0, slots=None, conv_out=FAKE, h_out=FAKE, ws_bytes=WS_BIG: (
        d, w, FAKE, FAKE, FAKE, FAKE, conv_out, FAKE, h_out, pool, slots, FAKE, ws_bytes, 0)
    f32 = _dims(batch=4, seqlen=1, d_inner=256, dt_rank=32, io_dtype=jm.JM_F32)
    assert jm.call_decode_step_single_kernel(*args(f32)) == _lib.JM_ERR_UNSUPPORTED
    narrow = _dims(batch=4, seqlen=1, d_inner=192, dt_rank=32, io_dtype=jm.JM_BF16)
    assert jm.call_decode_step_single_kernel(*args(narrow)) == _lib.JM_ERR_UNSUPPORTED
    rank8 = _dims(batch=4, seqlen=1, d_inner=256, dt_rank=8, io_dtype=jm.JM_BF16)
    assert jm.call_decode_step_single_kernel(*args(rank8)) == _lib.JM_ERR_UNSUPPORTED
    many = _dims(batch=1025, seqlen=1, d_inner=256, dt_rank=32, io_dtype=jm.JM_BF16)
    assert jm.call_decode_step_single_kernel(*args(many)) == _lib.JM_ERR_UNSUPPORTED
    ok = _dims(batch=4, seqlen=1, d_inner=256, dt_rank=32, io_dtype=jm.JM_BF16)
    # argument errors come first: pools must be updated in place, the workspace must be large enough
    assert jm.call_decode_step_single_kernel(*args(ok, pool=4, slots=FAKE, conv_out=FAKE + 256)) == \
        _lib.JM_ERR_INVALID_ARG
    assert jm.call_decode_step_single_kernel(*args(ok, ws_bytes=16)) == _lib.JM_ERR_WORKSPACE
    assert jm.call_decode_step_single_kernel(*args(_dims(d_state=8))) == _lib.JM_ERR_UNSUPPORTED
