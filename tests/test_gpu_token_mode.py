"""GPU parity of the literal token mode (read after update, LoLA notes
§2.4-§2.5): decode and C = 1 prefill through the C ABI against the float64
oracle with order="after", step by step with the oracle resynchronised from
the exported state.  Tolerances: 2e-3 per output row for bf16 inputs, 1e-5
for fp32; H and s as in the other parity tests."""

import numpy as np
import pytest
import torch

from oracle import lola as O
from sparse_kv_caching_amd.workloads import WORKLOADS, decode_inputs, make_inputs, to_f64

from lola_harness import dev, gpu_state, make_layer, membership, rel_fro, row_rel_err

pytestmark = pytest.mark.gpu


def _tol(wl):
    return 1e-5 if wl.dtype == "f32" else 2e-3


def _token_mode_decode(wl, steps, branches=7):
    print("token-mode decode", branches, wl, flush=True)
    from sparse_kv_caching_amd.lola import READ_AFTER_UPDATE
    inp = make_inputs(wl)
    layer = make_layer(wl, inp.W)
    layer.prefill(dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v), wl.C)
    layer.set_read_order(READ_AFTER_UPDATE)
    layer.set_read_branches(branches)
    st = gpu_state(layer, wl)
    Wf = inp.f64("W")
    tol = _tol(wl)
    for step in range(steps):
        q, k, v = decode_inputs(wl, step)
        yg = layer.decode(dev(wl, q), dev(wl, k), dev(wl, v)).cpu().numpy().astype(np.float64)
        logs = []
        yo = O.decode_step(st, to_f64(wl, q), to_f64(wl, k), to_f64(wl, v), Wf, logs=logs,
                           branches=branches, order="after")
        gst = gpu_state(layer, wl)
        ex, al, bad, msgs = membership(logs[0], [set(g.tolist()) for g in gst.g_pos], wl.lam)
        assert bad == 0, (step, msgs[:3])
        if al == 0:     # (a near-tie flip changes what the query reads)
            assert row_rel_err(yg, yo).max() <= tol, step
        assert rel_fro(gst.H, st.H) <= tol and rel_fro(gst.s, st.s) <= tol, step
        np.testing.assert_array_equal(gst.win_k, st.win_k)
        st = gst
    layer.free()


@pytest.mark.parametrize("name,eta,lam,T", [
    ("decode_b64", 16, 24, 96),      # one key chunk
    ("decode_b64", 96, 64, 192),     # lam + eta > 128: the chunked kernel
    ("decode_b64", 0, 24, 64),       # eta = 0: empty window after the update
    ("decode_b64", 16, 0, 64),       # lam = 0: the leaving pair is in H before the read
    ("decode_b64", 64, 64, 32),      # window and cache still filling
    ("tiny_fp32", 100, 40, 160),     # fp32, d = 64, chunked
])
def test_token_mode_decode(name, eta, lam, T):
    base = WORKLOADS[name]
    kw = dict(B=2, T=T, eta=eta, lam=lam, C=32)
    if name == "decode_b64":
        kw.update(Hq=8, Hkv=2)
    else:
        kw.update(planted=0)
    _token_mode_decode(base.scaled(**kw), 32)


@pytest.mark.parametrize("branches", [5, 6])
def test_token_mode_decode_with_masks(branches):
    wl = WORKLOADS["decode_b64"].scaled(B=2, Hq=8, Hkv=2, T=96, eta=16, lam=24, C=32)
    _token_mode_decode(wl, 24, branches)


def test_token_mode_prefill_c1_equals_decode_and_oracle():
    """C = 1 prefill in token mode is the decode loop (bitwise) and matches
    the oracle's read-after-update outputs (fp32, 1e-5)."""
    from sparse_kv_caching_amd.lola import READ_AFTER_UPDATE
    wl = WORKLOADS["tiny_fp32"].scaled(T=120, eta=16, lam=16, C=32, planted=0)
    inp = make_inputs(wl)
    a, b = make_layer(wl, inp.W), make_layer(wl, inp.W)
    a.set_read_order(READ_AFTER_UPDATE)
    b.set_read_order(READ_AFTER_UPDATE)
    q, k, v = dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v)
    ya = a.prefill(q, k, v, 1)
    yb = torch.stack([b.decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                               v[:, :, t].contiguous()) for t in range(wl.T)], dim=2)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)
    st = O.new_state(wl.units, wl.d, wl.D, wl.eta, wl.lam)
    yo = O.prefill(st, inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("W"), 1, order="after")
    assert row_rel_err(ya.cpu().numpy().astype(np.float64), yo).max() <= 1e-5
    a.free()
    b.free()


def test_token_mode_errors():
    from sparse_kv_caching_amd.lola import (LolaError, LOLA_ERR_INVALID_ARG, LOLA_ERR_UNSUPPORTED,
                                            READ_AFTER_UPDATE, READ_BEFORE_UPDATE)
    wl = WORKLOADS["llama8b_4k"].scaled(B=1, Hq=4, Hkv=1, T=64, eta=32, lam=32, C=64)
    inp = make_inputs(wl)
    layer = make_layer(wl, inp.W)
    for bad in (-1, 2, 7):
        with pytest.raises(LolaError) as ei:
            layer.set_read_order(bad)
        assert ei.value.code == LOLA_ERR_INVALID_ARG
    layer.set_read_order(READ_AFTER_UPDATE)
    q, k, v = dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v)
    with pytest.raises(LolaError) as ei:
        layer.prefill(q, k, v, 64)                 # chunked prefill reads before the update
    assert ei.value.code == LOLA_ERR_UNSUPPORTED
    assert layer.n == 0
    layer.set_read_order(READ_BEFORE_UPDATE)
    layer.free()
    # eta = 0, lam = 0: after the update only the state can be read
    wl0 = wl.scaled(eta=0, lam=0)
    L0 = make_layer(wl0, inp.W)
    L0.set_read_order(READ_AFTER_UPDATE)
    L0.set_read_branches(6)
    q1, k1, v1 = q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous()
    with pytest.raises(LolaError) as ei:
        L0.decode(q1, k1, v1)
    assert ei.value.code == LOLA_ERR_INVALID_ARG
    assert L0.n == 0
    L0.set_read_branches(7)
    L0.decode(q1, k1, v1)
    assert L0.n == 1
    L0.free()
