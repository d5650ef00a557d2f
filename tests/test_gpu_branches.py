"""GPU parity of the read-branch masks (LoLA notes §4.8, Table 12: queries
read only some memories, every update runs as before): the library through
its C ABI against the float64 oracle with the same mask, call by call with
the oracle resynchronised from the exported state.  Tolerances as in the
other parity tests: 2e-3 per output row for bf16 inputs, 1e-5 for fp32."""

import numpy as np
import pytest
import torch

from oracle import lola as O
from sparse_kv_caching_amd.workloads import WORKLOADS, decode_inputs, make_inputs, to_f64

from lola_harness import dev, gpu_state, make_layer, row_rel_err

pytestmark = pytest.mark.gpu


def _tol(wl):
    return 1e-5 if wl.dtype == "f32" else 2e-3


def _masked_prefill(wl, branches, calls):
    print("masked prefill", branches, wl, flush=True)
    inp = make_inputs(wl)
    qf, kf, vf, Wf = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("W")
    layer = make_layer(wl, inp.W)
    layer.set_read_branches(branches)
    st = O.new_state(wl.units, wl.d, wl.D, wl.eta, wl.lam)
    worst, t0 = 0.0, 0
    for tc in calls:
        t1 = min(wl.T, t0 + tc)
        sl = slice(t0, t1)
        yg = layer.prefill(dev(wl, inp.q[:, :, sl]), dev(wl, inp.k[:, :, sl]),
                           dev(wl, inp.v[:, :, sl]), wl.C).cpu().numpy().astype(np.float64)
        yo = O.prefill(st, qf[:, :, sl], kf[:, :, sl], vf[:, :, sl], Wf, wl.C, branches=branches)
        e = float(row_rel_err(yg, yo).max())
        worst = max(worst, e)
        assert e <= _tol(wl), (branches, t0, t1, e)
        st = gpu_state(layer, wl)
        t0 = t1
    final = layer.export()
    torch.cuda.synchronize()
    layer.free()
    print("max row error", worst, flush=True)
    return final


@pytest.mark.parametrize("branches", [4, 5, 6])
def test_masked_prefill_bf16_gqa(branches):
    """bf16, GQA 4:1, two sequences, ragged last chunk, several key tiles of
    cache and window: window only, state + window, cache + window."""
    wl = WORKLOADS["llama8b_4k"].scaled(B=2, Hq=8, Hkv=2, T=424, eta=64, lam=96, C=64)
    _masked_prefill(wl, branches, [64] * 7)


def test_masked_prefill_fp32():
    """fp32 (tolerance 1e-5), d = 64, cache hidden and state hidden."""
    wl = WORKLOADS["tiny_fp32"].scaled(T=256, eta=32, lam=48, C=32, planted=0)
    _masked_prefill(wl, 5, [96, 64, 96])
    _masked_prefill(wl, 6, [96, 64, 96])


def test_masks_leave_the_state_bitwise_unchanged():
    """Hiding memories from the read changes no update: H, s, the cache and
    the window after a masked prefill equal the unmasked run bit for bit."""
    wl = WORKLOADS["llama8b_4k"].scaled(B=1, Hq=4, Hkv=1, T=320, eta=64, lam=64, C=64)
    ref = _masked_prefill(wl, 7, [320])
    for br in (4, 6):
        got = _masked_prefill(wl, br, [320])
        for key in ("H", "s", "cache_pos", "cache_k", "win_k", "win_v"):
            assert torch.equal(got[key], ref[key]), (br, key)


@pytest.mark.parametrize("branches,eta,lam", [(4, 16, 24), (5, 16, 24), (6, 16, 24), (6, 96, 64),
                                               (4, 16, 64), (5, 16, 64), (5, 96, 64)])
def test_masked_decode(branches, eta, lam):
    """Decode with masks, through the one-chunk kernel and (lam + eta > 128)
    the chunked one; outputs per step against the oracle with the same mask.
    With lam >= 32 and the cache hidden, a wave's 32 keys can all be hidden
    (no visible key in its softmax)."""
    wl = WORKLOADS["decode_b64"].scaled(B=2, Hq=8, Hkv=2, T=192, eta=eta, lam=lam, C=32)
    print("masked decode", branches, wl, flush=True)
    inp = make_inputs(wl)
    layer = make_layer(wl, inp.W)
    layer.prefill(dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v), wl.C)
    layer.set_read_branches(branches)
    st = gpu_state(layer, wl)
    Wf = inp.f64("W")
    for step in range(24):
        q, k, v = decode_inputs(wl, step)
        yg = layer.decode(dev(wl, q), dev(wl, k), dev(wl, v)).cpu().numpy().astype(np.float64)
        yo = O.decode_step(st, to_f64(wl, q), to_f64(wl, k), to_f64(wl, v), Wf, branches=branches)
        assert row_rel_err(yg, yo).max() <= _tol(wl), step
        st = gpu_state(layer, wl)
    layer.free()


def test_invalid_masks_are_rejected():
    from sparse_kv_caching_amd.lola import LolaError, LOLA_ERR_INVALID_ARG
    wl = WORKLOADS["llama8b_4k"].scaled(B=1, Hq=4, Hkv=1, T=64, eta=32, lam=32, C=64)
    inp = make_inputs(wl)
    layer = make_layer(wl, inp.W)
    for bad in (0, 1, 2, 3, 8, 12, -1):
        with pytest.raises(LolaError) as ei:
            layer.set_read_branches(bad)
        assert ei.value.code == LOLA_ERR_INVALID_ARG
    layer.set_read_branches(4)
    layer.set_read_branches(7)
    layer.free()
