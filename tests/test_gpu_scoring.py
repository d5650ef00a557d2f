"""GPU parity of the alternative cache scoring rules (LoLA notes §4.5,
Table 4; lola_set_scoring): each rule's accumulated scores and cache
membership against the float64 oracle with the same rule, chunk by chunk
over two prefill calls (the window's running scores cross the call
boundary), with the outputs, window, cache, H per column and s per element
as in the other parity tests.  The scores are fp32 sums over the queries
that see a key through the window; compared to 1e-4 relative."""

import numpy as np
import pytest
import torch

from oracle import lola as O
from sparse_kv_caching_amd.lola import (LOLA_ERR_INVALID_ARG, LOLA_ERR_STATE, LOLA_ERR_UNSUPPORTED,
                                        LolaError)
from sparse_kv_caching_amd.workloads import WORKLOADS, decode_inputs, make_inputs, to_f64

from lola_harness import dev, gpu_state, make_layer, row_rel_err, slice_tokens
from test_gpu_parity import _tol, check_state, follow_call, new_stats

pytestmark = pytest.mark.gpu

RULES = {1: O.SCORE_KERNEL_SQ, 2: O.SCORE_KERNEL_ABS, 3: O.SCORE_KERNEL_RATIO,
         4: O.SCORE_LOCAL_ATTN}


@pytest.mark.parametrize("code", sorted(RULES))
@pytest.mark.parametrize("base,kw", [
    ("llama8b_4k", dict(B=2, Hq=8, Hkv=2, T=576, eta=64, lam=96, C=64)),
    ("tiny_fp32", dict(B=1, Hq=2, Hkv=1, d=128, T=320, eta=32, lam=48, C=32, planted=0)),
])
def test_scoring_rule_parity(code, base, kw):
    wl = WORKLOADS[base].scaled(**kw)
    rule = RULES[code]
    print("scoring", rule, wl, flush=True)
    inp = make_inputs(wl)
    qf, kf, vf, Wf = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("W")
    layer = make_layer(wl, inp.W)
    layer.set_scoring(code)
    st = O.new_state(wl.units, wl.d, wl.D, wl.eta, wl.lam, rule=rule)
    stats = new_stats()
    tol = _tol(wl)
    cut = (wl.T // 2) // wl.C * wl.C + wl.C // 2          # the second call starts mid-chunk
    for t0, t1 in ((0, cut), (cut, wl.T)):
        q = dev(wl, slice_tokens(inp.q, t0, t1))
        k = dev(wl, slice_tokens(inp.k, t0, t1))
        v = dev(wl, slice_tokens(inp.v, t0, t1))
        yg, snap, keys = layer.prefill_debug(q, k, v, wl.C)
        yg = yg.cpu().numpy().astype(np.float64)
        gst = gpu_state(layer, wl)
        sl = slice(t0, t1)
        yo = follow_call(st, wl, qf[:, :, sl], kf[:, :, sl], vf[:, :, sl], Wf, wl.C,
                         snap.cpu().numpy(), keys.cpu().numpy(),
                         [set(g.tolist()) for g in gst.g_pos], stats, score_tol=1e-4)
        e = float(row_rel_err(yg, yo).max())
        stats["y_max"] = max(stats["y_max"], e)
        assert e <= tol, e
        check_state(gst, st, tol, stats)
    print("PARITY scoring", rule, wl.name, stats, flush=True)
    assert stats["scored"] > 0
    layer.free()


def test_scoring_rule_rules():
    wl = WORKLOADS["llama8b_4k"].scaled(B=1, Hq=4, Hkv=1, T=128, eta=32, lam=32, C=64)
    inp = make_inputs(wl)
    L = make_layer(wl, inp.W)
    with pytest.raises(LolaError) as ei:
        L.set_scoring(7)
    assert ei.value.code == LOLA_ERR_INVALID_ARG
    L.set_scoring(4)
    q, k, v = dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v)
    with pytest.raises(LolaError) as ei:
        L.prefill(q, k, v, 1)
    assert ei.value.code == LOLA_ERR_UNSUPPORTED
    L.prefill(q, k, v, 64)
    with pytest.raises(LolaError) as ei:
        L.set_scoring(0)
    assert ei.value.code == LOLA_ERR_STATE
    qd, kd, vd = decode_inputs(wl, 0)
    with pytest.raises(LolaError) as ei:
        L.decode(dev(wl, qd), dev(wl, kd), dev(wl, vd))
    assert ei.value.code == LOLA_ERR_UNSUPPORTED
    snap = L.export()
    with pytest.raises(LolaError) as ei:
        L.import_(snap)
    assert ei.value.code == LOLA_ERR_UNSUPPORTED
    # the rule is kept across reset: the same run gives the same cache
    L.reset()
    L.prefill(q, k, v, 64)
    again = L.export()
    assert torch.equal(again["cache_pos"], snap["cache_pos"])
    L.reset()
    L.set_scoring(0)
    L.prefill(q, k, v, 64)
    L.check()
    L.free()
