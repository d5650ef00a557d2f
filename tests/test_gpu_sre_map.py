"""GPU parity of the SRE diagnostics (LoLA notes §4.4, Fig. 3; Eq. (26)):
lola_prefill_sre_map against the float64 oracle's sre_map on the same
inputs.  Fold chunks must be identical; each map entry is compared relative
to SRE + ||v_p||^2 (the scale of the terms whose difference SRE measures):
1e-3 for bf16 inputs (the chunk snapshots hold H_j as 16-bit hi/lo planes,
phi likewise, fp32 sums), 1e-5 for fp32 inputs (fp16 hi/lo planes)."""

import numpy as np
import pytest
import torch

from oracle import lola as O
from sparse_kv_caching_amd.workloads import WORKLOADS, make_inputs

from lola_harness import dev, make_layer, row_rel_err

pytestmark = pytest.mark.gpu


def _check(wl, tol):
    print("sre map", wl, flush=True)
    inp = make_inputs(wl)
    layer = make_layer(wl, inp.W)
    y, m, fold = layer.prefill_sre_map(dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v), wl.C)
    torch.cuda.synchronize()
    m, fold = m.cpu().numpy().astype(np.float64), fold.cpu().numpy()
    st = O.new_state(wl.units, wl.d, wl.D, wl.eta, wl.lam)
    mo, fo = O.sre_map(st, inp.f64("k"), inp.f64("v"), inp.f64("W"), wl.C)
    np.testing.assert_array_equal(fold, fo)
    assert (fo >= 0).sum() > 0
    v = inp.f64("v").reshape(wl.units, wl.T, wl.d)
    scale = mo + (v ** 2).sum(-1)[:, None, :]
    err = np.abs(m - mo) / scale
    print("max relative map error", err.max(), flush=True)
    assert err.max() <= tol
    assert np.all(m[mo == 0] == 0)
    # the outputs of the call are those of lola_prefill_chunk
    st2 = O.new_state(wl.units, wl.d, wl.D, wl.eta, wl.lam)
    yo = O.prefill(st2, inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("W"), wl.C)
    assert row_rel_err(y.cpu().numpy().astype(np.float64), yo).max() <= (2e-3 if wl.dtype == "bf16" else 1e-5)
    layer.free()


@pytest.mark.parametrize("eta,lam", [(64, 64), (32, 0)])
def test_sre_map_bf16(eta, lam):
    wl = WORKLOADS["llama8b_4k"].scaled(B=1, Hq=4, Hkv=1, T=448, eta=eta, lam=lam, C=64)
    _check(wl, 1e-3)


def test_sre_map_fp32():
    wl = WORKLOADS["tiny_fp32"].scaled(T=320, eta=32, lam=32, C=32, planted=0)
    _check(wl, 1e-5)
