"""Failure handling through the C ABI, forced from the host so that every
kernel exits normally:

* the chain's exchange gives up (a debug step at which every workgroup
  declares its partner lost, or a spin limit of one poll): the chain sets its
  device flag and ends, the attention and write-back kernels of the call
  return without touching anything, lola_state_check reports STATE, and reset
  or import recovers a state that then computes exactly what a fresh one does;
* imports that break the state's composition (LoLA notes §2.7: window, cache,
  H and s) are rejected and leave the state as it was;
* decode of sequences at different positions with window + cache > 128 keys
  is refused (UNSUPPORTED) before any launch.

Also the numerical edge of the running maximum: logits far below zero with
no linear term in the normaliser (an empty state, or the state hidden from
the read) must not underflow every weight (LoLA notes §2.5, Eq. (14))."""

import numpy as np
import pytest
import torch

from oracle import lola as O
from sparse_kv_caching_amd.lola import (DEBUG_CHAIN_FAIL_AT, DEBUG_SPIN_LIMIT, LOLA_ERR_INVALID_ARG,
                                        LOLA_ERR_STATE, LOLA_ERR_UNSUPPORTED, LolaError)
from sparse_kv_caching_amd.workloads import WORKLOADS, bf16_bits, decode_inputs, make_inputs, to_f64

from lola_harness import dev, gpu_state, make_layer, row_rel_err

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(B=1, Hq=8, Hkv=2, T=512, eta=64, lam=64, C=64)
    base.update(kw)
    return WORKLOADS["llama8b_4k"].scaled(**base)


def _expect(code, fn, *a):
    with pytest.raises(LolaError) as ei:
        fn(*a)
    assert ei.value.code == code, ei.value
    return ei.value


def _reference(wl, inp, parts):
    """Outputs and final export of an untouched state over the same calls."""
    L = make_layer(wl, inp.W)
    ys = [L.prefill(dev(wl, inp.q[:, :, a:b]), dev(wl, inp.k[:, :, a:b]), dev(wl, inp.v[:, :, a:b]),
                    wl.C).clone() for a, b in parts]
    fin = L.export()
    L.free()
    return ys, fin


@pytest.mark.parametrize("B,Hkv", [(1, 2), (33, 4)])   # 8 cooperating workgroups per unit; 1
def test_chain_give_up_and_recovery(B, Hkv):
    wl = _wl(B=B, Hkv=Hkv, Hq=4 * Hkv, T=384)
    print("give-up", wl, flush=True)
    inp = make_inputs(wl)
    parts = [(0, 192), (192, 384)]
    ys, fin = _reference(wl, inp, parts)
    L = make_layer(wl, inp.W)
    L.prefill(dev(wl, inp.q[:, :, :192]), dev(wl, inp.k[:, :, :192]), dev(wl, inp.v[:, :, :192]),
              wl.C)
    snap = L.export()
    # the second call scores at every chunk: give up at its second exchange
    L.debug_set(DEBUG_CHAIN_FAIL_AT, 1)
    L.prefill(dev(wl, inp.q[:, :, 192:]), dev(wl, inp.k[:, :, 192:]), dev(wl, inp.v[:, :, 192:]),
              wl.C)
    e = _expect(LOLA_ERR_STATE, L.check)
    assert "exchange" in str(e)
    _expect(LOLA_ERR_STATE, L.export)          # the binding checks first
    # poisoned: prefill and decode refuse until import or reset
    _expect(LOLA_ERR_STATE, L.prefill, dev(wl, inp.q[:, :, :64]), dev(wl, inp.k[:, :, :64]),
            dev(wl, inp.v[:, :, :64]), wl.C)
    # import clears the poison and the device flag
    L.debug_set(DEBUG_CHAIN_FAIL_AT, -1)
    L.import_(snap)
    L.check()
    y2 = L.prefill(dev(wl, inp.q[:, :, 192:]), dev(wl, inp.k[:, :, 192:]),
                   dev(wl, inp.v[:, :, 192:]), wl.C)
    assert torch.equal(y2, ys[1])
    got = L.export()
    for key in ("H", "s", "cache_pos", "cache_k", "win_k"):
        assert torch.equal(got[key], fin[key]), key
    # reset clears it too (the whole sequence: its first scored chunk gives up)
    L.debug_set(DEBUG_CHAIN_FAIL_AT, 0)
    L.reset()
    L.prefill(dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v), wl.C)
    _expect(LOLA_ERR_STATE, L.check)
    L.debug_set(DEBUG_CHAIN_FAIL_AT, -1)
    L.reset()
    L.check()
    y0 = L.prefill(dev(wl, inp.q[:, :, :192]), dev(wl, inp.k[:, :, :192]),
                   dev(wl, inp.v[:, :, :192]), wl.C)
    assert torch.equal(y0, ys[0])
    L.free()


def test_chain_tiny_spin_limit_ends_normally():
    """A spin limit of one poll: partners that are merely late count as
    lost.  Whether or not that happens, every kernel ends, and the state is
    either correct or reported and recoverable."""
    wl = _wl()
    inp = make_inputs(wl)
    ys, fin = _reference(wl, inp, [(0, wl.T)])
    L = make_layer(wl, inp.W)
    L.debug_set(DEBUG_SPIN_LIMIT, 1)
    q, k, v = dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v)
    outcomes = set()
    for _ in range(3):
        L.reset()
        y = L.prefill(q, k, v, wl.C)
        try:
            L.check()
            assert torch.equal(y, ys[0])
            outcomes.add("ok")
        except LolaError as err:
            assert err.code == LOLA_ERR_STATE
            outcomes.add("gave up")
    print("spin limit 1:", outcomes, flush=True)
    L.debug_set(DEBUG_SPIN_LIMIT, 0)
    L.reset()
    assert torch.equal(L.prefill(q, k, v, wl.C), ys[0])
    L.check()
    _expect(LOLA_ERR_INVALID_ARG, L.debug_set, 7, 1)
    _expect(LOLA_ERR_INVALID_ARG, L.debug_set, DEBUG_SPIN_LIMIT, -3)
    L.free()


def test_import_rejects_broken_states():
    wl = _wl(T=320)
    inp = make_inputs(wl)
    L = make_layer(wl, inp.W)
    L.prefill(dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v), wl.C)
    good = L.export()
    gs = min(wl.lam, wl.T - wl.eta)

    def broken(**changes):
        d = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in good.items()}
        for k, f in changes.items():
            f(d)
        return d

    def swap_pos(d):
        d["cache_pos"][0, [3, 4]] = d["cache_pos"][0, [4, 3]]

    def dup_pos(d):
        d["cache_pos"][1, 5] = d["cache_pos"][1, 4]

    def young_pos(d):
        d["cache_pos"][0, gs - 1] = wl.T - 1          # inside the window

    def pad_pos(d):
        d["cache_pos"][0, gs - 1] = -1                # a cached pair missing

    def s_mass(d):
        d["s"][1, 7] += 0.5                            # 1^T s != 2 N_fold

    def s_neg(d):
        d["s"][0, 0] = -1e-3

    def h_nan(d):
        d["H"][1, 3, 9] = float("nan")

    for name, f in [("swap", swap_pos), ("dup", dup_pos), ("young", young_pos), ("pad", pad_pos),
                    ("mass", s_mass), ("neg", s_neg), ("nan", h_nan)]:
        _expect(LOLA_ERR_STATE, L.import_, broken(x=f))
        after = L.export()                             # unchanged, not poisoned
        for key in ("H", "s", "cache_pos", "win_k"):
            assert torch.equal(after[key], good[key]), (name, key)
    L.import_(good)
    L.free()


def test_ragged_chunked_decode_is_refused():
    """Sequences at different positions with window + cache > 128 keys: the
    decode call returns UNSUPPORTED before any launch.  The batch is built
    from one-sequence views written on the host (no prefill)."""
    eta, lam, d, Hkv = 96, 64, 128, 2
    wl = WORKLOADS["decode_b64"].scaled(B=2, Hq=8, Hkv=Hkv, T=1, eta=eta, lam=lam, C=32)
    inp = make_inputs(wl)
    L = make_layer(wl, inp.W)
    n1 = 5                                             # window only: no cache, H = s = 0
    rng = np.random.default_rng(0)
    win = np.zeros((Hkv, eta, d), np.float32)
    win[:, :n1] = rng.standard_normal((Hkv, n1, d), dtype=np.float32)
    view = dict(n=n1, H=torch.zeros((Hkv, 128, d), device="cuda"),
                s=torch.zeros((Hkv, 128), device="cuda"),
                win_k=dev(wl, bf16_bits(win)), win_v=dev(wl, bf16_bits(win)),
                cache_pos=torch.full((Hkv, lam), -1, dtype=torch.int32, device="cuda"),
                cache_k=torch.zeros((Hkv, lam, d), dtype=torch.bfloat16, device="cuda"),
                cache_v=torch.zeros((Hkv, lam, d), dtype=torch.bfloat16, device="cuda"))
    L.import_sequence(1, view)
    assert L.positions() == [0, n1] and L.n == -1
    q, k, v = decode_inputs(wl, 0)
    e = _expect(LOLA_ERR_UNSUPPORTED, L.decode, dev(wl, q), dev(wl, k), dev(wl, v))
    assert "128" in str(e)
    assert L.positions() == [0, n1]
    # equal positions again: a uniform state
    L.import_sequence(0, view)
    assert L.n == n1 and L.positions() == [n1, n1]
    L.check()
    L.free()


@pytest.mark.parametrize("branches", [7, 6])
def test_far_negative_logits_do_not_underflow(branches):
    """Every key equal to one vector k0 and the queries -20 k0: all logits
    are about -226 (e^-226 underflows fp32).  With an empty state (the first
    chunks) or the state hidden, the normaliser has no linear term; the
    weights are then relative to the largest logit, and y is the mean of the
    visible values, as the float64 oracle gives."""
    wl = _wl(B=1, Hq=4, Hkv=1, T=192, eta=32, lam=32, C=32)
    inp = make_inputs(wl)
    k0 = np.ones(wl.d, np.float32)
    kk = np.broadcast_to(k0, (1, 1, wl.T, wl.d)).copy()
    qq = np.broadcast_to(-20.0 * k0, (1, wl.Hq, wl.T, wl.d)).copy()
    kb, qb = bf16_bits(kk), bf16_bits(qq)
    L = make_layer(wl, inp.W)
    L.set_read_branches(branches)
    y = L.prefill(dev(wl, qb), dev(wl, kb), dev(wl, inp.v), wl.C).cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y))
    st = O.new_state(wl.units, wl.d, wl.D, wl.eta, wl.lam)
    yo = O.prefill(st, to_f64(wl, qb), to_f64(wl, kb), inp.f64("v"), inp.f64("W"), wl.C,
                   branches=branches)
    assert row_rel_err(y, yo).max() <= 2e-3
    # decode from there: the same keys, so every logit stays far below zero
    st = gpu_state(L, wl)
    for step in range(6):
        _, _, vn = decode_inputs(wl, step)
        q1 = bf16_bits(np.broadcast_to(-20.0 * k0, (1, wl.Hq, wl.d)).copy())
        k1 = bf16_bits(np.broadcast_to(k0, (1, 1, wl.d)).copy())
        yd = L.decode(dev(wl, q1), dev(wl, k1), dev(wl, vn)).cpu().numpy().astype(np.float64)
        yod = O.decode_step(st, to_f64(wl, q1), to_f64(wl, k1), to_f64(wl, vn), inp.f64("W"),
                            branches=branches)
        assert np.all(np.isfinite(yd)) and row_rel_err(yd, yod).max() <= 2e-3, step
        st = gpu_state(L, wl)
    L.free()
