"""The two prefill schedules (the chain over every chunk, then the read; or
the read of each finished chunk beside the chain in one launch, the chain on
half of the compute units) give bitwise the same outputs, states and
per-chunk records: the chain's results do not depend on its workgroup
count, and the read sees the same snapshots.  Shapes cover the three chain
instances the concurrent schedule can pick (one column slab per workgroup
with candidate groups, two slabs, all slabs), fp32 inputs, a second call on a
non-empty state, and the failure path (a read that cannot wait for its
chunk ends, and the state reports the fault); and the two work splits of
the chain's workgroups.  Parity with the oracle of the
concurrent schedule itself is covered where the automatic choice takes it:
the full-size long-context and Llama-shaped calls in test_gpu_parity and
test_gpu_fullsize follow every chunk against the oracle."""

import numpy as np
import pytest
import torch

from sparse_kv_caching_amd.lola import (DEBUG_CHAIN_SPLIT, DEBUG_CHAIN_WORKGROUPS, DEBUG_OVERLAP,
                                        DEBUG_SPIN_LIMIT, LolaError)
from sparse_kv_caching_amd.workloads import WORKLOADS, make_inputs

from lola_harness import dev, make_layer

pytestmark = pytest.mark.gpu


def _run(wl, overlap, calls=1, split=-1, k=0):
    inp = make_inputs(wl)
    layer = make_layer(wl, inp.W)
    layer.debug_set(DEBUG_OVERLAP, overlap)
    layer.debug_set(DEBUG_CHAIN_SPLIT, split)
    layer.debug_set(DEBUG_CHAIN_WORKGROUPS, k)
    q, k, v = dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v)
    outs, recs = [], []
    T = wl.T
    bounds = [0, T] if calls == 1 else [0, T // 2 // wl.C * wl.C, T]
    for c in range(calls):
        t0, t1 = bounds[c], bounds[c + 1]
        y, sp, ck = layer.prefill_debug(q[:, :, t0:t1].contiguous(), k[:, :, t0:t1].contiguous(),
                                        v[:, :, t0:t1].contiguous(), wl.C)
        outs.append(y.cpu())
        recs.append((sp.cpu(), ck.cpu()))
    st = {n: t.cpu() for n, t in layer.export().items() if isinstance(t, torch.Tensor)}
    layer.free()
    return outs, recs, st


def _same(wl, calls=1, a_args=(0, -1, 0), b_args=(1, -1, 0)):
    """a_args / b_args: (schedule, work split, workgroups per unit; 0 auto)."""
    a = _run(wl, a_args[0], calls, a_args[1], a_args[2])
    b = _run(wl, b_args[0], calls, b_args[1], b_args[2])
    for ya, yb in zip(a[0], b[0]):
        assert torch.equal(ya, yb), "outputs differ between the schedules"
    for (spa, cka), (spb, ckb) in zip(a[1], b[1]):
        assert torch.equal(spa, spb), "per-chunk cache positions differ"
        assert torch.equal(cka, ckb), "per-chunk candidate keys differ"
    for n in a[2]:
        assert torch.equal(a[2][n], b[2][n]), "state %s differs" % n
    y = a[0][-1].numpy()
    assert np.isfinite(y).all()


def test_overlap_slab_per_workgroup():
    """Two units, 32 workgroups each (one slab, eight candidate groups of one
    tile) in both schedules."""
    _same(WORKLOADS["llama8b_4k"].scaled(B=1, Hq=8, Hkv=2, T=1024, eta=128, lam=192, C=64))


def test_overlap_two_slabs():
    """48 units: four workgroups per unit (one slab each) in the sequential
    schedule, two (two slabs each, column split) in the one-launch one."""
    _same(WORKLOADS["llama8b_4k"].scaled(B=6, Hq=16, Hkv=8, T=256, eta=64, lam=64, C=32),
          b_args=(1, 0, 2))


def test_overlap_one_workgroup_per_unit():
    """80 units of head dim 64: two workgroups per unit (one slab each)
    sequentially, one (no exchange) in the one-launch schedule."""
    _same(WORKLOADS["llama8b_4k"].scaled(B=10, Hq=8, Hkv=8, d=64, T=192, eta=32, lam=32, C=32),
          b_args=(1, -1, 1))


def test_overlap_fp32_and_gqa():
    _same(WORKLOADS["tiny_fp32"].scaled(B=2, Hq=4, Hkv=2, d=128, T=300, eta=32, lam=48, C=32))


def test_overlap_second_call():
    """Two calls: the second starts from a full cache and window."""
    _same(WORKLOADS["llama8b_4k"].scaled(B=1, Hq=4, Hkv=1, T=640, eta=64, lam=96, C=64), calls=2)


# The two ways the chain's workgroups of a unit share the work (column slabs
# times candidate groups, or candidate groups holding all of H, whose parts
# meet in LDS and whose phi tiles are staged there) give bitwise the same
# results, in either schedule.
SPLIT_SHAPES = {
    "two_units": WORKLOADS["llama8b_4k"].scaled(B=1, Hq=8, Hkv=2, T=1024, eta=128, lam=192, C=64),
    "k2": WORKLOADS["llama8b_4k"].scaled(B=6, Hq=16, Hkv=8, T=256, eta=64, lam=64, C=32),
    "d64": WORKLOADS["llama8b_4k"].scaled(B=2, Hq=8, Hkv=4, d=64, T=640, eta=64, lam=96, C=64),
    "fp32": WORKLOADS["tiny_fp32"].scaled(B=2, Hq=4, Hkv=2, d=128, T=300, eta=32, lam=48, C=32),
}


@pytest.mark.parametrize("shape", list(SPLIT_SHAPES))
@pytest.mark.parametrize("overlap", [0, 1])
def test_chain_split_same(shape, overlap):
    _same(SPLIT_SHAPES[shape], a_args=(overlap, 0, 0), b_args=(overlap, 1, 0))


def test_chain_workgroup_counts_same():
    """Forced workgroups per unit (candidate groups not a power of two: 12 =
    4 slabs x 3 groups with the column split; 6, 3 (one snapshot writer) and
    2 with the candidate split), bitwise the same as the automatic count."""
    wl = SPLIT_SHAPES["two_units"]
    _same(wl, a_args=(0, -1, 0), b_args=(0, 0, 12))
    _same(wl, a_args=(1, -1, 0), b_args=(1, 1, 6))
    _same(wl, a_args=(1, -1, 0), b_args=(1, 1, 3))
    _same(wl, a_args=(1, -1, 0), b_args=(1, 1, 2))


def test_overlap_read_gives_up():
    """A one-poll limit: the read's workgroups and the chain's exchange give
    up instead of waiting; every workgroup ends and the state reports the
    fault, then a reset recovers it."""
    wl = WORKLOADS["llama8b_4k"].scaled(B=1, Hq=8, Hkv=2, T=512, eta=64, lam=64, C=64)
    inp = make_inputs(wl)
    layer = make_layer(wl, inp.W)
    layer.debug_set(DEBUG_OVERLAP, 1)
    layer.debug_set(DEBUG_SPIN_LIMIT, 1)
    q, k, v = dev(wl, inp.q), dev(wl, inp.k), dev(wl, inp.v)
    layer.prefill(q, k, v, wl.C)
    with pytest.raises(LolaError):
        layer.check()
    layer.debug_set(DEBUG_SPIN_LIMIT, 0)
    layer.reset()
    y = layer.prefill(q, k, v, wl.C)
    layer.check()
    assert torch.isfinite(y).all()
    layer.free()
