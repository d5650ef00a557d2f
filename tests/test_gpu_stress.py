"""Parity stress inputs (seeded structures of the input module, not of the
pages' workloads), through the C ABI against the float64 oracle:

* clustered keys with values tied to the cluster, so that the prediction
  H^T phi(k) / phi(k)^T s carries signal and cache membership depends on it
  rather than on ||v||^2 alone (LoLA notes §2.3, Eq. (10));
* a pool of six (k, v) pairs per unit, so that candidates tie exactly: the
  top-lambda set must then be the oracle's bit for bit, the older position
  winning a tie at the capacity boundary (LoLA notes §2.6 on ties; the
  decode step folds the newer of tied lowest candidates);
* the chain instances of the two grid splits not reached by the other
  shapes: two cooperating workgroups per unit (96 units) and one (512 units,
  the 4096-token prefill of the decode workload).
"""

import pytest

from sparse_kv_caching_amd.workloads import WORKLOADS

from test_gpu_parity import _decode_lockstep, _full_size_single_call, run_lockstep

pytestmark = pytest.mark.gpu


def test_clustered_keys_lockstep_bf16():
    wl = WORKLOADS["llama8b_4k"].scaled(B=2, Hq=8, Hkv=2, T=704, eta=64, lam=96, C=64,
                                        keys="clustered")
    s = run_lockstep(wl)
    assert s["scored"] >= 8


def test_clustered_keys_lockstep_fp32():
    wl = WORKLOADS["tiny_fp32"].scaled(B=1, Hq=2, Hkv=1, d=128, T=384, eta=32, lam=64, C=32,
                                       planted=0, keys="clustered")
    run_lockstep(wl)


def test_exact_ties_lockstep():
    """Every candidate ties with others; membership must be exact."""
    wl = WORKLOADS["llama8b_4k"].scaled(B=2, Hq=8, Hkv=2, T=640, eta=64, lam=96, C=64,
                                        keys="pool")
    s = run_lockstep(wl, strict=True, check_continuous=False)
    assert s["ties"] > 0, "no tie group straddled the boundary"


def test_exact_ties_decode():
    wl = WORKLOADS["decode_b64"].scaled(B=2, Hq=8, Hkv=2, T=128, eta=16, lam=32, C=32,
                                        keys="pool")
    _decode_lockstep(wl, 48, strict=True)


def test_two_workgroups_per_unit():
    """96 units (12 sequences x 8 KV heads): the chain runs two cooperating
    workgroups per unit (two column slabs each); sequences 0 and 11 followed
    chunk by chunk."""
    wl = WORKLOADS["llama8b_4k"].scaled(B=12, T=1024, eta=64, lam=128, C=64)
    _full_size_single_call(wl, units=[0, 11])


@pytest.mark.timeout(900)
def test_one_workgroup_per_unit_decode_prefill():
    """The decode workload's 4096-token prefill (512 units, eta = lambda = 64,
    C = 64): one workgroup per unit holding all four column slabs; sequences
    0, 31 and 63 followed chunk by chunk (q = 0, as in the benchmark)."""
    _full_size_single_call(WORKLOADS["decode_b64"], units=[0, 31, 63], q_zero=True)
