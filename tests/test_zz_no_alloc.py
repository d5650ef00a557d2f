"""lola_prefill_chunk_noalloc (the prefill entry point for callers that
cannot allocate device memory: its workspace is the library's static device
array) against lola_prefill_chunk with the library's own workspace, through
the C ABI: outputs and exported states bitwise equal over consecutive calls,
the second smaller than the first, then another configuration on the same
array, a token-by-token call, and a call whose workspace would not fit
(rejected, state unchanged)."""

import pytest
import torch

from sparse_kv_caching_amd.lola import LOLA_ERR_WORKSPACE, LolaError
from sparse_kv_caching_amd.workloads import WORKLOADS, make_inputs

from lola_harness import dev, make_layer

pytestmark = pytest.mark.gpu

KEYS = ("H", "s", "win_k", "win_v", "cache_pos", "cache_k", "cache_v")


def _same_state(a, b):
    ea, eb = a.export(), b.export()
    assert ea["n"] == eb["n"]
    for key in KEYS:
        assert torch.equal(ea[key], eb[key]), key


def _pair(wl, calls):
    inp = make_inputs(wl)
    A, B = make_layer(wl, inp.W), make_layer(wl, inp.W)
    for t0, t1, C in calls:
        print("no-alloc call", wl.name, wl.B, wl.Hkv, t0, t1, C, flush=True)
        q = dev(wl, inp.q[:, :, t0:t1])
        k = dev(wl, inp.k[:, :, t0:t1])
        v = dev(wl, inp.v[:, :, t0:t1])
        ya = A.prefill_noalloc(q, k, v, C, out=torch.empty(q.shape, dtype=torch.float32,
                                                            device="cuda"))
        yb = B.prefill(q, k, v, C)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), (t0, t1, C)
        _same_state(A, B)
    return A, B


def test_noalloc_equals_prefill():
    wl = WORKLOADS["llama8b_4k"].scaled(B=2, Hq=8, Hkv=2, T=704, eta=64, lam=96, C=64)
    A, B = _pair(wl, [(0, 512, 64), (512, 704, 64)])        # second call smaller
    A.free()
    B.free()
    # another configuration on the same array, then token by token
    wl2 = WORKLOADS["tiny_fp32"].scaled(T=200, eta=32, lam=48, C=32, planted=0)
    A, B = _pair(wl2, [(0, 160, 32), (160, 196, 32), (196, 200, 1)])
    A.free()
    B.free()


def test_noalloc_rejects_a_call_beyond_its_workspace():
    wl = WORKLOADS["llama8b_4k"].scaled(B=2)                 # about 107 MB of workspace
    inp = make_inputs(wl.scaled(T=64))
    L = make_layer(wl, inp.W)
    assert L.workspace_bytes(wl.T, wl.C) > 64 << 20
    q = torch.empty((wl.B, wl.Hq, wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((wl.B, wl.Hkv, wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(LolaError) as ei:
        L.prefill_noalloc(q, k, k, wl.C, out=out)
    assert ei.value.code == LOLA_ERR_WORKSPACE
    assert L.n == 0
    L.check()
    L.free()
