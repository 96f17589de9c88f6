"""GPU check of tq_decode_attn_noalloc, the decode entry point that allocates
nothing (its workspace is a static device array of TQ_NOALLOC_SCRATCH_BYTES):
called through the C ABI, its output must equal tq_decode_attn's with a
caller-allocated workspace bit for bit, on two calls in a row (the second with
fewer sequences and tokens, so it runs over what the first left in the
scratch), and a call that needs more workspace than the scratch holds is
refused on the host before anything is launched (a CPU test)."""
import ctypes

import numpy as np
import pytest
import torch

from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import layout_of, say

DEV = "cuda"
SCRATCH_BYTES = 32 << 20  # TQ_NOALLOC_SCRATCH_BYTES


def _noalloc(prm, q, cache, n_comp, rk, rv, n_ring, out):
    L = tq.lib()
    lay, p, cc = prm.layout.c(), prm.c(), cache.c()
    b = cache.batch
    nc = (ctypes.c_int64 * b)(*n_comp)
    nr = (ctypes.c_int32 * b)(*n_ring)
    stream = torch.cuda.current_stream().cuda_stream
    return L.tq_decode_attn_noalloc(ctypes.byref(lay), ctypes.byref(p), q.data_ptr(), tq._dtype_code(q), q.shape[1],
                                    ctypes.byref(cc), nc, None if rk is None else rk.data_ptr(),
                                    None if rv is None else rv.data_ptr(), 0 if rk is None else rk.shape[1], nr,
                                    1.0 / np.sqrt(q.shape[-1]), out.data_ptr(), stream)


def _case(w, n_comp, n_ring, tag):
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cap = ((max(n_comp) + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    tq.encode_kv(prm, k[:, :cap].contiguous().to(DEV), v[:, :cap].contiguous().to(DEV), [0] * w.batch, cache)
    rng = np.random.default_rng(5)
    rk = torch.from_numpy(rng.standard_normal((w.batch, 128, w.h_kv, w.d))).to(torch.bfloat16).to(DEV)
    rv = torch.from_numpy(rng.standard_normal((w.batch, 128, w.h_kv, w.d))).to(torch.bfloat16).to(DEV)
    q = wl.query(w).to(DEV)
    ref = tq.decode_attn(prm, q, cache, n_comp, rk, rv, n_ring)
    out = torch.full_like(ref, float("nan"))
    rc = _noalloc(prm, q, cache, n_comp, rk, rv, n_ring, out)
    assert rc == tq.TQ_OK, tq.lib().tq_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(out, ref), f"{tag}: max |diff| {float((out - ref).abs().max()):.3e}"
    say(f"[no-alloc decode] {tag}: B={w.batch} n_comp={n_comp} n_ring={n_ring}: equal to tq_decode_attn")


@pytest.mark.gpu
def test_noalloc_decode_equals_workspace_decode_twice():
    w = wl.WORKLOADS[3].replace(batch=5, n_tokens=3000, decode_steps=1)
    _case(w, [3000, 2048, 1, 777, 0], [3, 0, 128, 17, 5], "first call")
    w2 = wl.WORKLOADS[3].replace(batch=2, n_tokens=300, decode_steps=1)
    _case(w2, [300, 64], [1, 0], "second, smaller call")


def test_noalloc_decode_refuses_oversize_workspace():
    # host check, no device touched: 64 sequences x 64 KV heads x 8 query
    # heads each need more than the 32 MiB scratch
    lay = tq.Layout()
    need = tq.decode_workspace_bytes(lay, 64, 512, 64, 1 << 20)
    assert need > SCRATCH_BYTES
    L = tq.lib()
    lc, p = lay.c(), tq._Params()
    p.pi, p.s, p.derived = 16, 16, 16  # never dereferenced: the call fails its size check first
    cc = tq._Cache(16, 16, 16, 16, 16, 0, 64, 64, 1 << 20)
    nc = (ctypes.c_int64 * 64)(*([1 << 20] * 64))
    rc = L.tq_decode_attn_noalloc(ctypes.byref(lc), ctypes.byref(p), 16, tq.TQ_F32, 512, ctypes.byref(cc), nc,
                                  None, None, 0, None, 0.1, 16, None)
    assert rc == tq.TQ_ERR_WORKSPACE
    assert "static scratch" in L.tq_last_error().decode()
