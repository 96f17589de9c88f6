"""GPU parity on the method's degenerate inputs, through both encode kernels
and the decode:

- an all-zero key and value (norm 0: y = 0 lies on the middle threshold of a
  symmetric table; both kernels put it in the lower cell, as #{t < y} does,
  and the window would excuse it anyway; its score is 0 whatever the code);
- a value group that is constant (delta 0: every code 0, the value is the
  stored minimum);
- a key a thousand times larger than the rest, and one 1e-12 times smaller
  (its squares stay in the fp32 normal range).

Codes are checked against the oracle outside the boundary window after the bulk
encode and again after the same tokens are re-encoded one at a time by the
few-token kernel; the decode (queries along the large key, along a plain
key, and random) is compared with the oracle on the GPU's codes.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import (OUT_RTOL, books, check_encode_slot, dequant_slot, encode_slot, layout_of, max_rel_err,
                        say, slot_from_cache)

pytestmark = pytest.mark.gpu

DEV = "cuda"
ZERO, CONST, BIG, TINY = 5, 40, 61, 77

CASES = {
    "2+1-bit keys, min/max values": wl.WORKLOADS[3].replace(batch=1, h_q=8, h_kv=2, n_tokens=96, decode_steps=1),
    "3+1-bit keys, MSE values": wl.WORKLOADS[4].replace(h_q=8, h_kv=2, n_tokens=96, decode_steps=1),
    "qwen layer, fp16 scalars": wl.by_name("qwen2.5-1.5b-layer-n512").replace(n_tokens=96),
    "3.5-bit keys": wl.WORKLOADS[3].replace(batch=1, h_q=8, h_kv=2, n_tokens=96, decode_steps=1, key_half=1),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.lib()


def _inputs(w):
    k, v = wl.prefill_kv(w)
    k, v = k.clone(), v.clone()
    k[:, ZERO] = 0
    v[:, ZERO] = 0
    v[:, CONST, :, 0:32] = 1.5
    k[:, BIG] = k[:, BIG] * 1000
    k[:, TINY] = (k[:, TINY].double() * 1e-12).to(k.dtype)
    return k, v


def _check_codes(w, bk, pi, s, cache, k, v, tag):
    tot = np.zeros(3, dtype=np.int64)
    for h in range(w.h_kv):
        ref = encode_slot(w, bk, pi, s, k[0, :, h].double().numpy(), v[0, :, h].double().numpy())
        tot += check_encode_slot(w, bk, cache, 0, h, ref, 0, w.n_tokens, f"{tag} h{h}")
    return tot


@pytest.mark.parametrize("name", list(CASES))
def test_degenerate_tokens(name):
    w = CASES[name]
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = _inputs(w)
    cache = tq.Cache(layout_of(w), 1, w.h_kv, 96, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0], cache)
    torch.cuda.synchronize()
    bulk = _check_codes(w, bk, pi, s, cache, k, v, f"{name} bulk")
    for t in (ZERO, CONST, BIG, TINY):  # the same tokens again, one per call
        tq.encode_kv(prm, k[:, t:t + 1].contiguous().to(DEV), v[:, t:t + 1].contiguous().to(DEV), [t], cache)
    torch.cuda.synchronize()
    small = _check_codes(w, bk, pi, s, cache, k, v, f"{name} few-token")
    # the constant group decodes to its minimum exactly; the zero value to 0
    if w.value_kind == "minmax":
        meta = cache.v_meta[0, :, CONST, 0].cpu()
        assert torch.all(meta[:, 0] == 0) and torch.all(meta[:, 1].float() == 1.5)
    kn = cache.k_norm[0, :, ZERO].float().cpu()
    assert torch.all(kn == 0)
    # decode on the GPU's codes
    kd, vd = [[]], [[]]
    for h in range(w.h_kv):
        a_, c_ = dequant_slot(w, bk, pi, s, slot_from_cache(w, cache, 0, h, w.n_tokens))
        kd[0].append(a_)
        vd[0].append(c_)
    g = w.h_q // w.h_kv
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, w.h_q, w.d))
    for hq in range(w.h_q):
        h = hq // g
        if hq % g == 0:
            q[0, hq] = k[0, BIG, h].double().numpy() * 1e-3   # points at the large key
        elif hq % g == 1:
            q[0, hq] = k[0, 10, h].double().numpy()           # a plain key
    qt = torch.from_numpy(q).to(w.torch_dtype)
    out = tq.decode_attn(prm, qt.to(DEV), cache, [w.n_tokens])
    torch.cuda.synchronize()
    ref = oracle.decode_attention(qt.double().numpy(), kd, vd)
    err = max_rel_err(out.cpu().double().numpy(), ref)
    say(f"[degenerate] {name}: excused flips bulk {bulk.tolist()}, few-token {small.tolist()}; "
        f"decode max rel err {err.max():.2e}")
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert err.max() <= OUT_RTOL


QUERY_SCALES = (0.0, 1e-6, 1.0, 4.0, 16.0, 64.0)


@pytest.mark.parametrize("path", ["mfma", "generic"])
@pytest.mark.parametrize("name", ["2+1-bit keys, min/max values", "3+1-bit keys, MSE values", "qwen layer, fp16 scalars"])
def test_query_scales(name, path, monkeypatch):
    """Queries over nine decades of magnitude, one scale per query head: a
    zero query (uniform attention), 1e-6 (nearly uniform) and 1 .. 64 times a
    unit Gaussian (ever more peaked softmax, where the score precision of the
    query's digit expansion decides the output).  Decode of the GPU's codes
    against the oracle, on both scan paths."""
    from tq_testlib import set_decode_path
    set_decode_path(monkeypatch, path)
    w = CASES[name].replace(n_tokens=96)
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cache = tq.Cache(layout_of(w), 1, w.h_kv, 96, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0], cache)
    torch.cuda.synchronize()
    kd, vd = [[]], [[]]
    for h in range(w.h_kv):
        a_, c_ = dequant_slot(w, bk, pi, s, slot_from_cache(w, cache, 0, h, w.n_tokens))
        kd[0].append(a_)
        vd[0].append(c_)
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, w.h_q, w.d))
    for hq in range(w.h_q):
        q[0, hq] *= QUERY_SCALES[hq % len(QUERY_SCALES)]
    qt = torch.from_numpy(q).to(w.torch_dtype)
    out = tq.decode_attn(prm, qt.to(DEV), cache, [w.n_tokens])
    torch.cuda.synchronize()
    ref = oracle.decode_attention(qt.double().numpy(), kd, vd)
    err = max_rel_err(out.cpu().double().numpy(), ref)
    per_scale = {sc: float(err[0, [hq for hq in range(w.h_q) if hq % len(QUERY_SCALES) == i]].max())
                 for i, sc in enumerate(QUERY_SCALES) if i < w.h_q}
    say(f"[query scales] {name} ({path}): " + ", ".join(f"{sc:g}: {e:.1e}" for sc, e in per_scale.items()))
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert err.max() <= OUT_RTOL
