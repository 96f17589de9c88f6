"""GPU parity when a call covers more sequences than one launch carries
(per-sequence lengths travel in kernel arguments, 64 sequences per launch):
70 sequences, so every entry point runs two launch groups that share the
workspace.  Bulk encode, a one-token encode, single-query decode with ragged
lengths and ragged rings, multi-query decode and the fused append, against the
oracle."""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import OUT_RTOL, books, dequant_slot, layout_of, max_rel_err, say, slot_from_cache

pytestmark = pytest.mark.gpu

DEV = "cuda"
B = 70


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.lib()


@pytest.fixture(scope="module")
def setup():
    w = wl.WORKLOADS[1].replace(batch=B, n_tokens=72, h_q=2, h_kv=1)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cache = tq.Cache(layout_of(w), B, w.h_kv, 96, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * B, cache)
    # one more token per sequence through the few-token encode, at position 72
    rng = np.random.default_rng(5)
    kn = torch.from_numpy(rng.standard_normal((B, 1, w.h_kv, w.d))).to(torch.float32)
    vn = torch.from_numpy(rng.standard_normal((B, 1, w.h_kv, w.d))).to(torch.float32)
    tq.encode_kv(prm, kn.to(DEV), vn.to(DEV), [72] * B, cache)
    torch.cuda.synchronize()
    return w, pi, s, prm, cache


def _oracle_kv(w, pi, s, cache, n_comp):
    bk = books(w)
    kd, vd = [], []
    for b in range(B):
        a_, c_ = dequant_slot(w, bk, pi, s, slot_from_cache(w, cache, b, 0, n_comp[b]))
        kd.append([a_])
        vd.append([c_])
    return kd, vd


def _ring(w):
    rng = np.random.default_rng(9)
    rk = torch.from_numpy(rng.standard_normal((B, 8, w.h_kv, w.d))).to(torch.bfloat16)
    rv = torch.from_numpy(rng.standard_normal((B, 8, w.h_kv, w.d))).to(torch.bfloat16)
    return rk, rv


def test_large_batch_decode(setup):
    w, pi, s, prm, cache = setup
    n_comp = [73 - (b % 41) for b in range(B)]
    n_ring = [b % 5 for b in range(B)]
    rk, rv = _ring(w)
    q = wl.query(w)
    out = tq.decode_attn(prm, q.to(DEV), cache, n_comp, rk.to(DEV), rv.to(DEV), n_ring)
    torch.cuda.synchronize()
    kd, vd = _oracle_kv(w, pi, s, cache, n_comp)
    ref = oracle.decode_attention(q.double().numpy(), kd, vd, rk.double().numpy(), rv.double().numpy(), n_ring)
    err = max_rel_err(out.cpu().double().numpy(), ref)
    say(f"[large batch] {B} sequences decode: max rel err {err.max():.2e}")
    assert err.max() <= OUT_RTOL


def test_large_batch_multi_query(setup):
    w, pi, s, prm, cache = setup
    n_comp = [73 - (b % 29) for b in range(B)]
    n_ring = [b % 3 for b in range(B)]
    rk, rv = _ring(w)
    rng = np.random.default_rng(13)
    q = torch.from_numpy(rng.standard_normal((B, 3, w.h_q, w.d))).to(torch.float32)
    out = tq.decode_attn(prm, q.to(DEV), cache, n_comp, rk.to(DEV), rv.to(DEV), n_ring)
    torch.cuda.synchronize()
    kd, vd = _oracle_kv(w, pi, s, cache, n_comp)
    ref = oracle.decode_attention_multi(q.double().numpy(), kd, vd, rk.double().numpy(), rv.double().numpy(),
                                        n_ring)
    err = max_rel_err(out.cpu().double().numpy(), ref)
    say(f"[large batch] {B} sequences, 3 queries each: max rel err {err.max():.2e}")
    assert err.max() <= OUT_RTOL


def test_large_batch_fused_append(setup):
    w, pi, s, prm, cache = setup
    n_comp = [73] * B
    n_ring = [b % 7 for b in range(B)]
    rk, rv = _ring(w)
    rk, rv = rk.to(DEV), rv.to(DEV)
    rk2, rv2 = rk.clone(), rv.clone()
    rng = np.random.default_rng(17)
    kn = torch.from_numpy(rng.standard_normal((B, 1, w.h_kv, w.d))).to(torch.bfloat16).to(DEV)
    vn = torch.from_numpy(rng.standard_normal((B, 1, w.h_kv, w.d))).to(torch.bfloat16).to(DEV)
    q = wl.query(w).to(DEV)
    fused = tq.decode_attn_append(prm, q, cache, n_comp, kn, vn, rk, rv, n_ring)
    tq.ring_append(kn, vn, rk2, rv2, n_ring)
    sep = tq.decode_attn(prm, q, cache, n_comp, rk2, rv2, [x + 1 for x in n_ring])
    torch.cuda.synchronize()
    assert torch.equal(rk, rk2) and torch.equal(rv, rv2)
    assert torch.equal(fused, sep)
