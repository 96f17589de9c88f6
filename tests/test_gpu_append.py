"""GPU checks of the fused decode step (tq_decode_attn_append): the ring append
done by the decode's query-preparation kernel must equal tq_ring_append
followed by tq_decode_attn with one more ring token, bit for bit (outputs and
ring contents), on both scan paths, for bf16 and fp32 new tokens, with ragged
ring lengths; and the result must match the oracle's attention over the same
keys.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import DECODE_PATHS, set_decode_path, OUT_RTOL, books, dequant_slot, layout_of, max_rel_err, say, slot_from_cache

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.lib()


def _setup(w, n_comp, n_ring, new_dtype):
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cap = ((max(n_comp) + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    rng = np.random.default_rng(41)
    ring_k = torch.from_numpy(rng.standard_normal((w.batch, 128, w.h_kv, w.d))).to(torch.bfloat16).to(DEV)
    ring_v = torch.from_numpy(rng.standard_normal((w.batch, 128, w.h_kv, w.d))).to(torch.bfloat16).to(DEV)
    kn = torch.from_numpy(rng.standard_normal((w.batch, 1, w.h_kv, w.d))).to(new_dtype).to(DEV)
    vn = torch.from_numpy(rng.standard_normal((w.batch, 1, w.h_kv, w.d))).to(new_dtype).to(DEV)
    q = wl.query(w).to(DEV)
    return prm, cache, ring_k, ring_v, kn, vn, q


@pytest.mark.parametrize("path", DECODE_PATHS)
@pytest.mark.parametrize("new_dtype", [torch.bfloat16, torch.float32])
def test_fused_append_equals_append_then_decode(path, new_dtype, monkeypatch):
    set_decode_path(monkeypatch, path)
    w = wl.WORKLOADS[1].replace(batch=3, n_tokens=700)
    n_comp = [700, 333, 64]
    n_ring = [0, 17, 127]  # empty ring, ragged, the last free slot
    say(f"[fused append] path={path} new={new_dtype} n_comp={n_comp} n_ring={n_ring}")
    prm, cache, rk, rv, kn, vn, q = _setup(w, n_comp, n_ring, new_dtype)
    rk2, rv2 = rk.clone(), rv.clone()
    fused = tq.decode_attn_append(prm, q, cache, n_comp, kn, vn, rk, rv, n_ring)
    tq.ring_append(kn, vn, rk2, rv2, n_ring)
    sep = tq.decode_attn(prm, q, cache, n_comp, rk2, rv2, [x + 1 for x in n_ring])
    torch.cuda.synchronize()
    assert torch.equal(rk, rk2) and torch.equal(rv, rv2)
    for b, p in enumerate(n_ring):
        assert torch.equal(rk[b, p], kn[b, 0].to(torch.bfloat16))
        assert torch.equal(rv[b, p], vn[b, 0].to(torch.bfloat16))
    assert torch.equal(fused, sep)


def test_fused_append_against_oracle():
    w = wl.WORKLOADS[3].replace(batch=2, n_tokens=640, decode_steps=1)
    n_comp = [640, 200]
    n_ring = [5, 0]
    prm, cache, rk, rv, kn, vn, q = _setup(w, n_comp, n_ring, torch.bfloat16)
    out = tq.decode_attn_append(prm, q, cache, n_comp, kn, vn, rk, rv, n_ring)
    torch.cuda.synchronize()
    bk = books(w)
    pi, s = wl.params(w)
    kd, vd = [], []
    for b in range(w.batch):
        kr, vr = [], []
        for h in range(w.h_kv):
            a_, c_ = dequant_slot(w, bk, pi, s, slot_from_cache(w, cache, b, h, n_comp[b]))
            kr.append(a_)
            vr.append(c_)
        kd.append(kr)
        vd.append(vr)
    rkn = rk.cpu().double().numpy()
    rvn = rv.cpu().double().numpy()
    ref = oracle.decode_attention(q.cpu().double().numpy(), kd, vd, rkn, rvn, [x + 1 for x in n_ring])
    err = max_rel_err(out.cpu().double().numpy(), ref)
    say(f"[fused append] against the oracle: max rel err {err.max():.2e} (bound {OUT_RTOL})")
    assert err.max() <= OUT_RTOL


def _oracle_decode(w, bk, pi, s, cache, q, n_comp, rk, rv, n_ring):
    """The oracle's attention over the GPU's own codes of every slot plus the
    first n_ring[b] ring tokens."""
    kd, vd = [], []
    for b in range(w.batch):
        kr, vr = [], []
        for h in range(w.h_kv):
            a_, c_ = dequant_slot(w, bk, pi, s, slot_from_cache(w, cache, b, h, n_comp[b]))
            kr.append(a_)
            vr.append(c_)
        kd.append(kr)
        vd.append(vr)
    return oracle.decode_attention(q.cpu().double().numpy(), kd, vd, rk.cpu().double().numpy(),
                                   rv.cpu().double().numpy(), list(n_ring))


def test_ring_fill_flush_then_decode():
    """The store's life cycle over one full ring (page "turboquant/audit_claims.py",
    AUDIT 1: the most recent 128 tokens stay uncompressed in bf16): 128 fused
    decode steps fill the ring, the full ring is flushed through tq_encode_kv
    at each sequence's compressed length (ragged, not 32-aligned), and the next
    step starts a new ring.  Checked against the oracle: decode outputs at
    ring lengths 1, 64 and 128 and after the flush, and the flushed tokens'
    codes against the oracle's encode of the same bf16 ring contents."""
    from tq_testlib import check_encode_slot, encode_slot

    w = wl.WORKLOADS[3].replace(batch=2, n_tokens=640, decode_steps=1)
    n_comp = [640, 501]
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, 800, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    # sequence 1 holds 501 compressed tokens: its positions 501.. are rewritten by the flush
    rk = torch.zeros((w.batch, 128, w.h_kv, w.d), dtype=torch.bfloat16, device=DEV)
    rv = torch.zeros_like(rk)
    worst = 0.0
    for i in range(129):
        if i == 128:  # the ring is full: flush it, then the step appends to an empty ring
            flushed_k, flushed_v = rk.clone(), rv.clone()
            tq.encode_kv(prm, rk, rv, n_comp, cache)
            torch.cuda.synchronize()
            for b in range(w.batch):
                for h in range(w.h_kv):
                    ref = encode_slot(w, bk, pi, s, flushed_k[b, :, h].cpu().double().numpy(),
                                      flushed_v[b, :, h].cpu().double().numpy())
                    check_encode_slot(w, bk, cache, b, h, ref, n_comp[b], 128, f"flush b{b} h{h}")
            n_comp = [n + 128 for n in n_comp]
        n_r = i % 128
        kn, vn = (x.to(DEV).contiguous() for x in wl.step_kv(w, i))
        q = wl.query(w, i).to(DEV)
        out = tq.decode_attn_append(prm, q, cache, n_comp, kn, vn, rk, rv, [n_r] * w.batch)
        if i in (0, 63, 127, 128):
            torch.cuda.synchronize()
            ref = _oracle_decode(w, bk, pi, s, cache, q, n_comp, rk, rv, [n_r + 1] * w.batch)
            err = float(max_rel_err(out.cpu().double().numpy(), ref).max())
            worst = max(worst, err)
            say(f"[ring flush] step {i}: compressed {n_comp}, ring {n_r + 1}, max rel err {err:.2e}")
            assert err <= OUT_RTOL
    say(f"[ring flush] worst {worst:.2e} (bound {OUT_RTOL})")

