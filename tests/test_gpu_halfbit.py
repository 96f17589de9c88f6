"""GPU parity of the fractional (half-bit) key widths: TurboQuantProd(3.5) =
2.5 MSE bits + QJL and TurboQuantProd(2.5) = 1.5 MSE bits + QJL, where the
rotated coordinates i with i mod 32 < 16 carry one more Lloyd-Max bit.

- Encode: GPU codes against the oracle's, bit-exact outside the boundary
  window of each coordinate's own table, norms to rounding.
- Decode: caches holding the oracle's codes, decoded on the GPU, within 2e-3
  of the oracle's attention; min/max and MSE values.
- End to end: GPU encode, read back, oracle decode of those codes against the
  GPU decode.
- The generic scan has no half-bit path: forcing it is an error, not a silent
  fallback.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import (gamma_report, OUT_RTOL, books, check_encode_slot, dequant_slot, encode_slot, layout_of, max_rel_err,
                        say, slot_from_cache, upload_slot)

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    "3.5-bit keys, min/max values": wl.WORKLOADS[3].replace(batch=2, n_tokens=600, decode_steps=1, key_half=1),
    "2.5-bit keys, min/max values": wl.WORKLOADS[3].replace(batch=2, n_tokens=600, decode_steps=1, key_half=1,
                                                           key_mse_bits=1),
    "3.5-bit keys, MSE values": wl.WORKLOADS[4].replace(n_tokens=700, decode_steps=1, key_half=1, key_mse_bits=2),
    "2.5-bit keys, fp32 inputs": wl.WORKLOADS[1].replace(batch=1, n_tokens=500, key_half=1, key_mse_bits=1),
    # six query heads per KV head: two head tiles on the shared half/parity word
    "3.5-bit keys, Qwen layer": wl.by_name("qwen2.5-1.5b-layer-n4096-k3.5bit").replace(n_tokens=700),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.lib()


def _setup(w):
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    return bk, pi, s, prm, k, v


@pytest.mark.parametrize("name", list(CASES))
def test_half_bit_encode_parity(name):
    w = CASES[name]
    bk, pi, s, prm, k, v = _setup(w)
    cap = ((w.n_tokens + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    torch.cuda.synchronize()
    tot = np.zeros(3, dtype=np.int64)
    for b in range(w.batch):
        for h in range(w.h_kv):
            ref = encode_slot(w, bk, pi, s, k[b, :, h].double().numpy(), v[b, :, h].double().numpy())
            tot += check_encode_slot(w, bk, cache, b, h, ref, 0, w.n_tokens, f"{name} b{b} h{h}")
    say(f"[half-bit encode] {name}: every slot matches outside the window; excused flips "
        f"MSE {tot[0]}, QJL {tot[1]}, values {tot[2]}")
    say("  " + gamma_report())


@pytest.mark.parametrize("name", list(CASES))
def test_half_bit_decode_parity(name):
    w = CASES[name]
    bk, pi, s, prm, k, v = _setup(w)
    n_comp = [w.n_tokens - 37 * b for b in range(w.batch)]
    cap = ((w.n_tokens + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    kd, vd = [], []
    for b in range(w.batch):
        kr, vr = [], []
        for h in range(w.h_kv):
            sc = encode_slot(w, bk, pi, s, k[b, :n_comp[b], h].double().numpy(), v[b, :n_comp[b], h].double().numpy())
            upload_slot(cache, w, b, h, sc)
            a_, c_ = dequant_slot(w, bk, pi, s, sc)
            kr.append(a_)
            vr.append(c_)
        kd.append(kr)
        vd.append(vr)
    q = wl.query(w)
    out = tq.decode_attn(prm, q.to(DEV), cache, n_comp)
    torch.cuda.synchronize()
    ref = oracle.decode_attention(q.double().numpy(), kd, vd)
    err = max_rel_err(out.cpu().double().numpy(), ref)
    say(f"[half-bit decode] {name}: max rel err {err.max():.2e} (bound {OUT_RTOL})")
    assert err.max() <= OUT_RTOL


@pytest.mark.parametrize("name", list(CASES))
def test_half_bit_end_to_end(name):
    w = CASES[name]
    bk, pi, s, prm, k, v = _setup(w)
    cap = ((w.n_tokens + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    q = wl.query(w)
    out = tq.decode_attn(prm, q.to(DEV), cache, [w.n_tokens] * w.batch)
    torch.cuda.synchronize()
    kd, vd = [], []
    for b in range(w.batch):
        kr, vr = [], []
        for h in range(w.h_kv):
            a_, c_ = dequant_slot(w, bk, pi, s, slot_from_cache(w, cache, b, h, w.n_tokens))
            kr.append(a_)
            vr.append(c_)
        kd.append(kr)
        vd.append(vr)
    ref = oracle.decode_attention(q.double().numpy(), kd, vd)
    err = max_rel_err(out.cpu().double().numpy(), ref)
    say(f"[half-bit end to end] {name}: max rel err {err.max():.2e} (bound {OUT_RTOL})")
    assert err.max() <= OUT_RTOL


def test_half_bit_generic_scan_is_refused(monkeypatch):
    w = CASES["3.5-bit keys, min/max values"].replace(batch=1, n_tokens=64)
    bk, pi, s, prm, k, v = _setup(w)
    cache = tq.Cache(layout_of(w), 1, w.h_kv, 64, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0], cache)
    monkeypatch.setenv("TQ_DECODE_PATH", "generic")
    with pytest.raises(tq.TqError) as e:
        tq.decode_attn(prm, wl.query(w).to(DEV), cache, [64])
    assert e.value.code == tq.TQ_ERR_UNSUPPORTED
    del bk
