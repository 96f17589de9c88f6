"""GPU parity of multi-query decode (T causal queries per sequence over the same
cache, tq_decode_attn_multi) against the oracle's decode_attention_multi.

The caches hold the oracle's codes, as in the single-query decode parity
tests, so the comparison isolates the decode.  Cases:

- T = 2 with four query heads per KV head (eight (query, head) pairs: one pass
  over the compressed cache), on both scan paths;
- T = 3 (twelve pairs: two passes), with ring lengths on either side of T - 1
  so that the causal tail lies in the ring or reaches into the compressed part;
- no ring at all (every hidden key is a compressed token), the Qwen-shaped
  layer (six heads per KV head, MSE values), and a sequence whose earliest
  queries see no key (zero output).
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import DECODE_PATHS, set_decode_path, OUT_RTOL, books, dequant_slot, encode_slot, layout_of, max_rel_err, say, upload_slot

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.lib()


def _multi_case(w, nq, n_comp, n_ring, tag):
    say(f"[multi-query parity] {tag}: T={nq} B={w.batch} H_q={w.h_q} H_kv={w.h_kv} n={n_comp} ring={n_ring}")
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cap = max(32, ((max(n_comp) + 31) // 32) * 32)
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    kd, vd = [], []
    for b in range(w.batch):
        kr, vr = [], []
        for h in range(w.h_kv):
            n = n_comp[b]
            sc = encode_slot(w, bk, pi, s, k[b, :n, h].double().numpy(), v[b, :n, h].double().numpy())
            if n > 0:
                upload_slot(cache, w, b, h, sc)
            a_, c_ = dequant_slot(w, bk, pi, s, sc)
            kr.append(a_)
            vr.append(c_)
        kd.append(kr)
        vd.append(vr)
    rng = np.random.default_rng(23)
    q = torch.from_numpy(rng.standard_normal((w.batch, nq, w.h_q, w.d))).to(w.torch_dtype)
    rk = rv = None
    if max(n_ring) > 0:
        rk = torch.from_numpy(rng.standard_normal((w.batch, 128, w.h_kv, w.d))).to(torch.bfloat16)
        rv = torch.from_numpy(rng.standard_normal((w.batch, 128, w.h_kv, w.d))).to(torch.bfloat16)
    out = tq.decode_attn(prm, q.to(DEV), cache, n_comp, None if rk is None else rk.to(DEV),
                         None if rv is None else rv.to(DEV), n_ring)
    torch.cuda.synchronize()
    ref = oracle.decode_attention_multi(q.double().numpy(), kd, vd,
                                        None if rk is None else rk.double().numpy(),
                                        None if rv is None else rv.double().numpy(), n_ring)
    got = out.cpu().double().numpy()
    assert got.shape == ref.shape
    for b in range(w.batch):
        for t in range(nq):
            if n_comp[b] + n_ring[b] - (nq - 1 - t) <= 0:
                assert np.all(got[b, t] == 0), (b, t)
    err = max_rel_err(got, ref)
    say(f"  max rel err {err.max():.2e} (bound {OUT_RTOL})")
    assert err.max() <= OUT_RTOL
    return got


@pytest.mark.parametrize("path", DECODE_PATHS)
def test_multi_query_two_queries_one_pass(path, monkeypatch):
    set_decode_path(monkeypatch, path)
    w = wl.WORKLOADS[1].replace(batch=2, n_tokens=700)
    _multi_case(w, 2, [700, 513], [3, 1], f"gqa4 ({path})")


def test_multi_query_three_queries_two_passes_causal_into_compressed():
    w = wl.WORKLOADS[3].replace(batch=3, n_tokens=640, decode_steps=1)
    # ring 5 >= T - 1; ring 1 and 0: the hidden keys reach the compressed tail
    _multi_case(w, 3, [640, 333, 64], [5, 1, 0], "batched minmax")


def test_multi_query_without_ring():
    w = wl.WORKLOADS[4].replace(n_tokens=1024, decode_steps=1)
    _multi_case(w, 4, [1000], [0], "long mse, no ring")


def test_multi_query_half_bit_keys():
    # T = 2 over four query heads per KV head: eight virtual heads, two head
    # tiles on the shared half/parity operand word of 3.5-bit keys
    w = wl.WORKLOADS[3].replace(batch=2, n_tokens=600, decode_steps=1, key_half=1)
    _multi_case(w, 2, [600, 411], [3, 0], "batched minmax, 3.5-bit keys")


def test_multi_query_qwen_layer():
    w = wl.by_name("qwen2.5-1.5b-layer-n4096").replace(n_tokens=1536)
    _multi_case(w, 2, [1536], [0], "qwen, six heads per KV head")


def test_multi_query_earliest_queries_see_nothing():
    w = wl.WORKLOADS[1].replace(batch=2, n_tokens=64)
    # sequence 0: one compressed token and no ring, T = 3: queries 0 and 1 see no key
    _multi_case(w, 3, [1, 64], [0, 2], "empty prefix")


def test_multi_query_of_one_matches_single_query():
    w = wl.WORKLOADS[1].replace(batch=2, n_tokens=300)
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, 320, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    q = wl.query(w).to(DEV)
    one = tq.decode_attn(prm, q, cache, [300, 300])
    multi = tq.decode_attn(prm, q[:, None].contiguous(), cache, [300, 300])
    torch.cuda.synchronize()
    assert torch.equal(one, multi[:, 0])
    del bk
