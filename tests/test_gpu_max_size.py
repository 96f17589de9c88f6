"""GPU parity at the far end of a cache slot whose planes exceed 2^31 bytes
(75,497,472 token positions of one KV head: 3.6 GB of key planes, 2.4 GB of
value planes), so every byte offset of the encode and the decode needs 64-bit
arithmetic.

- 64 tokens encoded at the last positions of the slot (bulk kernel), checked
  against the oracle outside the boundary window; the last one encoded again
  by the few-token kernel.
- One decode over all positions.  The positions never written are zero: their
  stored norm 0 gives score 0 and their zero min/max groups give value 0, so
  the expected output is the softmax over the 64 tokens' scores plus that many
  zero scores, in closed form from the oracle's dequantization of the 64
  tokens' GPU codes.
"""
import numpy as np
import pytest
import torch

from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import (OUT_RTOL, books, check_encode_slot, dequant_slot, encode_slot, layout_of, max_rel_err,
                        say, slot_from_cache)

pytestmark = pytest.mark.gpu

DEV = "cuda"
CAP = 72 << 20
N = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.lib()


@pytest.mark.timeout(300)
def test_offsets_beyond_2_gib():
    w = wl.WORKLOADS[3].replace(batch=1, h_q=4, h_kv=1, n_tokens=N, decode_steps=1)
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    cache = tq.Cache(layout_of(w), 1, 1, CAP, device=DEV)
    assert cache.k_planes.numel() > 2 ** 31 and cache.v_planes.numel() * 4 > 2 ** 31
    k, v = wl.prefill_kv(w)
    start = CAP - N
    say(f"[max size] slot of {CAP} positions: encode {N} tokens at {start}")
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [start], cache)
    torch.cuda.synchronize()
    ref = encode_slot(w, bk, pi, s, k[0, :, 0].double().numpy(), v[0, :, 0].double().numpy())
    ex = check_encode_slot(w, bk, cache, 0, 0, ref, start, N, "end of the slot")
    tq.encode_kv(prm, k[:, N - 1:N].contiguous().to(DEV), v[:, N - 1:N].contiguous().to(DEV), [CAP - 1], cache)
    torch.cuda.synchronize()
    ex_last = check_encode_slot(w, bk, cache, 0, 0, ref, start, N, "last position, few-token kernel")

    q = wl.query(w)
    out = tq.decode_attn(prm, q.to(DEV), cache, [CAP])
    torch.cuda.synchronize()
    kd, vd = dequant_slot(w, bk, pi, s, slot_from_cache(w, cache, 0, 0, N, start=start))
    qd = q.double().numpy()[0]
    sc = qd @ kd.T / np.sqrt(w.d)                      # [h_q, N]
    m = np.maximum(sc.max(axis=1), 0.0)                 # the zero positions score 0
    e = np.exp(sc - m[:, None])
    expect = (e @ vd) / (e.sum(axis=1) + (CAP - N) * np.exp(-m))[:, None]
    got = out.cpu().double().numpy()[0]
    err = max_rel_err(got, expect)
    say(f"  codes match outside the window (excused {list(ex)}, {list(ex_last)}); decode over {CAP} "
        f"positions: max rel err {err.max():.2e}")
    assert err.max() <= OUT_RTOL
