"""GPU parity of the few-token encode (calls with at most 4 new tokens per
sequence, as in a decode step that encodes its token directly, and any call
under TQ_ENCODE_PATH=small): codes bit-exact with the oracle outside the
boundary window, norms to rounding, and the neighbouring positions of the
shared 32-token value blocks preserved.

- A prefix encoded by the bulk (MFMA) kernel, then three one-token appends per
  sequence at ragged positions through the few-token kernel; every position
  of the slot is checked, so the appended tokens and their neighbours are.
- Whole sequences forced through the few-token kernel (several tokens per
  work-group, partial blocks at both ends).
Layouts: 2+1-bit keys with min/max values (fp32 inputs), 3+1-bit keys with
3-bit MSE values (bf16), fp16 scalars, and the 3.5- and 2.5-bit key widths.
"""
import numpy as np
import pytest
import torch

from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import books, check_encode_slot, encode_slot, layout_of, say

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    "2+1-bit keys, min/max values, fp32 inputs": wl.WORKLOADS[1].replace(batch=2, n_tokens=300),
    "3+1-bit keys, MSE values": wl.WORKLOADS[4].replace(n_tokens=260, decode_steps=1),
    "qwen layer, fp16 scalars": wl.by_name("qwen2.5-1.5b-layer-n512").replace(n_tokens=200),
    "3.5-bit keys": wl.WORKLOADS[3].replace(batch=2, n_tokens=230, decode_steps=1, key_half=1),
    "2.5-bit keys": wl.WORKLOADS[3].replace(batch=2, n_tokens=230, decode_steps=1, key_half=1, key_mse_bits=1),
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


def _check(w, bk, pi, s, cache, k, v, b, h, start, n, tag):
    ref = encode_slot(w, bk, pi, s, k[b, start:start + n, h].double().numpy(), v[b, start:start + n, h].double().numpy())
    return check_encode_slot(w, bk, cache, b, h, ref, start, n, tag)


@pytest.mark.parametrize("name", list(CASES))
def test_one_token_appends_after_bulk_prefix(name):
    w = CASES[name]
    bk, pi, s, prm, k, v = _setup(w)
    cap = ((w.n_tokens + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    P = w.n_tokens - 40                      # bulk prefix (many tokens: the bulk kernel)
    offs = [0, 13][:w.batch]                 # ragged append positions, sharing value blocks with the prefix
    tq.encode_kv(prm, k[:, :P].contiguous().to(DEV), v[:, :P].contiguous().to(DEV), [0] * w.batch, cache)
    for j in range(3):                       # one token per call: the few-token kernel
        pos = [P + offs[b] + j for b in range(w.batch)]
        kn = torch.stack([k[b, pos[b]:pos[b] + 1] for b in range(w.batch)]).contiguous()
        vn = torch.stack([v[b, pos[b]:pos[b] + 1] for b in range(w.batch)]).contiguous()
        tq.encode_kv(prm, kn.to(DEV), vn.to(DEV), pos, cache)
    torch.cuda.synchronize()
    tot = np.zeros(3, dtype=np.int64)
    for b in range(w.batch):
        for h in range(w.h_kv):
            tot += _check(w, bk, pi, s, cache, k, v, b, h, 0, P, f"{name} prefix b{b} h{h}")
            tot += _check(w, bk, pi, s, cache, k, v, b, h, P + offs[b], 3, f"{name} appended b{b} h{h}")
    say(f"[few-token encode] {name}: prefix {P}, appends at {[P + o for o in offs]}; excused flips "
        f"MSE {tot[0]}, QJL {tot[1]}, values {tot[2]}")


@pytest.mark.parametrize("name", list(CASES))
def test_whole_sequences_through_the_few_token_kernel(name, monkeypatch):
    w = CASES[name]
    bk, pi, s, prm, k, v = _setup(w)
    n = w.n_tokens - 10
    start = 5                                 # partial first and last 32-token blocks
    cap = ((start + n + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    monkeypatch.setenv("TQ_ENCODE_PATH", "small")
    kin = torch.zeros((w.batch, n, w.h_kv, w.d), dtype=k.dtype)
    vin = torch.zeros_like(kin)
    kin[:] = k[:, start:start + n]
    vin[:] = v[:, start:start + n]
    tq.encode_kv(prm, kin.to(DEV), vin.to(DEV), [start] * w.batch, cache)
    torch.cuda.synchronize()
    tot = np.zeros(3, dtype=np.int64)
    for b in range(w.batch):
        for h in range(w.h_kv):
            tot += _check(w, bk, pi, s, cache, k, v, b, h, start, n, f"{name} forced b{b} h{h}")
    say(f"[few-token encode, forced] {name}: {n} tokens from position {start}; excused flips "
        f"MSE {tot[0]}, QJL {tot[1]}, values {tot[2]}")


def _hip_events():
    import ctypes
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    a, b = ctypes.c_void_p(), ctypes.c_void_p()
    assert h.hipEventCreate(ctypes.byref(a)) == 0 and h.hipEventCreate(ctypes.byref(b)) == 0
    return h, a, b


@pytest.mark.parametrize("name", ["3+1-bit keys, MSE values", "qwen layer, fp16 scalars"])
def test_one_launch_and_two_launches_write_the_same_codes(name):
    """Few-token calls with MSE values encode keys and values in one launch;
    a call that asks to time the key kernel takes two launches instead.  Both
    run the same per-token code, so the caches must agree bit for bit."""
    w = CASES[name]
    _, _, _, prm, k, v = _setup(w)
    cap = ((w.n_tokens + 31) // 32) * 32
    P = w.n_tokens - 6
    caches = []
    h, ea, eb = _hip_events()
    for timed in (False, True):
        cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
        tq.encode_kv(prm, k[:, :P].contiguous().to(DEV), v[:, :P].contiguous().to(DEV), [0] * w.batch, cache)
        for j in range(3):
            pos = [P + j] * w.batch
            if timed:
                tq.time_next_launch(tq.TQ_KERNEL_ENCODE_KEYS, ea, eb)
            tq.encode_kv(prm, k[:, P + j:P + j + 1].contiguous().to(DEV), v[:, P + j:P + j + 1].contiguous().to(DEV),
                         pos, cache)
        torch.cuda.synchronize()
        caches.append(cache)
    h.hipEventDestroy(ea)
    h.hipEventDestroy(eb)
    a, b = caches
    for field in ("k_planes", "k_norm", "k_rnorm", "v_planes", "v_norm"):
        assert torch.equal(getattr(a, field), getattr(b, field)), field
    say(f"[few-token encode] {name}: one launch and two launches give identical caches")
