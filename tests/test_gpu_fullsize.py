"""GPU parity at full size, on sampled outputs.

Workloads:

- Batched decode: 32 sequences x 8 KV heads x 32768 tokens, keys 2-bit
  Lloyd-Max + QJL, values 2-bit min/max.
- Long context: 1 x 8 x 131072, keys 3-bit Lloyd-Max + QJL, values 3-bit
  Lloyd-Max.
- The Qwen2.5-1.5B-shaped layer (12 query heads, 2 KV heads) at N = 16384, and
  its literal 3-bit-MSE + QJL key variant with fp32 scalars.

All run with the launch shapes bench.py times (the same library calls on the
same tensor sizes; the split of the decode grid follows from the sizes).

Checks:

- The whole cache is encoded on the GPU.
- Sampled (sequence, KV head) slots are checked against the oracle: codes
  bit-exact outside the boundary window, norms to rounding.
- Decode steps run as in bench.py (ring append or direct encode, then decode).
- Each sampled slot's query heads are compared with the oracle decoding that
  slot's GPU codes, read back from the cache, so that the decode is compared on
  identical codes, within 2e-3 max relative error.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import (gamma_report, OUT_RTOL, books, check_encode_slot, dequant_slot, encode_slot, layout_of, max_rel_err,
                        say, slot_from_cache)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.lib()


def _sample_slots(w, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [(0, 0), (w.batch - 1, w.h_kv - 1)]
    extra = {(int(rng.integers(w.batch)), int(rng.integers(w.h_kv))) for _ in range(n)}
    return list(dict.fromkeys(fixed + sorted(extra)))[: n + 2]


def _check_decode(w, bk, pi, s, cache, q, out, slots, n_c, ring_k=None, ring_v=None, n_r=0, tag=""):
    """Oracle decode of the GPU-encoded codes of each sampled slot against the
    GPU output of that slot's query heads."""
    worst = 0.0
    G = w.group
    for b, h in slots:
        sc = slot_from_cache(w, cache, b, h, n_c)
        kd, vd = dequant_slot(w, bk, pi, s, sc)
        qs = q[b:b + 1, G * h:G * h + G].double().numpy()
        rk = rv = None
        if n_r:
            rk = ring_k[b:b + 1, :n_r, h:h + 1].cpu().double().numpy()
            rv = ring_v[b:b + 1, :n_r, h:h + 1].cpu().double().numpy()
        ref = oracle.decode_attention(qs, [[kd]], [[vd]], rk, rv, [n_r] if n_r else None)
        got = out[b:b + 1, G * h:G * h + G].cpu().double().numpy()
        err = max_rel_err(got, ref).max()
        worst = max(worst, err)
        assert err <= OUT_RTOL, f"{tag} slot (b={b}, h={h}): max rel err {err:.2e}"
    say(f"  {tag}: decode max rel err {worst:.2e} over {len(slots)} slots x {G} heads (bound {OUT_RTOL})")


@pytest.mark.timeout(600)
def test_fullsize_batched_b32_hkv8_n32768():
    w = wl.by_name("batched-b32-hkv8-n32768")
    say(f"[full size] {w.name}: generating {w.batch}x{w.n_tokens}x{w.h_kv}x{w.d} K and V")
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cap = w.n_tokens + w.ring_cap  # room for one ring flush, as bench.py sizes it
    cap = ((cap + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    say("  bulk encode on the GPU")
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    torch.cuda.synchronize()
    slots = _sample_slots(w, 3, seed=41)
    tot = np.zeros(3, dtype=np.int64)
    for b, h in slots:
        ref = encode_slot(w, bk, pi, s, k[b, :, h].double().numpy(), v[b, :, h].double().numpy())
        tot += check_encode_slot(w, bk, cache, b, h, ref, 0, w.n_tokens, f"b{b} h{h}")
    say(f"  encode: slots {slots} match outside the window; excused flips key MSE {tot[0]}, "
        f"key QJL {tot[1]} of {len(slots) * w.n_tokens * w.d} coordinates")
    say("  " + gamma_report())
    del k, v

    # decode steps as bench.py runs them: one call appends the step token to
    # the ring and attends (step 1 takes the two-call form, which must agree)
    rk = torch.zeros((w.batch, w.ring_cap, w.h_kv, w.d), dtype=torch.bfloat16, device=DEV)
    rv = torch.zeros_like(rk)
    ws = torch.empty(tq.decode_workspace_bytes(layout_of(w), w.batch, w.h_q, w.h_kv, cap),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((w.batch, w.h_q, w.d), dtype=torch.float32, device=DEV)
    n_r = 0
    for step in range(3):
        kn, vn = wl.step_kv(w, step)
        q = wl.query(w, step)
        if step == 1:
            tq.ring_append(kn.to(DEV).contiguous(), vn.to(DEV).contiguous(), rk, rv, [n_r] * w.batch)
            tq.decode_attn(prm, q.to(DEV), cache, [w.n_tokens] * w.batch, rk, rv, [n_r + 1] * w.batch, out=out,
                           workspace=ws)
        else:
            tq.decode_attn_append(prm, q.to(DEV), cache, [w.n_tokens] * w.batch, kn.to(DEV).contiguous(),
                                  vn.to(DEV).contiguous(), rk, rv, [n_r] * w.batch, out=out, workspace=ws)
        n_r += 1
        torch.cuda.synchronize()
        if step in (0, 2):
            _check_decode(w, bk, pi, s, cache, q, out, slots, w.n_tokens, rk, rv, n_r, tag=f"step {step}")


@pytest.mark.timeout(600)
def test_fullsize_long_b1_hkv8_n131072():
    w = wl.by_name("long-b1-hkv8-n131072")
    say(f"[full size] {w.name}: generating {w.batch}x{w.n_tokens}x{w.h_kv}x{w.d} K and V")
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cap = ((w.n_tokens + w.decode_steps + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    say("  bulk encode on the GPU")
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    torch.cuda.synchronize()
    slots = [(0, 0), (0, 3), (0, 7)]
    tot = np.zeros(3, dtype=np.int64)
    for b, h in slots:
        ref = encode_slot(w, bk, pi, s, k[b, :, h].double().numpy(), v[b, :, h].double().numpy())
        tot += check_encode_slot(w, bk, cache, b, h, ref, 0, w.n_tokens, f"b{b} h{h}")
    say(f"  encode: slots {slots} match outside the window; excused flips key MSE {tot[0]}, "
        f"key QJL {tot[1]}, value {tot[2]} of {len(slots) * w.n_tokens * w.d} coordinates")
    say("  " + gamma_report())
    del k, v

    ws = torch.empty(tq.decode_workspace_bytes(layout_of(w), w.batch, w.h_q, w.h_kv, cap),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((w.batch, w.h_q, w.d), dtype=torch.float32, device=DEV)
    n_c = w.n_tokens
    for step in range(3):
        # bench.py's step for this workload: encode the step token in place, then attend
        kn, vn = wl.step_kv(w, step)
        tq.encode_kv(prm, kn.to(DEV).contiguous(), vn.to(DEV).contiguous(), [n_c] * w.batch, cache)
        n_c += 1
        q = wl.query(w, step)
        tq.decode_attn(prm, q.to(DEV), cache, [n_c] * w.batch, out=out, workspace=ws)
        torch.cuda.synchronize()
        if step in (0, 2):
            _check_decode(w, bk, pi, s, cache, q, out, slots, n_c, tag=f"step {step}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["qwen2.5-1.5b-layer-n16384", "qwen2.5-1.5b-layer-n4096-k4bit-f32scalars"])
def test_fullsize_qwen_layer(name):
    """The Qwen2.5-1.5B-shaped layer (12 query heads on 2 KV heads: 6 per KV
    head, two 4-head MFMA tiles) at its longest sweep length, and the literal
    3-bit-MSE + QJL key variant with fp32 scalars; every slot checked."""
    w = wl.by_name(name)
    say(f"[full size] {w.name}")
    bk = books(w)
    pi, s = wl.params(w)
    prm = tq.Params(layout_of(w), pi, s, device=DEV)
    k, v = wl.prefill_kv(w)
    cap = ((w.n_tokens + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    torch.cuda.synchronize()
    slots = [(b, h) for b in range(w.batch) for h in range(w.h_kv)]
    tot = np.zeros(3, dtype=np.int64)
    for b, h in slots:
        ref = encode_slot(w, bk, pi, s, k[b, :, h].double().numpy(), v[b, :, h].double().numpy())
        tot += check_encode_slot(w, bk, cache, b, h, ref, 0, w.n_tokens, f"b{b} h{h}")
    say(f"  encode: all {len(slots)} slots match outside the window; excused flips key MSE {tot[0]}, "
        f"key QJL {tot[1]}, value {tot[2]} of {len(slots) * w.n_tokens * w.d} coordinates")
    say("  " + gamma_report())
    q = wl.query(w, 0)
    out = tq.decode_attn(prm, q.to(DEV), cache, [w.n_tokens] * w.batch)
    torch.cuda.synchronize()
    _check_decode(w, bk, pi, s, cache, q, out, slots, w.n_tokens, tag="decode")
