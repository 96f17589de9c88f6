"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Encode: packed codes bit-exact except where the oracle's rotated coordinate (or
QJL projection) lies within 1e-5 of a decision boundary, mismatch counts
printed; min/max value codes and fp16 scale/zero bit-exact; stored norms within
fp32 rounding (fp16: one ulp).  Decode: both sides read the same oracle-packed
cache, each attention output vector within 2e-3 max relative error.
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl
from tq_testlib import (DECODE_PATHS, set_decode_path, gamma_report, OUT_RTOL, books, check_encode_slot, dequant_slot, encode_slot, key_plane_mismatches, key_records,
                        layout_of, max_rel_err, read_value_planes, say, slot_from_cache, upload_slot)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.lib()


SMALL = {
    "single": wl.WORKLOADS[0],
    "gqa4": wl.WORKLOADS[1],
    "qwen_k3_f16": wl.QWEN_VARIANTS[0].replace(n_tokens=2048),
    "qwen_k3_f32": wl.QWEN_VARIANTS[2].replace(n_tokens=1024),
    "qwen": wl.by_name("qwen2.5-1.5b-layer-n4096").replace(n_tokens=1536),
    "batched_small": wl.WORKLOADS[3].replace(batch=3, n_tokens=640, decode_steps=1),
    "long_small": wl.WORKLOADS[4].replace(n_tokens=1024, decode_steps=1),
}


def _params(w):
    pi, s = wl.params(w)
    return pi, s, tq.Params(layout_of(w), pi, s, device=DEV)


@pytest.mark.parametrize("name", list(SMALL))
def test_encode_parity(name):
    w = SMALL[name]
    say(f"[encode parity] {name}: B={w.batch} H_kv={w.h_kv} N={w.n_tokens} {w.in_dtype}")
    bk = books(w)
    pi, s, prm = _params(w)
    k, v = wl.prefill_kv(w)
    cap = ((w.n_tokens + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    torch.cuda.synchronize()
    tot = np.zeros(3, dtype=np.int64)
    for b in range(w.batch):
        for h in range(w.h_kv):
            ref = encode_slot(w, bk, pi, s, k[b, :, h].double().numpy(), v[b, :, h].double().numpy())
            tot += check_encode_slot(w, bk, cache, b, h, ref, 0, w.n_tokens, f"{name} b{b} h{h}")
    n_coord = w.batch * w.h_kv * w.n_tokens * w.d
    say(f"  excused flips: key MSE {tot[0]}, key QJL {tot[1]}, value {tot[2]} of {n_coord} coordinates")
    say("  " + gamma_report())


@pytest.mark.parametrize("bits,group", [(1, 32), (2, 16), (2, 64), (3, 32), (4, 16), (4, 64)])
def test_encode_minmax_widths_and_groups(bits, group):
    """GPU min/max value codes for every width and group size, against the
    oracle (codes bit-exact outside the window, fp16 delta and minimum exact),
    with a ragged start so the first and last 32-token blocks are partial."""
    w = SMALL["batched_small"].replace(batch=2, h_kv=2, h_q=8, n_tokens=150, value_bits=bits, value_group=group)
    say(f"[encode min/max] {bits}-bit values, groups of {group}")
    bk = books(w)
    pi, s, prm = _params(w)
    k, v = wl.prefill_kv(w)
    start = 7
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, 192, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [start] * w.batch, cache)
    torch.cuda.synchronize()
    tot = np.zeros(3, dtype=np.int64)
    for b in range(w.batch):
        for h in range(w.h_kv):
            ref = encode_slot(w, bk, pi, s, k[b, :, h].double().numpy(), v[b, :, h].double().numpy())
            tot += check_encode_slot(w, bk, cache, b, h, ref, start, w.n_tokens, f"{bits}b g{group} b{b} h{h}")
    say(f"  excused value flips {tot[2]}")
    say("  " + gamma_report())


@pytest.mark.parametrize("path", ["mfma", "small"])
@pytest.mark.parametrize("kbits,qjl,vbits", [(1, 1, 1), (2, 0, 2), (3, 0, 4), (4, 1, 2), (4, 0, 3), (1, 0, 4)])
def test_encode_key_and_mse_value_widths(kbits, qjl, vbits, path, monkeypatch):
    """GPU key codes for every index width with and without the QJL bit, and
    MSE value codes for every width, on the bulk (MFMA) and the few-token
    kernels, against the oracle outside the boundary window."""
    monkeypatch.setenv("TQ_ENCODE_PATH", path)
    w = SMALL["long_small"].replace(batch=2, n_tokens=100, key_mse_bits=kbits, key_qjl=qjl, value_bits=vbits)
    say(f"[encode widths] keys {kbits}{'+1' if qjl else ''}, MSE values {vbits} ({path})")
    bk = books(w)
    pi, s, prm = _params(w)
    k, v = wl.prefill_kv(w)
    start = 3
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, 128, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [start] * w.batch, cache)
    torch.cuda.synchronize()
    tot = np.zeros(3, dtype=np.int64)
    for b in range(w.batch):
        for h in range(w.h_kv):
            ref = encode_slot(w, bk, pi, s, k[b, :, h].double().numpy(), v[b, :, h].double().numpy())
            tot += check_encode_slot(w, bk, cache, b, h, ref, start, w.n_tokens, f"k{kbits} q{qjl} v{vbits} b{b} h{h}")
    say(f"  excused flips: key MSE {tot[0]}, key QJL {tot[1]}, value {tot[2]}")
    say("  " + gamma_report())


@pytest.mark.parametrize("value_kind", ["minmax", "mse"])
def test_encode_ragged_positions_preserve_neighbours(value_kind):
    base = SMALL["batched_small"] if value_kind == "minmax" else SMALL["long_small"]
    w = base.replace(batch=3, h_kv=2, h_q=8, n_tokens=77)
    say(f"[encode ragged] {value_kind}")
    bk = books(w)
    pi, s, prm = _params(w)
    k, v = wl.prefill_kv(w)
    cap = 256
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(5)
    for t in (cache.k_planes, cache.v_planes):
        t.copy_(torch.randint(0, 255 if t.dtype == torch.uint8 else 2 ** 31 - 1, t.shape, generator=g, dtype=t.dtype))
    before = {n: getattr(cache, n).clone() for n in ("k_planes", "v_planes")}
    pos = [0, 45, 179]
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), pos, cache)
    torch.cuda.synchronize()
    for b in range(3):
        p0 = pos[b]
        # key records outside the written range are untouched
        kp = key_records(w, cache.k_planes[b])
        kb = key_records(w, before["k_planes"][b])
        mask = torch.ones(cap, dtype=torch.bool)
        mask[p0:p0 + 77] = False
        assert np.array_equal(kp[:, mask.numpy()], kb[:, mask.numpy()])
        # value bits of untouched tokens in shared blocks are preserved
        for h in range(w.h_kv):
            va = read_value_planes(cache.v_planes[b, h].cpu().numpy(), cap, w)
            vbh = read_value_planes(before["v_planes"][b, h].cpu().numpy(), cap, w)
            assert np.array_equal(va[mask.numpy()], vbh[mask.numpy()])
            ref = encode_slot(w, bk, pi, s, k[b, :, h].double().numpy(), v[b, :, h].double().numpy())
            check_encode_slot(w, bk, cache, b, h, ref, p0, 77, f"ragged b{b} h{h}")


def _oracle_cache(w, bk, pi, s, k, v, n_comp):
    """Oracle codes per slot and their dequantized K/V."""
    codes, kd, vd = {}, [], []
    for b in range(w.batch):
        kr, vr = [], []
        for h in range(w.h_kv):
            n = n_comp[b]
            sc = encode_slot(w, bk, pi, s, k[b, :n, h].double().numpy(), v[b, :n, h].double().numpy())
            codes[b, h] = sc
            a, c = dequant_slot(w, bk, pi, s, sc)
            kr.append(a)
            vr.append(c)
        kd.append(kr)
        vd.append(vr)
    return codes, kd, vd


def _decode_case(w, n_comp, n_ring, tag, steps_kv=None):
    say(f"[decode parity] {tag}: B={w.batch} H_q={w.h_q} H_kv={w.h_kv} n={n_comp} ring={n_ring}")
    bk = books(w)
    pi, s, prm = _params(w)
    k, v = wl.prefill_kv(w)
    cap = max(32, ((max(n_comp) + 31) // 32) * 32)
    codes, kd, vd = _oracle_cache(w, bk, pi, s, k, v, n_comp)
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    for (b, h), sc in codes.items():
        if n_comp[b] > 0:
            upload_slot(cache, w, b, h, sc)
    q = wl.query(w)
    rk = rv = None
    if max(n_ring) > 0:
        g = np.random.default_rng(11)
        rk = torch.from_numpy(g.standard_normal((w.batch, 128, w.h_kv, w.d))).to(torch.bfloat16)
        rv = torch.from_numpy(g.standard_normal((w.batch, 128, w.h_kv, w.d))).to(torch.bfloat16)
    out = tq.decode_attn(prm, q.to(DEV), cache, n_comp, None if rk is None else rk.to(DEV),
                         None if rv is None else rv.to(DEV), n_ring)
    torch.cuda.synchronize()
    ref = oracle.decode_attention(q.double().numpy(), kd, vd,
                                  None if rk is None else rk.double().numpy(),
                                  None if rv is None else rv.double().numpy(), n_ring)
    got = out.cpu().double().numpy()
    err = max_rel_err(got, ref)
    say(f"  max rel err {err.max():.2e} (bound {OUT_RTOL})")
    for b in range(w.batch):
        if n_comp[b] == 0 and n_ring[b] == 0:
            assert np.all(got[b] == 0)
    assert err.max() <= OUT_RTOL
    return got


@pytest.mark.parametrize("path", DECODE_PATHS)
@pytest.mark.parametrize("name", list(SMALL))
def test_decode_parity(name, path, monkeypatch):
    """Both decode paths: the int8-MFMA bit-plane scan (taken for symmetric
    codebooks) and the generic scan (forced with TQ_DECODE_PATH=generic)."""
    set_decode_path(monkeypatch, path)
    w = SMALL[name]
    nr = [1] * w.batch if w.ring_cap else [0] * w.batch
    _decode_case(w, [w.n_tokens] * w.batch, nr, f"{name} ({path})")


def test_decode_ragged_lengths_and_ring_sizes():
    w = SMALL["batched_small"].replace(batch=5, n_tokens=1000)
    _decode_case(w, [0, 37, 1000, 513, 64], [5, 0, 128, 127, 1], "ragged minmax")
    w = SMALL["long_small"].replace(batch=3, n_tokens=700)
    _decode_case(w, [700, 1, 256], [0, 0, 0], "ragged mse")


def test_decode_layouts_outside_the_mfma_path():
    """Layouts the MFMA scan does not cover run on the generic scan."""
    base = SMALL["batched_small"].replace(batch=2, n_tokens=300)
    _decode_case(base.replace(key_mse_bits=1, value_bits=4, value_group=16), [300, 200], [2, 0], "k1 v4 g16")
    _decode_case(base.replace(key_mse_bits=4, value_bits=1, value_group=64), [300, 5], [0, 1], "k4 v1 g64")
    _decode_case(SMALL["long_small"].replace(value_bits=2, key_mse_bits=1, n_tokens=300), [300], [0], "k1 mse v2")


@pytest.mark.parametrize("path", DECODE_PATHS)
def test_decode_two_bit_mse_values(path, monkeypatch):
    """2-bit MSE values (two value planes) with 2+1- and 3+1-bit keys, on both
    scan paths."""
    set_decode_path(monkeypatch, path)
    w = SMALL["long_small"].replace(value_bits=2, n_tokens=300)
    _decode_case(w, [300], [0], f"3+1-bit keys, 2-bit MSE values ({path})")
    _decode_case(w.replace(key_mse_bits=2, batch=2), [300, 97], [0, 0], f"2+1-bit keys, 2-bit MSE values ({path})")


@pytest.mark.parametrize("path", DECODE_PATHS)
def test_decode_four_bit_minmax_values(path, monkeypatch):
    """4-bit min/max values in groups of 32 (packed, eight tokens per word),
    with 2+1-, 3+1- and 3.5-bit keys, on both scan paths (the generic scan has
    no half-bit keys)."""
    set_decode_path(monkeypatch, path)
    base = SMALL["batched_small"].replace(batch=2, n_tokens=300, value_bits=4)
    _decode_case(base, [300, 133], [3, 0], f"4-bit values ({path})")
    _decode_case(base.replace(key_mse_bits=3), [300, 64], [0, 2], f"3+1-bit keys, 4-bit values ({path})")
    if path == "mfma":
        _decode_case(base.replace(key_half=1), [257, 300], [1, 0], "3.5-bit keys, 4-bit values (mfma)")


def test_four_bit_minmax_values_end_to_end():
    """GPU encode of 4-bit min/max values (packed words) then GPU decode,
    against the oracle decoding the GPU's codes."""
    w = SMALL["batched_small"].replace(batch=2, n_tokens=320, value_bits=4)
    bk = books(w)
    pi, s, prm = _params(w)
    k, v = wl.prefill_kv(w)
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, 320, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    n_comp = [320, 201]
    tot = np.zeros(3, dtype=np.int64)
    for b in range(w.batch):
        for h in range(w.h_kv):
            ref = encode_slot(w, bk, pi, s, k[b, :, h].double().numpy(), v[b, :, h].double().numpy())
            tot += check_encode_slot(w, bk, cache, b, h, ref, 0, w.n_tokens, f"4-bit values b{b} h{h}")
    q = wl.query(w)
    out = tq.decode_attn(prm, q.to(DEV), cache, n_comp)
    torch.cuda.synchronize()
    kd, vd = [], []
    for b in range(w.batch):
        kr, vr = [], []
        for h in range(w.h_kv):
            a_, c_ = dequant_slot(w, bk, pi, s, slot_from_cache(w, cache, b, h, n_comp[b]))
            kr.append(a_)
            vr.append(c_)
        kd.append(kr)
        vd.append(vr)
    ref = oracle.decode_attention(q.double().numpy(), kd, vd)
    err = max_rel_err(out.cpu().double().numpy(), ref)
    say(f"[4-bit values end to end] codes match (excused {tot.tolist()}); decode max rel err {err.max():.2e}")
    say("  " + gamma_report())
    assert err.max() <= OUT_RTOL


@pytest.mark.parametrize("path", DECODE_PATHS)
def test_decode_one_bit_keys(path, monkeypatch):
    """1-bit key indices (TurboQuantProd(2) and the 1-bit MSE-only keys), with
    min/max and MSE values, on both scan paths."""
    set_decode_path(monkeypatch, path)
    base = SMALL["batched_small"].replace(batch=2, n_tokens=300, key_mse_bits=1)
    _decode_case(base, [300, 190], [2, 0], f"1+1-bit keys ({path})")
    _decode_case(base.replace(key_qjl=0), [300, 64], [0, 1], f"1-bit keys, no qjl ({path})")
    mse = SMALL["long_small"].replace(n_tokens=300, key_mse_bits=1)
    _decode_case(mse, [300], [0], f"1+1-bit keys, MSE values ({path})")


@pytest.mark.parametrize("path", DECODE_PATHS)
def test_decode_keys_without_qjl(path, monkeypatch):
    """MSE-only keys (no QJL bit), 2 and 3 index bits, with min/max and MSE
    values, on both scan paths."""
    set_decode_path(monkeypatch, path)
    base = SMALL["batched_small"].replace(batch=2, n_tokens=300, key_qjl=0)
    _decode_case(base, [300, 256], [1, 1], f"no qjl, 2-bit keys ({path})")
    _decode_case(base.replace(key_mse_bits=3), [300, 77], [0, 3], f"no qjl, 3-bit keys ({path})")
    mse = SMALL["long_small"].replace(n_tokens=300, key_qjl=0)
    _decode_case(mse, [300], [0], f"no qjl, MSE values ({path})")
    _decode_case(mse.replace(key_mse_bits=2), [211], [0], f"no qjl, 2-bit keys, MSE values ({path})")


@pytest.mark.parametrize("path", DECODE_PATHS)
@pytest.mark.parametrize("kbits,qjl,vkind,vbits,group", [
    (4, 1, "minmax", 3, 32), (4, 0, "minmax", 1, 16), (3, 0, "minmax", 3, 64), (1, 1, "minmax", 1, 32),
    (2, 1, "minmax", 2, 16), (2, 1, "minmax", 4, 64), (4, 1, "mse", 1, 32), (1, 0, "mse", 4, 32),
    (3, 1, "mse", 2, 32), (4, 0, "mse", 4, 32)])
def test_decode_layout_sweep(kbits, qjl, vkind, vbits, group, path, monkeypatch):
    """Decode of oracle-encoded caches over key widths with and without QJL,
    min/max widths and group sizes and MSE value widths, on both scan paths
    (layouts the MFMA scan does not cover run on the generic scan either way)."""
    set_decode_path(monkeypatch, path)
    base = SMALL["batched_small"] if vkind == "minmax" else SMALL["long_small"]
    w = base.replace(batch=2, n_tokens=260, key_mse_bits=kbits, key_qjl=qjl, value_bits=vbits, value_group=group)
    nr = [2, 0] if w.ring_cap else [0, 0]
    _decode_case(w, [260, 131], nr, f"k{kbits}{'+1' if qjl else ''} {vkind} v{vbits} g{group} ({path})")


def test_decode_empty_sequence_gives_zero():
    w = SMALL["batched_small"].replace(batch=2, n_tokens=64)
    _decode_case(w, [0, 64], [0, 3], "empty")


def test_decode_group_sizes():
    for g, hk in ((1, 4), (2, 2), (3, 2), (5, 1), (8, 1)):
        w = SMALL["gqa4"].replace(h_kv=hk, h_q=g * hk, n_tokens=300)
        _decode_case(w, [300], [1], f"G={g}")


@pytest.mark.parametrize("n", [8192, 8448, 32768])
@pytest.mark.parametrize("name", ["batched_small", "long_small"])
def test_decode_combine_split_counts(name, n):
    """One slot of n tokens in 256-token splits: 32 splits (the combine's
    short prefetch, eight per quarter), 33 (its long prefetch) and 128 (past
    the long prefetch's 24 per quarter, so the rest come in batches), with
    min/max and MSE values and five ring tokens."""
    w = SMALL[name].replace(batch=1, h_kv=1, h_q=4, n_tokens=n)
    _decode_case(w, [n], [5], f"{name} n={n}")


def test_decode_split_invariance_and_determinism():
    """The same slot decoded alone (sixteen 256-token splits) and among 192
    copies (four 1024-token splits) gives the same output to fp32 rounding;
    repeated calls are bitwise identical."""
    w = SMALL["batched_small"].replace(batch=1, h_kv=1, h_q=4, n_tokens=4096)
    bk = books(w)
    pi, s, prm = _params(w)
    k, v = wl.prefill_kv(w)
    codes, _, _ = _oracle_cache(w, bk, pi, s, k, v, [4096])
    say("[decode split invariance]")
    outs = []
    for copies in (1, 192):
        cache = tq.Cache(layout_of(w), copies, 1, 4096, device=DEV)
        for b in range(copies):
            upload_slot(cache, w, b, 0, codes[0, 0])
        q = wl.query(w).repeat(copies, 1, 1)
        o1 = tq.decode_attn(prm, q.to(DEV), cache, [4096] * copies)
        o2 = tq.decode_attn(prm, q.to(DEV), cache, [4096] * copies)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        outs.append(o1[0].cpu().double().numpy())
    assert np.max(max_rel_err(outs[0], outs[1])) < 1e-5


@pytest.mark.parametrize("name", ["single", "gqa4", "qwen", "batched_small", "long_small"])
def test_end_to_end(name):
    """GPU encode + ring append + GPU decode against oracle encode + oracle decode
    from the same raw inputs (rare boundary-window code flips included)."""
    w = SMALL[name]
    # sizes with few enough boundary flips to leave clean KV slots to compare
    w = w.replace(n_tokens=min(w.n_tokens, 1024)) if name != "qwen" else w.replace(batch=4, n_tokens=256)
    say(f"[end to end] {name}")
    bk = books(w)
    pi, s, prm = _params(w)
    k, v = wl.prefill_kv(w)
    n = w.n_tokens
    cap = ((n + 31) // 32) * 32
    cache = tq.Cache(layout_of(w), w.batch, w.h_kv, cap, device=DEV)
    tq.encode_kv(prm, k.to(DEV), v.to(DEV), [0] * w.batch, cache)
    q = wl.query(w)
    n_ring = [0] * w.batch
    rk = rv = None
    if w.step_mode == "ring":
        kn, vn = wl.step_kv(w, 0)
        rk = torch.zeros((w.batch, w.ring_cap, w.h_kv, w.d), dtype=torch.bfloat16, device=DEV)
        rv = torch.zeros_like(rk)
        tq.ring_append(kn.to(DEV).contiguous(), vn.to(DEV).contiguous(), rk, rv, n_ring)
        n_ring = [1] * w.batch
    out = tq.decode_attn(prm, q.to(DEV), cache, [n] * w.batch, rk, rv, n_ring)
    torch.cuda.synchronize()
    _, kd, vd = _oracle_cache(w, bk, pi, s, k, v, [n] * w.batch)
    ring_k = ring_v = None
    if rk is not None:
        # the ring holds bf16(k_new): the oracle reads the same rounding of the step token
        ring_k = np.zeros((w.batch, 1, w.h_kv, w.d))
        ring_v = np.zeros_like(ring_k)
        ring_k[:, 0] = kn[:, 0].to(torch.bfloat16).double().numpy()
        ring_v[:, 0] = vn[:, 0].to(torch.bfloat16).double().numpy()
        assert torch.equal(rk[:, 0].cpu(), kn[:, 0].to(torch.bfloat16))
    ref = oracle.decode_attention(q.double().numpy(), kd, vd, ring_k, ring_v, n_ring)
    err = max_rel_err(out.cpu().double().numpy(), ref)
    # a key whose code flipped inside the boundary window (allowed by the
    # encode parity rule) changes its score; the 2e-3 output bound applies to
    # the query heads whose KV slot has no such flip
    codes, _, _ = _oracle_cache(w, bk, pi, s, k, v, [n] * w.batch)
    flipped = np.zeros((w.batch, w.h_kv), dtype=bool)
    for (b, h), sc in codes.items():
        _, ex_m, ex_q = key_plane_mismatches(w, bk, key_records(w, cache.k_planes[b, h])[:n], sc.key)
        idx_g = read_value_planes(cache.v_planes[b, h].cpu().numpy(), n, w)
        ex_v = int(np.sum(idx_g != (sc.val.code if w.value_kind == "minmax" else sc.val.idx)))
        flipped[b, h] = (ex_m + ex_q + ex_v) > 0
    hq_flip = np.repeat(flipped, w.group, axis=1)
    say(f"  max rel err {err[~hq_flip].max() if (~hq_flip).any() else 0:.2e} over {int((~hq_flip).sum())} heads "
        f"without boundary flips; {err[hq_flip].max() if hq_flip.any() else 0:.2e} over {int(hq_flip.sum())} "
        f"heads whose KV slot has flips")
    assert (~hq_flip).any(), "every KV slot has a boundary flip: nothing left to compare"
    assert err[~hq_flip].max() <= OUT_RTOL
