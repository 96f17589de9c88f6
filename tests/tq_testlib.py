"""Shared helpers of the GPU parity tests: oracle-side encoding of whole cache
slots, upload of oracle-packed caches into device tensors, and the comparison
rules (boundary windows for codes, relative bounds for outputs)."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import oracle
from compressed_kv_decode_tq_amd import tq
from compressed_kv_decode_tq_amd import workloads as wl

WINDOW = 1e-5          # codes may differ only where the oracle's coordinate is this close to a boundary
OUT_RTOL = 2e-3        # max relative error of an attention output vector

# Largest |gamma_gpu - gamma_oracle| seen by check_encode_slot (fp32 scalars),
# reported by gamma_report().
_GAMMA_ERR = {"max": 0.0, "tokens": 0}


def gamma_report() -> str:
    """Largest residual-norm error seen since the last report, then reset."""
    r = (f"max |gamma - gamma_oracle| {_GAMMA_ERR['max']:.2e} over {_GAMMA_ERR['tokens']} tokens "
         f"(bound {WINDOW:g} * sqrt(d))")
    _GAMMA_ERR.update(max=0.0, tokens=0)
    return r


#: Decode paths the parity tests run: the MFMA scan ("mfma") and the VALU
#: scan ("generic").
DECODE_PATHS = ["mfma", "generic"]


def set_decode_path(monkeypatch, path: str):
    """Force one decode path for the rest of the test."""
    if path == "generic":
        monkeypatch.setenv("TQ_DECODE_PATH", "generic")
    else:
        monkeypatch.delenv("TQ_DECODE_PATH", raising=False)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def layout_of(w: wl.Workload) -> tq.Layout:
    return tq.Layout(head_dim=w.d, key_mse_bits=w.key_mse_bits, key_qjl=w.key_qjl,
                     value_kind=tq.TQ_V_MINMAX if w.value_kind == "minmax" else tq.TQ_V_MSE,
                     value_bits=w.value_bits, value_group=w.value_group,
                     scalar_dtype=tq.TQ_F32 if w.scalar_dtype == "f32" else tq.TQ_F16, key_half=w.key_half)


def olayout_of(w: wl.Workload) -> oracle.Layout:
    return oracle.Layout(d=w.d, key_mse_bits=w.key_mse_bits, key_qjl=w.key_qjl,
                         value_kind=w.value_kind, value_bits=w.value_bits,
                         value_group=w.value_group, scalar_dtype=w.scalar_dtype, key_half=w.key_half)


@dataclasses.dataclass
class OracleBooks:
    k: oracle.Codebook
    v: oracle.Codebook | None
    k_hi: oracle.Codebook | None = None  # half-bit keys: the (key_mse_bits + 1)-bit table


def books(w: wl.Workload) -> OracleBooks:
    return OracleBooks(oracle.lloyd_max(w.d, w.key_mse_bits),
                       oracle.lloyd_max(w.d, w.value_bits) if w.value_kind == "mse" else None,
                       oracle.lloyd_max(w.d, w.key_mse_bits + 1) if w.key_half else None)


def _hi(bk: OracleBooks):
    return (bk.k_hi.centroids, bk.k_hi.thresholds) if bk.k_hi is not None else (None, None)


@dataclasses.dataclass
class SlotCode:
    """Oracle encoding of the tokens of one (sequence, KV head) slot."""
    key: oracle.KeyCode
    val: object  # ValueMinMax | ValueMSE


def encode_slot(w: wl.Workload, bk: OracleBooks, pi, s, k: np.ndarray, v: np.ndarray) -> SlotCode:
    ch, th = _hi(bk)
    key = oracle.encode_keys(k, pi, s, bk.k.centroids, bk.k.thresholds, w.scalar_dtype, qjl=bool(w.key_qjl),
                             centroids_hi=ch, thresholds_hi=th)
    if w.value_kind == "minmax":
        val = oracle.encode_values_minmax(v, w.value_bits, w.value_group)
    else:
        val = oracle.encode_values_mse(v, pi, bk.v.centroids, bk.v.thresholds, w.scalar_dtype)
    return SlotCode(key, val)


def dequant_slot(w: wl.Workload, bk: OracleBooks, pi, s, sc: SlotCode):
    kd = oracle.dequantize_keys(sc.key, pi, s, bk.k.centroids, qjl=bool(w.key_qjl), centroids_hi=_hi(bk)[0])
    if w.value_kind == "minmax":
        vd = oracle.dequantize_values_minmax(sc.val, w.value_group)
    else:
        vd = oracle.dequantize_values_mse(sc.val, pi, bk.v.centroids)
    return kd, vd


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def key_records(w: wl.Workload, blocks: torch.Tensor | np.ndarray) -> np.ndarray:
    """The token records ([..., 64 B, record]) of key-plane storage blocks
    ([..., B, 64 record], e.g. cache.k_planes[b, h])."""
    if isinstance(blocks, torch.Tensor):
        blocks = blocks.cpu().numpy()
    return oracle.key_blocks_to_records(blocks, w.d, w.key_mse_bits, bool(w.key_qjl), bool(w.key_half))


def put_key_records(cache: tq.Cache, w: wl.Workload, b: int, h: int, start: int, records: np.ndarray):
    """Write token records at positions start .. start + T - 1 of slot (b, h)."""
    allrec = key_records(w, cache.k_planes[b, h])
    allrec[start:start + records.shape[0]] = records
    blocks = oracle.key_records_to_blocks(allrec, w.d, w.key_mse_bits, bool(w.key_qjl), bool(w.key_half))
    cache.k_planes[b, h] = torch.from_numpy(blocks).to(cache.k_planes.device)


def upload_slot(cache: tq.Cache, w: wl.Workload, b: int, h: int, sc: SlotCode, start: int = 0):
    """Write the oracle-packed codes of one slot into the device cache at
    positions start .. start + T - 1 (start a multiple of 32)."""
    assert start % 32 == 0
    t = sc.key.idx.shape[0]
    dev = cache.k_planes.device
    kp = oracle.pack_key_planes(sc.key.idx, sc.key.qjl if w.key_qjl else None, w.key_mse_bits, half=bool(w.key_half))
    put_key_records(cache, w, b, h, start, kp)
    sd = np.float32 if w.scalar_dtype == "f32" else np.float16
    cache.k_norm[b, h, start:start + t] = torch.from_numpy(sc.key.norm.astype(sd)).to(dev)
    if w.key_qjl:
        cache.k_rnorm[b, h, start:start + t] = torch.from_numpy(sc.key.rnorm.astype(sd)).to(dev)
    if w.value_kind == "minmax":
        codes = sc.val.code
        meta = np.stack([sc.val.scale16, sc.val.min16], axis=-1)
        cache.v_meta[b, h, start:start + t] = torch.from_numpy(meta).to(dev)
    else:
        codes = sc.val.idx
        cache.v_norm[b, h, start:start + t] = torch.from_numpy(sc.val.norm.astype(sd)).to(dev)
    cap = ((t + 31) // 32) * 32
    words = oracle.pack_value_words(codes, w.value_bits, w.value_kind, cap).view(np.int32)
    cache.v_planes[b, h, start // 32:start // 32 + cap // 32] = torch.from_numpy(words).to(dev)


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per output vector: |got - ref|_inf / |ref|_inf (last axis)."""
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def read_key_planes(planes: np.ndarray, d: int, mse_bits: int, qjl: bool, half: bool = False):
    """Read codes back from key plane bytes (bit i%8 of byte i/8 of plane p is
    bit p of coordinate i's index; with the half-bit layout a d/16-byte plane
    follows holding bit mse_bits of coordinate i (i mod 32 < 16) at bit
    16*(i//32) + i%32; the last plane holds QJL bits)."""
    bits = np.unpackbits(np.ascontiguousarray(planes, dtype=np.uint8), axis=1, bitorder="little").astype(np.int64)
    idx = sum(bits[:, p * d:(p + 1) * d] << p for p in range(mse_bits))
    off = mse_bits * d
    if half:
        for i in range(d):
            if i % 32 < 16:
                idx[:, i] |= bits[:, off + 16 * (i // 32) + i % 32] << mse_bits
        off += d // 2
    return idx, (bits[:, off:off + d].astype(np.uint8) if qjl else None)


def read_value_planes(words: np.ndarray, n_tokens: int, w: wl.Workload) -> np.ndarray:
    """Codes [n_tokens, d] from the value words [blocks, bits, d] of the
    workload's layout.  Bit planes: bit p of token slot u of a block sits in
    bit 8*(u%4) + 4*(u//16) + (u//4)%4 of word p.  Packed codes (min/max values
    of width b = 2 or 4): word h holds tokens (32/b)*h + i, token i's code in
    bits 8*(i%4) + b*(i//4) upward."""
    x = np.ascontiguousarray(words).view(np.uint32).astype(np.uint64)
    nblk, bits, d = x.shape
    code = np.zeros((nblk, 32, d), dtype=np.int64)
    if w.value_kind == "minmax" and bits in (2, 4):
        per = 32 // bits
        for u in range(32):
            h, i = divmod(u, per)
            sh = np.uint64(8 * (i % 4) + bits * (i // 4))
            code[:, u, :] = ((x[:, h, :] >> sh) & np.uint64((1 << bits) - 1)).astype(np.int64)
    else:
        u = np.arange(32)
        t = (8 * (u % 4) + 4 * (u // 16) + (u // 4) % 4).astype(np.uint64)
        for p in range(bits):
            code |= ((x[:, p, None, :] >> t[None, :, None]) & 1).astype(np.int64) << p
    return code.reshape(-1, d)[:n_tokens]


def key_plane_mismatches(w: wl.Workload, bk: OracleBooks, gpu_planes: np.ndarray, ref: oracle.KeyCode):
    """Compare GPU key planes with the oracle's code bit by bit.  Returns
    (unexcused, excused_mse, excused_qjl): a mismatching MSE bit is excused when
    the oracle's rotated coordinate lies within WINDOW of a decision boundary; a
    mismatching QJL bit when |z_i| < WINDOW or the token has an excused MSE flip."""
    t, d = ref.idx.shape
    idx_g, qjl_g = read_key_planes(gpu_planes, d, w.key_mse_bits, bool(w.key_qjl), bool(w.key_half))
    mse_bad = idx_g != ref.idx
    near = np.min(np.abs(ref.y[..., None] - bk.k.thresholds[None, None, :]), axis=-1) < WINDOW
    if w.key_half:  # the half-bit coordinates decide against the larger table
        near_hi = np.min(np.abs(ref.y[..., None] - bk.k_hi.thresholds[None, None, :]), axis=-1) < WINDOW
        near = np.where(oracle.half_bit_coordinates(d)[None, :], near_hi, near)
    unexcused = int(np.sum(mse_bad & ~near))
    excused_mse = int(np.sum(mse_bad & near))
    excused_qjl = 0
    if w.key_qjl:
        q_bad = qjl_g != ref.qjl
        tok_flip = np.any(mse_bad & near, axis=1)
        ok = (np.abs(ref.z) < WINDOW) | tok_flip[:, None]
        unexcused += int(np.sum(q_bad & ~ok))
        excused_qjl = int(np.sum(q_bad & ok))
    return unexcused, excused_mse, excused_qjl


def check_encode_slot(w, bk, cache, b, h, ref, start, n, tag):
    """Compare the device cache slot (b, h) positions start..start+n-1 with the
    oracle code `ref`; returns the excused counts (key MSE bits, key QJL bits,
    value codes: MSE or min/max)."""
    kp = key_records(w, cache.k_planes[b, h])[start:start + n]
    bad, ex_m, ex_q = key_plane_mismatches(w, bk, kp, ref.key)
    assert bad == 0, f"{tag}: {bad} key bits differ outside the {WINDOW} window"
    flip = np.any(_flip_mask(w, bk, kp, ref), axis=1)
    f16 = w.scalar_dtype == "f16"
    kn = cache.k_norm[b, h, start:start + n].float().cpu().double().numpy()
    if f16:
        ulp = np.spacing(ref.key.norm.astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(kn - ref.key.norm) <= ulp * 1.01), tag
    else:
        assert np.max(np.abs(kn - ref.key.norm) / np.maximum(ref.key.norm, 1e-30)) <= 1e-6, tag
    if w.key_qjl:
        kr = cache.k_rnorm[b, h, start:start + n].float().cpu().double().numpy()
        ok = ~flip
        if f16:
            ulp = np.spacing(ref.key.rnorm.astype(np.float16)).astype(np.float64)
            assert np.all(np.abs(kr - ref.key.rnorm)[ok] <= ulp[ok] * 1.01), tag
        else:
            # The encode rule lets a rotated coordinate y_i move by up to WINDOW
            # (a code may flip only that close to a boundary).  gamma is the norm
            # of the residual y - c[idx] in rotated coordinates, so on a token with
            # no flipped code such a perturbation moves it by at most
            # |dy| <= WINDOW * sqrt(d) (triangle inequality).
            bound = WINDOW * np.sqrt(w.d)
            err = np.abs(kr - ref.key.rnorm)[ok]
            if err.size:
                _GAMMA_ERR["max"] = max(_GAMMA_ERR["max"], float(err.max()))
                _GAMMA_ERR["tokens"] += int(err.size)
            assert np.all(err <= bound), (tag, float(err.max()), bound)
    # values
    blk0 = start // 32
    nblk = (start + n + 31) // 32 - blk0
    words = cache.v_planes[b, h, blk0:blk0 + nblk].cpu().numpy()
    codes = read_value_planes(words, nblk * 32, w)[start - blk0 * 32: start - blk0 * 32 + n]
    if w.value_kind == "minmax":
        # a code may differ only where the oracle's ratio (v - min16) / delta16
        # lies within WINDOW (in code units) of a rounding midpoint k + 1/2, and
        # then only to the other neighbour of that midpoint
        bad_v = codes != ref.val.code
        r = ref.val.ratio
        near = np.abs(r - np.floor(r) - 0.5) < WINDOW
        assert np.sum(bad_v & ~near) == 0, \
            f"{tag}: {int(np.sum(bad_v & ~near))} min/max codes differ outside the window"
        assert np.all(np.abs(codes[bad_v] - ref.val.code[bad_v]) == 1), f"{tag}: min/max code off by more than 1"
        ex_v = int(np.sum(bad_v))
        meta = cache.v_meta[b, h, start:start + n].cpu().numpy()
        assert np.array_equal(meta[..., 0].view(np.uint16), ref.val.scale16.view(np.uint16)), tag
        assert np.array_equal(meta[..., 1].view(np.uint16), ref.val.min16.view(np.uint16)), tag
    else:
        bad_v = codes != ref.val.idx
        near = np.min(np.abs(ref.val.y[..., None] - bk.v.thresholds[None, None, :]), axis=-1) < WINDOW
        assert np.sum(bad_v & ~near) == 0, f"{tag}: MSE value codes differ outside the window"
        ex_v = int(np.sum(bad_v))
        vn = cache.v_norm[b, h, start:start + n].float().cpu().double().numpy()
        if f16:
            ulp = np.spacing(ref.val.norm.astype(np.float16)).astype(np.float64)
            assert np.all(np.abs(vn - ref.val.norm) <= ulp * 1.01), tag
        else:
            assert np.max(np.abs(vn - ref.val.norm) / np.maximum(ref.val.norm, 1e-30)) <= 1e-6, tag
    return ex_m, ex_q, ex_v


def _flip_mask(w, bk, kp, ref):
    idx_g, _ = read_key_planes(kp, w.d, w.key_mse_bits, bool(w.key_qjl), bool(w.key_half))
    return idx_g != ref.key.idx


def slot_from_cache(w: wl.Workload, cache: tq.Cache, b: int, h: int, n: int, start: int = 0) -> SlotCode:
    """The codes of device cache slot (b, h), positions start..start+n-1, read
    back into the oracle's code records (so the oracle can decode a
    GPU-encoded cache)."""
    end = start + n
    kp = key_records(w, cache.k_planes[b, h])[start:end]
    idx, qjl = read_key_planes(kp, w.d, w.key_mse_bits, bool(w.key_qjl), bool(w.key_half))
    norm = cache.k_norm[b, h, start:end].float().cpu().double().numpy()
    rnorm = cache.k_rnorm[b, h, start:end].float().cpu().double().numpy() if w.key_qjl else None
    key = oracle.KeyCode(idx=idx, qjl=qjl, norm=norm, rnorm=rnorm, y=None, z=None)
    blk0, blk1 = start // 32, (end + 31) // 32
    words = cache.v_planes[b, h, blk0:blk1].cpu().numpy()
    codes = read_value_planes(words, (blk1 - blk0) * 32, w)[start - 32 * blk0:end - 32 * blk0]
    if w.value_kind == "minmax":
        meta = cache.v_meta[b, h, start:end].cpu().numpy()
        val = oracle.ValueMinMax(code=codes, scale16=meta[..., 0].copy(), min16=meta[..., 1].copy(), ratio=None)
    else:
        vn = cache.v_norm[b, h, start:end].float().cpu().double().numpy()
        val = oracle.ValueMSE(idx=codes, norm=vn, y=None)
    return SlotCode(key, val)
