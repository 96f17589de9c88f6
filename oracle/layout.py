"""Byte layout of the compressed cache and its byte accounting.

TEST INFRASTRUCTURE (see the package docstring).  The pages fix the bit
budgets but not the packing; the layout below is this implementation's
definition, written here independently of the HIP library so that packed bytes
can be compared bit for bit.

Per (sequence, KV head) slot of ``capacity`` tokens:

* key planes   one record per token, record = key_mse_bits full planes
  (d/8 bytes each), then with the half-bit layout one half plane (d/16 bytes),
  then the QJL plane (d/8 bytes) when key_qjl.  Full plane p holds bit p of
  every coordinate's Lloyd-Max index, coordinate i in bit i % 8 of byte
  i // 8 (LSB first).  The half plane holds bit key_mse_bits of the index of
  the half-bit coordinates (i mod 32 < 16), coordinate i at bit position
  h = 16 (i // 32) + i mod 32 (bit h % 8 of byte h // 8).  The QJL plane
  holds the sign bits (1 = non-negative) in the full-plane order.
  Stored as uint8 [ceil(capacity/64)][64 * record]: blocks of 64 token
  positions, interleaved by words.  The plane at record byte offset o (s bytes)
  fills bytes 64 o .. 64 (o + s) - 1 of its block, and its word w (4 bytes, 2
  in the half plane) of token 64 j + 16 c + n (c < 4, n < 16) is word
  4 (4 n + w) + c of that range (key_records_to_blocks).
* key norm, key residual norm   [capacity] fp32 or fp16.
* value words uint32 [capacity/32][value_bits][d], in one of two forms:
  - bit planes (MSE values, and min/max values of width 1 or 3): word (blk, p,
    c) holds bit p of the code of token 32*blk + u at channel c, for u = 0..31,
    in bit value_bit(u) = 8*(u % 4) + 4*(u // 16) + (u // 4) % 4 (a fixed
    permutation of the 32 token slots of a block);
  - packed codes (min/max values of width b = 2 or 4): word (blk, h, c) holds
    the b-bit codes of tokens 32*blk + (32/b)*h + i, i < 32/b, at channel c,
    the code of token i in bits 8*(i % 4) + b*(i // 4) .. + b - 1.  For b = 1
    this is the same as one bit plane.
* value meta (min/max values)   fp16 [capacity][d/group][2] = (scale, min).
* value norm (MSE values)       [capacity] fp32 or fp16.

``memory_bytes`` counts, as in [audit] AUDIT 1: the quantized data, the
per-layer parameters (Pi, S, codebook tables) and the bf16 ring.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Layout:
    d: int = 128
    key_mse_bits: int = 2
    key_qjl: int = 1
    value_kind: str = "minmax"  # "minmax" | "mse"
    value_bits: int = 2
    value_group: int = 32
    scalar_dtype: str = "f32"  # "f32" | "f16"
    key_half: int = 0  # 1: half of the rotated coordinates get key_mse_bits + 1 bits

    @property
    def scalar_bytes(self) -> int:
        return 4 if self.scalar_dtype == "f32" else 2

    @property
    def key_planes(self) -> int:
        return self.key_mse_bits + self.key_qjl


def bytes_per_token_head(lay: Layout) -> dict:
    """Stored bytes for one token of one KV head, by field."""
    s = lay.scalar_bytes
    k_bits = lay.key_planes * lay.d // 8 + lay.key_half * lay.d // 16
    k_scal = s * (1 + lay.key_qjl)
    v_bits = lay.value_bits * lay.d // 8
    if lay.value_kind == "minmax":
        v_scal = (lay.d // lay.value_group) * 2 * 2
    else:
        v_scal = s
    return {"k_bits": k_bits, "k_scalars": k_scal, "v_bits": v_bits, "v_scalars": v_scal,
            "total": k_bits + k_scal + v_bits + v_scal}


def codebook_table_bytes(bits: int) -> int:
    """fp32 centroids (2^b), boundaries (2^b + 1) and decision boundaries (2^b - 1)."""
    levels = 1 << bits
    return 4 * (levels + (levels + 1) + (levels - 1))


def memory_bytes(lay: Layout, batch: int, h_kv: int, n_tokens: int, what: str,
                 ring_cap: int = 128) -> int:
    """what: "data" (quantized tensors only), "params" (Pi and S in fp32 plus
    the codebook tables), "ring" (bf16 K and V ring of ring_cap tokens)."""
    if what == "data":
        return bytes_per_token_head(lay)["total"] * batch * h_kv * n_tokens
    if what == "params":
        p = 2 * lay.d * lay.d * 4 + codebook_table_bytes(lay.key_mse_bits)
        if lay.key_half:
            p += codebook_table_bytes(lay.key_mse_bits + 1)
        if lay.value_kind == "mse":
            p += codebook_table_bytes(lay.value_bits)
        return p
    if what == "ring":
        return batch * ring_cap * h_kv * lay.d * 2 * 2
    raise ValueError(what)


def half_plane_position(d: int) -> np.ndarray:
    """Coordinates of the half plane in order: entry h is the coordinate i with
    16 (i // 32) + i mod 32 == h (those with i mod 32 < 16)."""
    i = np.arange(d)
    return i[(i % 32) < 16]


def pack_key_planes(idx: np.ndarray, qjl: np.ndarray | None, mse_bits: int, half: bool = False) -> np.ndarray:
    """(T, d) indices and (T, d) sign bits -> (T, record) uint8 planes."""
    idx = np.asarray(idx, dtype=np.int64)
    t, d = idx.shape
    planes = [((idx >> p) & 1).astype(np.uint8) for p in range(mse_bits)]
    if half:
        planes.append(((idx[:, half_plane_position(d)] >> mse_bits) & 1).astype(np.uint8))
    if qjl is not None:
        planes.append(np.asarray(qjl, dtype=np.uint8) & 1)
    bits = np.concatenate(planes, axis=1)  # (T, record bits)
    return np.packbits(bits, axis=1, bitorder="little")


def key_record_planes(d: int, mse_bits: int, qjl: bool, half: bool = False) -> list[tuple[int, int, int]]:
    """(byte offset, bytes, word bytes) of every plane of a key record."""
    planes = [(p * d // 8, d // 8, 4) for p in range(mse_bits)]
    off = mse_bits * d // 8
    if half:
        planes.append((off, d // 16, 2))
        off += d // 16
    if qjl:
        planes.append((off, d // 8, 4))
    return planes


def key_block_positions(d: int, mse_bits: int, qjl: bool, half: bool = False) -> np.ndarray:
    """(64, record) array: the byte of a 64-token storage block that holds
    byte j of the record of token u (u < 64) of the block."""
    planes = key_record_planes(d, mse_bits, qjl, half)
    rec = sum(size for _, size, _ in planes)
    pos = np.zeros((64, rec), dtype=np.int64)
    for u in range(64):
        c, n = u // 16, u % 16
        for off, size, wb in planes:
            for w in range(size // wb):
                for byte in range(wb):
                    pos[u, off + w * wb + byte] = 64 * off + (4 * (4 * n + w) + c) * wb + byte
    return pos


def key_records_to_blocks(records: np.ndarray, d: int, mse_bits: int, qjl: bool, half: bool = False) -> np.ndarray:
    """(..., T, record) token records, T a multiple of 64 -> (..., T/64, 64 record) storage blocks."""
    records = np.asarray(records, dtype=np.uint8)
    *lead, t, rec = records.shape
    assert t % 64 == 0
    pos = key_block_positions(d, mse_bits, qjl, half)
    blocks = np.zeros((*lead, t // 64, 64 * rec), dtype=np.uint8)
    src = records.reshape(*lead, t // 64, 64, rec)
    blocks[..., pos] = src  # pos is (64, rec): scatter every token byte of every block
    return blocks


def key_blocks_to_records(blocks: np.ndarray, d: int, mse_bits: int, qjl: bool, half: bool = False) -> np.ndarray:
    """Inverse of key_records_to_blocks: (..., B, 64 record) -> (..., 64 B, record)."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    *lead, nb, width = blocks.shape
    pos = key_block_positions(d, mse_bits, qjl, half)
    rec = pos.shape[1]
    assert width == 64 * rec
    return blocks[..., pos].reshape(*lead, nb * 64, rec)


def unpack_key_planes(packed: np.ndarray, d: int, mse_bits: int, qjl: bool, half: bool = False):
    """Inverse of pack_key_planes: returns (idx, qjl_bits or None)."""
    bits = np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=1, bitorder="little").astype(np.int64)
    idx = np.zeros((bits.shape[0], d), dtype=np.int64)
    for p in range(mse_bits):
        idx |= bits[:, p * d:(p + 1) * d] << p
    off = mse_bits * d
    if half:
        idx[:, half_plane_position(d)] |= bits[:, off:off + d // 2] << mse_bits
        off += d // 2
    return idx, (bits[:, off:off + d].astype(np.uint8) if qjl else None)


def value_bit(u) -> np.ndarray:
    """Bit position, inside a value-plane word, of token slot u (0..31) of its block."""
    u = np.asarray(u)
    return 8 * (u % 4) + 4 * (u // 16) + (u // 4) % 4


def pack_value_planes(code: np.ndarray, bits: int, capacity: int | None = None) -> np.ndarray:
    """(T, d) codes -> (capacity/32, bits, d) uint32 token-transposed planes.
    Tokens T..capacity-1 are zero."""
    code = np.asarray(code, dtype=np.int64)
    t, d = code.shape
    cap = t if capacity is None else capacity
    if cap % 32 or cap < t:
        raise ValueError("capacity must be a multiple of 32 and hold every token")
    full = np.zeros((cap, d), dtype=np.int64)
    full[:t] = code
    blocks = full.reshape(cap // 32, 32, d)  # (blk, u, c)
    pos = value_bit(np.arange(32)).astype(np.uint64)
    out = np.zeros((cap // 32, bits, d), dtype=np.uint64)
    for p in range(bits):
        bit = ((blocks >> p) & 1).astype(np.uint64)  # (blk, u, c)
        out[:, p, :] = np.sum(bit << pos[None, :, None], axis=1)
    return out.astype(np.uint32)


def unpack_value_planes(words: np.ndarray, n_tokens: int) -> np.ndarray:
    """(capacity/32, bits, d) uint32 -> (n_tokens, d) codes."""
    w = np.asarray(words, dtype=np.uint64)
    nblk, bits, d = w.shape
    tt = value_bit(np.arange(32)).astype(np.uint64)
    code = np.zeros((nblk, 32, d), dtype=np.int64)
    for p in range(bits):
        code |= (((w[:, p, None, :] >> tt[None, :, None]) & 1).astype(np.int64)) << p
    return code.reshape(nblk * 32, d)[:n_tokens]


def value_words_packed(kind: str, bits: int) -> bool:
    """True where the value words hold packed codes rather than bit planes."""
    return kind == "minmax" and bits in (2, 4)


def packed_code_bit(i, bits: int) -> np.ndarray:
    """Lowest bit, inside its packed word, of the code of token i (< 32/bits)."""
    i = np.asarray(i)
    return 8 * (i % 4) + bits * (i // 4)


def pack_value_codes(code: np.ndarray, bits: int, capacity: int | None = None) -> np.ndarray:
    """(T, d) codes of width 1, 2 or 4 -> (capacity/32, bits, d) uint32 packed
    words.  Tokens T..capacity-1 are zero."""
    if bits not in (1, 2, 4):
        raise ValueError("packed codes have width 1, 2 or 4")
    code = np.asarray(code, dtype=np.int64)
    t, d = code.shape
    cap = t if capacity is None else capacity
    if cap % 32 or cap < t:
        raise ValueError("capacity must be a multiple of 32 and hold every token")
    full = np.zeros((cap, d), dtype=np.uint64)
    full[:t] = code
    per = 32 // bits
    blocks = full.reshape(cap // 32, bits, per, d)  # (blk, h, i, c)
    shift = packed_code_bit(np.arange(per), bits).astype(np.uint64)
    out = np.sum(blocks << shift[None, None, :, None], axis=2)
    return out.astype(np.uint32)


def unpack_value_codes(words: np.ndarray, n_tokens: int) -> np.ndarray:
    """(capacity/32, bits, d) uint32 packed words -> (n_tokens, d) codes."""
    w = np.asarray(words, dtype=np.uint64)
    nblk, bits, d = w.shape
    per = 32 // bits
    shift = packed_code_bit(np.arange(per), bits).astype(np.uint64)
    code = (w[:, :, None, :] >> shift[None, None, :, None]) & np.uint64((1 << bits) - 1)
    return code.astype(np.int64).reshape(nblk * 32, d)[:n_tokens]


def pack_value_words(code: np.ndarray, bits: int, kind: str, capacity: int | None = None) -> np.ndarray:
    """Value words of the layout's form (packed codes or bit planes)."""
    if value_words_packed(kind, bits):
        return pack_value_codes(code, bits, capacity)
    return pack_value_planes(code, bits, capacity)


def unpack_value_words(words: np.ndarray, n_tokens: int, kind: str) -> np.ndarray:
    """Inverse of pack_value_words."""
    if value_words_packed(kind, np.asarray(words).shape[1]):
        return unpack_value_codes(words, n_tokens)
    return unpack_value_planes(words, n_tokens)
