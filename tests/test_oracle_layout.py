"""Pins of the oracle's packed layout (round trips, bit positions worked by hand)
and of its byte accounting against the compression figures the pages print."""
import json
import os

import numpy as np

import oracle
from oracle.layout import Layout, bytes_per_token_head, memory_bytes


def test_key_planes_round_trip_and_bit_positions():
    rng = np.random.default_rng(0)
    for mse_bits in (1, 2, 3, 4):
        idx = rng.integers(0, 1 << mse_bits, size=(37, 128))
        qjl = rng.integers(0, 2, size=(37, 128)).astype(np.uint8)
        packed = oracle.pack_key_planes(idx, qjl, mse_bits)
        assert packed.shape == (37, (mse_bits + 1) * 16) and packed.dtype == np.uint8
        i2, q2 = oracle.unpack_key_planes(packed, 128, mse_bits, True)
        assert np.array_equal(i2, idx) and np.array_equal(q2, qjl)
    # worked example: 2-bit index 2 (binary 10) at coordinate 9 sets plane 1,
    # byte 9 // 8 = 1, bit 9 % 8 = 1 -> byte 16 + 1 = 17 holds 0b10; the QJL bit
    # of coordinate 127 is the top bit of the last byte
    idx = np.zeros((1, 128), dtype=np.int64)
    idx[0, 9] = 2
    qjl = np.zeros((1, 128), dtype=np.uint8)
    qjl[0, 127] = 1
    p = oracle.pack_key_planes(idx, qjl, 2)[0]
    expect = np.zeros(48, dtype=np.uint8)
    expect[17] = 0b10
    expect[47] = 0x80
    assert np.array_equal(p, expect)


def test_key_block_storage_positions():
    """Records in 64-token blocks, interleaved by words: the plane at record
    offset o fills block bytes 64 o .. 64 (o + size) - 1, and word w of token
    16 c + n of the block is word 4 (4 n + w) + c there (include/tq.h)."""
    for mse_bits, qjl, half in ((2, True, False), (1, True, True), (2, True, True), (3, False, False)):
        pos = oracle.key_block_positions(128, mse_bits, qjl, half)
        rec = pos.shape[1]
        assert rec == (mse_bits + qjl) * 16 + half * 8
        assert sorted(pos.ravel().tolist()) == list(range(64 * rec))  # a permutation of the block
        rng = np.random.default_rng(mse_bits + 10 * half)
        recs = rng.integers(0, 256, size=(3, 128, rec), dtype=np.uint8)
        blocks = oracle.key_records_to_blocks(recs, 128, mse_bits, qjl, half)
        assert blocks.shape == (3, 2, 64 * rec)
        assert np.array_equal(oracle.key_blocks_to_records(blocks, 128, mse_bits, qjl, half), recs)
    # worked examples, 2-bit index + QJL (record 48 bytes: planes at 0, 16, 32)
    pos = oracle.key_block_positions(128, 2, True)
    # token 37 = 16*2 + 5 (c = 2, n = 5), plane 1 (offset 16), record byte 16 + 9:
    # word w = 9 // 4 = 2, byte 1 of it -> 64*16 + (4*(4*5 + 2) + 2)*4 + 1
    assert pos[37, 25] == 1024 + (4 * 22 + 2) * 4 + 1
    # token 0, QJL plane byte 0 -> 64*32
    assert pos[0, 32] == 2048
    # token 63 = 16*3 + 15, plane 0, last byte (word 3, byte 3): 0 + (4*63 + 3)*4 + 3 = 1023
    assert pos[63, 15] == 1023
    # half-bit layout, 2 + 1/2 index bits + QJL (record 16+16+8+16 = 56): the
    # half plane at offset 32 has 2-byte words; token 17 = 16 + 1 (c = 1, n = 1),
    # half-plane record byte 32 + 5 (word 2, byte 1) -> 64*32 + (4*(4 + 2) + 1)*2 + 1;
    # the QJL plane at offset 40
    pos = oracle.key_block_positions(128, 2, True, True)
    assert pos[17, 37] == 2048 + (4 * 6 + 1) * 2 + 1
    assert pos[0, 40] == 64 * 40


def test_value_planes_round_trip_and_bit_positions():
    rng = np.random.default_rng(1)
    for bits in (1, 2, 3, 4):
        code = rng.integers(0, 1 << bits, size=(70, 128))
        words = oracle.pack_value_planes(code, bits, capacity=96)
        assert words.shape == (3, bits, 128) and words.dtype == np.uint32
        assert np.array_equal(oracle.unpack_value_planes(words, 70), code)
        assert np.all(oracle.unpack_value_planes(words, 96)[70:] == 0)
    # the token slots of a block map one to one onto the 32 bits of a word
    from oracle.layout import value_bit
    assert sorted(value_bit(np.arange(32)).tolist()) == list(range(32))
    # worked examples: token 33 (block 1, slot 1 -> bit 8*1 = 8), channel 5,
    # code 3 = planes 0 and 1; token 22 (block 0, slot 22 -> 8*2 + 4*1 + 1 = 21),
    # channel 0, code 2 = plane 1 only
    code = np.zeros((64, 128), dtype=np.int64)
    code[33, 5] = 3
    code[22, 0] = 2
    w = oracle.pack_value_planes(code, 2)
    assert w[1, 0, 5] == 1 << 8 and w[1, 1, 5] == 1 << 8
    assert w[0, 1, 0] == 1 << 21 and w[0, 0, 0] == 0
    assert np.count_nonzero(w) == 3


def test_packed_value_codes_round_trip_and_bit_positions():
    rng = np.random.default_rng(2)
    for bits in (1, 2, 4):
        code = rng.integers(0, 1 << bits, size=(70, 128))
        words = oracle.pack_value_codes(code, bits, capacity=96)
        assert words.shape == (3, bits, 128) and words.dtype == np.uint32
        assert np.array_equal(oracle.unpack_value_codes(words, 70), code)
        assert np.all(oracle.unpack_value_codes(words, 96)[70:] == 0)
    # width 1: packed codes and bit planes are the same words
    code = rng.integers(0, 2, size=(64, 128))
    assert np.array_equal(oracle.pack_value_codes(code, 1), oracle.pack_value_planes(code, 1))
    # worked examples, width 2 (16 tokens per word): token 33 = block 1, slot 1
    # -> word 0, bits 8..9; token 22 = block 0, slot 22 -> word 1, i = 6 -> bits
    # 8*2 + 2*1 = 18..19
    code = np.zeros((64, 128), dtype=np.int64)
    code[33, 5] = 3
    code[22, 0] = 2
    w = oracle.pack_value_codes(code, 2)
    assert w[1, 0, 5] == 3 << 8 and w[0, 1, 0] == 1 << 19
    assert np.count_nonzero(w) == 2
    # width 4 (8 tokens per word): token 13 -> word 1, i = 5 -> bits 8 + 4 = 12..15
    code = np.zeros((32, 128), dtype=np.int64)
    code[13, 7] = 0xB
    w = oracle.pack_value_codes(code, 4)
    assert w[0, 1, 7] == 0xB << 12 and np.count_nonzero(w) == 1
    # the layout picks packed codes for min/max widths 2 and 4 only
    assert [oracle.value_words_packed("minmax", b) for b in (1, 2, 3, 4)] == [False, True, False, True]
    assert not any(oracle.value_words_packed("mse", b) for b in (1, 2, 3, 4))


def _gold(golden_dir):
    return json.load(open(os.path.join(golden_dir, "byte_counts.json")))


def test_audit_data_only_ratio(golden_dir):
    g = _gold(golden_dir)["audit_data_only"]
    lay = Layout(**g["layout"])
    assert bytes_per_token_head(lay)["total"] == g["bytes_per_token_head"]
    n, h_kv = 4096, 8
    fp16 = n * h_kv * 128 * 2 * 2
    ratio = fp16 / memory_bytes(lay, 1, h_kv, n, "data")
    assert round(ratio, 1) == g["ratio_printed"]
    assert abs(ratio - 5.12) < 1e-12


def test_audit_all_in_ratios(golden_dir):
    gold = _gold(golden_dir)
    g = gold["audit_all_in"]
    lay = Layout(**gold["audit_data_only"]["layout"])
    h_kv = g["h_kv"]
    assert 2 * 128 * 128 * 4 == g["pi_plus_s_bytes"]
    params = memory_bytes(lay, 1, h_kv, 0, "params")
    assert params - g["pi_plus_s_bytes"] == 4 * (4 + 5 + 3)  # 2-bit MSE codebook tables
    ring_one_tensor = memory_bytes(lay, 1, h_kv, 0, "ring") // 2  # the audit's ring term
    got = {}
    for n_s, printed in g["ratios_printed"].items():
        n = int(n_s)
        total = memory_bytes(lay, 1, h_kv, n, "data") + params + ring_one_tensor
        got[n] = n * h_kv * 128 * 2 * 2 / total
        assert round(got[n], 1) == printed or (n == 32768 and 5.0 <= got[n] < 5.1)
    assert abs(got[4096] - 4.5713) < 1e-4 and abs(got[128] - 1.0578) < 1e-4
    assert abs(got[32768] - 5.0443) < 1e-4


def test_results_page_compression(golden_dir):
    g = _gold(golden_dir)["results_compression"]
    lay = Layout(**g["layout"])
    assert bytes_per_token_head(lay)["total"] == 102
    fp16 = g["layers"] * g["h_kv"] * g["tokens"] * 128 * 2 * 2
    tq = g["layers"] * memory_bytes(lay, 1, g["h_kv"], g["tokens"], "data")
    assert fp16 / 1024 == g["fp16_kib_printed"]
    assert round(tq / 1024) == g["tq_kb_printed"]
    assert round(fp16 / tq, 2) == g["ratio_printed"]


def test_workload_layouts_bytes():
    # bytes per token-head of the five workloads' layouts (fp32 scalars unless noted)
    assert bytes_per_token_head(Layout())["total"] == 104
    assert bytes_per_token_head(Layout(key_mse_bits=3, value_kind="mse", value_bits=3))["total"] == 124
    assert bytes_per_token_head(Layout(value_kind="mse", value_bits=3, scalar_dtype="f16"))["total"] == 102
    assert bytes_per_token_head(Layout(key_mse_bits=3, value_kind="mse", value_bits=3,
                                       scalar_dtype="f16"))["total"] == 118


def test_half_bit_key_planes_round_trip_and_bit_positions():
    rng = np.random.default_rng(3)
    d = 128
    mask = oracle.half_bit_coordinates(d)
    for mse_bits in (1, 2):
        idx = np.where(mask, rng.integers(0, 1 << (mse_bits + 1), size=(9, d)),
                       rng.integers(0, 1 << mse_bits, size=(9, d)))
        q = rng.integers(0, 2, size=(9, d)).astype(np.uint8)
        packed = oracle.pack_key_planes(idx, q, mse_bits, half=True)
        assert packed.shape == (9, (mse_bits * d + d // 2 + d) // 8)
        i2, q2 = oracle.unpack_key_planes(packed, d, mse_bits, True, half=True)
        assert np.array_equal(i2, idx) and np.array_equal(q2, q)
    # worked example, 2 full planes: coordinate 37 (32 + 5: half plane bit
    # 16 + 5 = 21 -> byte 32 + 2, bit 5) with index 4 = binary 100; coordinate
    # 20 (no half-plane bit) with index 3; QJL bit of coordinate 1
    idx = np.zeros((1, d), dtype=np.int64)
    idx[0, 37] = 4
    idx[0, 20] = 3
    q = np.zeros((1, d), dtype=np.uint8)
    q[0, 1] = 1
    p = oracle.pack_key_planes(idx, q, 2, half=True)[0]
    expect = np.zeros(56, dtype=np.uint8)
    expect[2] = 1 << 4          # plane 0, coordinate 20: byte 2, bit 4
    expect[16 + 2] = 1 << 4     # plane 1, coordinate 20
    expect[32 + 2] = 1 << 5     # half plane, coordinate 37
    expect[40] = 1 << 1         # QJL plane, coordinate 1
    assert np.array_equal(p, expect)
    assert oracle.bytes_per_token_head(oracle.Layout(key_half=1))["k_bits"] == 56
    assert oracle.bytes_per_token_head(oracle.Layout(key_mse_bits=1, key_half=1))["k_bits"] == 40
