"""Host tests of the Python binding's argument checks (no GPU, no library
call): every rejection below is raised before anything reaches libtq, whose C
entry points trust the sizes they are given (a q with fewer sequences than the
cache, a ring slice with the wrong row stride or a short per-sequence list
would otherwise make the kernels read or write past a buffer)."""
import types

import pytest
import torch

from compressed_kv_decode_tq_amd import tq

B, H_KV, H_Q, D, CAP, R = 2, 2, 8, 128, 64, 16


@pytest.fixture()
def setup():
    lay = tq.Layout()
    cache = tq.Cache(lay, B, H_KV, CAP, device="cpu")
    params = types.SimpleNamespace(layout=lay)  # the checks only read the layout
    q = torch.zeros(B, H_Q, D)
    rk = torch.zeros(B, R, H_KV, D, dtype=torch.bfloat16)
    rv = torch.zeros_like(rk)
    kn = torch.zeros(B, 1, H_KV, D)
    return lay, cache, params, q, rk, rv, kn


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_decode_rejects_bad_query(setup):
    _, cache, prm, q, rk, rv, _ = setup
    _raises(lambda: tq.decode_attn(prm, q[:1].contiguous(), cache, [4, 4]), "sequences")
    _raises(lambda: tq.decode_attn(prm, torch.zeros(B, H_Q, 64), cache, [4, 4]), "head_dim")
    _raises(lambda: tq.decode_attn(prm, torch.zeros(B, 3, D), cache, [4, 4]), "multiple of num_kv_heads")
    _raises(lambda: tq.decode_attn(prm, q.transpose(0, 1).contiguous().transpose(0, 1), cache, [4, 4]),
            "contiguous")
    _raises(lambda: tq.decode_attn(prm, q.half(), cache, [4, 4]), "fp32 or bf16")
    _raises(lambda: tq.decode_attn(prm, torch.zeros(B, D), cache, [4, 4]), r"\[B, H_q, d\]")


def test_decode_rejects_short_per_sequence_lists(setup):
    _, cache, prm, q, rk, rv, _ = setup
    _raises(lambda: tq.decode_attn(prm, q, cache, [4]), "n_compressed")
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], rk, rv, [1]), "n_ring")
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], None, None, [1, 0]), "without ring")


def test_decode_rejects_bad_output_and_workspace(setup):
    _, cache, prm, q, _, _, _ = setup
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], out=torch.zeros(B, H_Q, D, dtype=torch.bfloat16)), "out")
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], out=torch.zeros(B, H_Q - 1, D)), "out")
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], out=torch.zeros(B, D, H_Q).transpose(1, 2)), "out")
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], workspace=torch.zeros(64, dtype=torch.float32)),
            "workspace")


def test_decode_rejects_bad_rings(setup):
    _, cache, prm, q, rk, rv, _ = setup
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], rk, None, [1, 1]), "together")
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], rk[:, :4], rv[:, :4], [1, 1]), "contiguous")
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], rk.float(), rv.float(), [1, 1]), "bf16")
    bad = torch.zeros(B, R, H_KV + 1, D, dtype=torch.bfloat16)
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], bad, bad, [1, 1]), r"must be \[")
    _raises(lambda: tq.decode_attn(prm, q, cache, [4, 4], rk, rv[:, :8].contiguous(), [1, 1]), "same shape")


def test_fused_append_rejections(setup):
    _, cache, prm, q, rk, rv, kn = setup
    f = tq.decode_attn_append
    _raises(lambda: f(prm, q[:, None].contiguous(), cache, [4, 4], kn, kn, rk, rv, [0, 0]), "one query")
    _raises(lambda: f(prm, q, cache, [4, 4], kn, kn, None, None, [0, 0]), "ring buffers")
    _raises(lambda: f(prm, q, cache, [4, 4], kn[:, :, :1].contiguous(), kn[:, :, :1].contiguous(), rk, rv, [0, 0]),
            "k_new and v_new must be")
    _raises(lambda: f(prm, q, cache, [4, 4], kn, kn.bfloat16(), rk, rv, [0, 0]), "same dtype")
    _raises(lambda: f(prm, q, cache, [4, 4], kn.half(), kn.half(), rk, rv, [0, 0]), "fp32 or bf16")
    _raises(lambda: f(prm, q, cache, [4, 4], kn, kn, rk, rv, [0]), "n_ring")
    _raises(lambda: f(prm, q[:1].contiguous(), cache, [4, 4], kn, kn, rk, rv, [0, 0]), "sequences")


def test_encode_rejections(setup):
    _, cache, prm, _, _, _, _ = setup
    k = torch.zeros(B, 3, H_KV, D)
    _raises(lambda: tq.encode_kv(prm, torch.zeros(B, 3, H_KV, 64), torch.zeros(B, 3, H_KV, 64), [0, 0], cache),
            "head_dim")
    _raises(lambda: tq.encode_kv(prm, k, k, [0], cache), "dst_pos")
    _raises(lambda: tq.encode_kv(prm, k[:1], k[:1], [0], cache), "batch or head count")
    _raises(lambda: tq.encode_kv(prm, k.half(), k.half(), [0, 0], cache), "fp32 or bf16")
    _raises(lambda: tq.encode_kv(prm, k, k.bfloat16(), [0, 0], cache), "same dtype")


def test_ring_append_rejections(setup):
    _, _, _, _, rk, rv, kn = setup
    _raises(lambda: tq.ring_append(kn, kn, rk, rv, [0]), "n_ring")
    _raises(lambda: tq.ring_append(kn, kn.bfloat16(), rk, rv, [0, 0]), "must match")
    _raises(lambda: tq.ring_append(kn, kn, rk[:, :4], rv[:, :4], [0, 0]), "contiguous")
    _raises(lambda: tq.ring_append(kn, kn, rk, rv[:, :8].contiguous(), [0, 0]), "one shape")
    _raises(lambda: tq.ring_append(kn.half(), kn.half(), rk, rv, [0, 0]), "fp32 or bf16")
