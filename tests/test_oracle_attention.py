"""Pins of the oracle's decode attention: explicit loops on tiny inputs, closed-form
special cases, PyTorch's scaled-dot-product attention for the uncompressed case,
and invariance under token permutation."""
import numpy as np
import torch

import oracle


def _tiny(seed, b=2, h_kv=2, g=2, n=(5, 3), nr=(2, 3), d=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, h_kv * g, d))
    kc = [[rng.standard_normal((n[i], d)) for _ in range(h_kv)] for i in range(b)]
    vc = [[rng.standard_normal((n[i], d)) for _ in range(h_kv)] for i in range(b)]
    rk = rng.standard_normal((b, 4, h_kv, d))
    rv = rng.standard_normal((b, 4, h_kv, d))
    return q, kc, vc, rk, rv, list(nr)


def test_matches_explicit_loops():
    for seed in range(4):
        q, kc, vc, rk, rv, nr = _tiny(seed)
        out = oracle.decode_attention(q, kc, vc, rk, rv, nr, scale=0.37)
        b, hq, d = q.shape
        g = hq // len(kc[0])
        for bi in range(b):
            for h in range(hq):
                kv = h // g
                keys = list(kc[bi][kv]) + [rk[bi, j, kv] for j in range(nr[bi])]
                vals = list(vc[bi][kv]) + [rv[bi, j, kv] for j in range(nr[bi])]
                ref = oracle.decode_attention_bruteforce(q[bi, h], keys, vals, 0.37)
                assert np.max(np.abs(out[bi, h] - ref)) < 1e-13


def test_single_token_returns_its_value():
    q, kc, vc, _, _, _ = _tiny(1, n=(1, 1))
    out = oracle.decode_attention(q, kc, vc)
    for bi in range(2):
        for h in range(4):
            assert np.allclose(out[bi, h], vc[bi][h // 2][0], atol=1e-15)


def test_zero_query_averages_values():
    q, kc, vc, rk, rv, nr = _tiny(2)
    q[:] = 0
    out = oracle.decode_attention(q, kc, vc, rk, rv, nr)
    for bi in range(2):
        for h in range(4):
            kv = h // 2
            allv = np.concatenate([vc[bi][kv], rv[bi, : nr[bi], kv]])
            assert np.allclose(out[bi, h], allv.mean(0), atol=1e-14)


def test_ring_only_is_textbook_sdpa():
    q, kc, vc, rk, rv, nr = _tiny(3, n=(0, 0), nr=(4, 3))
    out = oracle.decode_attention(q, kc, vc, rk, rv, nr)
    for bi in range(2):
        for h in range(4):
            kv = h // 2
            qq = torch.tensor(q[bi, h][None, None, None, :])
            kk = torch.tensor(rk[bi, : nr[bi], kv][None, None])
            vv = torch.tensor(rv[bi, : nr[bi], kv][None, None])
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv).numpy()[0, 0, 0]
            assert np.max(np.abs(out[bi, h] - ref)) < 1e-13


def test_token_permutation_invariance():
    q, kc, vc, rk, rv, nr = _tiny(4, n=(7, 6))
    out = oracle.decode_attention(q, kc, vc, rk, rv, nr)
    rng = np.random.default_rng(0)
    kc2 = [[None] * 2 for _ in range(2)]
    vc2 = [[None] * 2 for _ in range(2)]
    for bi in range(2):
        for h in range(2):
            p = rng.permutation(len(kc[bi][h]))
            kc2[bi][h], vc2[bi][h] = kc[bi][h][p], vc[bi][h][p]
    out2 = oracle.decode_attention(q, kc2, vc2, rk, rv, nr)
    assert np.max(np.abs(out - out2)) < 1e-13


def test_empty_cache_gives_zero():
    q, kc, vc, rk, rv, _ = _tiny(5, n=(0, 0))
    out = oracle.decode_attention(q, kc, vc, rk, rv, [0, 0])
    assert np.all(out == 0)
