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


def _multi_tiny(seed, b=2, h_kv=2, g=2, t=3, n=(5, 2), nr=(2, 0), d=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, t, h_kv * g, d))
    kc = [[rng.standard_normal((n[i], d)) for _ in range(h_kv)] for i in range(b)]
    vc = [[rng.standard_normal((n[i], d)) for _ in range(h_kv)] for i in range(b)]
    rk = rng.standard_normal((b, 4, h_kv, d))
    rv = rng.standard_normal((b, 4, h_kv, d))
    return q, kc, vc, rk, rv, list(nr)


def test_multi_query_matches_explicit_causal_loops():
    # every key of a sequence gets its position in the compressed-then-ring
    # order; query t of T sees positions < L - (T - 1 - t), L = n_c + n_r
    for seed in range(4):
        q, kc, vc, rk, rv, nr = _multi_tiny(seed)
        out = oracle.decode_attention_multi(q, kc, vc, rk, rv, nr, scale=0.41)
        bsz, nq, hq, d = q.shape
        g = hq // len(kc[0])
        for bi in range(bsz):
            for t in range(nq):
                for h in range(hq):
                    kv = h // g
                    keys = list(kc[bi][kv]) + [rk[bi, j, kv] for j in range(nr[bi])]
                    vals = list(vc[bi][kv]) + [rv[bi, j, kv] for j in range(nr[bi])]
                    visible = len(keys) - (nq - 1 - t)
                    if visible <= 0:  # nothing visible: the output is zero
                        assert np.all(out[bi, t, h] == 0)
                        continue
                    ref = oracle.decode_attention_bruteforce(q[bi, t, h], keys[:visible], vals[:visible], 0.41)
                    assert np.max(np.abs(out[bi, t, h] - ref)) < 1e-13


def test_multi_query_needle_is_hidden_from_earlier_queries():
    # the last key of the sequence (the ring's last token, or the last
    # compressed token when the ring is empty) is aligned with every query and
    # carries a distinct value: only the last query sees it, and its output is
    # that value up to exp(-scale * margin)
    d, nq = 8, 3
    for use_ring in (True, False):
        rng = np.random.default_rng(5)
        q = np.zeros((1, nq, 1, d))
        q[..., 0] = 1.0
        kc = [[rng.standard_normal((6, d)) * 0.01]]
        vc = [[rng.standard_normal((6, d))]]
        rk = np.zeros((1, 4, 1, d))
        rv = np.zeros((1, 4, 1, d))
        needle_v = np.arange(1.0, d + 1.0)
        if use_ring:
            rk[0, 0, 0] = rng.standard_normal(d) * 0.01
            rv[0, 0, 0] = rng.standard_normal(d)
            rk[0, 1, 0, 0] = 200.0
            rv[0, 1, 0] = needle_v
            nr = [2]
        else:
            kc[0][0][-1] = 0.0
            kc[0][0][-1, 0] = 200.0
            vc[0][0][-1] = needle_v
            nr = [0]
        out = oracle.decode_attention_multi(q, kc, vc, rk, rv, nr, scale=1.0)
        assert np.max(np.abs(out[0, nq - 1, 0] - needle_v)) < 1e-12
        for t in range(nq - 1):
            assert np.max(np.abs(out[0, t, 0] - needle_v)) > 1.0


def test_multi_query_of_one_is_single_query():
    q, kc, vc, rk, rv, nr = _multi_tiny(7, t=1)
    a = oracle.decode_attention_multi(q, kc, vc, rk, rv, nr)
    b = oracle.decode_attention(q[:, 0], kc, vc, rk, rv, nr)
    assert np.max(np.abs(a[:, 0] - b)) < 1e-15
