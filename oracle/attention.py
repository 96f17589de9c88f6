"""Decode attention over a TurboQuant cache plus a bf16 ring: one query per
(sequence, query head), or T queries per sequence (multi-query decode).

TEST INFRASTRUCTURE (see the package docstring).

Structure: dequantize, then attend ([audit] AUDIT 2 and AUDIT 4: keys and values
are reconstructed in full and multiplied with the query, softmax, weighted sum).
The fused GPU kernel reaches the same result in the rotated-query form of
[explainer] "Tại sao nó hoạt động" and [results] "Latency Benchmarks"; the two
forms are algebraically equal, so this oracle is an independent cross-check.

Readings taken where the pages are silent:

* Query head h_q reads KV head h_q // G (G = H_q / H_kv, contiguous groups:
  the (H_kv, G, T, N) score layout of [audit] AUDIT 4).
* Softmax scale tau is an argument (1/sqrt(d) in every workload).
* The ring holds the most recent tokens uncompressed in bf16 in the original
  (unrotated) space ([audit] AUDIT 1 ring term); one softmax runs over the
  compressed tokens and the ring tokens together.
* Multi-query decode (T > 1 in the (H_kv, G, T, N) score layout of [audit]
  AUDIT 4): the T queries of a sequence are its last T positions, already
  appended to the cache or the ring.  The keys of a sequence are its
  compressed tokens followed by its ring tokens, and query t (0 <= t < T) sees
  every key except the last T - 1 - t of that order (causal among the new
  positions; all earlier tokens are visible to every query).
"""
from __future__ import annotations

import numpy as np


def decode_attention(q: np.ndarray, k_comp: list, v_comp: list, ring_k=None, ring_v=None,
                     n_ring=None, scale: float | None = None) -> np.ndarray:
    """Attention output for one query per (batch, query head).

    q: (B, H_q, d).  k_comp[b][h], v_comp[b][h]: dequantized compressed keys and
    values of sequence b, KV head h, each (n_c, d) float64 (n_c may be 0).
    ring_k, ring_v: (B, R, H_kv, d) arrays (bf16 values, any float dtype) or None;
    n_ring[b] of their rows are valid.  Returns (B, H_q, d) float64.
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, h_q, d = q.shape
    h_kv = len(k_comp[0])
    g = h_q // h_kv
    tau = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros((bsz, h_q, d))
    for b in range(bsz):
        for hq in range(h_q):
            h = hq // g
            keys = [np.asarray(k_comp[b][h], dtype=np.float64).reshape(-1, d)]
            vals = [np.asarray(v_comp[b][h], dtype=np.float64).reshape(-1, d)]
            if ring_k is not None and n_ring is not None and n_ring[b] > 0:
                keys.append(np.asarray(ring_k[b, : n_ring[b], h, :], dtype=np.float64))
                vals.append(np.asarray(ring_v[b, : n_ring[b], h, :], dtype=np.float64))
            kk = np.concatenate(keys, axis=0)
            vv = np.concatenate(vals, axis=0)
            if kk.shape[0] == 0:
                continue  # nothing to attend to: the output stays 0
            s = tau * (kk @ q[b, hq])
            p = np.exp(s - s.max())
            out[b, hq] = (p @ vv) / p.sum()
    return out


def decode_attention_multi(q: np.ndarray, k_comp: list, v_comp: list, ring_k=None, ring_v=None,
                           n_ring=None, scale: float | None = None) -> np.ndarray:
    """T queries per sequence.  q: (B, T, H_q, d); the other arguments as in
    decode_attention.  Query t sees all but the last T - 1 - t keys of the
    sequence's compressed-then-ring order.  Returns (B, T, H_q, d) float64."""
    q = np.asarray(q, dtype=np.float64)
    bsz, nq, h_q, d = q.shape
    h_kv = len(k_comp[0])
    out = np.zeros((bsz, nq, h_q, d))
    for b in range(bsz):
        nr = int(n_ring[b]) if (ring_k is not None and n_ring is not None) else 0
        for t in range(nq):
            hidden = nq - 1 - t
            hide_r = min(hidden, nr)
            hide_c = hidden - hide_r
            kc = [np.asarray(k_comp[b][h]).reshape(-1, d) for h in range(h_kv)]
            vc = [np.asarray(v_comp[b][h]).reshape(-1, d) for h in range(h_kv)]
            kc = [x[: x.shape[0] - hide_c] for x in kc]
            vc = [x[: x.shape[0] - hide_c] for x in vc]
            out[b, t] = decode_attention(q[b:b + 1, t], [kc], [vc],
                                         None if ring_k is None else ring_k[b:b + 1],
                                         None if ring_v is None else ring_v[b:b + 1],
                                         [nr - hide_r], scale)[0]
    return out


def decode_attention_bruteforce(q, keys, values, scale):
    """Textbook attention by explicit loops, for tiny inputs: o = sum_j p_j v_j with
    p_j = exp(s_j) / sum_i exp(s_i), s_j = scale * sum_c q_c k_jc."""
    n = len(keys)
    s = []
    for j in range(n):
        acc = 0.0
        for c in range(len(q)):
            acc += float(q[c]) * float(keys[j][c])
        s.append(scale * acc)
    m = max(s)
    w = [np.exp(x - m) for x in s]
    tot = sum(w)
    o = []
    for c in range(len(q)):
        acc = 0.0
        for j in range(n):
            acc += w[j] * float(values[j][c])
        o.append(acc / tot)
    return np.array(o)
