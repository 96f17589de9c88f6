"""Seeded synthetic workloads for TurboQuant KV encode and compressed decode.

This module only draws random numbers and shapes them: the per-layer random
rotation and QJL projection, the key/value/query tensors with their channel
structure, and the per-step decode tokens. It holds none of the method's
arithmetic (no quantisation, no rotation of data, no attention), so both the
float64 oracle and the HIP path can take their inputs from here.

Shapes follow the K/V chunk layout of the compressed store in the
``turboquant/audit_claims.py`` page (AUDIT 1: ``append_chunk`` takes
``(N, H_kv, d)``), with the batch in front: K, V are ``[B, N, H_kv, d]`` and q is
``[B, H_q, d]``.  Every tensor is generated in float64 and cast once to the
workload's input dtype (fp32 or bf16, round-to-nearest-even); the cast tensor
is the shared input and the oracle promotes it back to float64.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# Stream tags for SeedSequence spawning: one independent stream per role.
_TAG_PI, _TAG_S, _TAG_K, _TAG_V, _TAG_Q = 1, 2, 3, 4, 5
_TAG_OUTLIER, _TAG_SIGMA_K, _TAG_SIGMA_V, _TAG_SIGMA_Q, _TAG_STEP = 6, 7, 8, 9, 10


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark/parity configuration.

    ``key_mse_bits`` is the Lloyd-Max part of a TurboQuantProd key; the key
    also stores one QJL sign bit per coordinate when ``key_qjl`` is set.
    """

    name: str
    batch: int
    h_q: int
    h_kv: int
    n_tokens: int
    in_dtype: str  # "f32" | "bf16"
    key_mse_bits: int
    value_kind: str  # "minmax" | "mse"
    value_bits: int
    scalar_dtype: str  # "f32" | "f16"
    structure: str  # "iid" | "outliers" | "lognormal_kvq" | "lognormal_kv"
    ring_cap: int  # 0 = no ring buffer
    decode_steps: int
    step_mode: str  # "ring" (append new token to the bf16 ring) | "encode" | "none"
    seed: int
    d: int = 128
    key_qjl: int = 1
    value_group: int = 32
    key_half: int = 0  # 1: half of the rotated coordinates get key_mse_bits + 1 bits

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.in_dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _qwen_layer(n: int, key_mse_bits: int = 2, scalar_dtype: str = "f16") -> Workload:
    return Workload(
        name=f"qwen2.5-1.5b-layer-n{n}" + ("" if key_mse_bits == 2 else f"-k{key_mse_bits + 1}bit")
        + ("" if scalar_dtype == "f16" else "-f32scalars"),
        batch=1, h_q=12, h_kv=2, n_tokens=n, in_dtype="bf16", key_mse_bits=key_mse_bits,
        value_kind="mse", value_bits=3, scalar_dtype=scalar_dtype, structure="lognormal_kvq",
        ring_cap=0, decode_steps=1, step_mode="none", seed=20263)


#: The five workloads.  Index 0 is the small parity case, index 3 the batched
#: 32K-token decode that the headline metric is quoted on.
WORKLOADS: list[Workload] = [
    Workload(name="single-head-n512", batch=1, h_q=1, h_kv=1, n_tokens=512, in_dtype="f32",
             key_mse_bits=2, value_kind="minmax", value_bits=2, scalar_dtype="f32",
             structure="iid", ring_cap=0, decode_steps=1, step_mode="none", seed=20261),
    Workload(name="gqa4-hkv8-n4096-ring", batch=1, h_q=32, h_kv=8, n_tokens=4096, in_dtype="f32",
             key_mse_bits=2, value_kind="minmax", value_bits=2, scalar_dtype="f32",
             structure="outliers", ring_cap=128, decode_steps=1, step_mode="ring", seed=20262),
    _qwen_layer(4096),
    Workload(name="batched-b32-hkv8-n32768", batch=32, h_q=32, h_kv=8, n_tokens=32768,
             in_dtype="bf16", key_mse_bits=2, value_kind="minmax", value_bits=2,
             scalar_dtype="f32", structure="outliers", ring_cap=128, decode_steps=64,
             step_mode="ring", seed=20264),
    Workload(name="long-b1-hkv8-n131072", batch=1, h_q=32, h_kv=8, n_tokens=131072,
             in_dtype="bf16", key_mse_bits=3, value_kind="mse", value_bits=3,
             scalar_dtype="f32", structure="lognormal_kv", ring_cap=0, decode_steps=16,
             step_mode="encode", seed=20265),
]

#: The sequence-length sweep of the Qwen2.5-1.5B-shaped layer, with the
#: literal 3-bit-MSE + QJL key variant and fp32 scalars as extra cases.
QWEN_SWEEP = [_qwen_layer(n) for n in (512, 1024, 2048, 4096, 8192, 16384)]
QWEN_VARIANTS = [_qwen_layer(4096, key_mse_bits=3), _qwen_layer(4096, scalar_dtype="f32"),
                 _qwen_layer(4096, key_mse_bits=3, scalar_dtype="f32")]

#: Fractional key widths: the batched 32K-token decode and the Qwen-shaped
#: layer with 3.5-bit keys (2.5 MSE bits + QJL) and 2.5-bit keys (1.5 + QJL).
FRACTIONAL = [WORKLOADS[3].replace(name="batched-b32-hkv8-n32768-k3.5bit", key_half=1),
              WORKLOADS[3].replace(name="batched-b32-hkv8-n32768-k2.5bit", key_mse_bits=1, key_half=1),
              _qwen_layer(4096).replace(name="qwen2.5-1.5b-layer-n4096-k3.5bit", key_half=1)]


def by_name(name: str) -> Workload:
    for w in WORKLOADS + QWEN_SWEEP + QWEN_VARIANTS + FRACTIONAL:
        if w.name == name:
            return w
    raise KeyError(name)


def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *tags])))


def rotation(d: int, seed: int) -> np.ndarray:
    """A Haar-distributed random orthogonal d x d matrix in float64.

    Drawn as the Q factor of a QR decomposition of an i.i.d. N(0,1) matrix,
    with each column's sign fixed by the sign of R's diagonal (the standard way
    to sample the Haar measure).  This is the random draw of the rotation, not
    an application of it.
    """
    g = _rng(seed, _TAG_PI).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def qjl_matrix(d: int, seed: int) -> np.ndarray:
    """The QJL projection S: d x d i.i.d. N(0,1) entries, float64."""
    return _rng(seed, _TAG_S).standard_normal((d, d))


def channel_scales(w: Workload, which: str, n_heads: int) -> np.ndarray:
    """Per-(head, channel) multipliers applied to the N(0,1) draws.

    * ``outliers``: per KV head, 4 distinct channels drawn from the seed are
      scaled by 10 on both K and V (queries are left unscaled).
    * ``lognormal_*``: per (head, channel) std exp(N(0,1)), independent for K, V
      and (``lognormal_kvq`` only) q.
    """
    d = w.d
    out = np.ones((n_heads, d))
    if w.structure == "outliers" and which in ("k", "v"):
        rng = _rng(w.seed, _TAG_OUTLIER)
        for h in range(n_heads):
            out[h, rng.choice(d, size=4, replace=False)] = 10.0
    elif w.structure.startswith("lognormal"):
        if which == "q" and w.structure != "lognormal_kvq":
            return out
        tag = {"k": _TAG_SIGMA_K, "v": _TAG_SIGMA_V, "q": _TAG_SIGMA_Q}[which]
        out = np.exp(_rng(w.seed, tag).standard_normal((n_heads, d)))
    return out


def _cast(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def slot_tokens(w: Workload, which: str, b: int, h: int, n: int | None = None) -> torch.Tensor:
    """The first ``n`` prefill tokens of K or V for sequence b, KV head h:
    ``[n, d]`` in the workload dtype.  Generated per (b, h) so any slot can be
    regenerated alone."""
    n = w.n_tokens if n is None else n
    tag = _TAG_K if which == "k" else _TAG_V
    x = _rng(w.seed, tag, b, h).standard_normal((n, w.d))
    x *= channel_scales(w, which, w.h_kv)[h][None, :]
    return _cast(x, w.torch_dtype)


def prefill_kv(w: Workload, n: int | None = None, threads: int | None = None):
    """K and V prefill tensors ``[B, n, H_kv, d]`` (CPU, workload dtype)."""
    n = w.n_tokens if n is None else n
    k = torch.empty((w.batch, n, w.h_kv, w.d), dtype=w.torch_dtype)
    v = torch.empty_like(k)

    def fill(job):
        which, b, h = job
        dst = k if which == "k" else v
        dst[b, :, h, :] = slot_tokens(w, which, b, h, n)

    jobs = [(which, b, h) for which in ("k", "v") for b in range(w.batch) for h in range(w.h_kv)]
    threads = threads or min(16, os.cpu_count() or 1)
    if len(jobs) == 1 or threads == 1:
        for j in jobs:
            fill(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, jobs))
    return k, v


def query(w: Workload, step: int = 0) -> torch.Tensor:
    """The decode query of step ``step``: ``[B, H_q, d]`` in the workload dtype."""
    x = _rng(w.seed, _TAG_Q, step).standard_normal((w.batch, w.h_q, w.d))
    x *= channel_scales(w, "q", w.h_q)[None, :, :]
    return _cast(x, w.torch_dtype)


def step_kv(w: Workload, step: int):
    """The K/V of the token appended at decode step ``step``: ``[B, 1, H_kv, d]``
    each, drawn with the same per-channel structure as the prefill."""
    rng = _rng(w.seed, _TAG_STEP, step)
    k = rng.standard_normal((w.batch, 1, w.h_kv, w.d)) * channel_scales(w, "k", w.h_kv)[None, None]
    v = rng.standard_normal((w.batch, 1, w.h_kv, w.d)) * channel_scales(w, "v", w.h_kv)[None, None]
    return _cast(k, w.torch_dtype), _cast(v, w.torch_dtype)


def params(w: Workload):
    """(Pi, S) in float64 for the workload's layer."""
    return rotation(w.d, w.seed), qjl_matrix(w.d, w.seed)
