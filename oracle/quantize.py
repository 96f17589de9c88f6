"""TurboQuant encoders and dequantizers, float64, one vector per row.

TEST INFRASTRUCTURE (see the package docstring).

Keys use the product quantizer ``TurboQuantProd(bits=b)`` of [audit] AUDIT 3 /
AUDIT 5: a (b-1)-bit Lloyd-Max code of the rotated unit vector plus a 1-bit QJL
sign sketch of the residual and the residual's norm ([explainer] "Ý tưởng cốt
lõi", stages 1 and 2).  Values use either the asymmetric min/max group code
named by the store's ``value_bits`` / ``value_group_size`` ([audit] AUDIT 1), or
the same rotated Lloyd-Max code as the keys (MSE only).

Readings taken where the pages are silent:

* Pi rotates column vectors: y = Pi u.  S multiplies the residual in the
  original space: sigma = sign(S r), r = u - Pi^T c[idx].
* A coordinate equal to a threshold goes to the lower cell; sign(0) = +1.
* A zero vector has u = 0 (its codes come from y = 0); its norm 0 makes every
  score and every reconstructed value 0.
* QJL scale: sqrt(pi/2)/m with m = d rows of S, since for s ~ N(0, I)
  E[sign(<s,r>) <s,y>] = sqrt(2/pi) <r,y>/|r|.
* Fractional key widths (the pages' 2.5 and 3.5 bits per channel, [explainer]
  "Ý tưởng cốt lõi" / "Ý nghĩa thực tế"; the pages do not say how the half bit
  is spent): half of the rotated coordinates, those i with i mod 32 < 16, use a
  Lloyd-Max quantizer with one more bit than the rest.  After the rotation
  every coordinate has the same law, so which half gets the extra bit does
  not change the distortion.  TurboQuantProd(3.5) = 2.5 MSE bits + QJL,
  TurboQuantProd(2.5) = 1.5 MSE bits + QJL.
* Stored scalars (n, gamma, value norm) are rounded once to the layout's
  scalar dtype (fp32 or fp16, round-to-nearest-even); normalisation uses the
  unrounded norm, reconstruction the stored one.
* Min/max values: groups of ``group`` consecutive channels of one token.  The
  scale and zero are stored as fp16; the scale is the group's range over the
  2^b - 1 steps, formed in IEEE fp32 and then rounded to fp16, the zero is the
  group's minimum rounded to fp16.  The code of each channel is the nearest
  step from the STORED zero in units of the STORED scale, by plain division in
  float64 with ties to even:
      delta16 = fp16(fp32(fp32(max) - fp32(min)) / fp32(2^b - 1)), min16 = fp16(min)
      code    = clip(rint_half_even((v - min16) / delta16), 0, 2^b - 1)
  with code 0 wherever delta16 == 0.  Reconstruction: min16 + code * delta16.
  An implementation that forms the ratio in lower precision agrees with this
  except where the ratio lies within its rounding error of a half-integer.
"""
from __future__ import annotations

import dataclasses

import numpy as np

QJL_SCALE = np.sqrt(np.pi / 2.0)


def round_scalar(x: np.ndarray, scalar_dtype: str) -> np.ndarray:
    """Store a float64 scalar as fp32 or fp16 (round to nearest even) and read
    it back as float64."""
    if scalar_dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if scalar_dtype == "f16":
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
    raise ValueError(scalar_dtype)


def _normalize(x: np.ndarray):
    n = np.linalg.norm(x, axis=-1)
    safe = np.where(n > 0, n, 1.0)
    u = np.where(n[..., None] > 0, x / safe[..., None], 0.0)
    return n, u


def half_bit_coordinates(d: int) -> np.ndarray:
    """Mask of the rotated coordinates that get the extra bit in the fractional
    (half-bit) key layout: i mod 32 < 16."""
    return (np.arange(d) % 32) < 16


def _centroid_values(idx: np.ndarray, centroids: np.ndarray, centroids_hi=None) -> np.ndarray:
    """c[idx] per coordinate; with centroids_hi, the half-bit coordinates read
    the larger table."""
    if centroids_hi is None:
        return centroids[idx]
    mask = half_bit_coordinates(idx.shape[-1])
    out = np.empty(idx.shape, dtype=np.float64)
    out[..., ~mask] = centroids[idx[..., ~mask]]
    out[..., mask] = centroids_hi[idx[..., mask]]
    return out


def _bucketize(y: np.ndarray, thresholds: np.ndarray) -> np.ndarray:
    """idx = #{k : t_k < y}; a value equal to a threshold stays in the lower cell."""
    return np.searchsorted(thresholds, y, side="left").astype(np.int64)


@dataclasses.dataclass
class KeyCode:
    idx: np.ndarray  # (T, d) int, Lloyd-Max cell of each rotated coordinate
    qjl: np.ndarray  # (T, d) uint8, 1 where (S r)_i >= 0
    norm: np.ndarray  # (T,) stored |k|
    rnorm: np.ndarray  # (T,) stored gamma = |r|
    # unrounded intermediates, used by the tests' boundary windows
    y: np.ndarray  # (T, d) rotated unit vector Pi u
    z: np.ndarray  # (T, d) QJL projection S r


def encode_keys(k: np.ndarray, Pi: np.ndarray, S: np.ndarray, centroids: np.ndarray,
                thresholds: np.ndarray, scalar_dtype: str = "f32", qjl: bool = True,
                centroids_hi=None, thresholds_hi=None) -> KeyCode:
    """TurboQuantProd encode of the rows of k (any float dtype, promoted to float64).

    Steps, in the order of [explainer] "Ý tưởng cốt lõi" / "Tại sao nó hoạt động":
      1. n = |k|, u = k / n
      2. y = Pi u                         (rotate)
      3. idx_i = #{t : t < y_i}          (one scalar quantizer for every coordinate)
      4. r = u - Pi^T c[idx], gamma = |r| (residual of the MSE stage)
      5. sigma = sign(S r)               (1-bit QJL sketch of the residual)
    With centroids_hi / thresholds_hi (one more bit), the half-bit coordinates
    of half_bit_coordinates use those tables in step 3.
    """
    k = np.asarray(k, dtype=np.float64)
    n, u = _normalize(k)
    y = u @ Pi.T
    idx = _bucketize(y, thresholds)
    if thresholds_hi is not None:
        mask = half_bit_coordinates(y.shape[-1])
        idx = np.where(mask, _bucketize(y, thresholds_hi), idx)
    u_mse = _centroid_values(idx, centroids, centroids_hi) @ Pi
    r = u - u_mse
    gamma = np.linalg.norm(r, axis=-1)
    if qjl:
        z = r @ S.T
        bits = (z >= 0).astype(np.uint8)
    else:
        z = np.zeros_like(r)
        bits = np.zeros(r.shape, dtype=np.uint8)
        gamma = np.zeros_like(gamma)
    return KeyCode(idx=idx, qjl=bits, norm=round_scalar(n, scalar_dtype),
                   rnorm=round_scalar(gamma, scalar_dtype), y=y, z=z)


def dequantize_keys(code: KeyCode, Pi: np.ndarray, S: np.ndarray, centroids: np.ndarray,
                    qjl: bool = True, centroids_hi=None) -> np.ndarray:
    """k~ = n (Pi^T c[idx] + sqrt(pi/2)/d * gamma * S^T sigma), sigma = 2 bit - 1:
    the reconstruction whose inner product with any query is the unbiased
    TurboQuantProd score ([audit] AUDIT 2 dequantizes keys this way before
    its matmul; AUDIT 6 checks the unbiasedness)."""
    d = Pi.shape[0]
    k_mse = _centroid_values(code.idx, centroids, centroids_hi) @ Pi
    if qjl:
        sigma = 2.0 * code.qjl.astype(np.float64) - 1.0
        k_qjl = (QJL_SCALE / d) * code.rnorm[:, None] * (sigma @ S)
    else:
        k_qjl = 0.0
    return code.norm[:, None] * (k_mse + k_qjl)


def score_estimate(q: np.ndarray, code: KeyCode, Pi: np.ndarray, S: np.ndarray,
                   centroids: np.ndarray, qjl: bool = True, centroids_hi=None) -> np.ndarray:
    """<q, k> estimate for every key (the quantizer's ``attention_score`` of
    [audit] AUDIT 3/5/6): the query is rotated once and the keys are never
    reconstructed ([explainer] "Tại sao nó hoạt động", rotate the query at run
    time):  n (<Pi q, c[idx]> + sqrt(pi/2)/d * gamma <S q, sigma>)."""
    q = np.asarray(q, dtype=np.float64)
    d = Pi.shape[0]
    s = _centroid_values(code.idx, centroids, centroids_hi) @ (Pi @ q)
    if qjl:
        sigma = 2.0 * code.qjl.astype(np.float64) - 1.0
        s = s + (QJL_SCALE / d) * code.rnorm * (sigma @ (S @ q))
    return code.norm * s


@dataclasses.dataclass
class ValueMinMax:
    code: np.ndarray  # (T, d) int
    scale16: np.ndarray  # (T, d/group) float16 delta
    min16: np.ndarray  # (T, d/group) float16 zero
    ratio: np.ndarray  # (T, d) float64 (v - min16) / delta16, before rounding (0 where delta16 == 0)


def encode_values_minmax(v: np.ndarray, bits: int, group: int) -> ValueMinMax:
    """Asymmetric b-bit min/max code per group of ``group`` channels ([audit]
    AUDIT 1 store arguments ``value_bits``, ``value_group_size``), as stated
    in the module docstring: fp16 scale and zero, then each code by float64
    division against the stored fp16 values."""
    v64 = np.asarray(v, dtype=np.float64)
    t, d = v64.shape
    if d % group:
        raise ValueError("group must divide d")
    g = v64.reshape(t, d // group, group)
    # scale and zero: the range is formed in fp32 (the inputs are fp32 or
    # bf16, so their fp32 values are exact), then stored as fp16
    mn32 = g.min(axis=-1).astype(np.float32)
    mx32 = g.max(axis=-1).astype(np.float32)
    levels = (1 << bits) - 1
    delta32 = (mx32 - mn32) / np.float32(levels)
    scale16 = delta32.astype(np.float16)
    min16 = mn32.astype(np.float16)
    s64 = scale16.astype(np.float64)[..., None]
    m64 = min16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(s64 > 0, (g - m64) / np.where(s64 > 0, s64, 1.0), 0.0)
    code = np.clip(np.rint(ratio), 0, levels).astype(np.int64)
    return ValueMinMax(code=code.reshape(t, d), scale16=scale16, min16=min16,
                       ratio=ratio.reshape(t, d))


def dequantize_values_minmax(code: ValueMinMax, group: int) -> np.ndarray:
    t, d = code.code.shape
    c = code.code.reshape(t, d // group, group).astype(np.float64)
    v = code.min16.astype(np.float64)[..., None] + c * code.scale16.astype(np.float64)[..., None]
    return v.reshape(t, d)


@dataclasses.dataclass
class ValueMSE:
    idx: np.ndarray  # (T, d) int
    norm: np.ndarray  # (T,) stored |v|
    y: np.ndarray  # (T, d) rotated unit vector, for boundary windows


def encode_values_mse(v: np.ndarray, Pi: np.ndarray, centroids: np.ndarray,
                      thresholds: np.ndarray, scalar_dtype: str = "f32") -> ValueMSE:
    """TurboQuant-MSE code of a value vector: n_v = |v|, idx = Q(Pi v / n_v)
    ([explainer] "Ý tưởng cốt lõi", stage 1 alone)."""
    v = np.asarray(v, dtype=np.float64)
    n, u = _normalize(v)
    y = u @ Pi.T
    return ValueMSE(idx=_bucketize(y, thresholds), norm=round_scalar(n, scalar_dtype), y=y)


def dequantize_values_mse(code: ValueMSE, Pi: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """v~ = n_v Pi^T c[idx]."""
    return code.norm[:, None] * (centroids[code.idx] @ Pi)
