"""Host-side checks of libtq (no GPU needed): the library loads and exports every
symbol include/tq.h declares, its Lloyd-Max tables match the oracle's, its byte
accounting matches the oracle's recount, and bad arguments are rejected before
anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from compressed_kv_decode_tq_amd import tq
from oracle.layout import Layout as OLayout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = tq.lib()
    declared = _declared_symbols()
    assert set(declared) == set(tq.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert tq.version().startswith("tq ")


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [3, 4, 5, 8, 16, 128])
def test_codebook_matches_oracle(d, bits):
    c, t = tq.make_codebook(d, bits)
    ref = oracle.lloyd_max(d, bits)
    # double-precision solve rounded once to fp32: within one fp32 ulp of the oracle
    ulp_c = np.spacing(np.abs(ref.centroids).astype(np.float32))
    assert np.all(np.abs(c.astype(np.float64) - ref.centroids) <= ulp_c)
    ulp_t = np.spacing(np.maximum(np.abs(ref.thresholds), 1e-30).astype(np.float32))
    # the oracle does not impose symmetry, so its middle threshold is zero only to
    # its iteration tolerance (a few 1e-15); near zero the bound is absolute
    assert np.all(np.abs(t.astype(np.float64) - ref.thresholds) <= np.maximum(ulp_t, 1e-13))
    # exact symmetry of the table
    assert np.array_equal(c, -c[::-1])


def _lay(**kw):
    base = dict(head_dim=128, key_mse_bits=2, key_qjl=1, value_kind=tq.TQ_V_MINMAX, value_bits=2,
                value_group=32, scalar_dtype=tq.TQ_F32)
    base.update(kw)
    return tq.Layout(**base)


def _olay(l: tq.Layout) -> OLayout:
    return OLayout(d=l.head_dim, key_mse_bits=l.key_mse_bits, key_qjl=l.key_qjl,
                   value_kind="minmax" if l.value_kind == tq.TQ_V_MINMAX else "mse",
                   value_bits=l.value_bits, value_group=l.value_group,
                   scalar_dtype="f32" if l.scalar_dtype == tq.TQ_F32 else "f16", key_half=l.key_half)


@pytest.mark.parametrize("kw", [{}, {"scalar_dtype": tq.TQ_F16},
                                {"value_kind": tq.TQ_V_MSE, "value_bits": 3, "scalar_dtype": tq.TQ_F16},
                                {"key_mse_bits": 3, "value_kind": tq.TQ_V_MSE, "value_bits": 3},
                                {"key_qjl": 0, "value_bits": 4, "value_group": 16},
                                {"key_half": 1}, {"key_mse_bits": 1, "key_half": 1, "scalar_dtype": tq.TQ_F16},
                                {"key_half": 1, "value_kind": tq.TQ_V_MSE, "value_bits": 3}])
def test_memory_bytes_matches_oracle(kw):
    l = _lay(**kw)
    ol = _olay(l)
    for b, h, n in [(1, 8, 4096), (32, 8, 32768), (1, 2, 46), (3, 1, 0)]:
        assert tq.memory_bytes(l, b, h, n, 128, tq.TQ_BYTES_DATA) == oracle.memory_bytes(ol, b, h, n, "data")
        assert tq.memory_bytes(l, b, h, n, 128, tq.TQ_BYTES_RING) == oracle.memory_bytes(ol, b, h, n, "ring")
    assert tq.memory_bytes(l, 1, 8, 0, 0, tq.TQ_BYTES_PARAMS) == oracle.memory_bytes(ol, 1, 8, 0, "params")


def test_bad_layouts_are_rejected():
    for kw, code in [({"head_dim": 96}, tq.TQ_ERR_UNSUPPORTED), ({"head_dim": 100}, tq.TQ_ERR_INVALID),
                     ({"key_mse_bits": 0}, tq.TQ_ERR_INVALID), ({"key_mse_bits": 5}, tq.TQ_ERR_INVALID),
                     ({"value_bits": 0}, tq.TQ_ERR_INVALID), ({"value_group": 48}, tq.TQ_ERR_INVALID),
                     ({"value_group": 128}, tq.TQ_ERR_UNSUPPORTED), ({"scalar_dtype": 7}, tq.TQ_ERR_INVALID),
                     ({"value_kind": 3}, tq.TQ_ERR_INVALID), ({"key_qjl": 2}, tq.TQ_ERR_INVALID),
                     ({"key_half": 2}, tq.TQ_ERR_INVALID), ({"key_half": 1, "key_qjl": 0}, tq.TQ_ERR_UNSUPPORTED),
                     ({"key_half": 1, "key_mse_bits": 3}, tq.TQ_ERR_UNSUPPORTED)]:
        l = _lay(**kw)
        lay = l.c()
        r = tq.lib().tq_memory_bytes(ctypes.byref(lay), 1, 1, 1, 0, tq.TQ_BYTES_DATA)
        if code == tq.TQ_ERR_UNSUPPORTED:
            assert r > 0  # byte counts are defined for any valid layout
        else:
            assert r == code, (kw, r)
        # decode rejects it before touching any pointer
        cache = tq._Cache(1, 1, 1, 1, 1, 1, 1, 1, 32)
        prm = tq._Params()
        nc = (ctypes.c_int64 * 1)(0)
        rc = tq.lib().tq_decode_attn(ctypes.byref(lay), ctypes.byref(prm), 1, tq.TQ_F32, 1, ctypes.byref(cache),
                                     nc, None, None, 0, None, 1.0, 1, 1, 1 << 20, None)
        assert rc == code, (kw, rc, tq.lib().tq_last_error())
    assert tq.lib().tq_make_codebook(2, 2, None, None) == tq.TQ_ERR_INVALID
    assert tq.lib().tq_make_codebook(128, 5, None, None) == tq.TQ_ERR_INVALID


def test_encode_and_decode_argument_checks():
    lay = _lay().c()
    prm = tq._Params()
    prm.pi, prm.s, prm.derived = 16, 16, 16  # never dereferenced: every call below fails its checks first
    cache = tq._Cache(16, 16, 16, 16, 16, 0, 2, 1, 64)
    L = tq.lib()
    pos = (ctypes.c_int64 * 2)(0, 60)
    # positions 60..67 exceed capacity 64
    assert L.tq_encode_kv(ctypes.byref(lay), ctypes.byref(prm), 16, 16, tq.TQ_BF16, 8, pos,
                          ctypes.byref(cache), None) == tq.TQ_ERR_CAPACITY
    assert "capacity" in L.tq_last_error().decode()
    # bad dtype, NULL inputs, negative n
    assert L.tq_encode_kv(ctypes.byref(lay), ctypes.byref(prm), 16, 16, tq.TQ_F16, 1, pos,
                          ctypes.byref(cache), None) == tq.TQ_ERR_INVALID
    assert L.tq_encode_kv(ctypes.byref(lay), ctypes.byref(prm), None, 16, tq.TQ_BF16, 1, pos,
                          ctypes.byref(cache), None) == tq.TQ_ERR_INVALID
    assert L.tq_encode_kv(ctypes.byref(lay), ctypes.byref(prm), 16, 16, tq.TQ_BF16, -1, pos,
                          ctypes.byref(cache), None) == tq.TQ_ERR_INVALID
    # zero new tokens is a no-op
    assert L.tq_encode_kv(ctypes.byref(lay), ctypes.byref(prm), 16, 16, tq.TQ_BF16, 0, pos,
                          ctypes.byref(cache), None) == tq.TQ_OK
    # capacity not a multiple of 32
    bad = tq._Cache(16, 16, 16, 16, 16, 0, 2, 1, 48)
    assert L.tq_encode_kv(ctypes.byref(lay), ctypes.byref(prm), 16, 16, tq.TQ_BF16, 1, pos,
                          ctypes.byref(bad), None) == tq.TQ_ERR_INVALID
    # min/max values need v_meta
    nometa = tq._Cache(16, 16, 16, 16, 0, 0, 2, 1, 64)
    assert L.tq_encode_kv(ctypes.byref(lay), ctypes.byref(prm), 16, 16, tq.TQ_BF16, 1, pos,
                          ctypes.byref(nometa), None) == tq.TQ_ERR_INVALID
    # decode: h_q not a multiple of h_kv, too many heads per group, short workspace, n beyond capacity
    nc = (ctypes.c_int64 * 2)(64, 10)
    nr = (ctypes.c_int32 * 2)(0, 0)
    args = lambda hq, ws, ncv=nc: (ctypes.byref(lay), ctypes.byref(prm), 16, tq.TQ_F32, hq, ctypes.byref(cache),  # noqa: E731
                                   ncv, None, None, 0, nr, 0.1, 16, 16, ws, None)
    assert L.tq_decode_attn(*args(9, 1 << 30)) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_decode_attn(*args(4, 8)) == tq.TQ_ERR_WORKSPACE
    big = (ctypes.c_int64 * 2)(65, 0)
    assert L.tq_decode_attn(*args(4, 1 << 30, big)) == tq.TQ_ERR_CAPACITY
    need = L.tq_decode_workspace_bytes(ctypes.byref(lay), 2, 4, 1, 64)
    assert need > 0
    # multi-query: one query is the single-query size; more need at least as much
    margs = lambda nq, ws: (ctypes.byref(lay), ctypes.byref(prm), 16, tq.TQ_F32, 4, nq,  # noqa: E731
                            ctypes.byref(cache), nc, None, None, 0, nr, 0.1, 16, 16, ws, None)
    assert L.tq_decode_workspace_bytes_multi(ctypes.byref(lay), 2, 4, 1, 64, 1) == need
    assert L.tq_decode_workspace_bytes_multi(ctypes.byref(lay), 2, 4, 1, 64, 3) >= need
    assert L.tq_decode_workspace_bytes_multi(ctypes.byref(lay), 2, 4, 1, 64, 0) == 0
    assert L.tq_decode_attn_multi(*margs(0, 1 << 30)) == tq.TQ_ERR_INVALID
    assert L.tq_decode_attn_multi(*margs(3, 8)) == tq.TQ_ERR_WORKSPACE
    # fused append: NULL token, bad dtype, no ring, a ring with no room left;
    # each fails its checks before any launch
    rk = ctypes.c_void_p(16)
    aargs = lambda kn, dt, rcap, nrv: (ctypes.byref(lay), ctypes.byref(prm), 16, tq.TQ_F32, 4,  # noqa: E731
                                       ctypes.byref(cache), nc, kn, kn, dt, rk, rk, rcap, nrv, 0.1, 16, 16,
                                       1 << 30, None)
    assert L.tq_decode_attn_append(*aargs(None, tq.TQ_BF16, 128, nr)) == tq.TQ_ERR_INVALID
    assert L.tq_decode_attn_append(*aargs(16, tq.TQ_F16, 128, nr)) == tq.TQ_ERR_INVALID
    assert L.tq_decode_attn_append(*aargs(16, tq.TQ_BF16, 0, nr)) == tq.TQ_ERR_INVALID
    nr_last = (ctypes.c_int32 * 2)(0, 128)
    assert L.tq_decode_attn_append(*aargs(16, tq.TQ_BF16, 128, nr_last)) == tq.TQ_ERR_CAPACITY
    assert "appended" in L.tq_last_error().decode()
    # ring append bounds
    nr_full = (ctypes.c_int32 * 2)(0, 128)
    assert L.tq_ring_append(16, 16, tq.TQ_BF16, 2, 1, 128, 16, 16, 128, nr_full, None) == tq.TQ_ERR_CAPACITY
    assert L.tq_ring_append(16, 16, tq.TQ_BF16, 2, 1, 64, 16, 16, 128, nr, None) == tq.TQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("batch,h_q,h_kv", [(1, 1, 1), (1, 32, 8), (32, 32, 8), (1, 12, 2), (100, 32, 8)])
def test_decode_workspace_never_shrinks_with_more_tokens(batch, h_q, h_kv):
    """A workspace sized for a capacity fits every call with fewer tokens: the
    required size never decreases as max_tokens grows (the split count of a
    shorter sequence can exceed that of a longer one, so the bound must cover
    all lengths up to max_tokens)."""
    lay = tq.Layout()
    prev = 0
    for n in list(range(0, 5000, 37)) + [32768, 32769, 32896, 131072, 131088, 1 << 20]:
        need = tq.decode_workspace_bytes(lay, batch, h_q, h_kv, n)
        assert need >= prev, (n, need, prev)
        prev = need


def test_product_path_fails_loudly_without_the_library(monkeypatch):
    """No fallback: with libtq.so absent every call of the binding raises."""
    monkeypatch.setattr(tq, "_LIB_PATH", os.path.join(ROOT, "no-such-dir", "libtq.so"))
    monkeypatch.setattr(tq, "_lib", None)
    with pytest.raises(ImportError):
        tq.lib()
    with pytest.raises(ImportError):
        tq.make_codebook(128, 2)
    with pytest.raises(ImportError):
        tq.memory_bytes(_lay(), 1, 1, 1, 0, tq.TQ_BYTES_DATA)


def test_product_package_does_not_import_the_oracle():
    """The product path (the binding, the build, the input generators) never
    imports the oracle; only tests, the smoke test and the CPU baseline of the
    bench do."""
    import ast
    pkg = os.path.join(ROOT, "compressed_kv_decode_tq_amd")
    for fn in sorted(os.listdir(pkg)):
        if not fn.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(pkg, fn)).read())
        for node in ast.walk(tree):
            names = []
            if isinstance(node, ast.Import):
                names = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                names = [node.module or ""]
            assert not any(n == "oracle" or n.startswith("oracle.") for n in names), (fn, names)
