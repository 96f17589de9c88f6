// Host-only exercise of the libtq C ABI (include/tq.h) under AddressSanitizer
// and UndefinedBehaviorSanitizer, linked against the stand-in launchers of
// stub_launch.cpp.  Every "device" buffer is a host allocation of exactly the
// size the header documents, so the stubs' first/last-byte touches turn any
// host offset mistake into a sanitizer report.  Prints "host ABI checks: N
// passed" and exits 0 when every check holds; a failed check exits 1.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <vector>

#include "stub_launch.h"
#include "tq.h"

namespace {

int g_checks = 0;

#define CHECK(cond)                                                                  \
  do {                                                                               \
    ++g_checks;                                                                      \
    if (!(cond)) {                                                                   \
      std::fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__, \
                   __LINE__, #cond, tq_last_error());                                \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

// A heap block of exactly n bytes (at least one, so the pointer is non-NULL).
struct Buf {
  std::unique_ptr<unsigned char[]> p;
  size_t n = 0;
  explicit Buf(size_t bytes = 0) : p(new unsigned char[bytes ? bytes : 1]), n(bytes) {}
  void* get() const { return p.get(); }
};

tq_layout layout(int kbits, int qjl, int vkind, int vbits, int vgroup, int sdt, int half = 0) {
  tq_layout l;
  std::memset(&l, 0, sizeof(l));
  l.head_dim = 128;
  l.key_mse_bits = kbits;
  l.key_qjl = qjl;
  l.value_kind = vkind;
  l.value_bits = vbits;
  l.value_group = vgroup;
  l.scalar_dtype = sdt;
  l.key_half = half;
  return l;
}

size_t ssz(const tq_layout& l) { return l.scalar_dtype == TQ_F32 ? 4 : 2; }
size_t key_rec(const tq_layout& l) {
  return (size_t)(l.key_mse_bits + l.key_qjl) * 16 + (size_t)l.key_half * 8;
}

// A cache whose arrays have exactly the documented sizes.
struct HostCache {
  Buf kp, kn, kr, vp, vm, vn;
  tq_cache c;
  HostCache(const tq_layout& l, int batch, int h_kv, int64_t cap) {
    const size_t slots = (size_t)batch * h_kv * cap;
    kp = Buf((size_t)batch * h_kv * ((cap + 63) / 64 * 64) * key_rec(l));  // whole 64-token blocks
    kn = Buf(slots * ssz(l));
    if (l.key_qjl) kr = Buf(slots * ssz(l));
    vp = Buf(slots * (size_t)l.value_bits * 16);
    if (l.value_kind == TQ_V_MINMAX) vm = Buf(slots * (size_t)(128 / l.value_group) * 4);
    if (l.value_kind == TQ_V_MSE) vn = Buf(slots * ssz(l));
    std::memset(&c, 0, sizeof(c));
    c.k_planes = (uint8_t*)kp.get();
    c.k_norm = kn.get();
    c.k_rnorm = l.key_qjl ? kr.get() : nullptr;
    c.v_planes = (uint32_t*)vp.get();
    c.v_meta = l.value_kind == TQ_V_MINMAX ? (uint16_t*)vm.get() : nullptr;
    c.v_norm = l.value_kind == TQ_V_MSE ? vn.get() : nullptr;
    c.batch = batch;
    c.num_kv_heads = h_kv;
    c.capacity = cap;
  }
};

struct HostParams {
  Buf pi{128 * 128 * 4}, s{128 * 128 * 4}, derived;
  tq_params p;
  explicit HostParams(const tq_layout& l) {
    derived = Buf(tq_params_derived_bytes(128));
    std::memset(&p, 0, sizeof(p));
    p.pi = (const float*)pi.get();
    p.s = (const float*)s.get();
    p.derived = derived.get();
    CHECK(tq_make_codebook(128, l.key_mse_bits, p.k_centroids, p.k_thresholds) == TQ_OK);
    if (l.key_half) CHECK(tq_make_codebook(128, l.key_mse_bits + 1, p.k_centroids_hi, p.k_thresholds_hi) == TQ_OK);
    if (l.value_kind == TQ_V_MSE) CHECK(tq_make_codebook(128, l.value_bits, p.v_centroids, p.v_thresholds) == TQ_OK);
  }
};

void reset_log() { stub::g_log = stub::Log{}; }

void test_codebook() {
  for (int d : {3, 4, 5, 64, 128, 1024}) {
    for (int bits = 1; bits <= 4; ++bits) {
      float c[16], t[15];
      CHECK(tq_make_codebook(d, bits, c, t) == TQ_OK);
      const int L = 1 << bits;
      for (int i = 0; i < L; ++i) {
        CHECK(std::isfinite(c[i]) && std::fabs(c[i]) < 1.f);
        CHECK(std::fabs(c[i] + c[L - 1 - i]) <= 1e-6f * (1.f + std::fabs(c[i])));  // symmetric law
        if (i + 1 < L) {
          CHECK(c[i] < c[i + 1]);
          CHECK(std::fabs(t[i] - 0.5f * (c[i] + c[i + 1])) <= 1e-6f);  // midpoint condition
        }
      }
    }
  }
  float c[16], t[15];
  CHECK(tq_make_codebook(2, 2, c, t) == TQ_ERR_INVALID);
  CHECK(std::strlen(tq_last_error()) > 0);
  CHECK(tq_make_codebook(128, 0, c, t) == TQ_ERR_INVALID);
  CHECK(tq_make_codebook(128, 5, c, t) == TQ_ERR_INVALID);
  CHECK(tq_make_codebook(128, 2, nullptr, t) == TQ_ERR_INVALID);
  CHECK(tq_make_codebook(128, 2, c, nullptr) == TQ_ERR_INVALID);
  CHECK(tq_make_codebook(128, 2, c, t) == TQ_OK && tq_last_error()[0] == 0);
}

void test_memory_bytes() {
  const tq_layout a = layout(2, 1, TQ_V_MINMAX, 2, 32, TQ_F32);
  // keys 2 + 1 bits (48 B) + two fp32 scalars; values 2 bits (32 B) + 4 groups x (fp16 scale, fp16 min)
  CHECK(tq_memory_bytes(&a, 1, 1, 1, 0, TQ_BYTES_DATA) == 48 + 8 + 32 + 16);
  CHECK(tq_memory_bytes(&a, 32, 8, 32768, 0, TQ_BYTES_DATA) == (int64_t)104 * 32 * 8 * 32768);
  const tq_layout b = layout(3, 1, TQ_V_MSE, 3, 32, TQ_F16);
  CHECK(tq_memory_bytes(&b, 2, 3, 5, 0, TQ_BYTES_DATA) == (int64_t)(64 + 4 + 48 + 2) * 2 * 3 * 5);
  const tq_layout h = layout(2, 1, TQ_V_MINMAX, 2, 32, TQ_F32, 1);
  CHECK(tq_memory_bytes(&h, 1, 1, 1, 0, TQ_BYTES_DATA) == 48 + 8 + 8 + 32 + 16);
  CHECK(tq_memory_bytes(&a, 4, 8, 0, 128, TQ_BYTES_RING) == (int64_t)4 * 128 * 8 * 128 * 2 * 2);
  CHECK(tq_memory_bytes(&a, 1, 1, 1, 0, TQ_BYTES_PARAMS) > 2 * 128 * 128 * 4);
  CHECK(tq_memory_bytes(&a, -1, 1, 1, 0, TQ_BYTES_DATA) == TQ_ERR_INVALID);
  CHECK(tq_memory_bytes(&a, 1, 1, -5, 0, TQ_BYTES_DATA) == TQ_ERR_INVALID);
  CHECK(tq_memory_bytes(&a, 1, 1, 1, 0, 99) == TQ_ERR_INVALID);
  CHECK(tq_memory_bytes(nullptr, 1, 1, 1, 0, TQ_BYTES_DATA) == TQ_ERR_INVALID);
  tq_layout bad = a;
  bad.value_group = 48;
  CHECK(tq_memory_bytes(&bad, 1, 1, 1, 0, TQ_BYTES_DATA) == TQ_ERR_INVALID);
}

void test_prepare() {
  Buf pi(128 * 128 * 4), s(128 * 128 * 4), derived(tq_params_derived_bytes(128));
  CHECK(tq_params_derived_bytes(128) > 0 && tq_params_derived_bytes(64) == 0);
  reset_log();
  CHECK(tq_prepare_params(128, (const float*)pi.get(), (const float*)s.get(), derived.get(), derived.n, nullptr) == TQ_OK);
  CHECK(stub::g_log.prepare == 1);
  CHECK(tq_prepare_params(64, (const float*)pi.get(), (const float*)s.get(), derived.get(), derived.n, nullptr) ==
        TQ_ERR_UNSUPPORTED);
  CHECK(tq_prepare_params(100, (const float*)pi.get(), (const float*)s.get(), derived.get(), derived.n, nullptr) ==
        TQ_ERR_INVALID);
  CHECK(tq_prepare_params(128, nullptr, (const float*)s.get(), derived.get(), derived.n, nullptr) == TQ_ERR_INVALID);
  CHECK(tq_prepare_params(128, (const float*)pi.get(), (const float*)s.get(), derived.get(), derived.n - 1, nullptr) ==
        TQ_ERR_INVALID);
  CHECK(stub::g_log.prepare == 1);  // rejected calls launch nothing
}

void test_layout_checks() {
  Buf k(1024), v(1024);
  int64_t pos[1] = {0};
  const tq_layout ok = layout(2, 1, TQ_V_MINMAX, 2, 32, TQ_F32);
  HostParams hp(ok);
  HostCache hc(ok, 1, 1, 32);
  struct Bad { tq_layout l; int code; };
  std::vector<Bad> bad;
  auto with = [&](auto f, int code) { tq_layout l = ok; f(l); bad.push_back({l, code}); };
  with([](tq_layout& l) { l.head_dim = 64; }, TQ_ERR_UNSUPPORTED);
  with([](tq_layout& l) { l.head_dim = 100; }, TQ_ERR_INVALID);
  with([](tq_layout& l) { l.key_mse_bits = 0; }, TQ_ERR_INVALID);
  with([](tq_layout& l) { l.key_mse_bits = 5; }, TQ_ERR_INVALID);
  with([](tq_layout& l) { l.key_qjl = 2; }, TQ_ERR_INVALID);
  with([](tq_layout& l) { l.value_kind = 7; }, TQ_ERR_INVALID);
  with([](tq_layout& l) { l.value_bits = 0; }, TQ_ERR_INVALID);
  with([](tq_layout& l) { l.value_group = 0; }, TQ_ERR_INVALID);
  with([](tq_layout& l) { l.value_group = 8; }, TQ_ERR_UNSUPPORTED);
  with([](tq_layout& l) { l.scalar_dtype = 9; }, TQ_ERR_INVALID);
  with([](tq_layout& l) { l.key_half = 3; }, TQ_ERR_INVALID);
  with([](tq_layout& l) { l.key_half = 1; l.key_mse_bits = 3; }, TQ_ERR_UNSUPPORTED);
  with([](tq_layout& l) { l.key_half = 1; l.key_qjl = 0; }, TQ_ERR_UNSUPPORTED);
  reset_log();
  for (const Bad& b : bad)
    CHECK(tq_encode_kv(&b.l, &hp.p, k.get(), v.get(), TQ_F32, 1, pos, &hc.c, nullptr) == b.code);
  CHECK(stub::g_log.encode_keys.empty() && stub::g_log.encode_values == 0);
}

// Bulk and few-token encodes over several batch sizes (launches of at most 64
// sequences) and layouts, each against exactly sized buffers.
void test_encode() {
  const tq_layout layouts[] = {
      layout(2, 1, TQ_V_MINMAX, 2, 32, TQ_F32), layout(3, 1, TQ_V_MSE, 3, 32, TQ_F16),
      layout(1, 0, TQ_V_MINMAX, 4, 16, TQ_F16), layout(2, 1, TQ_V_MINMAX, 4, 64, TQ_F32, 1),
      layout(4, 0, TQ_V_MSE, 2, 32, TQ_F32)};
  for (const tq_layout& l : layouts) {
    HostParams hp(l);
    for (int batch : {1, 3, 64, 65, 130}) {
      const int h_kv = 2;
      const int64_t cap = 96;
      HostCache hc(l, batch, h_kv, cap);
      for (int64_t n_new : {1, 5, 40}) {
        for (int dt : {TQ_F32, TQ_BF16}) {
          const size_t esz = dt == TQ_F32 ? 4 : 2;
          Buf k((size_t)batch * n_new * h_kv * 128 * esz), v((size_t)batch * n_new * h_kv * 128 * esz);
          std::vector<int64_t> pos(batch);
          for (int b = 0; b < batch; ++b) pos[b] = (b * 37) % (cap - n_new + 1);  // unaligned starts
          for (bool small : {false, true}) {
            stub::g_small_supported = small;
            reset_log();
            CHECK(tq_encode_kv(&l, &hp.p, k.get(), v.get(), dt, n_new, pos.data(), &hc.c, nullptr) == TQ_OK);
            const int launches = (batch + 63) / 64;
            const bool fused = small && l.value_kind == TQ_V_MSE;
            CHECK((int)stub::g_log.encode_keys.size() == (fused ? 0 : launches));
            CHECK(stub::g_log.encode_values == (fused ? 0 : launches));
            CHECK(stub::g_log.encode_small == (fused ? launches : 0));
            int seen = 0;
            for (const tq::EncodeArgs& a : stub::g_log.encode_keys) {
              CHECK(a.batch == std::min(64, batch - seen));
              for (int b = 0; b < a.batch; ++b) CHECK(a.pos.v[b] == pos[seen + b]);
              seen += a.batch;
            }
          }
          stub::g_small_supported = false;
        }
      }
      // errors: nothing launched
      Buf k((size_t)batch * 4 * h_kv * 128 * 4), v(k.n);
      std::vector<int64_t> pos(batch, 0);
      reset_log();
      pos[batch - 1] = cap - 3;
      CHECK(tq_encode_kv(&l, &hp.p, k.get(), v.get(), TQ_F32, 4, pos.data(), &hc.c, nullptr) == TQ_ERR_CAPACITY);
      pos[batch - 1] = -1;
      CHECK(tq_encode_kv(&l, &hp.p, k.get(), v.get(), TQ_F32, 4, pos.data(), &hc.c, nullptr) == TQ_ERR_INVALID);
      pos[batch - 1] = 0;
      CHECK(tq_encode_kv(&l, &hp.p, nullptr, v.get(), TQ_F32, 4, pos.data(), &hc.c, nullptr) == TQ_ERR_INVALID);
      CHECK(tq_encode_kv(&l, &hp.p, k.get(), v.get(), 5, 4, pos.data(), &hc.c, nullptr) == TQ_ERR_INVALID);
      CHECK(tq_encode_kv(&l, &hp.p, k.get(), v.get(), TQ_F32, -1, pos.data(), &hc.c, nullptr) == TQ_ERR_INVALID);
      CHECK(tq_encode_kv(&l, &hp.p, k.get(), v.get(), TQ_F32, 0, pos.data(), &hc.c, nullptr) == TQ_OK);
      tq_params np = hp.p;
      np.derived = nullptr;
      CHECK(tq_encode_kv(&l, &np, k.get(), v.get(), TQ_F32, 4, pos.data(), &hc.c, nullptr) == TQ_ERR_INVALID);
      tq_cache nc = hc.c;
      nc.capacity = 40;
      CHECK(tq_encode_kv(&l, &hp.p, k.get(), v.get(), TQ_F32, 4, pos.data(), &nc, nullptr) == TQ_ERR_INVALID);
      if (l.key_qjl) {
        nc = hc.c;
        nc.k_rnorm = nullptr;
        CHECK(tq_encode_kv(&l, &hp.p, k.get(), v.get(), TQ_F32, 4, pos.data(), &nc, nullptr) == TQ_ERR_INVALID);
      }
      CHECK(stub::g_log.encode_keys.empty() && stub::g_log.encode_values == 0);
    }
  }
}

void test_ring_append() {
  for (int batch : {1, 64, 65, 130}) {
    const int h_kv = 3, cap = 17;
    for (int dt : {TQ_F32, TQ_BF16}) {
      const size_t esz = dt == TQ_F32 ? 4 : 2;
      Buf k((size_t)batch * h_kv * 128 * esz), v(k.n);
      Buf rk((size_t)batch * cap * h_kv * 128 * 2), rv(rk.n);
      std::vector<int32_t> nr(batch);
      for (int b = 0; b < batch; ++b) nr[b] = b % cap;
      reset_log();
      CHECK(tq_ring_append(k.get(), v.get(), dt, batch, h_kv, 128, rk.get(), rv.get(), cap, nr.data(), nullptr) == TQ_OK);
      CHECK((int)stub::g_log.ring_batches.size() == (batch + 63) / 64);
      nr[batch - 1] = cap;
      CHECK(tq_ring_append(k.get(), v.get(), dt, batch, h_kv, 128, rk.get(), rv.get(), cap, nr.data(), nullptr) ==
            TQ_ERR_CAPACITY);
      nr[batch - 1] = 0;
      CHECK(tq_ring_append(k.get(), v.get(), dt, batch, h_kv, 64, rk.get(), rv.get(), cap, nr.data(), nullptr) ==
            TQ_ERR_UNSUPPORTED);
      CHECK(tq_ring_append(nullptr, v.get(), dt, batch, h_kv, 128, rk.get(), rv.get(), cap, nr.data(), nullptr) ==
            TQ_ERR_INVALID);
      CHECK(tq_ring_append(k.get(), v.get(), dt, batch, h_kv, 128, rk.get(), rv.get(), 0, nr.data(), nullptr) ==
            TQ_ERR_INVALID);
      CHECK((int)stub::g_log.ring_batches.size() == (batch + 63) / 64);
    }
  }
}

// One decode configuration: exact-size q, out, workspace, cache and ring.
struct DecodeCase {
  tq_layout l;
  int batch, h_q, h_kv, nq, ring_cap;
  int64_t cap;
};

int run_decode(const DecodeCase& dc, const HostParams& hp, const std::vector<int64_t>& n_comp,
               const std::vector<int32_t>& n_ring, size_t ws_bytes, bool append, bool noalloc = false) {
  HostCache hc(dc.l, dc.batch, dc.h_kv, dc.cap);
  const size_t rows = (size_t)dc.batch * dc.nq * dc.h_q;
  Buf q(rows * 128 * 2), out(rows * 128 * 4), ws(ws_bytes);
  const size_t ring = (size_t)dc.batch * dc.ring_cap * dc.h_kv * 128 * 2;
  Buf rk(ring), rv(ring), kn((size_t)dc.batch * dc.h_kv * 128 * 4), vnw(kn.n);
  const int32_t* nr = dc.ring_cap > 0 ? n_ring.data() : nullptr;
  if (noalloc)
    return tq_decode_attn_noalloc(&dc.l, &hp.p, q.get(), TQ_BF16, dc.h_q, &hc.c, n_comp.data(), rk.get(), rv.get(),
                                  dc.ring_cap, nr, 0.088f, (float*)out.get(), nullptr);
  if (append)
    return tq_decode_attn_append(&dc.l, &hp.p, q.get(), TQ_BF16, dc.h_q, &hc.c, n_comp.data(), kn.get(), vnw.get(),
                                 TQ_F32, rk.get(), rv.get(), dc.ring_cap, nr, 0.088f, (float*)out.get(), ws.get(),
                                 ws_bytes, nullptr);
  if (dc.nq > 1)
    return tq_decode_attn_multi(&dc.l, &hp.p, q.get(), TQ_BF16, dc.h_q, dc.nq, &hc.c, n_comp.data(), rk.get(),
                                rv.get(), dc.ring_cap, nr, 0.088f, (float*)out.get(), ws.get(), ws_bytes, nullptr);
  return tq_decode_attn(&dc.l, &hp.p, q.get(), TQ_BF16, dc.h_q, &hc.c, n_comp.data(), rk.get(), rv.get(), dc.ring_cap,
                        nr, 0.088f, (float*)out.get(), ws.get(), ws_bytes, nullptr);
}

void test_decode() {
  const tq_layout layouts[] = {layout(2, 1, TQ_V_MINMAX, 2, 32, TQ_F32), layout(3, 1, TQ_V_MSE, 3, 32, TQ_F16),
                               layout(2, 1, TQ_V_MINMAX, 4, 32, TQ_F32, 1), layout(1, 0, TQ_V_MINMAX, 2, 16, TQ_F16)};
  for (const tq_layout& l : layouts) {
    HostParams hp(l);
    for (int batch : {1, 5, 64, 65, 130}) {
      for (int h_q : {1, 4, 12, 32}) {
        const int h_kv = h_q >= 4 ? h_q / 4 : 1;
        for (int nq : {1, 3}) {
          for (int ring_cap : {0, 7, 128}) {
            const int64_t cap = 640;
            const DecodeCase dc{l, batch, h_q, h_kv, nq, ring_cap, cap};
            std::vector<int64_t> n_comp(batch);
            std::vector<int32_t> n_ring(batch);
            for (int b = 0; b < batch; ++b) {
              n_comp[b] = b == 0 ? cap : (b * 131) % (cap + 1);  // includes 0 and the capacity
              n_ring[b] = ring_cap > 0 ? (b * 5) % ring_cap : 0;
            }
            const size_t need = nq > 1 ? tq_decode_workspace_bytes_multi(&l, batch, h_q, h_kv, cap, nq)
                                       : tq_decode_workspace_bytes(&l, batch, h_q, h_kv, cap);
            CHECK(need > 0);
            // a shorter cache never needs more workspace
            CHECK(tq_decode_workspace_bytes_multi(&l, batch, h_q, h_kv, cap / 3, nq) <= need);
            for (bool mfma : {true, false}) {
              stub::g_mfma_supported = mfma;
              reset_log();
              const int rc = run_decode(dc, hp, n_comp, n_ring, need, false);
              if (!mfma && l.key_half) {
                CHECK(rc == TQ_ERR_UNSUPPORTED);
                continue;
              }
              CHECK(rc == TQ_OK);
              const auto& log = mfma ? stub::g_log.decode_mfma : stub::g_log.decode_generic;
              const int nvirt = (h_q / h_kv) * nq, vg = std::min(8, nvirt);
              CHECK((int)log.size() == ((batch + 63) / 64) * ((nvirt + vg - 1) / vg));
              int vseen = 0;
              for (const tq::DecodeArgs& a : log) {
                CHECK(a.vbase == vseen);
                CHECK(a.group == std::min(vg, nvirt - vseen));
                vseen = a.vbase + a.group >= nvirt ? 0 : a.vbase + a.group;
              }
              // one byte short: refused before any launch
              reset_log();
              CHECK(run_decode(dc, hp, n_comp, n_ring, need - 1, false) == TQ_ERR_WORKSPACE);
              CHECK(stub::g_log.decode_mfma.empty() && stub::g_log.decode_generic.empty());
              if (nq == 1 && ring_cap > 0) {
                reset_log();
                std::vector<int32_t> nr1 = n_ring;
                for (int32_t& x : nr1) x = std::min(x, ring_cap - 1);
                CHECK(run_decode(dc, hp, n_comp, nr1, need, true) == TQ_OK);
                if (!mfma) CHECK((int)stub::g_log.ring_batches.size() == (batch + 63) / 64);
                nr1[batch - 1] = ring_cap;
                CHECK(run_decode(dc, hp, n_comp, nr1, need, true) == TQ_ERR_CAPACITY);
              }
            }
            stub::g_mfma_supported = true;
          }
        }
      }
    }
  }
}

void test_decode_errors() {
  const tq_layout l = layout(2, 1, TQ_V_MINMAX, 2, 32, TQ_F32);
  HostParams hp(l);
  const DecodeCase dc{l, 3, 32, 8, 1, 128, 256};
  std::vector<int64_t> n_comp = {256, 10, 0};
  std::vector<int32_t> n_ring = {0, 127, 128};
  const size_t need = tq_decode_workspace_bytes(&l, 3, 32, 8, 256);
  reset_log();
  CHECK(run_decode(dc, hp, n_comp, n_ring, need, false) == TQ_OK);
  n_comp[1] = 257;
  CHECK(run_decode(dc, hp, n_comp, n_ring, need, false) == TQ_ERR_CAPACITY);
  n_comp[1] = -1;
  CHECK(run_decode(dc, hp, n_comp, n_ring, need, false) == TQ_ERR_CAPACITY);
  n_comp[1] = 10;
  n_ring[2] = 129;
  CHECK(run_decode(dc, hp, n_comp, n_ring, need, false) == TQ_ERR_CAPACITY);
  n_ring[2] = 128;
  // the fused append needs room for one more ring token
  CHECK(run_decode(dc, hp, n_comp, n_ring, need, true) == TQ_ERR_CAPACITY);
  const DecodeCase wide{l, 3, 32, 2, 1, 0, 256};  // 16 query heads per KV head
  CHECK(run_decode(wide, hp, n_comp, n_ring, 1 << 20, false) == TQ_ERR_UNSUPPORTED);
  const DecodeCase odd{l, 3, 30, 8, 1, 0, 256};  // 30 query heads over 8 KV heads
  CHECK(run_decode(odd, hp, n_comp, n_ring, 1 << 20, false) == TQ_ERR_INVALID);
  const DecodeCase big_ring{l, 3, 32, 8, 1, 200, 256};
  std::vector<int32_t> over = {0, 150, 3};
  CHECK(run_decode(big_ring, hp, n_comp, over, 1 << 22, false) == TQ_ERR_UNSUPPORTED);
  CHECK(stub::g_log.decode_mfma.size() == 1);  // only the first call launched

  HostCache hc(l, 3, 8, 256);
  Buf q(3 * 32 * 128 * 4), out(q.n), ws(need), rk(3 * 128 * 8 * 128 * 2), rv(rk.n);
  n_ring = {0, 1, 2};
  CHECK(tq_decode_attn(&l, &hp.p, q.get(), TQ_F32, 32, &hc.c, n_comp.data(), rk.get(), rv.get(), 128, n_ring.data(),
                       NAN, (float*)out.get(), ws.get(), need, nullptr) == TQ_ERR_INVALID);
  CHECK(tq_decode_attn(&l, &hp.p, q.get(), 3, 32, &hc.c, n_comp.data(), rk.get(), rv.get(), 128, n_ring.data(), 1.f,
                       (float*)out.get(), ws.get(), need, nullptr) == TQ_ERR_INVALID);
  CHECK(tq_decode_attn(&l, &hp.p, q.get(), TQ_F32, 32, &hc.c, n_comp.data(), rk.get(), rv.get(), 128, nullptr, 1.f,
                       (float*)out.get(), ws.get(), need, nullptr) == TQ_ERR_INVALID);
  CHECK(tq_decode_attn(&l, &hp.p, q.get(), TQ_F32, 32, &hc.c, n_comp.data(), rk.get(), rv.get(), 128, n_ring.data(),
                       1.f, nullptr, ws.get(), need, nullptr) == TQ_ERR_INVALID);
  CHECK(tq_decode_attn_multi(&l, &hp.p, q.get(), TQ_F32, 32, 0, &hc.c, n_comp.data(), rk.get(), rv.get(), 128,
                             n_ring.data(), 1.f, (float*)out.get(), ws.get(), need, nullptr) == TQ_ERR_INVALID);
  CHECK(tq_decode_attn_append(&l, &hp.p, q.get(), TQ_F32, 32, &hc.c, n_comp.data(), nullptr, rv.get(), TQ_F32,
                              rk.get(), rv.get(), 128, n_ring.data(), 1.f, (float*)out.get(), ws.get(), need,
                              nullptr) == TQ_ERR_INVALID);
  CHECK(tq_decode_attn_append(&l, &hp.p, q.get(), TQ_F32, 32, &hc.c, n_comp.data(), rk.get(), rv.get(), TQ_F32,
                              rk.get(), rv.get(), 0, n_ring.data(), 1.f, (float*)out.get(), ws.get(), need,
                              nullptr) == TQ_ERR_INVALID);
  tq_params np = hp.p;
  np.derived = nullptr;
  CHECK(tq_decode_attn(&l, &np, q.get(), TQ_F32, 32, &hc.c, n_comp.data(), rk.get(), rv.get(), 128, n_ring.data(),
                       1.f, (float*)out.get(), ws.get(), need, nullptr) == TQ_ERR_INVALID);
  CHECK(tq_decode_workspace_bytes(&l, 0, 32, 8, 256) == 0);
  CHECK(tq_decode_workspace_bytes(&l, 3, 30, 8, 256) == 0);
  CHECK(tq_decode_workspace_bytes(nullptr, 3, 32, 8, 256) == 0);
}

void test_noalloc() {
  const tq_layout l = layout(2, 1, TQ_V_MINMAX, 2, 32, TQ_F32);
  HostParams hp(l);
  const DecodeCase small{l, 4, 32, 8, 1, 16, 2048};
  std::vector<int64_t> n_comp = {2048, 5, 0, 1000};
  std::vector<int32_t> n_ring = {0, 3, 15, 1};
  reset_log();
  CHECK(run_decode(small, hp, n_comp, n_ring, 0, false, true) == TQ_OK);
  CHECK(stub::g_log.decode_mfma.size() == 1 && stub::g_log.noalloc_lookups == 1);
  // a call whose workspace exceeds the static scratch is refused before any lookup
  // (64 sequences x 64 KV heads x 8 query heads: 32 MiB of rotated queries alone)
  const DecodeCase big{l, 64, 512, 64, 1, 0, 64};
  std::vector<int64_t> nbig(64, 64);
  std::vector<int32_t> nr0(64, 0);
  CHECK(tq_decode_workspace_bytes(&l, 64, 512, 64, 64) > TQ_NOALLOC_SCRATCH_BYTES);
  reset_log();
  CHECK(run_decode(big, hp, nbig, nr0, 0, false, true) == TQ_ERR_WORKSPACE);
  CHECK(stub::g_log.decode_mfma.empty() && stub::g_log.noalloc_lookups == 0);
}

void test_timing_hooks() {
  const tq_layout l = layout(2, 1, TQ_V_MINMAX, 2, 32, TQ_F32);
  HostParams hp(l);
  int e0, e1;  // any non-NULL handles: the stubs only record them
  CHECK(tq_time_next_launch(3, &e0, &e1) == TQ_ERR_INVALID);
  CHECK(tq_time_next_launch(-1, &e0, &e1) == TQ_ERR_INVALID);
  CHECK(tq_time_next_launch(TQ_KERNEL_DECODE_SCAN, &e0, &e1) == TQ_OK);
  const DecodeCase dc{l, 2, 8, 2, 1, 0, 256};
  std::vector<int64_t> n_comp = {100, 256};
  std::vector<int32_t> n_ring = {0, 0};
  const size_t need = tq_decode_workspace_bytes(&l, 2, 8, 2, 256);
  reset_log();
  CHECK(run_decode(dc, hp, n_comp, n_ring, need, false) == TQ_OK);
  CHECK(stub::g_log.last_timed.begin == (hipEvent_t)(void*)&e0 && stub::g_log.last_timed.end == (hipEvent_t)(void*)&e1);
  reset_log();
  CHECK(run_decode(dc, hp, n_comp, n_ring, need, false) == TQ_OK);  // consumed by the first call
  CHECK(stub::g_log.last_timed.begin == nullptr && stub::g_log.last_timed.end == nullptr);
  CHECK(std::strlen(tq_version()) > 0);
}

}  // namespace

int main() {
  test_codebook();
  test_memory_bytes();
  test_prepare();
  test_layout_checks();
  test_encode();
  test_ring_append();
  test_decode();
  test_decode_errors();
  test_noalloc();
  test_timing_hooks();
  std::printf("host ABI checks: %d passed\n", g_checks);
  return 0;
}
