// Stand-ins for the kernel launchers of libtq, for a host-only build of the C
// ABI (tq_api.cpp, tq_codebook.cpp, tq_plan.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  No GPU is used: each launcher reads and writes
// back one byte at the first and at the last address of every buffer extent
// the real kernel would touch, computed from the launch arguments the way the
// kernels index them.  The driver hands host allocations of exactly the
// documented sizes as "device" buffers, so an offset mistake in the host code
// shows up as a heap-buffer-overflow report.  Launches are also counted and
// their arguments kept for the driver's checks.
#include "stub_launch.h"

#include <cstdio>
#include <cstdlib>

namespace stub {
Log g_log;
bool g_mfma_supported = true;
bool g_small_supported = false;
}  // namespace stub

namespace {

// The combine step stages at most this many splits per head.
constexpr int kCombineSplits = 2048;

[[noreturn]] void die(const char* what) {
  std::fprintf(stderr, "stub launch check failed: %s\n", what);
  std::exit(3);
}

void touch(const void* p, size_t bytes) {
  if (bytes == 0) return;
  if (!p) die("null buffer with a non-empty extent");
  volatile unsigned char* c = (volatile unsigned char*)p;
  c[0] = c[0];
  c[bytes - 1] = c[bytes - 1];
}

size_t key_rec(int mse_bits, int qjl, int half) { return tq::key_record_bytes(mse_bits, qjl, half); }

// Cache extents of `slots` (sequence, head) slots of `cap` tokens.
void touch_cache_keys(const uint8_t* planes, const void* norm, const void* rnorm, size_t slots, int64_t cap,
                      size_t kpb, int qjl, size_t ssz) {
  touch(planes, slots * (size_t)tq::key_slot_tokens(cap) * kpb);  // whole 64-token key blocks
  touch(norm, slots * cap * ssz);
  if (qjl) touch(rnorm, slots * cap * ssz);
}
void touch_cache_values(const uint32_t* planes, const uint16_t* meta, const void* vnorm, size_t slots, int64_t cap,
                        int vmse, int vbits, int group, size_t ssz) {
  touch(planes, slots * cap * (size_t)vbits * tq::kD / 8);
  if (vmse)
    touch(vnorm, slots * cap * ssz);
  else
    touch(meta, slots * cap * (size_t)(tq::kD / group) * 4);
}

void check_encode(const tq::EncodeArgs& a, size_t in_esz) {
  if (a.batch < 1 || a.batch > tq::kMaxSeqPerLaunch) die("encode batch outside 1..64");
  if (a.n_new <= 0) die("encode launched with no tokens");
  int64_t tiles = 0;
  for (int b = 0; b < a.batch; ++b) {
    if (a.tile_start.v[b] != tiles) die("tile_start is not the prefix count of tiles");
    const int64_t pos = a.pos.v[b];
    if (pos < 0 || pos + a.n_new > a.capacity) die("encode positions outside the capacity");
    tiles += (int64_t)a.h_kv * (((pos + a.n_new + 31) >> 5) - (pos >> 5));
  }
  if (tiles != a.num_tiles) die("num_tiles does not count the tiles");
  touch(a.k, (size_t)a.batch * a.n_new * a.h_kv * tq::kD * in_esz);
  touch(a.v, (size_t)a.batch * a.n_new * a.h_kv * tq::kD * in_esz);
  touch(a.derived, tq::kDerivedBytes);
  touch(a.pi, (size_t)tq::kD * tq::kD * 4);
}

void check_decode(const tq::DecodeArgs& a, size_t kpb, int qjl, int vmse, int vbits, int npl) {
  if (a.batch < 1 || a.batch > tq::kMaxSeqPerLaunch) die("decode batch outside 1..64");
  if (a.group < 1 || a.group > tq::kMaxGroup) die("decode group outside 1..8");
  if (a.split_len <= 0 || a.split_len % 64) die("split length is not a positive multiple of 64");
  if (a.splits < 1 || a.splits > kCombineSplits) die("split count outside what the combine stages");
  for (int b = 0; b < a.batch; ++b) {
    if (a.n_comp.v[b] < 0 || a.n_comp.v[b] > a.capacity) die("n_comp outside the capacity");
    if ((int64_t)a.splits * a.split_len < a.n_comp.v[b]) die("the splits do not cover every compressed token");
    if (a.n_ring.v[b] < 0 || a.n_ring.v[b] > (a.ring_cap > 0 ? a.ring_cap : 0)) die("n_ring outside the ring");
    if (a.n_ring.v[b] > tq::kMaxRing) die("more ring tokens than the combine attends");
  }
  const size_t qsz = a.q_bf16 ? 2 : 4;
  const size_t last_q = tq::q_row(a, a.batch - 1, a.nq - 1, a.h_q - 1) + 1;
  touch(a.q, last_q * tq::kD * qsz);
  touch(a.out, last_q * tq::kD * 4);
  const size_t rows = tq::ws_row(a, a.batch - 1, a.h_kv - 1, a.group - 1) + 1;
  touch(a.qprep, rows * 2 * tq::kD * 4);
  touch(a.partial, ((size_t)(a.splits - 1) * a.batch * a.h_kv * a.group + rows) * (tq::kD + 2) * 4);
  if (npl > 0) {
    const size_t nht = a.group > 4 ? 2 : 1;
    touch(a.qdig, (size_t)a.batch * a.h_kv * nht * npl * 2 * 64 * 16);
    touch(a.qconst, rows * 4 * 4);
  }
  const size_t slots = (size_t)a.batch * a.h_kv;
  const size_t ssz = a.scalar_f16 ? 2 : 4;
  touch_cache_keys(a.k_planes, a.k_norm, a.k_rnorm, slots, a.capacity, kpb, qjl, ssz);
  touch_cache_values(a.v_planes, a.v_meta, a.v_norm, slots, a.capacity, vmse, vbits, a.value_group, ssz);
  touch(a.pi, (size_t)tq::kD * tq::kD * 4);
  touch(a.s, (size_t)tq::kD * tq::kD * 4);
  touch(a.mat_t, (size_t)2 * tq::kD * tq::kD * 4);
  if (a.ring_cap > 0) {
    const size_t ring = (size_t)a.batch * a.ring_cap * a.h_kv * tq::kD * 2;
    touch(a.ring_k, ring);
    touch(a.ring_v, ring);
  }
  if (a.app_k) {
    const size_t esz = a.app_bf16 ? 2 : 4;
    touch(a.app_k, slots * tq::kD * esz);
    touch(a.app_v, slots * tq::kD * esz);
    if (a.app_ring_k != a.ring_k || a.app_ring_v != a.ring_v) die("the append ring is not the attended ring");
  }
}

}  // namespace

extern "C" const char* hipGetErrorString(hipError_t e) {
  return e == hipSuccess ? "no error" : "stub launch error";
}

namespace tq {

hipError_t launch_prepare_params(const float* pi, const float* s, uint16_t* derived, hipStream_t) {
  touch(pi, (size_t)kD * kD * 4);
  touch(s, (size_t)kD * kD * 4);
  touch(derived, kDerivedBytes);
  ++stub::g_log.prepare;
  return hipSuccess;
}

hipError_t launch_encode_keys(const EncodeArgs& a, int in_bf16, int mse_bits, int qjl, int half, hipStream_t,
                              TimedLaunch t) {
  check_encode(a, in_bf16 ? 2 : 4);
  const size_t ssz = a.scalar_f16 ? 2 : 4;
  touch_cache_keys(a.k_planes, a.k_norm, a.k_rnorm, (size_t)a.batch * a.h_kv, a.capacity,
                   key_rec(mse_bits, qjl, half), qjl, ssz);
  stub::g_log.encode_keys.push_back(a);
  stub::g_log.last_timed = t;
  return hipSuccess;
}

hipError_t launch_encode_small_kv(const EncodeArgs& a, int in_bf16, int key_mse_bits, int key_qjl, int key_half,
                                  int value_bits, hipStream_t) {
  if (!stub::g_small_supported) return hipErrorNotSupported;
  check_encode(a, in_bf16 ? 2 : 4);
  const size_t ssz = a.scalar_f16 ? 2 : 4;
  const size_t slots = (size_t)a.batch * a.h_kv;
  touch_cache_keys(a.k_planes, a.k_norm, a.k_rnorm, slots, a.capacity, key_rec(key_mse_bits, key_qjl, key_half),
                   key_qjl, ssz);
  touch_cache_values(a.v_planes, a.v_meta, a.v_norm, slots, a.capacity, 1, value_bits, a.value_group, ssz);
  ++stub::g_log.encode_small;
  return hipSuccess;
}

hipError_t launch_encode_values_mse(const EncodeArgs& a, int in_bf16, int bits, hipStream_t, TimedLaunch) {
  check_encode(a, in_bf16 ? 2 : 4);
  touch_cache_values(a.v_planes, a.v_meta, a.v_norm, (size_t)a.batch * a.h_kv, a.capacity, 1, bits,
                     a.value_group, a.scalar_f16 ? 2 : 4);
  ++stub::g_log.encode_values;
  return hipSuccess;
}

hipError_t launch_encode_values_minmax(const EncodeArgs& a, int in_bf16, int bits, hipStream_t, TimedLaunch) {
  check_encode(a, in_bf16 ? 2 : 4);
  touch_cache_values(a.v_planes, a.v_meta, a.v_norm, (size_t)a.batch * a.h_kv, a.capacity, 0, bits,
                     a.value_group, a.scalar_f16 ? 2 : 4);
  ++stub::g_log.encode_values;
  return hipSuccess;
}

hipError_t launch_ring_append(const void* k_new, const void* v_new, int in_bf16, int batch, int h_kv,
                              uint16_t* ring_k, uint16_t* ring_v, int ring_cap, const SeqValues& n_ring,
                              hipStream_t) {
  if (batch < 1 || batch > kMaxSeqPerLaunch) die("ring append batch outside 1..64");
  for (int b = 0; b < batch; ++b)
    if (n_ring.v[b] < 0 || n_ring.v[b] >= ring_cap) die("ring position outside the ring");
  const size_t esz = in_bf16 ? 2 : 4;
  touch(k_new, (size_t)batch * h_kv * kD * esz);
  touch(v_new, (size_t)batch * h_kv * kD * esz);
  touch(ring_k, (size_t)batch * ring_cap * h_kv * kD * 2);
  touch(ring_v, (size_t)batch * ring_cap * h_kv * kD * 2);
  stub::g_log.ring_batches.push_back(batch);
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int key_mse_bits, int key_qjl, int value_mse, int value_bits,
                         hipStream_t, TimedLaunch scan) {
  check_decode(a, key_rec(key_mse_bits, key_qjl, 0), key_qjl, value_mse, value_bits, 0);
  stub::g_log.decode_generic.push_back(a);
  stub::g_log.last_timed = scan;
  return hipSuccess;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int key_mse_bits, int key_qjl, int value_mse, int value_bits,
                              int key_planes, int value_planes, hipStream_t, TimedLaunch scan) {
  if (!stub::g_mfma_supported) return hipErrorNotSupported;
  if (key_planes < 1 || key_planes > 4 || (value_mse && value_planes < 1)) die("MFMA scan without plane weights");
  const int base_bits = key_mse_bits - a.key_half;
  check_decode(a, key_rec(base_bits, key_qjl, a.key_half), key_qjl, value_mse, value_bits, key_planes + key_qjl);
  stub::g_log.decode_mfma.push_back(a);
  stub::g_log.last_timed = scan;
  return hipSuccess;
}

hipError_t launch_combine(const DecodeArgs&, int, hipStream_t) { return hipSuccess; }

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  static unsigned char* scratch = static_cast<unsigned char*>(std::malloc(TQ_NOALLOC_SCRATCH_BYTES));
  *ptr = scratch;
  *bytes = TQ_NOALLOC_SCRATCH_BYTES;
  ++stub::g_log.noalloc_lookups;
  return scratch ? hipSuccess : hipErrorOutOfMemory;
}

}  // namespace tq
