// Host-side planning of a decode launch: how the token range of each
// (sequence, KV head) is split over work-groups, and the workspace the MFMA
// path needs for its query digit operands.  Pure host arithmetic with no HIP
// calls, kept apart from the kernels so it can be built and checked on its own.
#include "tq_internal.h"

namespace tq {

// Split of the token range for the decode grid, in whole 64-token chunks
// (the waves of a work-group take the chunks of its split in turn).  About
// kSplitTarget work-groups over the device: 768 is three per compute unit, one
// round at the scan's three waves per SIMD, so no second, partly filled round
// of work-groups trails the first (32 sequences of 8 KV heads at 32768 tokens:
// 3 splits of 10944 tokens per sequence-head, 166 against 167-170 us for 8
// splits and 2048 work-groups, 171-175 us for 1024).  When that makes splits
// shorter than kLongSplit tokens, they are lengthened towards kLongSplit as long
// as at least kFloorGroups work-groups remain, so per-work-group set-up and the
// combine's merge stay small next to the scan while a few long sequences still
// fill every compute unit.  8 sequence-heads of 131072 tokens: 1408-token
// splits, 752 work-groups (about three per compute unit), against 1536-token
// splits and 688 work-groups with whole 256-token rounds (5% less scan time)
// and 512-token splits and 2048 work-groups for a floor of eight per compute
// unit (4% more time per step, most of it in the combine).
constexpr int64_t kFloorGroups = 768;
constexpr int64_t kLongSplit = 2048;
constexpr int64_t kMinSplit = 256;

void decode_split(int64_t max_tokens, int64_t units, int32_t* splits, int32_t* split_len) {
  if (units < 1) units = 1;
  int64_t want = (kSplitTarget + units - 1) / units;
  if (want < 1) want = 1;
  int64_t len = (max_tokens + want - 1) / want;
  int64_t floor_len = (max_tokens * units + kFloorGroups - 1) / kFloorGroups;  // keeps >= kFloorGroups groups
  if (floor_len > kLongSplit) floor_len = kLongSplit;
  if (len < floor_len) len = floor_len;
  len = ((len + 63) / 64) * 64;
  if (len < kMinSplit) len = kMinSplit;
  int64_t n = (max_tokens + len - 1) / len;
  if (n < 1) n = 1;
  *splits = (int32_t)n;
  *split_len = (int32_t)len;
}

// The split count of decode_split for any token count up to max_tokens is at
// most this bound (len >= n / want gives at most `want` splits, len >= kMinSplit
// at most ceil(max_tokens / kMinSplit)); the bound never decreases as
// max_tokens grows, so a workspace sized for a capacity fits every shorter call.
int32_t decode_max_splits(int64_t max_tokens, int64_t units) {
  int64_t want = units > 0 ? (kSplitTarget + units - 1) / units : 1;
  if (want < 1) want = 1;
  int64_t by_len = (max_tokens + kMinSplit - 1) / kMinSplit;
  int64_t n = want < by_len ? want : by_len;
  return (int32_t)(n < 1 ? 1 : n);
}

// Query digit operands (up to five score planes, two halves, 64 lanes of
// 16 bytes per tile of four virtual heads) and four per-head constants.
size_t mfma_workspace_bytes(int batch, int h_q, int group) {
  const int nht = (group + 3) / 4;
  const int h_kv = h_q / group;
  const size_t dig = (size_t)batch * h_kv * nht * 5 * 2 * 64 * 16;  // up to 5 score planes
  const size_t cst = (size_t)batch * h_q * 4 * 4;
  return dig + cst + 256;
}

}  // namespace tq
