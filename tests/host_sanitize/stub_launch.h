// Launch log of the stand-in launchers (stub_launch.cpp), read by driver.cpp.
#pragma once

#include <vector>

#include "tq_internal.h"

namespace stub {

struct Log {
  int prepare = 0;
  int encode_small = 0;
  int encode_values = 0;
  int noalloc_lookups = 0;
  std::vector<tq::EncodeArgs> encode_keys;
  std::vector<tq::DecodeArgs> decode_mfma;
  std::vector<tq::DecodeArgs> decode_generic;
  std::vector<int> ring_batches;
  tq::TimedLaunch last_timed;
};

extern Log g_log;
extern bool g_mfma_supported;   // false: launch_decode_mfma declines every layout
extern bool g_small_supported;  // true: launch_encode_small_kv takes every MSE-value call

}  // namespace stub
