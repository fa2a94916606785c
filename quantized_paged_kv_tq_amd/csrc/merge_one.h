// Stage 2 of the multi-query (prefill) attention: entries of one query token
// with a single split each (D = 128), one wave per (entry, query head).
#pragma once
#include <hip/hip_runtime.h>

namespace tqk {

struct DecodeParams;
hipError_t launch_merge_one_split(const DecodeParams& p, hipStream_t st);

}  // namespace tqk
