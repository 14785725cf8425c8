// Internal launch interface of the metadata value checks (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace lmx {

struct MetaArgs {
  const int* seg_indptr;
  const int* weight_indices;
  const int* permutation;    // null: not checked (identity)
  const int* lora_ranks;
  const int* slice_offsets;  // null: not checked
  int64_t N;
  int T, G, L, R, S;
};

// flag: one device int that receives a bit per broken rule (bit k = rule k); counts: T device ints
// (used when the permutation is checked). Three launches on st.
hipError_t launch_metadata_check(const MetaArgs& a, int* flag, int* counts, hipStream_t st);

}  // namespace lmx
