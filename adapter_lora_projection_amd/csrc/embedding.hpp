// Internal launch interface of the embedding LoRA-A kernel (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmx {

struct EmbeddingArgs {
  const int* input_ids;
  const void* w_a;  // A[a][j][v] at element a*stride_l + j*stride_r + v*stride_v
  const int* seg_indptr;
  const int* weight_indices;
  const int* permutation;  // null: identity
  const int* lora_ranks;
  void* h;
  int64_t stride_l, stride_r, stride_v, ldh;
  int T, R, G, L, V;
};

// esize: bytes per element (2 or 4). vec: 16-byte rows (unit rank stride, R, ldh and the other
// strides multiples of 16 bytes, w_a and h 16-byte aligned; the caller checks).
hipError_t launch_embedding_a(const EmbeddingArgs& a, int esize, bool vec, hipStream_t st);

}  // namespace lmx
