// KV-cache write for gfx950 (mini_engine, "Custom CUDA kernels", KV-cache
// write; miniserve, "Engine" flowchart: new K/V rows are copied into the paged
// pool at slot = block_id * block_size + offset, padded rows skipped).
//
// A pure byte copy: each thread moves one 16-byte piece of one K or V row, so
// the result is bit-exact.  Threads are numbered over (token, piece) with the
// K pieces of a row followed by its V pieces, so a workgroup covers whole rows
// when rows are small and part of a row when they are large; consecutive
// lanes touch consecutive 16-byte pieces of the same row on both sides.

#include "device_common.h"
#include "launch.h"

namespace pka {

constexpr int kKvWriteThreads = 256;

__global__ void __launch_bounds__(kKvWriteThreads)
kv_cache_write_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                      const int64_t* __restrict__ slot_mapping, int64_t total_pieces, int32_t row_pieces,
                      int64_t num_slots, uint4* __restrict__ k_cache, uint4* __restrict__ v_cache) {
  const int64_t idx = (int64_t)blockIdx.x * kKvWriteThreads + threadIdx.x;
  if (idx >= total_pieces) return;
  const int32_t per_token = 2 * row_pieces;
  const int64_t tok = idx / per_token;
  const int32_t piece = (int32_t)(idx - tok * per_token);
  const int64_t slot = slot_mapping[tok];
  // Padded row; a slot past the pool (a broken precondition) is skipped too
  // rather than written out of bounds.
  if (slot < 0 || slot >= num_slots) return;
  if (piece < row_pieces) {
    k_cache[slot * row_pieces + piece] = key[tok * row_pieces + piece];
  } else {
    const int32_t p = piece - row_pieces;
    v_cache[slot * row_pieces + p] = value[tok * row_pieces + p];
  }
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
  const int32_t row_pieces = a.row_bytes / 16;
  const int64_t total = (int64_t)a.num_tokens * 2 * row_pieces;
  const int64_t blocks = (total + kKvWriteThreads - 1) / kKvWriteThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3((unsigned)blocks), dim3(kKvWriteThreads), 0, stream,
                     static_cast<const uint4*>(a.key), static_cast<const uint4*>(a.value), a.slot_mapping, total,
                     row_pieces, a.num_slots, static_cast<uint4*>(a.k_cache), static_cast<uint4*>(a.v_cache));
  return hipGetLastError();
}

}  // namespace pka
