// Rotary embedding fused into the KV-cache write, for gfx950.
//
// mini_engine ("Roadmap") folds RoPE into the QKV split / KV-cache write, and
// miniserve's "Engine" flowchart orders one layer as fused qkv projection,
// RoPE, then the copy of each new token's K and V rows into its pool slot
// (block_id * block_size + offset).  One pass here reads the fused
// projection rows [q heads | k heads | v heads] once, writes the rotated q
// heads to a contiguous q tensor, and scatters the rotated k heads and the
// untouched v heads into their cache slots (negative slots are padding).
//
// The rotation is the rotate-half rotary embedding over the whole head:
// element i < D/2 pairs with i + D/2 and the pair turns by
// pos * theta^(-2 i / D).  Its cos/sin come from a table filled once per
// (theta, D) by pka_rope_table, in double precision, stored as fp32 pairs.
//
// Work item = (token, head, 8-element piece of the first half): the thread
// loads the piece and its partner piece D/2 further (16 bytes each), the 8
// (cos, sin) pairs of its position, rotates in fp32 and rounds to the input
// type once.  v pieces are plain 16-byte copies, so V lands bit-exact.

#include "device_common.h"
#include "launch.h"

namespace pka {

constexpr int kRopeThreads = 256;

template <typename T>
__global__ void __launch_bounds__(kRopeThreads)
rope_kv_write_kernel(const uint16_t* __restrict__ qkv, int64_t row_stride, const int64_t* __restrict__ positions,
                     const int64_t* __restrict__ slot_mapping, const float* __restrict__ table, int64_t total,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_position,
                     int64_t num_slots, uint16_t* __restrict__ q_out,
                     uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache) {
  using E = Elem<T>;
  const int64_t idx = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  if (idx >= total) return;
  const int32_t half = head_dim / 2;
  const int32_t pieces = half / 8;  // pieces per half head
  const int32_t heads = num_q_heads + 2 * num_kv_heads;
  const int64_t tok = idx / ((int64_t)heads * pieces);
  const int32_t rem = (int32_t)(idx - tok * heads * pieces);
  const int32_t head = rem / pieces;
  const int32_t piece = rem - head * pieces;
  const int32_t e0 = piece * 8;  // first element of this thread's piece in the first half

  const uint16_t* src = qkv + tok * row_stride + (int64_t)head * head_dim;
  const uint4 lo = *reinterpret_cast<const uint4*>(src + e0);
  const uint4 hi = *reinterpret_cast<const uint4*>(src + half + e0);

  const bool is_v = head >= num_q_heads + num_kv_heads;
  int64_t slot = 0;
  if (head >= num_q_heads) {
    slot = slot_mapping[tok];
    // Padded token: nothing goes to the cache (nor for a slot past the pool,
    // a broken precondition).
    if (slot < 0 || slot >= num_slots) return;
  }
  const int64_t kv_row = (int64_t)num_kv_heads * head_dim;  // elements per cache row (slot)
  if (is_v) {
    uint16_t* dst = v_cache + slot * kv_row + (int64_t)(head - num_q_heads - num_kv_heads) * head_dim;
    *reinterpret_cast<uint4*>(dst + e0) = lo;
    *reinterpret_cast<uint4*>(dst + half + e0) = hi;
    return;
  }

  // (cos, sin) pairs of elements e0 .. e0 + 7 at this token's position (a
  // position outside the table, a broken precondition, is clamped into it).
  const int64_t pos = min(max(positions[tok], (int64_t)0), (int64_t)max_position - 1);
  const float4* cs = reinterpret_cast<const float4*>(table + (pos * half + e0) * 2);
  float c[8], s[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 v = cs[j];
    c[2 * j] = v.x;
    s[2 * j] = v.y;
    c[2 * j + 1] = v.z;
    s[2 * j + 1] = v.w;
  }
  const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w};
  const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
  uint32_t olo[4], ohi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a0 = E::lo(lw[j]), a1 = E::hi(lw[j]);  // first-half elements 2j, 2j+1
    const float b0 = E::lo(hw[j]), b1 = E::hi(hw[j]);  // their partners in the second half
    const float c0 = c[2 * j], s0 = s[2 * j], c1 = c[2 * j + 1], s1 = s[2 * j + 1];
    olo[j] = E::pack2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
    ohi[j] = E::pack2(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
  }
  uint16_t* dst;
  if (head < num_q_heads) {
    dst = q_out + (tok * num_q_heads + head) * head_dim;
  } else {
    dst = k_cache + slot * kv_row + (int64_t)(head - num_q_heads) * head_dim;
  }
  *reinterpret_cast<uint4*>(dst + e0) = make_uint4(olo[0], olo[1], olo[2], olo[3]);
  *reinterpret_cast<uint4*>(dst + half + e0) = make_uint4(ohi[0], ohi[1], ohi[2], ohi[3]);
}

// table[p][i] = (cos a, sin a), a = p * theta^(-2 i / D), i < D/2, in double.
__global__ void __launch_bounds__(kRopeThreads)
rope_table_kernel(float* __restrict__ table, int32_t max_position, int32_t head_dim, double theta) {
  const int64_t idx = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  const int32_t half = head_dim / 2;
  if (idx >= (int64_t)max_position * half) return;
  const int64_t p = idx / half;
  const int32_t i = (int32_t)(idx - p * half);
  const double inv_freq = pow(theta, -2.0 * i / head_dim);
  double sn, cn;
  sincos((double)p * inv_freq, &sn, &cn);
  *reinterpret_cast<float2*>(table + 2 * idx) = make_float2((float)cn, (float)sn);
}

hipError_t launch_rope_table(float* table, int max_position, int head_dim, double theta, hipStream_t stream) {
  const int64_t total = (int64_t)max_position * (head_dim / 2);
  const int64_t blocks = (total + kRopeThreads - 1) / kRopeThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(kRopeThreads), 0, stream, table, max_position,
                     head_dim, theta);
  return hipGetLastError();
}

hipError_t launch_rope_kv_write(const RopeKvArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.num_tokens * (a.num_q_heads + 2 * a.num_kv_heads) * (a.head_dim / 16);
  const int64_t blocks = (total + kRopeThreads - 1) / kRopeThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (a.bf16)
    hipLaunchKernelGGL(rope_kv_write_kernel<BF16>, dim3((unsigned)blocks), dim3(kRopeThreads), 0, stream, a.qkv,
                       a.row_stride, a.positions, a.slot_mapping, a.table, total, a.num_q_heads, a.num_kv_heads,
                       a.head_dim, a.max_position, a.num_slots, a.q_out, a.k_cache, a.v_cache);
  else
    hipLaunchKernelGGL(rope_kv_write_kernel<F16>, dim3((unsigned)blocks), dim3(kRopeThreads), 0, stream, a.qkv,
                       a.row_stride, a.positions, a.slot_mapping, a.table, total, a.num_q_heads, a.num_kv_heads,
                       a.head_dim, a.max_position, a.num_slots, a.q_out, a.k_cache, a.v_cache);
  return hipGetLastError();
}

}  // namespace pka
