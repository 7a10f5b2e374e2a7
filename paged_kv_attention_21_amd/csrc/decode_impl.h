// Paged decode attention for gfx950: kernel templates, instantiated per
// (element type, head size) by the decode_*.hip files.
//
// What it computes (MiniLLM Runtime, "CUDA PagedAttention scope"; mini_engine,
// "Custom CUDA kernels", paged decode v1 and v2): for one query row per
// sequence, softmax(scale * q . k_t) over the sequence's context, then the
// weighted sum of v_t, reading every K/V row in place through the block table
// (MiniLLM Runtime, "Core class relationships").
//
// Work decomposition.  One workgroup per (KV head, sequence) - or per
// (KV head, 256-token partition, sequence) for split-K.  Split-K either leaves
// the partition states for a separate reduce kernel, or (the single-launch
// form the dispatcher uses) counts the partitions of each (sequence, KV head)
// as they finish and lets the workgroup whose partition arrives last merge
// them all and write the output.  The G query heads of
// the GQA group ride along, so every K/V byte is loaded once and used G times.
// The workgroup's W wavefronts take the range's KV blocks round-robin.  The
// single pass runs the sequences longest first (see heavy_first_seq).
//
// Two per-wavefront computations share that frame: the vector path below for
// groups of one and two query heads, and for groups of four and eight - whose
// dot products and weighted sums would bound the vector path - the
// matrix-core path (see DecodeMfma), which streams 16-key units instead of
// blocks.
//
// Lane layout inside a wavefront (vector path).  One 16-byte load per lane (8 elements)
// makes a token row of D elements span LPT = D / 8 lanes, so one wave load
// covers TPL = 64 / LPT tokens and a 16-token block of one head takes
// LPB = 16 / TPL loads per tensor (D = 128: 16 lanes, 4 tokens, 4 loads);
// 8- and 32-token blocks take half and twice as many.
// Each group of LPT lanes ("row") sums its dot-product pieces with DPP and
// keeps its own online-softmax state (max, exp-sum, 8 accumulator dims per
// head) over the tokens it sees; rows, then wavefronts, are merged once at the
// end with the same max/exp-sum rule the split-K reduce uses.
//
// Memory: the caches are token-major ([block][slot][kv head][dim]), so a
// (block, head) is 16 rows of D*2 bytes at a stride of num_kv_heads*D*2 bytes;
// each row is fetched as whole 16-byte pieces by consecutive lanes.  Each
// wavefront keeps the next block's K and V loads in flight while it computes
// on the current one.  K/V are read exactly once, so the loads are marked
// non-temporal (measured on MI355X: the paged read pattern streams at ~5.9 TB/s
// with them and ~5.2 TB/s without).  Block-table entries are fetched 64 at a time with one
// vector load per wavefront and broadcast with readlane.
//
// Numerics: q.k in fp32 with v_dot2 on the raw fp16/bf16 pairs (matrix-core
// path: MFMA, fp32 accumulation of exact products); softmax in the
// base-2 domain (scale * log2 e folded into the logit); fp32 accumulation;
// tokens past the context are selected out (never multiplied by a zero
// weight), so NaN garbage in unowned slots cannot leak in.

#pragma once

#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace pka {

template <int D, int BS>
struct DecodeLayout {
  static constexpr int LPT = D / 8;       // lanes per token row
  static constexpr int TPL = kWave / LPT;  // token rows per wave load
  static constexpr int LPB = BS / TPL;     // wave loads per block per tensor
  static_assert(kWave % LPT == 0 && BS % TPL == 0 && kPartitionSize % BS == 0, "unsupported head_dim / block");
};

// Wave loads per tensor in one streaming tile of the vector path (see
// paged_decode_kernel): the whole block up to four loads (two for groups of
// eight query heads, whose accumulators and scores take twice the registers
// of a group of four).
template <int D, int G, int BS>
constexpr int decode_tile_loads() {
  constexpr int cap = G >= 8 ? 2 : 4;
  return DecodeLayout<D, BS>::LPB < cap ? DecodeLayout<D, BS>::LPB : cap;
}

// ---------------------------------------------------------------------------
// Matrix-core path (groups of four and eight query heads).
//
// With G query heads per K/V byte the vector path's dot products, row sums and
// weighted sums grow with G, and at G = 8 they - not HBM - bound the kernel.
// Groups of four and more run on the matrix cores instead, in units of 16
// consecutive keys:
//   S^T[16 keys][16 cols] = K[16 keys][D] . Q^T[D][16 cols]
//     (v_mfma_f32_16x16x32, the group's G heads in the first G columns of the
//     B operand, the other columns zero and never stored),
//   O^T[D][16 cols] += V^T[D][16 keys] . P^T[16 keys][16 cols]
//     (v_mfma_f32_16x16x16; the accumulator layout of S^T - lane l holds keys
//     4 (l / 16) .. +3 of column l % 16 - is exactly the B operand layout of
//     this product, so the weights never leave the lane).
// The weights are split into a high part (rounded to the input type) and the
// rounded remainder, two products per unit, so they keep about 16 bits: the
// result carries the same single output rounding as the vector path.
// K and V rows are loaded with whole-row 16-byte pieces per lane (the same
// coalesced pattern as the vector path), staged in a wavefront-private LDS
// tile, and read back as operands: K rows as 16-byte A-operand pieces, V
// through the transposing read.  Row strides of 2D + 16 bytes (K) and 2D + 32
// bytes (V) keep both read patterns free of bank conflicts.
// ---------------------------------------------------------------------------
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct DecodeMfma;

template <>
struct DecodeMfma<BF16> {
  typedef __bf16 x8_t __attribute__((ext_vector_type(8)));
  typedef short s4_t __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(x8_t, a), __builtin_bit_cast(x8_t, b), c, 0, 0,
                                                   0);
  }
  static __device__ __forceinline__ f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a), __builtin_bit_cast(s4_t, b), c, 0,
                                                     0, 0);
  }
};

template <>
struct DecodeMfma<F16> {
  typedef _Float16 x8_t __attribute__((ext_vector_type(8)));
  typedef _Float16 x4_t __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(x8_t, a), __builtin_bit_cast(x8_t, b), c, 0, 0,
                                                  0);
  }
  static __device__ __forceinline__ f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(x4_t, a), __builtin_bit_cast(x4_t, b), c, 0, 0,
                                                 0);
  }
};

// Growth of a column's max (base 2) tolerated before the accumulators are
// rescaled: weights stay below 2^8, well inside the input type's range.
constexpr float kMcSlack = 8.f;

// Groups that take the matrix-core path.
template <int G>
constexpr bool decode_uses_mfma() {
  return G >= 4;
}

// Wavefronts per SIMD the kernel is compiled for at least: two for the
// matrix-core path up to 128 dims, whose ring of loads and accumulators would
// otherwise spread over the accumulation registers and run one wavefront per
// SIMD.  At 256 dims one unit's loads and the accumulators alone take 128
// registers, so those instances keep one wavefront per SIMD.
template <int D, int G>
constexpr int decode_min_waves() {
  return decode_uses_mfma<G>() && D <= 128 ? 2 : 1;
}

// Geometry of the matrix-core path for head size D.
template <int D>
struct McGeom {
  static constexpr int NL = D / 32;            // 16-byte loads per lane, per tensor and unit (= QK k-steps)
  static constexpr int KSTR = 2 * D + 16;      // LDS row stride of the K tile, bytes
  static constexpr int VSTR = 2 * D + 32;      // LDS row stride of the V tile, bytes
  static constexpr int TILE = 16 * (KSTR + VSTR);  // one wavefront's K and V tiles
  // Register buffers of the load ring (8 * NL registers each): while one
  // unit is computed, the next one's loads are in flight.  Two: measured at
  // 64 dims, rings of three and four cost occupancy (three and four
  // wavefronts per SIMD against four) and ran 2-4 % slower.  One at 256 dims,
  // where a wavefront already holds the whole register file (one per SIMD):
  // a second unit's 64 registers made the partition-only form with 32-token
  // blocks spill, and measured no faster (group 8, 32-token blocks: 206.7
  // against 208.2 us).
  static constexpr int RING = D == 256 ? 1 : 2;
};

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// output lane i gets element i % 4 of the 8-byte pieces read by input lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4: when input lane L reads row
// r0 + L / 4, columns c0 + 4 (L % 4) .. +3 of a row-major [key][dim] tile,
// output lane i holds keys r0 .. r0 + 3 of column c0 + i.
__device__ __forceinline__ uint2 lds_read_tr_b16(const void* p) {
  typedef short short4v __attribute__((ext_vector_type(4)));
  const auto r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(const_cast<void*>(p)));
  return __builtin_bit_cast(uint2, r);
}

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Heavy-first order of the single-pass grid.  Workgroups start in grid order
// as earlier ones finish, and a long sequence that starts last sets the
// kernel's tail, so grid row r is given the r-th sequence in decreasing
// order of context length - approximated by kOrderBuckets equal buckets of
// [0, max_ctx], equal buckets in index order (longest-processing-time-first
// list scheduling).  Every workgroup derives the same order from
// context_lens: one load per sequence and thread group, a histogram in LDS
// and one scan by the first wavefront.  Returns a wavefront-uniform index.
constexpr int kOrderBuckets = kWave;  // one bucket per lane of the scan
template <int NT>
__device__ __forceinline__ int heavy_first_seq(const int32_t* __restrict__ context_lens, int num_seqs, int max_ctx,
                                               int rank, int* lds /* kOrderBuckets + 1 ints */) {
  const int tid = threadIdx.x;
  auto bucket = [&](int i) {  // 0 holds the longest contexts
    const long long c = max(context_lens[i], 0);
    const int b = (int)(c * kOrderBuckets / ((long long)max_ctx + 1));
    return kOrderBuckets - 1 - min(b, kOrderBuckets - 1);
  };
  if (tid < kOrderBuckets) lds[tid] = 0;
  __syncthreads();
  for (int i = tid; i < num_seqs; i += NT) atomicAdd(&lds[bucket(i)], 1);
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    const int cnt = lds[lane];
    int incl = cnt;  // inclusive prefix sum over the buckets
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const int excl = incl - cnt;
    const unsigned long long hit = __ballot(cnt > 0 && excl <= rank && rank < incl);
    int found = rank;  // unreachable fallback: the given order
    if (hit) {
      const int k = __ffsll((long long)hit) - 1;  // the bucket holding position `rank`
      int target = rank - __shfl(excl, k);
      for (int base = 0; base < num_seqs; base += kWave) {
        const int i = base + lane;
        const bool match = i < num_seqs && bucket(i) == k;
        const unsigned long long mask = __ballot(match);
        const int n = __popcll(mask);
        if (target < n) {
          const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
          found = base + __ffsll((long long)__ballot(match && pos == target)) - 1;
          break;
        }
        target -= n;
      }
    }
    if (lane == 0) lds[kOrderBuckets] = found;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(lds[kOrderBuckets]);
}

// Stores and loads of partition states that other workgroups read within the
// same launch (the single-launch split-K).  They are device-scope relaxed
// atomics, which gfx950 performs coherently past the XCD's L2 (the sc1 form of
// the store and the load), so publishing a state needs no write-back of the L2
// and reading one no L2 invalidation: only a wait for the stores to complete
// before the arrival is counted.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge, in the workgroup that arrived last, the P states of query heads
// kvh*G .. kvh*G+G-1 of one sequence (row stride `rows` in the workspace),
// with the same max / exp-sum rule as the split-K reduce: M = max_p m_p,
// w_p = l_p exp(m_p - M), out = sum_p w_p o_p / sum_p w_p.  Each thread owns
// CPT 4-dim columns over the group's heads and every PP-th state (PP groups
// of threads per column).  States go in passes of CH: a pass first issues the
// thread's o loads into registers (they do not depend on the weights), then
// stages the pass's max logits and exp-sums in LDS, where one wavefront per
// head forms the pass max and the weights (a running max rescales earlier
// passes) - so a pass costs one round trip to memory.  The PP groups are
// summed through LDS at the end.
template <typename T, int D, int G, int W>
__device__ __forceinline__ void merge_group_partitions(const float* __restrict__ tmp_out,
                                                       const float* __restrict__ max_logits,
                                                       const float* __restrict__ exp_sums, int seq, int kvh,
                                                       int num_q_heads, int rows, int P,
                                                       uint16_t* __restrict__ out) {
  typedef float float4v_t __attribute__((ext_vector_type(4)));
  constexpr int NT = W * kWave;
  constexpr int COLS = G * D / 4;                // 4-dim columns over the group's heads
  constexpr int CPT = COLS > NT ? COLS / NT : 1;  // columns per thread
  constexpr int PP = COLS >= NT ? 1 : NT / COLS;  // partition groups
  constexpr int VPT = 8;                          // o vectors per column and pass, per thread
  constexpr int CH = VPT * PP;                    // states per pass
  static_assert(COLS % NT == 0 || NT % COLS == 0, "whole columns per thread");
  __shared__ float s_w[G][CH], s_l[G][CH];
  __shared__ float s_run[3][G];  // running max, running weight sum, this pass's rescale
  __shared__ float4v_t s_red[PP > 1 ? NT : 1];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = wave_id();
  const int pg = PP > 1 ? tid / COLS : 0;
  const size_t row0 = ((size_t)seq * num_q_heads + (size_t)kvh * G) * rows;  // head g: + g * rows
  float4v_t acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = float4v_t{0.f, 0.f, 0.f, 0.f};
  if (tid < G) {
    s_run[0][tid] = -INFINITY;
    s_run[1][tid] = 0.f;
  }
  for (int p0 = 0; p0 < P; p0 += CH) {
    const int n = min(CH, P - p0);
    // This thread's o vectors of the pass (states pg, pg + PP, ...).
    float4v_t ov[CPT][VPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int col = PP > 1 ? tid % COLS : tid + c * NT;
      const int g = col / (D / 4), d4 = col % (D / 4);
      const float* po = tmp_out + (row0 + (size_t)g * rows + p0) * D + 4 * d4;
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        const int p = pg + v * PP;
        ov[c][v] = float4v_t{0.f, 0.f, 0.f, 0.f};
        if (p < n) {
          const float* src = po + (size_t)p * D;
          ov[c][v] = float4v_t{load_coherent(src), load_coherent(src + 1), load_coherent(src + 2),
                               load_coherent(src + 3)};
        }
      }
    }
    for (int i = tid; i < G * n; i += NT) {
      const int g = i / n, p = i - g * n;
      const size_t idx = row0 + (size_t)g * rows + p0 + p;
      s_w[g][p] = load_coherent(max_logits + idx);
      s_l[g][p] = load_coherent(exp_sums + idx);
    }
    __syncthreads();
    for (int g = wave; g < G; g += W) {
      float mx = -INFINITY;
      for (int p = lane; p < n; p += kWave) mx = fmaxf(mx, s_w[g][p]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_old = s_run[0][g];
      const float m_new = fmaxf(m_old, mx);
      float ls = 0.f;
      for (int p = lane; p < n; p += kWave) {
        const float w = s_l[g][p] * fast_exp2((s_w[g][p] - m_new) * kLog2e);
        s_w[g][p] = w;
        ls += w;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ls += __shfl_xor(ls, off);
      if (lane == 0) {
        const float a = m_old == -INFINITY ? 0.f : fast_exp2((m_old - m_new) * kLog2e);
        s_run[2][g] = a;
        s_run[1][g] = s_run[1][g] * a + ls;
        s_run[0][g] = m_new;
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int col = PP > 1 ? tid % COLS : tid + c * NT;
      const int g = col / (D / 4);
      acc[c] *= s_run[2][g];
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        const int p = pg + v * PP;
        if (p < n) acc[c] += s_w[g][p] * ov[c][v];
      }
    }
    __syncthreads();  // s_w and s_l are rewritten by the next pass
  }
  if constexpr (PP > 1) {
    s_red[tid] = acc[0];
    __syncthreads();
    if (tid >= COLS) return;
#pragma unroll
    for (int q = 1; q < PP; ++q) acc[0] += s_red[q * COLS + tid];
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int col = PP > 1 ? tid : tid + c * NT;
    const int g = col / (D / 4), d4 = col % (D / 4);
    const float lt = s_run[1][g];
    const float4v_t o = lt > 0.f ? acc[c] / lt : float4v_t{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<uint2*>(out + ((size_t)seq * num_q_heads + (size_t)kvh * G + g) * D + 4 * d4) =
        make_uint2(Elem<T>::pack2(o[0], o[1]), Elem<T>::pack2(o[2], o[3]));
  }
}

// Launch forms of the decode kernel.
enum DecodeMode : int {
  kDecodeSingle = kLaunchSingle,          // one workgroup per (KV head, sequence), writes out
  kDecodeSplit = kLaunchSplit,            // partitions only: states for the separate reduce
  kDecodeSplitFused = kLaunchSplitFused,  // partitions, then the last one of each (sequence, KV head) merges
};

// BS = tokens per KV block (8, 16 or 32).
//
// Single pass and split-K partition pass: the workgroup's range is the
// sequence (or one 256-token partition of it) and its W wavefronts take the
// range's blocks round-robin; the wavefronts' states are merged through LDS.
// Single-launch split-K (MODE kDecodeSplitFused): grid (KV head, Y, sequence);
// each wavefront takes whole 256-token partitions, wavefront w of workgroup y
// partitions y*W + w, y*W + w + Y*W, ..., streaming each partition's blocks on
// its own; the workgroup merges its wavefronts' states through LDS, publishes
// the result as one state (row y of the workspace), and the last of the
// sequence's workgroups to arrive merges those states into the output.
template <typename T, int D, int G, int W, int MODE, int BS>
__global__ void __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(decode_min_waves<D, G>())))
paged_decode_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                    const int32_t* __restrict__ context_lens, int32_t max_blocks_per_seq,
                    int32_t num_kv_heads, float scale_log2, uint16_t* __restrict__ out,
                    float* __restrict__ tmp_out, float* __restrict__ max_logits,
                    float* __restrict__ exp_sums, int32_t max_num_partitions, int32_t order_max_ctx,
                    const uint16_t* __restrict__ new_k, const uint16_t* __restrict__ new_v,
                    uint16_t* __restrict__ k_store, uint16_t* __restrict__ v_store, int32_t pair_from,
                    uint32_t* __restrict__ counters, int32_t split_chunk) {
  constexpr bool SPLIT = MODE != kDecodeSingle;
  constexpr bool FUSED = MODE == kDecodeSplitFused;
  using L = DecodeLayout<D, BS>;
  constexpr int kBlockSize = BS;
  using E = Elem<T>;
  constexpr int LPT = L::LPT, TPL = L::TPL, LPB = L::LPB;

  const int kvh = blockIdx.x;
  const int part = MODE == kDecodeSplit ? (int)blockIdx.y : 0;
  int seq = SPLIT ? (int)blockIdx.z : (int)blockIdx.y;
  if constexpr (!SPLIT) {
    __shared__ int order_lds[kOrderBuckets + 1];
    // When the whole grid is resident at once and some compute units hold two
    // workgroups (see launch_decode_t), the rows that take a unit's second
    // slot run in reverse rank order, so a unit pairs a long sequence with a
    // short one instead of two long ones.
    if (pair_from > 0 && seq >= pair_from) seq = (int)gridDim.y + pair_from - 1 - seq;
    if (order_max_ctx > 0) seq = heavy_first_seq<W * kWave>(context_lens, gridDim.y, order_max_ctx, seq, order_lds);
  }
  const int num_q_heads = num_kv_heads * G;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_id();

  // The first 64 block-table entries this wavefront will stream (lane k: its
  // k-th block), fetched before the context length is known so the two loads
  // overlap instead of following each other.  The entries lie inside the
  // sequence's table row; those past the context are never used.
  // Single-launch split-K: each wavefront takes chunks of `chunk` tokens -
  // the 256-token partition, or a power-of-two fraction of it (at least one
  // KV block) when the device would otherwise be short of wavefronts; the
  // host keeps the workgroup count within the workspace's rows.
  // The matrix-core path streams 16-key units instead of blocks: lane k then
  // holds the entry of the wavefront's k-th unit (and, with 8-token blocks,
  // of the unit's second block in pre_win2).
  constexpr bool kMfma = decode_uses_mfma<G>();
  const int chunk = FUSED ? split_chunk : kPartitionSize;
  constexpr int kStep = kMfma ? 16 : BS;  // tokens per streaming step
  const int pre_first = FUSED ? ((int)blockIdx.y * W + wave) * (chunk / kStep)
                              : (MODE == kDecodeSplit ? part * (kPartitionSize / kStep) : 0) + wave;
  const int pre_step = pre_first + lane * (FUSED ? 1 : W);
  const int pre_idx = !kMfma ? pre_step : (BS == 8 ? 2 * pre_step : (BS == 32 ? pre_step >> 1 : pre_step));
  const int32_t* const tbl_row = block_tables + (size_t)seq * max_blocks_per_seq;
  const int pre_win = pre_idx < max_blocks_per_seq ? tbl_row[pre_idx] : 0;
  const int pre_win2 = kMfma && BS == 8 && pre_idx + 1 < max_blocks_per_seq ? tbl_row[pre_idx + 1] : 0;

  const int ctx = context_lens[seq];
  // Single-launch split-K: the sequence's chunks (no more than the host-sized
  // workspace's partitions cover) and the workgroups that hold some of them.
  const int num_parts =
      FUSED ? min((max(ctx, 0) + chunk - 1) / chunk, max_num_partitions * (kPartitionSize / chunk)) : 0;
  const int wg_active = FUSED ? min((int)gridDim.y, (num_parts + W - 1) / W) : 0;
  if constexpr (FUSED) {
    if ((int)blockIdx.y >= wg_active) {  // no partition for this workgroup
      if (ctx <= 0 && blockIdx.y == 0) {
        // An empty context has no partition to merge: its output is 0.
        for (int t = threadIdx.x; t < G * D; t += W * kWave)
          out[((size_t)seq * num_q_heads + (size_t)kvh * G + t / D) * D + t % D] = 0;
      }
      return;
    }
  }
  int tok_begin = 0, tok_end = ctx;
  if constexpr (MODE == kDecodeSplit) {
    tok_begin = part * kPartitionSize;
    if (tok_begin >= ctx) return;  // past this sequence's end: nothing to write
    tok_end = min(ctx, tok_begin + kPartitionSize);
  }

  const int row = lane / LPT;
  const int col = lane % LPT;  // this lane's 8 dims: col*8 .. col*8+7

  // Appended token (when new_k is given): position ctx - 1 of every sequence
  // is the row new_k / new_v [seq][kvh] - the decode step's KV-cache write
  // folded into the attention that reads it.  The wavefront that consumes
  // the range's last block takes that position's K/V from registers (the
  // cached copy may be stale or NaN until then: it is loaded and selected
  // out, never read back) and stores the row to its slot, whose block it
  // already holds, so no extra table lookup delays the start of the loop.
  // (The matrix-core path loads it where it is used.)
  uint4 app_k = make_uint4(0, 0, 0, 0), app_v = app_k;
  if (!kMfma && new_k != nullptr && ctx > 0 && (FUSED || tok_end == ctx)) {
    const size_t src = ((size_t)seq * num_kv_heads + kvh) * D + col * 8;
    app_k = *reinterpret_cast<const uint4*>(new_k + src);
    app_v = *reinterpret_cast<const uint4*>(new_v + src);
  }

  // Per-wavefront states (running max in base 2, exp-sum, accumulators),
  // merged through LDS below.  The matrix-core path keeps its K/V tiles in
  // s_kv and writes its states over them.
  __shared__ float s_m[W][G], s_l[W][G];
  __shared__ float s_acc_v[kMfma ? 1 : W][G][D];
  __shared__ __align__(16) char s_kv[kMfma ? W * McGeom<D>::TILE : 16];
  float(*const s_acc)[G][D] = kMfma ? reinterpret_cast<float(*)[G][D]>(s_kv) : s_acc_v;
  if constexpr (kMfma) {
    // Matrix-core path: the wavefront streams 16-key units (see the notes
    // above DecodeMfma); its state is the running max m_ref (base 2, per
    // column), the lane's share of the exp-sum and the O^T accumulators.
    using MC = DecodeMfma<T>;
    using MG = McGeom<D>;
    constexpr int NL = MG::NL, RING = MG::RING, KSTR = MG::KSTR, VSTR = MG::VSTR;
    constexpr int DT = D / 16;            // 16-dim tiles of the output
    constexpr int RB = BS == 8 ? 8 : 16;  // rows of a unit that lie in one block
    const int g4 = lane >> 4, c16 = lane & 15;
    char* const s_k = s_kv + wave * MG::TILE;
    char* const s_v = s_k + 16 * KSTR;
    const size_t row_elems = (size_t)num_kv_heads * D;  // elements between consecutive slots
    const size_t row_bytes = row_elems * 2;
    const size_t block_bytes = row_bytes * BS;
    const char* kbase = reinterpret_cast<const char*>(k_cache) + (size_t)kvh * D * 2;
    const char* vbase = reinterpret_cast<const char*>(v_cache) + (size_t)kvh * D * 2;
    // Unit row TPL * i + row is this lane's row of load i; its piece is dims
    // col * 8 .. +7.  Load i reads a uniform base plus this one lane offset.
    const uint32_t lane_off = (uint32_t)(((size_t)row * row_elems + (size_t)col * 8) * 2);

    // Q^T as the B operand: lane l holds dims 32 s + 8 (l / 16) .. +7 of the
    // group's head l % 16 (zero for columns past the group).
    uint4 qt[NL];
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      qt[s] = make_uint4(0, 0, 0, 0);
      if (c16 < G)
        qt[s] = *reinterpret_cast<const uint4*>(q + ((size_t)seq * num_q_heads + (size_t)kvh * G + c16) * D + 32 * s +
                                                8 * g4);
    }
    f32x4_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_ref = kNegBig, l_part = 0.f;

    // The range being streamed: units [u_first, u_first + u_count), tokens
    // up to e_tok, its last block, and whether it ends with the appended token.
    int u_first = 0, u_count = 0, e_tok = 0, last_blk = 0;
    bool append = false;
    auto set_range = [&](int b, int e) __attribute__((always_inline)) {  // b: a multiple of 16
      u_first = b / 16;
      u_count = e > b ? (e - b + 15) / 16 : 0;
      e_tok = e;
      last_blk = e > 0 ? (e - 1) / BS : 0;
      append = new_k != nullptr && ctx > 0 && e == ctx;
    };
    // Uniform byte offset of load i of unit u (blocks pb0 and, for 8-token
    // blocks, pb1); the lane adds lane_off.
    auto load_base = [&](int i, int u, int pb0, int pb1) __attribute__((always_inline)) {
      const size_t half = BS == 32 ? (size_t)((u & 1) * 16) * row_bytes : 0;
      const size_t base = (BS == 8 && TPL * i >= 8) ? (size_t)pb1 * block_bytes : (size_t)pb0 * block_bytes + half;
      return base + (size_t)((TPL * i) % RB) * row_bytes;
    };
    uint4 kb[RING][NL], vb[RING][NL];
    auto issue = [&](auto rb, int u, int pb0, int pb1) __attribute__((always_inline)) {
      constexpr int r = decltype(rb)::value;
#pragma unroll
      for (int i = 0; i < NL; ++i) kb[r][i] = load_nt16(kbase + load_base(i, u, pb0, pb1) + lane_off);
#pragma unroll
      for (int i = 0; i < NL; ++i) vb[r][i] = load_nt16(vbase + load_base(i, u, pb0, pb1) + lane_off);
    };

    // One unit: stage it in LDS, S^T by MFMA, online softmax per column,
    // O^T += V^T (hi + lo weights).  MASKED: the range's last unit, whose
    // rows from nvalid on lie past the range (their V rows are zeroed and
    // their logits selected out, so NaN garbage there cannot leak in) and
    // which may hold the appended token.
    auto consume_t = [&](auto masked, uint4 (&kk)[NL], uint4 (&vv)[NL], int u, int nvalid, int pb0,
                         int pb1) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked)::value;
      if constexpr (MASKED) {
        if (append && u == u_first + u_count - 1) {
          // The appended token is the range's last row: take it from
          // registers and store it to its slot (whose block this unit holds).
          const int ra = nvalid - 1;
          const size_t src = ((size_t)seq * num_kv_heads + kvh) * D + col * 8;
          const uint4 ak = *reinterpret_cast<const uint4*>(new_k + src);
          const uint4 av = *reinterpret_cast<const uint4*>(new_v + src);
#pragma unroll
          for (int i = 0; i < NL; ++i) {
            if (TPL * i + row == ra) {
              kk[i] = ak;
              vv[i] = av;
              const size_t off = (size_t)kvh * D * 2 + load_base(i, u, pb0, pb1) + lane_off;
              *reinterpret_cast<uint4*>(reinterpret_cast<char*>(k_store) + off) = ak;
              *reinterpret_cast<uint4*>(reinterpret_cast<char*>(v_store) + off) = av;
            }
          }
        }
#pragma unroll
        for (int i = 0; i < NL; ++i)
          if (TPL * i + row >= nvalid) vv[i] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int rr = TPL * i + row;
        *reinterpret_cast<uint4*>(s_k + rr * KSTR + col * 16) = kk[i];
        *reinterpret_cast<uint4*>(s_v + rr * VSTR + col * 16) = vv[i];
      }
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NL; ++s)
        sc = MC::qk(*reinterpret_cast<const uint4*>(s_k + c16 * KSTR + 64 * s + 16 * g4), qt[s], sc);
      float t[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        t[i] = sc[i] * scale_log2;
        if constexpr (MASKED) t[i] = 4 * g4 + i < nvalid ? t[i] : -INFINITY;
      }
      // Column max over the unit's 16 keys (lanes l, l ^ 16, l ^ 32, l ^ 48).
      const float mx = xor32_max(xor16_max(vmax(vmax(t[0], t[1]), vmax(t[2], t[3]))));
      // Rescale only when some column's max grew by more than kMcSlack.
      if (__ballot(mx > m_ref + kMcSlack)) {
        const float mn = fmaxf(m_ref, mx);
        const float alpha = fast_exp2(m_ref - mn);
        m_ref = mn;
        l_part *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(t[i] - m_ref);
      l_part += (p[0] + p[1]) + (p[2] + p[3]);
      const uint32_t h01 = E::pack2(p[0], p[1]), h23 = E::pack2(p[2], p[3]);
      const uint2 ph = make_uint2(h01, h23);
      const uint2 pl = make_uint2(E::pack2(p[0] - E::lo(h01), p[1] - E::hi(h01)),
                                  E::pack2(p[2] - E::lo(h23), p[3] - E::hi(h23)));
      // V^T operand of dim tile dt: input lane j of group g4 reads row
      // 4 g4 + j / 4, dims 16 dt + 4 (j % 4) .. +3.
      const char* vrow = s_v + (4 * g4 + c16 / 4) * VSTR + 8 * (c16 & 3);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 vt = lds_read_tr_b16(vrow + 32 * dt);
        o[dt] = MC::pv(vt, ph, o[dt]);
        o[dt] = MC::pv(vt, pl, o[dt]);
      }
    };
    auto consume = [&](auto rb, int u, int pb0, int pb1) __attribute__((always_inline)) {
      constexpr int r = decltype(rb)::value;
      const int nvalid = e_tok - 16 * u;
      if (nvalid < 16 || (append && u == u_first + u_count - 1))
        consume_t(std::true_type{}, kb[r], vb[r], u, nvalid, pb0, pb1);
      else
        consume_t(std::false_type{}, kb[r], vb[r], u, 16, pb0, pb1);
    };

    // Stream units first, first + stride, ... (< u_count) of the range, RING
    // units in flight.  Every path into the steady-state loop has issued the
    // same RING units (short windows repeat their last unit), so the waits
    // the compiler places there are exact; the units left at the end of a
    // window are consumed after the loop.  Table entries come 64 units at a
    // time (lane k: the wavefront's k-th unit of the window); with `pre`, the
    // first window's are already in pre_win / pre_win2.
    auto stream_units = [&](int first, int stride, bool pre) __attribute__((always_inline)) {
      const int nb = first < u_count ? (u_count - first + stride - 1) / stride : 0;
      for (int j0 = 0; j0 < nb; j0 += kWave) {
        const int jn = min(kWave, nb - j0);
        auto unit_of = [&](int k) __attribute__((always_inline)) { return u_first + first + (j0 + k) * stride; };
        int w0 = 0, w1 = 0;
        if (pre && j0 == 0) {
          w0 = pre_win;
          w1 = pre_win2;
        } else if (lane < jn) {
          const int u = unit_of(lane);
          w0 = tbl_row[BS == 8 ? 2 * u : (BS == 32 ? u >> 1 : u)];
          if constexpr (BS == 8) w1 = tbl_row[min(2 * u + 1, last_blk)];
        }
        // Blocks of unit k; an 8-token unit's second block past the range
        // (its entry may be unset) is replaced by its first (rows masked).
        auto blocks = [&](int k, int& pb0, int& pb1) __attribute__((always_inline)) {
          pb0 = uniform_lane(w0, k);
          pb1 = pb0;
          if constexpr (BS == 8) {
            if (2 * unit_of(k) + 1 <= last_blk) pb1 = uniform_lane(w1, k);
          }
        };
        auto iss = [&](auto rb, int k) __attribute__((always_inline)) {
          int pb0, pb1;
          blocks(k, pb0, pb1);
          issue(rb, unit_of(k), pb0, pb1);
        };
        auto con = [&](auto rb, int k) __attribute__((always_inline)) {
          int pb0, pb1;
          blocks(k, pb0, pb1);
          consume(rb, unit_of(k), pb0, pb1);
        };
        auto prologue = [&](auto rb) __attribute__((always_inline)) { iss(rb, min((int)decltype(rb)::value, jn - 1)); };
        static_for<0, RING>(prologue);
        int k = 0;
        for (; k + RING < jn; k += RING) {
          auto body = [&](auto rb) __attribute__((always_inline)) {
            constexpr int r = decltype(rb)::value;
            con(rb, k + r);
            iss(rb, min(k + r + RING, jn - 1));
          };
          static_for<0, RING>(body);
        }
        auto tail = [&](auto rb) __attribute__((always_inline)) {
          constexpr int r = decltype(rb)::value;
          if (k + r < jn) con(rb, k + r);
        };
        static_for<0, RING>(tail);
      }
    };

    if constexpr (FUSED) {
      const int wstride = (int)gridDim.y * W;
      const int p0 = (int)blockIdx.y * W + wave;
      for (int p = p0; p < num_parts; p += wstride) {
        set_range(p * chunk, min(ctx, (p + 1) * chunk));
        stream_units(0, 1, p == p0);
      }
    } else {
      set_range(tok_begin, tok_end);
      stream_units(wave, W, true);
    }

    // The column's exp-sum over the four lane groups; then the wavefront's
    // state goes to LDS, over the K/V tiles once every wavefront is done.
    const float l_tot = xor32_sum(xor16_sum(l_part));
    __syncthreads();
    if (c16 < G) {
      if (g4 == 0) {
        s_m[wave][c16] = m_ref;
        s_l[wave][c16] = l_tot;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t*>(&s_acc[wave][c16][16 * dt + 4 * g4]) = o[dt];
    }
  } else {
    // (Groups of four and eight take this path only where decode_uses_mfma
    // sends them here; it stays complete for every group.)
    // q pieces of the G heads of this group: in registers, or - for groups of
    // four and more, whose accumulators take 32+ registers per lane - in LDS,
    // read once per tile and head.
    constexpr bool kQLds = G >= 4 && !kMfma;
    __shared__ uint4 s_q[kQLds ? G : 1][kQLds ? D / 8 : 1];
    uint32_t qv[kQLds ? 1 : G][4];
    if constexpr (kQLds) {
      const uint16_t* qg = q + ((size_t)seq * num_q_heads + (size_t)kvh * G) * D;  // the group's G rows, contiguous
      for (int t = threadIdx.x; t < G * D / 8; t += W * kWave)
        s_q[t / (D / 8)][t % (D / 8)] = *reinterpret_cast<const uint4*>(qg + t * 8);
      __syncthreads();
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 t = *reinterpret_cast<const uint4*>(q + ((size_t)seq * num_q_heads + kvh * G + g) * D + col * 8);
        qv[g][0] = t.x; qv[g][1] = t.y; qv[g][2] = t.z; qv[g][3] = t.w;
      }
    }

    float m[G], lsum[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = kNegBig;
      lsum[g] = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[g][d] = 0.f;
    }

    const size_t row_elems = (size_t)num_kv_heads * D;        // elements between consecutive slots
    const size_t block_bytes = row_elems * kBlockSize * 2;    // bytes per physical block
    // The streaming unit is a tile: TT consecutive slots of one block, LPBT
    // wave loads per tensor (the whole block when it needs no more than
    // tile_loads() loads), so the load buffers and per-token scores stay within
    // the register budget for every head size, group and block size.
    constexpr int LPBT = decode_tile_loads<D, G, BS>();
    constexpr int TT = LPBT * TPL;  // slots per tile
    constexpr int TPB = LPB / LPBT;  // tiles per block
    const uint32_t tile_bytes = (uint32_t)(row_elems * TT * 2);
    // Per-lane byte offset of load i inside a tile: slot (i*TPL + row), dims col*8.
    uint32_t lane_off[LPBT];
#pragma unroll
    for (int i = 0; i < LPBT; ++i) lane_off[i] = (uint32_t)(((i * TPL + row) * row_elems + col * 8) * 2);
    const char* kbase = reinterpret_cast<const char*>(k_cache) + (size_t)kvh * D * 2;
    const char* vbase = reinterpret_cast<const char*>(v_cache) + (size_t)kvh * D * 2;

    // The range being streamed: its blocks, the tokens in its last block, and
    // whether it ends with the appended token.
    int nblk = 0, last_valid = 0;
    bool append = false;
    const int32_t* tbl = block_tables;
    auto set_range = [&](int b, int e) {
      const int lb_begin = b / kBlockSize;
      nblk = e > b ? (e - b + kBlockSize - 1) / kBlockSize : 0;
      last_valid = e - (lb_begin + nblk - 1) * kBlockSize;
      append = new_k != nullptr && ctx > 0 && e == ctx;
      tbl = block_tables + (size_t)seq * max_blocks_per_seq + lb_begin;
    };

    // Loads of tile `sub` of physical block pb.
    auto issue = [&](int pb, int sub, uint4 (&kk)[LPBT], uint4 (&vv)[LPBT]) {
      const size_t off = (size_t)pb * block_bytes + (size_t)sub * tile_bytes;
      const char* kb = kbase + off;
      const char* vb = vbase + off;
#pragma unroll
      for (int i = 0; i < LPBT; ++i) kk[i] = load_nt16(kb + lane_off[i]);
#pragma unroll
      for (int i = 0; i < LPBT; ++i) vv[i] = load_nt16(vb + lane_off[i]);
    };

    // MASKED is only taken for tiles of the range's last block that hold slots
    // past its last token (nvalid < TT; nvalid <= 0 masks the whole tile).
    auto consume_t = [&](auto masked, const uint4 (&kk)[LPBT], const uint4 (&vv)[LPBT], int nvalid) {
      constexpr bool MASKED = decltype(masked)::value;
      float s[G][LPBT];
      if constexpr (kQLds) {
        // Head by head, so only one head's q is live.
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint4 qq = s_q[g][col];
#pragma unroll
          for (int i = 0; i < LPBT; ++i) {
            const bool valid = !MASKED || (i * TPL + row) < nvalid;
            float d = E::dot2(qq.x, kk[i].x, 0.f);
            d = E::dot2(qq.y, kk[i].y, d);
            d = E::dot2(qq.z, kk[i].z, d);
            d = E::dot2(qq.w, kk[i].w, d);
            d = group_sum<LPT>(d) * scale_log2;
            s[g][i] = valid ? d : -INFINITY;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < LPBT; ++i) {
          const bool valid = !MASKED || (i * TPL + row) < nvalid;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float d = E::dot2(qv[g][0], kk[i].x, 0.f);
            d = E::dot2(qv[g][1], kk[i].y, d);
            d = E::dot2(qv[g][2], kk[i].z, d);
            d = E::dot2(qv[g][3], kk[i].w, d);
            d = group_sum<LPT>(d) * scale_log2;
            s[g][i] = valid ? d : -INFINITY;
          }
        }
      }
      float p[G][LPBT];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = m[g];
#pragma unroll
        for (int i = 0; i < LPBT; ++i) mx = fmaxf(mx, s[g][i]);
        const float alpha = fast_exp2(m[g] - mx);
        m[g] = mx;
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < LPBT; ++i) {
          p[g][i] = fast_exp2(s[g][i] - mx);
          ps += p[g][i];
        }
        lsum[g] = lsum[g] * alpha + ps;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[g][d] *= alpha;
      }
#pragma unroll
      for (int i = 0; i < LPBT; ++i) {
        const bool valid = !MASKED || (i * TPL + row) < nvalid;
        const uint32_t w4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
        float vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[2 * e] = E::lo(w4[e]);
          vf[2 * e + 1] = E::hi(w4[e]);
        }
        if (MASKED && !valid) {
#pragma unroll
          for (int d = 0; d < 8; ++d) vf[d] = 0.f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[g][d] = fmaf(p[g][i], vf[d], acc[g][d]);
      }
    };

    // Tile `sub` of the range's block blk (physical id pb, used only for the
    // appended token's store).
    auto consume = [&](const uint4 (&kk)[LPBT], const uint4 (&vv)[LPBT], int blk, int sub, int pb) {
      const bool last = blk == nblk - 1;
      const int nvalid = last ? last_valid - sub * TT : TT;
      const int r = last_valid - 1 - sub * TT;  // the appended slot's row in this tile, if in [0, TT)
      if (last && append && r >= 0 && r < TT) {
        // Load i = r / TPL, lane row r % TPL holds the appended token.
        uint4 ka2[LPBT], va2[LPBT];
#pragma unroll
        for (int i = 0; i < LPBT; ++i) {
          const bool mine = i * TPL + row == r;
          ka2[i] = mine ? app_k : kk[i];
          va2[i] = mine ? app_v : vv[i];
        }
        if (row == r % TPL) {
          const size_t off = (size_t)kvh * D * 2 + (size_t)pb * block_bytes + (size_t)sub * tile_bytes + lane_off[0] +
                             (size_t)((r / TPL) * TPL) * row_elems * 2;
          *reinterpret_cast<uint4*>(reinterpret_cast<char*>(k_store) + off) = app_k;
          *reinterpret_cast<uint4*>(reinterpret_cast<char*>(v_store) + off) = app_v;
        }
        if (nvalid < TT)
          consume_t(std::true_type{}, ka2, va2, nvalid);
        else
          consume_t(std::false_type{}, ka2, va2, TT);
      } else if (nvalid < TT) {
        consume_t(std::true_type{}, kk, vv, nvalid);
      } else {
        consume_t(std::false_type{}, kk, vv, TT);
      }
    };

    // Stream the tiles of blocks first, first + stride, ... (< nblk) of the
    // range: double buffered, so while a tile is consumed the next one's
    // 2*LPBT loads are in flight.  Every path into the steady-state body has
    // issued the same two tiles' loads (a one-tile window loads its tile
    // twice), so the waits the compiler places there are exact: each consume
    // waits for its own loads only, never for the tile behind it.  The 1-3
    // tiles left at the end of a window are peeled (their waits may be
    // conservative).  Table entries come 64 at a time (lane k holds the entry
    // of the wave's block j0 + k); with `pre`, the first window's are already
    // in pre_win.  Tile u of a window is tile u % TPB of its block u / TPB.
    auto stream_blocks = [&](int first, int stride, bool pre) {
      const int nb = first < nblk ? (nblk - first + stride - 1) / stride : 0;
      uint4 ka[LPBT], va[LPBT], kb2[LPBT], vb2[LPBT];
      for (int j0 = 0; j0 < nb; j0 += kWave) {
        const int jn = min(kWave, nb - j0);
        const int tbl_win = pre && j0 == 0 ? pre_win : (lane < jn ? tbl[first + (j0 + lane) * stride] : 0);
        const int blk_base = first + j0 * stride;  // range-relative index of the window's block 0
        const int nt = jn * TPB;
        auto pb_of = [&](int u) { return uniform_lane(tbl_win, u / TPB); };
        auto blk_of = [&](int u) { return blk_base + (u / TPB) * stride; };
        issue(pb_of(0), 0, ka, va);
        const int u1 = nt > 1 ? 1 : 0;
        issue(pb_of(u1), u1 % TPB, kb2, vb2);
        int u = 0;
        for (; u + 3 < nt; u += 2) {
          consume(ka, va, blk_of(u), u % TPB, pb_of(u));
          issue(pb_of(u + 2), (u + 2) % TPB, ka, va);
          consume(kb2, vb2, blk_of(u + 1), (u + 1) % TPB, pb_of(u + 1));
          issue(pb_of(u + 3), (u + 3) % TPB, kb2, vb2);
        }
        const int rem = nt - u;  // 1, 2 or 3 tiles left; ka holds u, kb2 holds u + 1
        consume(ka, va, blk_of(u), u % TPB, pb_of(u));
        if (rem == 3) issue(pb_of(u + 2), (u + 2) % TPB, ka, va);
        if (rem >= 2) consume(kb2, vb2, blk_of(u + 1), (u + 1) % TPB, pb_of(u + 1));
        if (rem == 3) consume(ka, va, blk_of(u + 2), (u + 2) % TPB, pb_of(u + 2));
      }
    };

    if constexpr (FUSED) {
      // This wavefront's chunks, one running state over all of them.
      const int wstride = (int)gridDim.y * W;
      const int p0 = (int)blockIdx.y * W + wave;
      for (int p = p0; p < num_parts; p += wstride) {
        set_range(p * chunk, min(ctx, (p + 1) * chunk));
        stream_blocks(0, 1, p == p0);
      }
    } else {
      set_range(tok_begin, tok_end);
      stream_blocks(wave, W, true);
    }

    // Merge the rows of this wavefront (butterfly over lane ^ LPT, ^ 2 LPT, ...).
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mo = __shfl_xor(m[g], off);
        const float lo = __shfl_xor(lsum[g], off);
        const float mm = fmaxf(m[g], mo);
        const float fa = fast_exp2(m[g] - mm);
        const float fb = fast_exp2(mo - mm);
        lsum[g] = lsum[g] * fa + lo * fb;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[g][d] = acc[g][d] * fa + __shfl_xor(acc[g][d], off) * fb;
        m[g] = mm;
      }
    }

    // The wavefront's state to LDS.
    if (row == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int d = 0; d < 8; ++d) s_acc[wave][g][col * 8 + d] = acc[g][d];
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = lsum[g];
      }
    }
  }

  // Merge the wavefronts through LDS, normalise and store.
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += W * kWave) {
    const int g = t / D, d = t % D;
    float mm = kNegBig;
#pragma unroll
    for (int w = 0; w < W; ++w) mm = fmaxf(mm, s_m[w][g]);
    float lt = 0.f, at = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = fast_exp2(s_m[w][g] - mm);
      lt += s_l[w][g] * f;
      at += s_acc[w][g][d] * f;
    }
    const int h = kvh * G + g;
    const float o = lt > 0.f ? at / lt : 0.f;
    if constexpr (FUSED) {
      // The workgroup's state: row blockIdx.y of the (sequence, head).
      const size_t idx = ((size_t)seq * num_q_heads + h) * max_num_partitions + blockIdx.y;
      store_coherent(tmp_out + idx * D + d, o);
      if (d == 0) {
        store_coherent(max_logits + idx, mm * kLn2);  // back to natural-log units
        store_coherent(exp_sums + idx, lt);
      }
    } else if constexpr (SPLIT) {
      const size_t idx = ((size_t)seq * num_q_heads + h) * max_num_partitions + part;
      tmp_out[idx * D + d] = o;
      if (d == 0) {
        max_logits[idx] = mm * kLn2;  // back to natural-log units
        exp_sums[idx] = lt;
      }
    } else {
      out[((size_t)seq * num_q_heads + h) * D + d] = E::from_float(o);
    }
  }

  if constexpr (FUSED) {
    // Publish the workgroup's state: every wavefront waits until its coherent
    // stores have completed, then one thread counts the workgroup.  The
    // counter wraps to 0 on the last arrival, so every call leaves the
    // counters as it found them; the workgroup that sees the wrap merges the
    // sequence's workgroup states (reading them with coherent loads).
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t prev = __builtin_amdgcn_atomic_inc32(counters + (size_t)seq * num_kv_heads + kvh,
                                                          (uint32_t)(wg_active - 1), __ATOMIC_RELAXED, "agent");
      s_last = prev == (uint32_t)(wg_active - 1);
    }
    __syncthreads();
    if (!s_last) return;
    merge_group_partitions<T, D, G, W>(tmp_out, max_logits, exp_sums, seq, kvh, num_q_heads, max_num_partitions,
                                       wg_active, out);
  }
}

// Split-K reduce: one workgroup per (query head, sequence, chunk of
// ReduceGeom::DC dims).  Partitions are taken in passes of up to kReduceChunk:
// the threads find the pass's max logit and weights w_p = l_p exp(m_p - M) in
// parallel (weights kept in LDS; every dim chunk recomputes them, a few loads
// per partition), then thread t accumulates dim t % DC of the chunk over
// partitions t / DC, t / DC + GROUPS, ... with independent loads in flight; a
// running max rescales earlier passes.
constexpr int kReduceThreads = 256;
constexpr int kReduceChunk = 1024;

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* scratch) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();  // scratch may still be read by a previous reduction
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  v = scratch[0];
#pragma unroll
  for (int w = 1; w < kReduceThreads / kWave; ++w) v = is_max ? fmaxf(v, scratch[w]) : v + scratch[w];
  return v;
}

// Dims per reduce workgroup: the head's dims are spread over D / kReduceDims
// workgroups, so a few (sequence, head) pairs still fill the GPU and each
// thread walks a quarter of the partitions it would otherwise.
#ifndef PKA_REDUCE_DIMS
#define PKA_REDUCE_DIMS 32
#endif
template <int D>
struct ReduceGeom {
  static constexpr int DC = D < PKA_REDUCE_DIMS ? D : PKA_REDUCE_DIMS;  // dims per workgroup
  static constexpr int CHUNKS = D / DC;
};

template <typename T, int D>
__global__ void __launch_bounds__(kReduceThreads)
splitk_reduce_kernel(const float* __restrict__ tmp_out, const float* __restrict__ max_logits,
                     const float* __restrict__ exp_sums, const int32_t* __restrict__ context_lens,
                     int32_t num_q_heads, int32_t partition_size, int32_t max_num_partitions,
                     uint16_t* __restrict__ out) {
  constexpr int DC = ReduceGeom<D>::DC;
  constexpr int GROUPS = kReduceThreads / DC;
  __shared__ float s_w[kReduceChunk];
  __shared__ float s_red[kReduceThreads / kWave];
  __shared__ float s_acc[GROUPS][DC];
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int t = threadIdx.x;
  const int dl = t % DC, grp = t / DC;
  const int d = blockIdx.z * DC + dl;  // this thread's dim
  const int ctx = context_lens[seq];
  // A context past the host bound (a broken precondition) must not reach into
  // another row's partitions.
  const int P = ctx > 0 ? min((ctx + partition_size - 1) / partition_size, max_num_partitions) : 0;
  const size_t base = ((size_t)seq * num_q_heads + h) * max_num_partitions;

  float m_run = -INFINITY, l_run = 0.f, acc = 0.f;
  for (int p0 = 0; p0 < P; p0 += kReduceChunk) {
    const int n = min(kReduceChunk, P - p0);
    float mx = -INFINITY;
    for (int p = t; p < n; p += kReduceThreads) mx = fmaxf(mx, max_logits[base + p0 + p]);
    mx = block_reduce(mx, true, s_red);
    const float m_new = fmaxf(m_run, mx);
    const float rescale = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * kLog2e);
    float ls = 0.f;
    for (int p = t; p < n; p += kReduceThreads) {
      const float w = exp_sums[base + p0 + p] * fast_exp2((max_logits[base + p0 + p] - m_new) * kLog2e);
      s_w[p] = w;
      ls += w;
    }
    ls = block_reduce(ls, false, s_red);  // its barriers also publish s_w
    l_run = l_run * rescale + ls;
    acc *= rescale;
    m_run = m_new;
    const float* po = tmp_out + (base + p0) * D + d;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int p = grp;
    for (; p + 3 * GROUPS < n; p += 4 * GROUPS) {
      a0 += s_w[p] * po[(size_t)p * D];
      a1 += s_w[p + GROUPS] * po[(size_t)(p + GROUPS) * D];
      a2 += s_w[p + 2 * GROUPS] * po[(size_t)(p + 2 * GROUPS) * D];
      a3 += s_w[p + 3 * GROUPS] * po[(size_t)(p + 3 * GROUPS) * D];
    }
    for (; p < n; p += GROUPS) a0 += s_w[p] * po[(size_t)p * D];
    acc += (a0 + a1) + (a2 + a3);
    __syncthreads();  // s_w is rewritten by the next pass
  }
  s_acc[grp][dl] = acc;
  __syncthreads();
  if (t < DC) {
    float o = 0.f;
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) o += s_acc[g][t];
    out[((size_t)seq * num_q_heads + h) * D + blockIdx.z * DC + t] =
        Elem<T>::from_float(l_run > 0.f ? o / l_run : 0.f);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

#ifndef PKA_DECODE_WAVES
#define PKA_DECODE_WAVES 4
#endif
constexpr int kDecodeWaves = PKA_DECODE_WAVES;  // wavefronts per single-pass decode workgroup
#ifndef PKA_SPLIT_WAVES
#define PKA_SPLIT_WAVES 4
#endif
constexpr int kSplitWaves = PKA_SPLIT_WAVES;    // wavefronts per split-K partition workgroup
// Wavefronts per workgroup of the single-launch split-K.  Eight (one
// workgroup per compute unit, half the workgroup states to merge) where the
// kernel fits 256 registers per lane: measured on 4 x 16,384 tokens, 51.1
// against 52.6 us per call with four.  Instances whose load buffers and
// accumulators need more (16 registers per load of a block, 12 per query
// head of the group, beyond ~100) would spill with eight and keep four, which
// may use the accumulation registers as well.
template <int D, int G, int BS>
constexpr int fused_waves() {
  if (decode_uses_mfma<G>()) return 4;  // the matrix-core path's ring of loads fills the register budget
  return 16 * decode_tile_loads<D, G, BS>() + 12 * G <= 100 ? 8 : 4;
}
// Heavy-first ordering scans all context lengths in every workgroup; above
// this many sequences the grid order is kept.
constexpr int kOrderMaxSeqs = 1024;

template <typename T, int D, int G, int BS>
static hipError_t launch_decode_t(const DecodeArgs& a, int mode, hipStream_t stream) {
  const float scale_log2 = a.scale * kLog2e;
  if (mode == kDecodeSingle) {
    dim3 grid(a.num_kv_heads, a.num_seqs);
    // Longest-first pairing: a grid of more workgroups than compute units but
    // no more than two per unit starts all at once, the first CUs / H rows
    // taking one slot on every unit and the rest a second slot; those rows
    // are reversed (measured on the 64-sequence decode of the mixed step:
    // 7-11 % faster; grids of several rounds keep plain longest-first order).
    const int64_t wgs = (int64_t)a.num_seqs * a.num_kv_heads;
    // Ordering pays only when some workgroups wait for others to finish; with
    // no more workgroups than compute units all of them start at once.
    const bool order = a.order_max_ctx > 0 && a.num_seqs <= kOrderMaxSeqs && (a.num_cus <= 0 || wgs > a.num_cus);
    int32_t pair_from = 0;
    if (a.num_cus > 0 && wgs > a.num_cus && wgs <= 2 * (int64_t)a.num_cus) pair_from = a.num_cus / a.num_kv_heads;
    if (pair_from >= a.num_seqs) pair_from = 0;
    hipLaunchKernelGGL((paged_decode_kernel<T, D, G, kDecodeWaves, kDecodeSingle, BS>), grid,
                       dim3(kDecodeWaves * kWave), 0, stream, a.q, a.k_cache, a.v_cache, a.block_tables,
                       a.context_lens, a.max_blocks_per_seq, a.num_kv_heads, scale_log2, a.out, nullptr, nullptr,
                       nullptr, 0, order ? a.order_max_ctx : 0, a.new_k, a.new_v, a.k_store,
                       a.v_store, order ? pair_from : 0, nullptr, 0);
  } else if (mode == kDecodeSplit) {
    dim3 grid(a.num_kv_heads, a.max_num_partitions, a.num_seqs);
    hipLaunchKernelGGL((paged_decode_kernel<T, D, G, kSplitWaves, kDecodeSplit, BS>), grid,
                       dim3(kSplitWaves * kWave), 0, stream, a.q, a.k_cache, a.v_cache, a.block_tables,
                       a.context_lens, a.max_blocks_per_seq, a.num_kv_heads, scale_log2, nullptr, a.tmp_out,
                       a.max_logits, a.exp_sums, a.max_num_partitions, 0, a.new_k, a.new_v, a.k_store, a.v_store, 0,
                       nullptr, 0);
  } else {
    // Single launch: enough workgroups per (sequence, KV head) that every
    // wavefront of one resident round (one workgroup per compute unit) has a
    // chunk, and no more than the chunks need.  Chunks are 256-token
    // partitions unless that leaves wavefronts of the round idle; then they
    // are halved (down to 256 / FW tokens, so no more workgroups than the
    // workspace has partition rows, and at least one block).
    constexpr int FW = fused_waves<D, G, BS>();
    const int64_t pairs = (int64_t)a.num_seqs * a.num_kv_heads;
    const int64_t slots = (int64_t)(a.num_cus > 0 ? a.num_cus : 256) * (8 / FW);
    const int64_t max_ctx = a.max_context_len > 0 ? std::min<int64_t>(a.max_context_len, (int64_t)a.max_num_partitions *
                                                                                             kPartitionSize)
                                                  : (int64_t)a.max_num_partitions * kPartitionSize;
    int chunk = kPartitionSize;
    while (chunk / 2 >= std::max(BS, kPartitionSize / FW) && pairs * ((max_ctx + chunk - 1) / chunk) < slots * FW)
      chunk /= 2;
    const int64_t by_chunks = ((max_ctx + chunk - 1) / chunk + FW - 1) / FW;
    const int y = (int)std::max<int64_t>(
        1, std::min<int64_t>({by_chunks, slots / pairs, (int64_t)a.max_num_partitions}));
    dim3 grid(a.num_kv_heads, y, a.num_seqs);
    hipLaunchKernelGGL((paged_decode_kernel<T, D, G, FW, kDecodeSplitFused, BS>), grid,
                       dim3(FW * kWave), 0, stream, a.q, a.k_cache, a.v_cache, a.block_tables,
                       a.context_lens, a.max_blocks_per_seq, a.num_kv_heads, scale_log2, a.out, a.tmp_out,
                       a.max_logits, a.exp_sums, a.max_num_partitions, 0, a.new_k, a.new_v, a.k_store, a.v_store, 0,
                       a.counters, chunk);
  }
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t launch_decode_b(const DecodeArgs& a, int mode, hipStream_t stream) {
  switch (a.block_size) {
    case 8: return launch_decode_t<T, D, G, 8>(a, mode, stream);
    case 16: return launch_decode_t<T, D, G, 16>(a, mode, stream);
    case 32: return launch_decode_t<T, D, G, 32>(a, mode, stream);
  }
  return hipErrorInvalidValue;
}

// Every decode launch of one (element type, head size); instantiated by the
// decode_<type>_d<size>.hip files, dispatched to by launch_decode.
template <typename T, int D>
hipError_t launch_decode_td(const DecodeArgs& a, int mode, hipStream_t stream) {
  switch (a.group) {
    case 1: return launch_decode_b<T, D, 1>(a, mode, stream);
    case 2: return launch_decode_b<T, D, 2>(a, mode, stream);
    case 4: return launch_decode_b<T, D, 4>(a, mode, stream);
    case 8: return launch_decode_b<T, D, 8>(a, mode, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t launch_splitk_reduce_td(const ReduceArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((splitk_reduce_kernel<T, D>), dim3(a.num_q_heads, a.num_seqs, ReduceGeom<D>::CHUNKS),
                     dim3(kReduceThreads), 0, stream, a.tmp_out, a.max_logits, a.exp_sums, a.context_lens,
                     a.num_q_heads, a.partition_size, a.max_num_partitions, a.out);
  return hipGetLastError();
}

#define PKA_DECODE_FOR_ALL(X) X(F16, 64) X(F16, 128) X(F16, 256) X(BF16, 64) X(BF16, 128) X(BF16, 256)
#define PKA_DECODE_EXTERN(T, D)                                                          \
  extern template hipError_t launch_decode_td<T, D>(const DecodeArgs&, int, hipStream_t); \
  extern template hipError_t launch_splitk_reduce_td<T, D>(const ReduceArgs&, hipStream_t);
#define PKA_DECODE_INSTANTIATE(T, D)                                              \
  template hipError_t launch_decode_td<T, D>(const DecodeArgs&, int, hipStream_t); \
  template hipError_t launch_splitk_reduce_td<T, D>(const ReduceArgs&, hipStream_t);

}  // namespace pka
