// Paged decode attention for gfx950.
//
// What it computes (MiniLLM Runtime, "CUDA PagedAttention scope"; mini_engine,
// "Custom CUDA kernels", paged decode v1 and v2): for one query row per
// sequence, softmax(scale * q . k_t) over the sequence's context, then the
// weighted sum of v_t, reading every K/V row in place through the block table
// (MiniLLM Runtime, "Core class relationships").
//
// Work decomposition.  One workgroup per (KV head, sequence) - or per
// (KV head, 256-token partition, sequence) for split-K.  The G query heads of
// the GQA group ride along, so every K/V byte is loaded once and used G times.
// The workgroup's W wavefronts take the range's KV blocks round-robin.
//
// Lane layout inside a wavefront.  One 16-byte load per lane (8 elements)
// makes a token row of D elements span LPT = D / 8 lanes, so one wave load
// covers TPL = 64 / LPT tokens and a 16-token block of one head takes
// LPB = 16 / TPL loads per tensor (D = 128: 16 lanes, 4 tokens, 4 loads).
// Each group of LPT lanes ("row") sums its dot-product pieces with DPP and
// keeps its own online-softmax state (max, exp-sum, 8 accumulator dims per
// head) over the tokens it sees; rows, then wavefronts, are merged once at the
// end with the same max/exp-sum rule the split-K reduce uses.
//
// Memory: the caches are token-major ([block][slot][kv head][dim]), so a
// (block, head) is 16 rows of D*2 bytes at a stride of num_kv_heads*D*2 bytes;
// each row is fetched as whole 16-byte pieces by consecutive lanes.  Each
// wavefront keeps the next block's K and V loads in flight while it computes
// on the current one.  Block-table entries are fetched 64 at a time with one
// vector load per wavefront and broadcast with readlane.
//
// Numerics: q.k in fp32 with v_dot2 on the raw fp16/bf16 pairs; softmax in the
// base-2 domain (scale * log2 e folded into the logit); fp32 accumulation;
// tokens past the context are selected out (never multiplied by a zero
// weight), so NaN garbage in unowned slots cannot leak in.

#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace pka {

constexpr int kBlockSize = 16;

template <int D>
struct DecodeLayout {
  static constexpr int LPT = D / 8;       // lanes per token row
  static constexpr int TPL = kWave / LPT;  // token rows per wave load
  static constexpr int LPB = kBlockSize / TPL;  // wave loads per block per tensor
  static_assert(kWave % LPT == 0 && kBlockSize % TPL == 0, "unsupported head_dim");
};

template <typename T, int D, int G, int W, bool SPLIT>
__global__ void __launch_bounds__(W * kWave)
paged_decode_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                    const int32_t* __restrict__ context_lens, int32_t max_blocks_per_seq,
                    int32_t num_kv_heads, float scale_log2, uint16_t* __restrict__ out,
                    float* __restrict__ tmp_out, float* __restrict__ max_logits,
                    float* __restrict__ exp_sums, int32_t max_num_partitions) {
  using L = DecodeLayout<D>;
  using E = Elem<T>;
  constexpr int LPT = L::LPT, TPL = L::TPL, LPB = L::LPB;

  const int kvh = blockIdx.x;
  const int part = SPLIT ? (int)blockIdx.y : 0;
  const int seq = SPLIT ? (int)blockIdx.z : (int)blockIdx.y;
  const int num_q_heads = num_kv_heads * G;

  const int ctx = context_lens[seq];
  int tok_begin = 0, tok_end = ctx;
  if constexpr (SPLIT) {
    tok_begin = part * kPartitionSize;
    if (tok_begin >= ctx) return;  // past this sequence's end: nothing to write
    tok_end = min(ctx, tok_begin + kPartitionSize);
  }
  const int lb_begin = tok_begin / kBlockSize;
  const int nblk = tok_end > tok_begin ? (tok_end - tok_begin + kBlockSize - 1) / kBlockSize : 0;
  const int last_valid = tok_end - (lb_begin + nblk - 1) * kBlockSize;  // tokens in the range's last block

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int row = lane / LPT;
  const int col = lane % LPT;  // this lane's 8 dims: col*8 .. col*8+7

  // q pieces of the G heads of this group.
  uint32_t qv[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 t = *reinterpret_cast<const uint4*>(q + ((size_t)seq * num_q_heads + kvh * G + g) * D + col * 8);
    qv[g][0] = t.x; qv[g][1] = t.y; qv[g][2] = t.z; qv[g][3] = t.w;
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
  // Per-lane byte offset of load i inside a (block, head): row (i*TPL + row), dims col*8.
  uint32_t lane_off[LPB];
#pragma unroll
  for (int i = 0; i < LPB; ++i) lane_off[i] = (uint32_t)(((i * TPL + row) * row_elems + col * 8) * 2);
  const char* kbase = reinterpret_cast<const char*>(k_cache) + (size_t)kvh * D * 2;
  const char* vbase = reinterpret_cast<const char*>(v_cache) + (size_t)kvh * D * 2;
  const int32_t* tbl = block_tables + (size_t)seq * max_blocks_per_seq + lb_begin;

  // This wavefront's blocks are wave, wave + W, wave + 2W, ... (< nblk).
  const int nb_wave = wave < nblk ? (nblk - wave + W - 1) / W : 0;

  auto issue = [&](int pb, uint4 (&kk)[LPB], uint4 (&vv)[LPB]) {
    const char* kb = kbase + (size_t)pb * block_bytes;
    const char* vb = vbase + (size_t)pb * block_bytes;
#pragma unroll
    for (int i = 0; i < LPB; ++i) kk[i] = *reinterpret_cast<const uint4*>(kb + lane_off[i]);
#pragma unroll
    for (int i = 0; i < LPB; ++i) vv[i] = *reinterpret_cast<const uint4*>(vb + lane_off[i]);
  };

  // MASKED is only taken for the range's last block when it is partial.
  auto consume_t = [&](auto masked, const uint4 (&kk)[LPB], const uint4 (&vv)[LPB], int nvalid) {
    constexpr bool MASKED = decltype(masked)::value;
    float s[G][LPB];
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
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
    float p[G][LPB];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int i = 0; i < LPB; ++i) mx = fmaxf(mx, s[g][i]);
      const float alpha = fast_exp2(m[g] - mx);
      m[g] = mx;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        p[g][i] = fast_exp2(s[g][i] - mx);
        ps += p[g][i];
      }
      lsum[g] = lsum[g] * alpha + ps;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[g][d] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
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

  auto consume = [&](const uint4 (&kk)[LPB], const uint4 (&vv)[LPB], int blk) {
    if (blk == nblk - 1 && last_valid < kBlockSize)
      consume_t(std::true_type{}, kk, vv, last_valid);
    else
      consume_t(std::false_type{}, kk, vv, kBlockSize);
  };

  // Main loop: double-buffered over this wavefront's blocks; table entries
  // come 64 at a time (lane k holds the entry of the wave's block j0 + k).
  uint4 ka[LPB], va[LPB], kb2[LPB], vb2[LPB];
  for (int j0 = 0; j0 < nb_wave; j0 += kWave) {
    const int jn = min(kWave, nb_wave - j0);
    const int my_blk = wave + (j0 + lane) * W;
    const int tbl_win = lane < jn ? tbl[my_blk] : 0;
    issue(uniform_lane(tbl_win, 0), ka, va);
    int j = 0;
    for (; j + 1 < jn; j += 2) {
      issue(uniform_lane(tbl_win, j + 1), kb2, vb2);
      const int blk0 = wave + (j0 + j) * W;
      consume(ka, va, blk0);
      if (j + 2 < jn) issue(uniform_lane(tbl_win, j + 2), ka, va);
      const int blk1 = blk0 + W;
      consume(kb2, vb2, blk1);
    }
    if (j < jn) {
      const int blk0 = wave + (j0 + j) * W;
      consume(ka, va, blk0);
    }
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

  // Merge the wavefronts through LDS, normalise and store.
  __shared__ float s_m[W][G], s_l[W][G];
  __shared__ float s_acc[W][G][D];
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
    if constexpr (SPLIT) {
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
}

// Split-K reduce: one workgroup per (query head, sequence), one thread per dim.
template <typename T, int D>
__global__ void __launch_bounds__(D)
splitk_reduce_kernel(const float* __restrict__ tmp_out, const float* __restrict__ max_logits,
                     const float* __restrict__ exp_sums, const int32_t* __restrict__ context_lens,
                     int32_t num_q_heads, int32_t partition_size, int32_t max_num_partitions,
                     uint16_t* __restrict__ out) {
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int d = threadIdx.x;
  const int ctx = context_lens[seq];
  const int P = ctx > 0 ? (ctx + partition_size - 1) / partition_size : 0;
  const size_t base = ((size_t)seq * num_q_heads + h) * max_num_partitions;
  float mm = -INFINITY;
  for (int p = 0; p < P; ++p) mm = fmaxf(mm, max_logits[base + p]);
  float lt = 0.f, at = 0.f;
  for (int p = 0; p < P; ++p) {
    const float w = exp_sums[base + p] * fast_exp2((max_logits[base + p] - mm) * kLog2e);
    lt += w;
    at += w * tmp_out[(base + p) * D + d];
  }
  out[((size_t)seq * num_q_heads + h) * D + d] = Elem<T>::from_float(lt > 0.f ? at / lt : 0.f);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

constexpr int kDecodeWaves = 4;

template <typename T, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs& a, bool split, hipStream_t stream) {
  const float scale_log2 = a.scale * kLog2e;
  if (!split) {
    dim3 grid(a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((paged_decode_kernel<T, D, G, kDecodeWaves, false>), grid, dim3(kDecodeWaves * kWave), 0,
                       stream, a.q, a.k_cache, a.v_cache, a.block_tables, a.context_lens, a.max_blocks_per_seq,
                       a.num_kv_heads, scale_log2, a.out, nullptr, nullptr, nullptr, 0);
  } else {
    dim3 grid(a.num_kv_heads, a.max_num_partitions, a.num_seqs);
    hipLaunchKernelGGL((paged_decode_kernel<T, D, G, kDecodeWaves, true>), grid, dim3(kDecodeWaves * kWave), 0,
                       stream, a.q, a.k_cache, a.v_cache, a.block_tables, a.context_lens, a.max_blocks_per_seq,
                       a.num_kv_heads, scale_log2, nullptr, a.tmp_out, a.max_logits, a.exp_sums,
                       a.max_num_partitions);
  }
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_g(const DecodeArgs& a, bool split, hipStream_t stream) {
  switch (a.group) {
    case 1: return launch_decode_t<T, D, 1>(a, split, stream);
    case 2: return launch_decode_t<T, D, 2>(a, split, stream);
    case 4: return launch_decode_t<T, D, 4>(a, split, stream);
    case 8: return launch_decode_t<T, D, 8>(a, split, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, bool split, hipStream_t stream) {
  if (a.bf16) {
    if (a.head_dim == 64) return launch_decode_g<BF16, 64>(a, split, stream);
    if (a.head_dim == 128) return launch_decode_g<BF16, 128>(a, split, stream);
  } else {
    if (a.head_dim == 64) return launch_decode_g<F16, 64>(a, split, stream);
    if (a.head_dim == 128) return launch_decode_g<F16, 128>(a, split, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_splitk_reduce(const ReduceArgs& a, hipStream_t stream) {
  dim3 grid(a.num_q_heads, a.num_seqs);
#define PKA_REDUCE(T, D)                                                                                   \
  hipLaunchKernelGGL((splitk_reduce_kernel<T, D>), grid, dim3(D), 0, stream, a.tmp_out, a.max_logits,     \
                     a.exp_sums, a.context_lens, a.num_q_heads, a.partition_size, a.max_num_partitions, a.out)
  if (a.bf16) {
    if (a.head_dim == 64) PKA_REDUCE(BF16, 64);
    else if (a.head_dim == 128) PKA_REDUCE(BF16, 128);
    else return hipErrorInvalidValue;
  } else {
    if (a.head_dim == 64) PKA_REDUCE(F16, 64);
    else if (a.head_dim == 128) PKA_REDUCE(F16, 128);
    else return hipErrorInvalidValue;
  }
#undef PKA_REDUCE
  return hipGetLastError();
}

}  // namespace pka
