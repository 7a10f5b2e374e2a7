// Paged prefill attention for gfx950 on MFMA.
//
// What it computes (mini_engine, "Custom CUDA kernels", paged prefill
// attention; miniserve, "Engine" flowchart, bottom-right causal mask): for a
// ragged batch of query chunks, chunk j of q_len rows sits at the end of a
// sequence of context_lens[j] tokens; row i sees the c = ctx - q_len cached
// tokens and chunk rows 0..i.  K and V are read in place through the block
// table, softmax is online (running max / exp-sum per row), one launch covers
// every chunk of the batch.
//
// Tiling.  A workgroup (4 wavefronts) owns 128 "q-rows" of one chunk and one
// KV head: 128 / G query positions times the G query heads of the GQA group,
// so every K/V tile it stages serves all G heads.  It walks the visible keys
// in tiles of 32 (two KV blocks), staged in LDS: K row-major, V transposed.
// Each wavefront owns 32 q-rows (two 16-row MFMA tiles).
//
// Products (v_mfma_f32_16x16x32, fp32 accumulate):
//   S^T = K Q^T : A = 16 keys x 32 dims of K (LDS), B = Q^T fragment kept in
//                 registers for the whole kernel.  The C layout then gives each
//                 lane 4 keys of one q-row - exactly the lane's share of the
//                 B operand of the next product, so the softmax weights never
//                 leave registers.
//   O^T += V^T P^T : A = 16 dims x 32 keys of V^T (LDS), B = P^T (registers,
//                 rounded to the input type).
// Both products only need the two operands to agree on which K index each
// (lane group, element) holds; the key order inside a tile is permuted so the
// 8 keys a lane needs in PV are 8 consecutive rows of V^T (one 16-byte LDS read).
//
// Numerics: logits in fp32, softmax in base 2 with scale * log2 e folded in,
// masked keys selected out (-inf logit; K/V rows past the context are zeroed in
// LDS so no NaN garbage reaches the products), fp32 accumulators, one
// normalisation at the end, round to nearest even on store.

#include "device_common.h"
#include "launch.h"

namespace pka {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;

template <>
struct Mfma<BF16> {
  static __device__ __forceinline__ floatx4_t mma(const uint4& a, const uint4& b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return (uint32_t)Elem<BF16>::from_float(lo) | ((uint32_t)Elem<BF16>::from_float(hi) << 16);
  }
};

template <>
struct Mfma<F16> {
  static __device__ __forceinline__ floatx4_t mma(const uint4& a, const uint4& b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8_t, a), __builtin_bit_cast(halfx8_t, b),
                                                  c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return (uint32_t)Elem<F16>::from_float(lo) | ((uint32_t)Elem<F16>::from_float(hi) << 16);
  }
};

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfRows = 128;          // q-rows per workgroup (positions x group heads)
constexpr int kPfRowsPerWave = 32;    // two 16-row MFMA tiles
constexpr int kPfKeys = 32;           // keys per staged tile (two KV blocks)
constexpr int kPfBlock = 16;          // KV block size

template <int D>
struct PfLds {
  static constexpr int KROW = D + 8;         // K tile row stride (elements)
  static constexpr int VROW = kPfKeys + 8;   // V^T tile row stride (elements)
  static constexpr int KELEMS = kPfKeys * KROW;
  static constexpr int VELEMS = D * VROW;
  static constexpr int STAGE = KELEMS + VELEMS;
};

// Find the chunk and the query tile of workgroup `tile` (tiles of `bq`
// positions, numbered chunk by chunk).  Every wavefront runs the same scan.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ qsl, int num_seqs, int bq, int tile,
                                          int* seq, int* qtile) {
  const int lane = threadIdx.x & (kWave - 1);
  int before = 0;  // tiles of chunks already passed
  for (int base = 0; base < num_seqs; base += kWave) {
    const int s = base + lane;
    int n = 0;
    if (s < num_seqs) {
      const int ql = qsl[s + 1] - qsl[s];
      n = (ql + bq - 1) / bq;
    }
    int incl = n;  // inclusive prefix sum over the wavefront
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const int hit = before + incl > tile && before + incl - n <= tile && n > 0;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int first = __ffsll((long long)mask) - 1;
      const int excl = __shfl(before + incl - n, first);
      *seq = base + first;
      *qtile = tile - excl;
      return true;
    }
    before += __shfl(incl, kWave - 1);
  }
  return false;
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(kPfThreads)
paged_prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                     const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                     const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start_loc,
                     int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_kv_heads, float scale_log2,
                     uint16_t* __restrict__ out) {
  using MM = Mfma<T>;
  using LD = PfLds<D>;
  constexpr int BQ = kPfRows / G;     // query positions per workgroup
  constexpr int KSTEPS = D / 32;      // MFMA k-steps of QK^T
  constexpr int DTILES = D / 16;      // 16-dim tiles of the output
  constexpr int NT = kPfRowsPerWave / 16;

  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * LD::STAGE];

  const int kvh = blockIdx.x;
  int seq, qt;
  if (!find_tile(query_start_loc, num_seqs, BQ, blockIdx.y, &seq, &qt)) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_id();
  const int l16 = lane & 15;
  const int blk = lane >> 4;
  const int num_q_heads = num_kv_heads * G;

  const int qstart = query_start_loc[seq];
  const int qlen = query_start_loc[seq + 1] - qstart;
  const int ctx = context_lens[seq];
  const int cached = ctx - qlen;
  const int q0 = qt * BQ;
  const int nvalid = min(BQ, qlen - q0);
  const int kend = cached + q0 + nvalid;  // keys [0, kend) are visible to some row
  const int ntiles = (kend + kPfKeys - 1) / kPfKeys;
  const int32_t* tbl = block_tables + (size_t)seq * max_blocks_per_seq;
  const size_t row_elems = (size_t)num_kv_heads * D;

  // Q^T fragments (B operand): q-row n of this lane in tile nt, dims 32s + 8blk .. +7.
  uint4 qf[NT][KSTEPS];
  int pos_of[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = wave * kPfRowsPerWave + nt * 16 + l16;
    const int pos = q0 + n / G;
    const int g = n % G;
    pos_of[nt] = pos < qlen ? pos : -1;
    const uint16_t* qp = q + ((size_t)(qstart + pos) * num_q_heads + kvh * G + g) * D + 8 * blk;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (pos < qlen) v = *reinterpret_cast<const uint4*>(qp + 32 * s);
      qf[nt][s] = v;
    }
  }

  // ---- global -> register staging of one key tile ----
  constexpr int KCHUNKS = kPfKeys * D / 8;                  // 16-byte pieces of the K tile
  constexpr int KPER = (KCHUNKS + kPfThreads - 1) / kPfThreads;
  constexpr int VITEMS = (kPfKeys / 4) * (D / 4);            // 4 keys x 4 dims items of the V tile
  static_assert(VITEMS <= kPfThreads, "one V item per thread");
  uint4 kreg[KPER];
  uint2 vreg[4];

  auto row_ptr = [&](const uint16_t* cache, int key) -> const uint16_t* {
    const int pb = tbl[key / kPfBlock];
    return cache + ((size_t)pb * kPfBlock + key % kPfBlock) * row_elems + (size_t)kvh * D;
  };

  auto fetch = [&](int tile) {
    const int k0 = tile * kPfKeys;
#pragma unroll
    for (int r = 0; r < KPER; ++r) {
      const int c = threadIdx.x + r * kPfThreads;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < KCHUNKS) {
        const int key = k0 + c / (D / 8);
        if (key < ctx) v = *reinterpret_cast<const uint4*>(row_ptr(k_cache, key) + (c % (D / 8)) * 8);
      }
      kreg[r] = v;
    }
    const int t = threadIdx.x;
    if (t < VITEMS) {
      const int dg = t % (D / 4), kg = t / (D / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * kg + r;
        uint2 v = make_uint2(0, 0);
        if (key < ctx) v = *reinterpret_cast<const uint2*>(row_ptr(v_cache, key) + 4 * dg);
        vreg[r] = v;
      }
    }
  };

  auto stage = [&](int buf) {
    uint16_t* ks = lds + buf * LD::STAGE;
    uint16_t* vt = ks + LD::KELEMS;
#pragma unroll
    for (int r = 0; r < KPER; ++r) {
      const int c = threadIdx.x + r * kPfThreads;
      if (c < KCHUNKS) *reinterpret_cast<uint4*>(ks + (c / (D / 8)) * LD::KROW + (c % (D / 8)) * 8) = kreg[r];
    }
    const int t = threadIdx.x;
    if (t < VITEMS) {
      const int dg = t % (D / 4), kg = t / (D / 4);
      // 4 keys x 4 dims -> for each dim, the 4 keys side by side (V^T row).
      const uint32_t a0 = vreg[0].x, a1 = vreg[0].y, b0 = vreg[1].x, b1 = vreg[1].y;
      const uint32_t c0 = vreg[2].x, c1 = vreg[2].y, d0 = vreg[3].x, d1 = vreg[3].y;
      const uint2 col0 = make_uint2((a0 & 0xffffu) | (b0 << 16), (c0 & 0xffffu) | (d0 << 16));
      const uint2 col1 = make_uint2((a0 >> 16) | (b0 & 0xffff0000u), (c0 >> 16) | (d0 & 0xffff0000u));
      const uint2 col2 = make_uint2((a1 & 0xffffu) | (b1 << 16), (c1 & 0xffffu) | (d1 << 16));
      const uint2 col3 = make_uint2((a1 >> 16) | (b1 & 0xffff0000u), (c1 >> 16) | (d1 & 0xffff0000u));
      uint16_t* dst = vt + (4 * dg) * LD::VROW + 4 * kg;
      *reinterpret_cast<uint2*>(dst) = col0;
      *reinterpret_cast<uint2*>(dst + LD::VROW) = col1;
      *reinterpret_cast<uint2*>(dst + 2 * LD::VROW) = col2;
      *reinterpret_cast<uint2*>(dst + 3 * LD::VROW) = col3;
    }
  };

  floatx4_t o[NT][DTILES];
  float m[NT], lpart[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = kNegBig;
    lpart[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) o[nt][dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }

  // K row read by this lane in key half kt: key 8*(l16/4) + 4*kt + l16%4 of the tile.
  const int krow0 = 8 * (l16 >> 2) + (l16 & 3);

  if (ntiles > 0) fetch(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    stage(buf);
    __syncthreads();
    if (tile + 1 < ntiles) fetch(tile + 1);
    const uint16_t* ks = lds + buf * LD::STAGE;
    const uint16_t* vt = ks + LD::KELEMS;
    const int k0 = tile * kPfKeys;

    // S^T = K Q^T for both key halves and both q-row tiles.
    floatx4_t sacc[NT][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[nt][kt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const uint4 a = *reinterpret_cast<const uint4*>(ks + (krow0 + 4 * kt) * LD::KROW + 32 * s + 8 * blk);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sacc[nt][kt] = MM::mma(a, qf[nt][s], sacc[nt][kt]);
      }
    }

    // Online softmax per q-row; this lane holds keys 8*blk + 4*kt + i.
    const bool diag = k0 + kPfKeys - 1 > cached + q0;  // some key of the tile is past some row's limit
    uint4 pf[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float sv[2][4];
      float mx = kNegBig;
      const int limit = pos_of[nt] >= 0 ? cached + pos_of[nt] : -1;  // last visible key of this q-row
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[nt][kt][i] * scale_log2;
          if (diag && (k0 + 8 * blk + 4 * kt + i > limit)) v = -INFINITY;
          sv[kt][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[nt], mx);
      const float alpha = fast_exp2(m[nt] - mnew);
      m[nt] = mnew;
      float ps = 0.f;
      float p[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kt][i] = fast_exp2(sv[kt][i] - mnew);
          ps += p[kt][i];
        }
      lpart[nt] = lpart[nt] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) o[nt][dt] *= alpha;
      pf[nt] = make_uint4(MM::pack2(p[0][0], p[0][1]), MM::pack2(p[0][2], p[0][3]), MM::pack2(p[1][0], p[1][1]),
                          MM::pack2(p[1][2], p[1][3]));
    }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const uint4 a = *reinterpret_cast<const uint4*>(vt + (16 * dt + l16) * LD::VROW + 8 * blk);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt][dt] = MM::mma(a, pf[nt], o[nt][dt]);
    }
  }

  // Normalise and store: lane holds dims 16*dt + 4*blk + i of q-row l16 of tile nt.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = lpart[nt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (pos_of[nt] < 0) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int n = wave * kPfRowsPerWave + nt * 16 + l16;
    const int g = n % G;
    uint16_t* op = out + ((size_t)(qstart + pos_of[nt]) * num_q_heads + kvh * G + g) * D + 4 * blk;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const floatx4_t v = o[nt][dt] * inv;
      *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(MM::pack2(v[0], v[1]), MM::pack2(v[2], v[3]));
    }
  }
}

template <typename T, int D, int G>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  constexpr int BQ = kPfRows / G;
  const long long tiles = (long long)(a.num_q_tokens + BQ - 1) / BQ + a.num_seqs;
  if (tiles > 65535) return hipErrorInvalidValue;
  dim3 grid(a.num_kv_heads, (unsigned)tiles);
  hipLaunchKernelGGL((paged_prefill_kernel<T, D, G>), grid, dim3(kPfThreads), 0, stream, a.q, a.k_cache, a.v_cache,
                     a.block_tables, a.context_lens, a.query_start_loc, a.num_seqs, a.max_blocks_per_seq,
                     a.num_kv_heads, a.scale * kLog2e, a.out);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t stream) {
  switch (a.group) {
    case 1: return launch_prefill_t<T, D, 1>(a, stream);
    case 2: return launch_prefill_t<T, D, 2>(a, stream);
    case 4: return launch_prefill_t<T, D, 4>(a, stream);
    case 8: return launch_prefill_t<T, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

bool prefill_supported(bool bf16, int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.bf16) {
    if (a.head_dim == 64) return launch_prefill_g<BF16, 64>(a, stream);
    if (a.head_dim == 128) return launch_prefill_g<BF16, 128>(a, stream);
  } else {
    if (a.head_dim == 64) return launch_prefill_g<F16, 64>(a, stream);
    if (a.head_dim == 128) return launch_prefill_g<F16, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pka
