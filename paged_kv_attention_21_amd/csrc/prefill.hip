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
// Work items.  A query tile is 128 "q-rows" of one chunk and one KV head:
// 128 / G query positions times the G query heads of the GQA group, so every
// K/V tile staged in LDS serves all G heads.  The keys a query tile can see,
// [0, kend), are cut into splits of split_keys; one workgroup (4 wavefronts)
// takes one (KV head, query tile, split).  A tile with one split writes its
// output directly; otherwise every split leaves its unnormalised state (row
// max, exp-sum, O) in the workspace and a merge kernel combines them with the
// same max / exp-sum rule as the split-K decode.  Long chunks after a long
// cached prefix - the expensive ones - thereby spread over many compute units.
// Grid x is the KV head, so with 8 KV heads every tile of one head lands on the
// same XCD (workgroups are dealt to the 8 XCDs round robin) and its K/V tiles
// are shared through that XCD's L2.
//
// Inside a split the workgroup walks 64-key tiles, staged in LDS row-major
// (K and V alike, pieces swizzled per row) by buffer loads that write LDS
// directly, one tile ahead; a tile's physical blocks come from scalar loads of
// the block table, so their base addresses are wavefront-uniform (scalar
// registers).  Each wavefront owns 32 q-rows
// (two 16-row MFMA tiles; 16 q-rows at head size 256).
//
// Products (v_mfma_f32_16x16x32, fp32 accumulate):
//   S^T = K Q^T : A = 16 keys x 32 dims of K (LDS), B = Q^T fragment kept in
//                 registers for the whole split.  The C layout then gives each
//                 lane 4 keys of one q-row - exactly the lane's share of the
//                 B operand of the next product, so the softmax weights never
//                 leave registers.
//   O^T += V^T P^T : A = 16 dims x 32 keys of V^T, read from the row-major V
//                 tile with gfx950's transposing LDS read; B = P^T (registers,
//                 rounded to the input type).
// Both products only need the two operands to agree on which K index each
// (lane group, element) holds; the key order inside a tile is permuted so the
// 8 keys a lane needs in PV are 8 consecutive keys (two transposing reads).
//
// Numerics: logits in fp32, softmax in base 2 with scale * log2 e folded in,
// masked keys selected out (-inf logit; K/V rows past the context are zeroed in
// LDS so no NaN garbage reaches the products), fp32 accumulators, one
// normalisation at the end, round to nearest even on store.

#include <algorithm>

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
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return Elem<BF16>::pack2(lo, hi); }
  static constexpr uint32_t kOne2 = 0x3F803F80u;  // (1.0, 1.0)
};

template <>
struct Mfma<F16> {
  static __device__ __forceinline__ floatx4_t mma(const uint4& a, const uint4& b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8_t, a), __builtin_bit_cast(halfx8_t, b),
                                                  c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return Elem<F16>::pack2(lo, hi); }
  static constexpr uint32_t kOne2 = 0x3C003C00u;  // (1.0, 1.0)
};

#ifndef PKA_PREFILL_WAVES
#define PKA_PREFILL_WAVES 4
#endif
// Each wavefront owns 32 q-rows; all wavefronts of a workgroup share every
// staged K/V tile, so more wavefronts per tile means fewer K/V bytes pulled
// through L2 per MFMA flop (the kernel is bound by that traffic at 4 waves).
constexpr int kPfWaves = PKA_PREFILL_WAVES;
constexpr int kPfThreads = kPfWaves * kWave;  // threads of the merge kernel (and of the attention kernel, D <= 128)
constexpr int kPfRows = kPfWaves * 32;  // q-rows per query tile (positions x group heads)

// Attention-kernel geometry by head size.  Up to 128 dims a wavefront owns 32
// q-rows (two 16-row MFMA tiles); at 256 dims its output accumulators would
// take 128 registers, so a wavefront owns 16 q-rows and the workgroup has
// twice the wavefronts.  The query tile is kPfRows q-rows either way, which
// keeps the split state and the merge independent of the head size.
template <int D>
struct PfGeom {
  static constexpr int RPW = D == 256 ? 16 : 32;  // q-rows per wavefront
  static constexpr int WAVES = kPfRows / RPW;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int NT = RPW / 16;             // 16-row MFMA tiles per wavefront
  static_assert(THREADS <= 1024, "workgroup size");
};
// Wave priority around the MFMA stretches (s_setprio 1 while a wavefront
// issues its S or PV products, 0 for its softmax): the two wavefronts of a
// SIMD then tend to alternate - one issuing products back to back while the
// other fills the gaps with exp and conversion work - instead of contending
// for the same unit in the same phase.  Measured on the long prefill: 899 ->
// 968 TFLOP/s; raising only the S or only the PV stretch gains less, raising
// the softmax instead loses.
__device__ __forceinline__ void pf_prio_mfma() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void pf_prio_valu() { __builtin_amdgcn_s_setprio(0); }
constexpr int kPfKeys = 64;           // keys per staged tile (two 32-key halves)
// Word 3 of a raw buffer descriptor (gfx9 family: 32-bit data format, no
// swizzle, no stride).  Loads use offsets well inside num_records.
constexpr int kBufferFlags = 0x00020000;
constexpr float kPfSlack = 8.f;       // log2 growth of a row max tolerated before rescaling

// LDS tiles.  K and V rows are stored unpadded (D elements) and the 16-byte
// pieces of row r sit at piece index XOR pf_swz<D>(r), so that one wavefront's
// direct load (64 lanes x 16 bytes, written to 1 KB of consecutive LDS) fills
// whole rows.  gfx950's LDS serves a 16-byte read eight lanes per cycle and an
// 8-byte read sixteen lanes per cycle, from 64 four-byte banks; the swizzle
// spreads both read patterns of the kernel over distinct banks:
//  * K rows as the MFMA A operand: the eight lanes of a cycle read rows
//    {0, 1, 2, 3, 8, 9, 10, 11} (+ 16, + 4) at one piece index, so the eight
//    rows need distinct swizzles modulo 16 pieces;
//  * transposing V reads: the sixteen lanes of a cycle read rows
//    8 g + {0, 1, 2, 3} (+ 4), four lanes per row on a pair of adjacent
//    pieces, so the rows need distinct swizzles once halved.
// At 128 and 256 dims (16 or more pieces per row) the swizzle takes row bits
// 0, 1 to piece bits 1, 2 and row bit 3 to piece bit 3.  At 64 dims (eight
// pieces, two rows per 256 bytes) row bit 0 already picks the bank half, and
// the swizzle takes row bits 1 and 3 to piece bits 1 and 2.  Row bit 2 is
// left out, so K rows r and r + 4 share a swizzle.
template <int D>
struct PfLds {
  static_assert(D == 64 || D == 128 || D == 256, "supported head sizes");
  static constexpr int ROW = D;               // row stride in elements
  static constexpr int TILE = kPfKeys * ROW;  // one [64 keys][D] tile
  static constexpr int STAGE = 2 * TILE;      // K tile, then V tile
};
template <int D>
__device__ __forceinline__ int pf_swz(int row) {
  return D == 64 ? (row & 2) | ((row >> 1) & 4) : ((row & 3) << 1) | (row & 8);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// output lane i gets element i % 4 of the 8-byte pieces read by input lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4.  So when input lane L of group g
// reads row 8g + L / 4, columns 4 (L % 4) .. +3 of a row-major [key][dim]
// tile, output lane i holds keys 8g .. 8g + 3 of dim i: a column of V, i.e.
// four K-elements of the V^T MFMA operand.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef short short4v __attribute__((ext_vector_type(4)));
  const auto r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, r);
}

// Direct load of 16 bytes per lane from a buffer into LDS: lane i's bytes
// land at `lds` + 16 i (the LDS base is wavefront-uniform).
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rsrc, uint16_t* lds, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}

// Bytes of one split's saved state: O[128][D], then row max[128], exp-sum[128] (fp32).
__host__ __device__ constexpr size_t pf_slot_floats(int D) { return (size_t)kPfRows * (D + 2); }

// Find the chunk and the query tile of global tile index `tile` (tiles of
// `bq` positions, numbered chunk by chunk).  Every wavefront runs the same scan.
// Returns, besides the chunk and its query tile, the chunk's first row, row
// count and cached length, read in the same pass (one load round trip).
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens,
                                          int num_seqs, int bq, int tile, int* seq, int* qtile, int* qstart,
                                          int* qlen, int* cached) {
  const int lane = threadIdx.x & (kWave - 1);
  int before = 0;  // tiles of chunks already passed
  for (int base = 0; base < num_seqs; base += kWave) {
    const int s = base + lane;
    int n = 0, q0 = 0, ql = 0, cl = 0;
    if (s < num_seqs) {
      q0 = qsl[s];
      ql = qsl[s + 1] - q0;
      cl = context_lens[s];
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
      *qstart = __shfl(q0, first);
      *qlen = __shfl(ql, first);
      *cached = __shfl(cl - ql, first);
      return true;
    }
    before += __shfl(incl, kWave - 1);
  }
  return false;
}

// Geometry of one query tile, shared by the attention and merge kernels.
struct PfTile {
  int tile, seq, qt, qstart, qlen, cached, q0, kend, nsplit;  // tile: index in canonical order
};

__device__ __forceinline__ bool pf_tile(const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens,
                                        int num_seqs, int bq, int split_keys, int tile, PfTile* t) {
  int seq, qt, qstart, qlen, cached;
  if (!find_tile(qsl, context_lens, num_seqs, bq, tile, &seq, &qt, &qstart, &qlen, &cached)) return false;
  // Uniform across the wavefront: keep it (and all that follows) in scalar
  // registers so the loops and branches below are scalar-controlled.
  t->tile = tile;
  t->seq = __builtin_amdgcn_readfirstlane(seq);
  t->qt = __builtin_amdgcn_readfirstlane(qt);
  t->qstart = __builtin_amdgcn_readfirstlane(qstart);
  t->qlen = __builtin_amdgcn_readfirstlane(qlen);
  t->cached = __builtin_amdgcn_readfirstlane(cached);
  t->q0 = t->qt * bq;
  t->kend = t->cached + t->q0 + min(bq, t->qlen - t->q0);  // keys [0, kend) are visible to some row
  t->nsplit = (t->kend + split_keys - 1) / split_keys;
  return true;
}

// Heavy-first order of the (query tile, split) work items.  Workgroups start
// in grid order as slots free up, and an item with many key tiles that starts
// late sets the kernel's tail: in canonical order (tiles chunk by chunk) the
// last tiles of a chunk see the most keys, so on 4 chunks of 2,048 rows after
// 6,144 cached tokens they started last and ended ~60 us after the rest.  So
// grid row r takes the r-th item in decreasing order of its key tiles -
// kPfOrderBuckets buckets of that count over [1, split_keys / 64], equal
// buckets in canonical order (longest-processing-time-first list scheduling)
// - and the heaviest items of a mixed batch each start on their own compute
// unit.  Every workgroup derives the same order from query_start_loc and
// context_lens, in LDS scratch that the key tiles later overwrite.
constexpr int kPfOrderBuckets = kWave;
constexpr int kPfOrderMaxSeqs = 256;    // chunks the ordering handles; above, grid order is kept
// Query tiles likewise.  3,584 keeps the scratch (34 KB) within what a
// head-size-64 workgroup may take for three to share a compute unit.
constexpr int kPfOrderMaxTiles = 3584;

// Finds the item of rank `rank` and fills *t (as pf_tile) and *split; false
// when the batch has fewer items.  scratch: LDS for (4 kPfOrderMaxSeqs + 1 +
// 2 kPfOrderMaxTiles + kPfOrderBuckets + NT) ints; res: 8 ints of LDS apart
// from it.
//
// Every item is a full split (split_keys / 64 key tiles, bucket 0) except the
// last split of each query tile, which holds the tile's remaining keys.  The
// first wavefront lays out, per query tile, its split count and the key
// tiles of its last split (walking each chunk's tiles with running sums, no
// divisions); the workgroup builds the bucket histogram from that, the first
// wavefront finds the bucket holding `rank`, and a scan over per-thread runs
// of tiles finds the tile holding the item.
template <int NT>
__device__ bool pf_pick_item(const int32_t* __restrict__ qsl, const int32_t* __restrict__ context_lens,
                             int num_seqs, int bq, int split_keys, int rank, int* scratch, int* res, PfTile* t,
                             int* split) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  int* cached = scratch;                          // [kPfOrderMaxSeqs]
  int* qlen = cached + kPfOrderMaxSeqs;
  int* qstart = qlen + kPfOrderMaxSeqs;
  int* tile_start = qstart + kPfOrderMaxSeqs;     // [kPfOrderMaxSeqs + 1]
  int* tile_geo = tile_start + kPfOrderMaxSeqs + 1;  // [kPfOrderMaxTiles]: split count << 16 | last split's key tiles
  int* tile_chunk = tile_geo + kPfOrderMaxTiles;  // [kPfOrderMaxTiles]
  int* hist = tile_chunk + kPfOrderMaxTiles;      // [kPfOrderBuckets]
  int* part = hist + kPfOrderBuckets;             // [NT]
  const int max_w = (split_keys + kPfKeys - 1) / kPfKeys;
  // Buckets of width 2^sh over max_w - w, so that every weight lands in one.
  const int sh = max_w > kPfOrderBuckets ? 32 - __builtin_clz((unsigned)(max_w - 1)) - 6 : 0;
  auto bucket = [&](int w) { return min(kPfOrderBuckets - 1, (max_w - w) >> sh); };
  if (tid < kPfOrderBuckets) hist[tid] = 0;
  if (tid < kWave) {
    int before = 0;
    for (int base = 0; base < num_seqs; base += kWave) {
      const int c = base + lane;
      int n = 0, ql = 0, cach = 0;
      if (c < num_seqs) {
        const int q0 = qsl[c];
        ql = qsl[c + 1] - q0;
        cach = context_lens[c] - ql;
        qstart[c] = q0;
        qlen[c] = ql;
        cached[c] = cach;
        n = (ql + bq - 1) / bq;
      }
      int incl = n;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const int first = before + incl - n;
      before += __shfl(incl, kWave - 1);
      if (c < num_seqs) {
        tile_start[c] = first;
        if (before <= kPfOrderMaxTiles && n > 0) {
          // Tile i's keys end at cached + min((i + 1) bq, ql); rem = keys of
          // its last split, in (0, split_keys].
          int kend = cach + min(bq, ql);
          int ns = (kend + split_keys - 1) / split_keys;
          int rem = kend - (ns - 1) * split_keys;
          for (int i = 0; i < n; ++i) {
            tile_geo[first + i] = (ns << 16) | ((rem + kPfKeys - 1) / kPfKeys);
            tile_chunk[first + i] = c;
            const int step = min((i + 2) * bq, ql) - min((i + 1) * bq, ql);
            rem += step;
            while (rem > split_keys) {
              rem -= split_keys;
              ++ns;
            }
          }
        }
      }
    }
    if (lane == 0) tile_start[num_seqs] = before;
  }
  __syncthreads();
  const int total_tiles = tile_start[num_seqs];
  if (total_tiles > kPfOrderMaxTiles) return false;  // (the caller checks the bound first)
  for (int T = tid; T < total_tiles; T += NT) {
    const int g = tile_geo[T];
    if ((g >> 16) > 1) atomicAdd(&hist[0], (g >> 16) - 1);
    atomicAdd(&hist[bucket(g & 0xffff)], 1);
  }
  __syncthreads();
  // The bucket holding position `rank` (first wavefront); res[0] = bucket or
  // -1 past the last item, res[1] = position inside the bucket.
  if (tid < kWave) {
    const int cnt = hist[lane];
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const unsigned long long hit = __ballot(cnt > 0 && incl - cnt <= rank && rank < incl);
    if (lane == 0) res[0] = -1;
    if (hit) {
      const int k = __ffsll((long long)hit) - 1;
      if (lane == k) {
        res[0] = k;
        res[1] = rank - (incl - cnt);
      }
    }
  }
  __syncthreads();
  const int k = res[0];
  if (k < 0) return false;
  const int target = res[1];
  // Items of bucket k in canonical order (tiles in order, a tile's splits in
  // order): per tile, its full splits when k = 0, then its last split if it
  // falls in bucket k.  Each thread counts its run of tiles, a scan over the
  // runs finds the one holding the target, and its thread walks the run.
  auto n_in_k = [&](int g) { return (k == 0 ? (g >> 16) - 1 : 0) + (bucket(g & 0xffff) == k); };
  const int per = (total_tiles + NT - 1) / NT;
  const int T0 = min(total_tiles, tid * per), T1 = min(total_tiles, T0 + per);
  int cnt = 0;
  for (int T = T0; T < T1; ++T) cnt += n_in_k(tile_geo[T]);
  part[tid] = cnt;
  __syncthreads();
  if (tid < kWave) {
    int before = 0;
    for (int base = 0; base < NT; base += kWave) {
      const int v0 = part[base + lane];
      int incl = v0;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      part[base + lane] = before + incl - v0;
      before += __shfl(incl, kWave - 1);
    }
  }
  __syncthreads();
  if (cnt > 0 && part[tid] <= target && target < part[tid] + cnt) {
    int left = target - part[tid];
    for (int T = T0; T < T1; ++T) {
      const int g = tile_geo[T];
      const int n = n_in_k(g);
      if (left < n) {
        // The full splits come first (bucket 0 only), then the last split.
        const int sp = k == 0 ? left : (g >> 16) - 1;
        const int c = tile_chunk[T];
        res[0] = c;
        res[1] = T - tile_start[c];
        res[2] = sp;
        res[3] = qstart[c];
        res[4] = qlen[c];
        res[5] = cached[c];
        res[6] = T;
        break;
      }
      left -= n;
    }
  }
  __syncthreads();
  t->tile = __builtin_amdgcn_readfirstlane(res[6]);
  t->seq = __builtin_amdgcn_readfirstlane(res[0]);
  t->qt = __builtin_amdgcn_readfirstlane(res[1]);
  *split = __builtin_amdgcn_readfirstlane(res[2]);
  t->qstart = __builtin_amdgcn_readfirstlane(res[3]);
  t->qlen = __builtin_amdgcn_readfirstlane(res[4]);
  t->cached = __builtin_amdgcn_readfirstlane(res[5]);
  t->q0 = t->qt * bq;
  t->kend = t->cached + t->q0 + min(bq, t->qlen - t->q0);
  t->nsplit = (t->kend + split_keys - 1) / split_keys;
  return true;
}

// Wavefronts per SIMD the kernel is compiled for: two (a workgroup of four
// takes up to 200 registers a lane and 66 KB of LDS at head size 128, 128 KB
// at 256), three at head size 64 (136 registers, 50 KB: three workgroups per
// compute unit; measured 785 -> 872 TFLOP/s on the long prefill's chunks).
template <int D>
constexpr int pf_waves_per_simd() { return D == 64 ? 3 : 2; }

// BS = tokens per KV block (8, 16 or 32): a 64-key tile spans 64 / BS blocks.
template <typename T, int D, int G, int BS>
__global__ void __launch_bounds__(PfGeom<D>::THREADS)
    __attribute__((amdgpu_waves_per_eu(pf_waves_per_simd<D>(), pf_waves_per_simd<D>())))
paged_prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                     const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                     const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start_loc,
                     int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_kv_heads, int32_t split_keys,
                     int32_t max_splits, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ partial) {
  using MM = Mfma<T>;
  using EL = Elem<T>;
  constexpr uint32_t kOnes2 = MM::kOne2;
  const float slack_raw = kPfSlack / scale_log2;  // kPfSlack in raw score units
  using LD = PfLds<D>;
  constexpr int BQ = kPfRows / G;     // query positions per tile
  constexpr int KSTEPS = D / 32;      // MFMA k-steps of QK^T
  constexpr int DTILES = D / 16;      // 16-dim tiles of the output
  constexpr int NT = PfGeom<D>::NT;
  constexpr int RPW = PfGeom<D>::RPW;
  constexpr int THREADS = PfGeom<D>::THREADS;
  constexpr int KH = kPfKeys / 32;    // 32-key halves of a key tile

  // Two stages of (K, V) tiles, as two arrays: the compiler can then see that
  // the direct loads into one stage do not touch the stage being read, and
  // issues no wait for them before those reads.  The item ordering uses stage
  // 0's memory first.
  constexpr int kOrderElems = (4 * kPfOrderMaxSeqs + 1 + 2 * kPfOrderMaxTiles + kPfOrderBuckets + THREADS) * 2;
  __shared__ __attribute__((aligned(16))) uint16_t lds0[std::max(LD::STAGE, kOrderElems)];
  __shared__ __attribute__((aligned(16))) uint16_t lds1[LD::STAGE];

  const int kvh = blockIdx.x;
  // Grid row blockIdx.y is an item rank: heavy-first when the batch is small
  // enough for the ordering, else tile blockIdx.y / max_splits, split
  // blockIdx.y % max_splits.  (The host sizes the grid for the upper bound.)
  __shared__ int pick_res[8];
  PfTile tl;
  int split;
  if (num_seqs <= kPfOrderMaxSeqs && (int)gridDim.y / max(max_splits, 1) <= kPfOrderMaxTiles) {
    // (gridDim.y / max_splits bounds the batch's query tiles.)
    if (!pf_pick_item<THREADS>(query_start_loc, context_lens, num_seqs, BQ, split_keys, (int)blockIdx.y,
                               reinterpret_cast<int*>(lds0), pick_res, &tl, &split))
      return;
  } else {
    split = (int)blockIdx.y % max_splits;
    if (!pf_tile(query_start_loc, context_lens, num_seqs, BQ, split_keys, (int)blockIdx.y / max_splits, &tl)) return;
  }
  const int tile_id = tl.tile;
  if (split >= tl.nsplit) return;  // this tile sees fewer keys
  if (tl.nsplit > max_splits) return;  // context longer than max_context_len: precondition broken

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_id();
  const int l16 = lane & 15;
  const int blk = lane >> 4;
  const int num_q_heads = num_kv_heads * G;
  const int ctx = tl.cached + tl.qlen;
  const int k_lo = split * split_keys;
  const int k_hi = min(tl.kend, k_lo + split_keys);
  const int ntiles = (k_hi - k_lo + kPfKeys - 1) / kPfKeys;
  const size_t row_elems = (size_t)num_kv_heads * D;

  // The Q^T B-operand fragments stay in registers for the whole split: lane
  // (blk, l16) holds dims 32 s + 8 blk .. +7 of q-row l16 of row tile nt
  // (q-row n = position n / G, head n % G of the group; rows past the chunk
  // are zero).
  int pos_of[NT];
  uint4 qf[KSTEPS][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = wave * RPW + nt * 16 + l16;
    const int pos = tl.q0 + n / G;
    pos_of[nt] = pos < tl.qlen ? pos : -1;
    const uint16_t* qrow = q + ((size_t)(tl.qstart + (pos < tl.qlen ? pos : 0)) * num_q_heads + kvh * G + n % G) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qf[s][nt] = make_uint4(0, 0, 0, 0);
      if (pos < tl.qlen) qf[s][nt] = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * blk);
    }
  }

  // ---- global -> LDS staging of one key tile (direct loads) ----
  // Every 16-byte piece goes from memory straight into LDS: a buffer load that
  // writes LDS puts lane i's 16 bytes at the wavefront's LDS base + 16 i.
  // Wavefront w's r-th load covers the RPI = 64 / (D/8) consecutive tile rows
  // from RPI w + r ROWS_PER_PASS; lane i fills piece slot i % (D/8) of row
  // i / (D/8), so it loads that row's global piece slot ^ pf_swz(row).  A
  // wavefront's rows of one load never straddle a KV block, so the block is
  // wavefront-uniform: its base address sits in a buffer descriptor (scalar
  // registers) and each load adds the lane's constant 32-bit offset.
  constexpr int PPR = D / 8;                // 16-byte pieces per row
  constexpr int RPI = kWave / PPR;          // rows per wavefront load
  constexpr int CHUNKS = kPfKeys * PPR;     // pieces per tile
  static_assert(CHUNKS % THREADS == 0, "whole passes over the tile");
  constexpr int PER = CHUNKS / THREADS;     // loads per wavefront, tile and cache
  constexpr int ROWS_PER_PASS = THREADS / PPR;
  static_assert(BS % RPI == 0, "a wavefront's rows of one load lie in one KV block");
  const int my_row = threadIdx.x / PPR;     // row of pass 0
  const int my_slot = threadIdx.x % PPR;    // LDS piece slot this lane fills
  const size_t blk_elems = (size_t)BS * row_elems;
  // A block past the context is replaced by the context's last block (only
  // table entries inside the context are read): its rows come from memory the
  // sequence owns; V rows past the context are then zeroed, K rows there are
  // masked out of the scores.

  // The physical blocks come from the block table through scalar loads; each
  // block's base address goes into a buffer descriptor.  K and V of one tile
  // use the same blocks and the same lane offsets.
  const int32_t* __restrict__ tbl_row = block_tables + (size_t)tl.seq * max_blocks_per_seq;
  const int lb_last = (ctx - 1) / BS;  // last logical block inside the context
  // Byte offset of pass r's piece inside its block (the row's offset in the
  // block, then the head and the swizzled piece).
  uint32_t goff_bytes[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int row = my_row + r * ROWS_PER_PASS;
    goff_bytes[r] = (uint32_t)(((row % BS) * row_elems + (size_t)kvh * D + 8 * (my_slot ^ pf_swz<D>(row))) * 2);
  }
  const uint32_t blk_bytes = (uint32_t)(blk_elems * 2);
  // Physical blocks of this wavefront's loads of key tile `tile` (scalar
  // loads, issued a step before the loads that use them so their latency is
  // hidden behind a whole tile of work).
  auto lookup = [&](int tile, uint32_t (&pb)[PER]) {
    const int lb0 = (k_lo + tile * kPfKeys) / BS;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      // KV block of this load inside the tile: the same for the whole
      // wavefront, so it follows from the scalar wavefront index alone.
      const int blk_of = (wave * RPI + r * ROWS_PER_PASS) / BS;
      pb[r] = (uint32_t)tbl_row[min(lb0 + blk_of, lb_last)];
    }
  };
  // The K and V rows of the key tile whose blocks `lookup` put in `pb`, into
  // the stage at (kdst, vdst).
  auto load_tile = [&](const uint32_t (&pb)[PER], uint16_t* kdst, uint16_t* vdst) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const uint64_t off = (uint64_t)pb[r] * blk_bytes;
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(k_cache) + off), (short)0, 0x7fffffff, kBufferFlags);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(v_cache) + off), (short)0, 0x7fffffff, kBufferFlags);
      const int row0 = wave * RPI + r * ROWS_PER_PASS;  // the load's first row (wavefront-uniform)
      lds_load16(kr, kdst + row0 * LD::ROW, goff_bytes[r]);
      lds_load16(vr, vdst + row0 * LD::ROW, goff_bytes[r]);
    }
  };
  // Once this wavefront's loads of key tile `tile` have landed (vmcnt 0):
  // zero its V pieces of rows past the context, each lane the piece it loaded.
  auto finish_tile = [&](int tile, uint16_t* vdst) {
    const int k0 = k_lo + tile * kPfKeys;
    if (k0 + kPfKeys > ctx) {  // the context ends inside this tile
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int row = my_row + r * ROWS_PER_PASS;
        if (k0 + row >= ctx) *reinterpret_cast<uint4*>(vdst + row * LD::ROW + 8 * my_slot) = make_uint4(0, 0, 0, 0);
      }
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

  // K row read by this lane in key quarter kt of a 32-key half: key
  // 8*(l16/4) + 4*kt + l16%4 of the half; its pieces 4s + blk are swizzled by
  // ksw (the half's base row is a multiple of 32 and the swizzle leaves out
  // row bit 2, so both key quarters and both halves share it).
  const int krow0 = 8 * (l16 >> 2) + (l16 & 3);
  const int ksw = pf_swz<D>(krow0);

  auto qk = [&](const uint16_t* ks, floatx4_t (&sacc)[NT][2]) {
    // S^T = K Q^T over one 32-key half and both q-row tiles.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sacc[nt][0] = sacc[nt][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint4 a = *reinterpret_cast<const uint4*>(ks + (krow0 + 4 * kt) * LD::ROW +
                                                        8 * ((4 * s + blk) ^ ksw));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sacc[nt][kt] = MM::mma(a, qf[s][nt], sacc[nt][kt]);
      }
    }
  };

  // Online softmax per q-row, one 32-key half at a time; this lane holds keys
  // 8*blk + 4*kt + i of the half.  The running max m is kept in raw score
  // units (the scale is positive), so a weight is exp2(s * c - m * c) with
  // c = scale * log2(e): one fma and one exp per score.
  //
  // Part 1: causal mask (only on halves that reach the diagonal, a
  // wavefront-uniform test), row max, and the lazy rescale: the reference max
  // only moves when some row's max grows by more than kPfSlack in log2 units,
  // so the accumulators are rescaled on a handful of halves instead of on
  // every one; weights stay below 2^kPfSlack, harmless for fp32 sums and for
  // the (relative) bf16/fp16 rounding of P.
  auto row_max = [&](int k0, floatx4_t (&sacc)[NT][2]) {
    const bool diag = k0 + 31 > tl.cached + tl.q0;
    if (diag) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int limit = pos_of[nt] >= 0 ? tl.cached + pos_of[nt] : -1;  // last visible key of this q-row
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + 8 * blk + 4 * kt + i > limit) sacc[nt][kt][i] = -INFINITY;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const floatx4_t& s0 = sacc[nt][0];
      const floatx4_t& s1 = sacc[nt][1];
      // This lane's max over its 8 keys; only when some lane exceeds the slack
      // is the full row max (over the row's four lanes) formed and the row
      // rescaled, so the common half needs no cross-lane traffic.
      const float lmx = vmax(vmax3(vmax3(vmax3(s0[0], s0[1], s0[2]), s0[3], s1[0]), s1[1], s1[2]), s1[3]);
      if (__ballot(lmx > m[nt] + slack_raw)) {
        const float mx = xor32_max(xor16_max(lmx));
        const float mnew = fmaxf(m[nt], mx);
        const float alpha = fast_exp2((m[nt] - mnew) * scale_log2);
        m[nt] = mnew;
        lpart[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) o[nt][dt] *= alpha;
      }
    }
  };

  // Part 2, branch-free: weights, rounded to the input type, and their row sums
  // (of the rounded values, the ones the PV product uses).
  auto weights = [&](const floatx4_t (&sacc)[NT][2], uint4 (&pf)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mc = -m[nt] * scale_log2;
      float p[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[kt][i] = fast_exp2(__builtin_fmaf(sacc[nt][kt][i], scale_log2, mc));
      pf[nt] = make_uint4(MM::pack2(p[0][0], p[0][1]), MM::pack2(p[0][2], p[0][3]), MM::pack2(p[1][0], p[1][1]),
                          MM::pack2(p[1][2], p[1][3]));
      lpart[nt] = EL::dot2(pf[nt].x, kOnes2, lpart[nt]);
      lpart[nt] = EL::dot2(pf[nt].y, kOnes2, lpart[nt]);
      lpart[nt] = EL::dot2(pf[nt].z, kOnes2, lpart[nt]);
      lpart[nt] = EL::dot2(pf[nt].w, kOnes2, lpart[nt]);
    }
  };

  auto pv = [&](const uint16_t* vs, const uint4 (&pf)[NT]) {
    // O^T += V^T P^T over one 32-key half; the V^T operand (dims 16 dt + l16,
    // keys 8 blk .. +7) comes from the row-major V tile through two
    // transposing reads.  This lane reads rows 8 blk + l16/4 (+4 for the
    // upper half: the same swizzle), dims 16 dt + 4 (l16 % 4) .. +3, i.e.
    // piece 2 dt + (l16 % 4) / 2 at element 4 (l16 % 2).  The swizzle is
    // even, so the swizzled piece is 2 (dt ^ vh) + (l16 % 4) / 2.
    const int vh = pf_swz<D>(8 * blk + (l16 >> 2)) >> 1;
    const uint16_t* vrd = vs + (8 * blk + (l16 >> 2)) * LD::ROW + 8 * ((l16 & 3) >> 1) + 4 * (l16 & 1);
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const uint16_t* vp = vrd + 16 * (dt ^ vh);
      const uint2 lo = lds_read_tr16(vp);
      const uint2 hi = lds_read_tr16(vp + 4 * LD::ROW);
      const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt][dt] = MM::mma(a, pf[nt], o[nt][dt]);
    }
  };

  // Key tiles of 64 keys, double-buffered in LDS, one barrier per tile.  Step
  // t computes on tile t (both halves) while tile t+1 loads straight into the
  // other stage (free since the last barrier): the loads have the whole step
  // to land, and each wavefront waits for its own before the barrier that
  // hands the tile to the others.  Within the step the two halves are
  // interleaved so the softmax of one half can overlap the MFMAs of the
  // other: S of both halves, then softmax + PV of half 0, then softmax + PV
  // of half 1.
  const int last_tile = ntiles - 1;
  uint32_t pb_next[PER];  // blocks of the tile the next step loads
  if (ntiles > 0) {
    uint32_t pb0[PER];
    lookup(0, pb0);
    lookup(min(1, last_tile), pb_next);
    load_tile(pb0, lds0, lds0 + LD::TILE);
    __builtin_amdgcn_s_waitcnt(0);
    finish_tile(0, lds0 + LD::TILE);
    __syncthreads();
  }
  // (The stage pointers are restrict: once inlined, that tells the compiler
  // the direct loads into `next` do not alias the reads of `kt_lds`.)
  auto step = [&](int t, const uint16_t* __restrict__ kt_lds, uint16_t* __restrict__ next)
                  __attribute__((always_inline)) {
    const uint16_t* vt_lds = kt_lds + LD::TILE;
    const bool more = t < last_tile;  // wavefront-uniform
    if (more) {
      load_tile(pb_next, next, next + LD::TILE);
      lookup(min(t + 2, last_tile), pb_next);
    }
    // Scheduler hint: interleave the tile's MFMAs with its exp work (the
    // compiler's strategy for softmax-between-products loops).  Measured:
    // long prefill 1,012 -> 1,019-1,021 TFLOP/s, mixed-step prefill call
    // 40.1-40.3 -> 39.3 us; strategies 0 and 2 gain about the same.
    __builtin_amdgcn_iglp_opt(3);
    floatx4_t sh[KH][NT][2];
    pf_prio_mfma();
#pragma unroll
    for (int h = 0; h < KH; ++h) qk(kt_lds + h * 32 * LD::ROW, sh[h]);
    pf_prio_valu();
#pragma unroll
    for (int h = 0; h < KH; ++h) {
      uint4 pf[NT];
      row_max(k_lo + t * kPfKeys + 32 * h, sh[h]);
      weights(sh[h], pf);
      pf_prio_mfma();
      pv(vt_lds + h * 32 * LD::ROW, pf);
      pf_prio_valu();
    }
    // This wavefront's loads have landed (unconditional, so no load counts as
    // outstanding into the next step on any path).
    __builtin_amdgcn_s_waitcnt(0);
    if (more) finish_tile(t + 1, next + LD::TILE);
    __syncthreads();
  };
  // Even tiles sit in stage 0, odd tiles in stage 1.
  for (int t = 0; t < ntiles; t += 2) {
    step(t, lds0, lds1);
    if (t + 1 < ntiles) step(t + 1, lds1, lds0);
  }

  // Lane holds dims 16*dt + 4*blk + i of q-row l16 of tile nt.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = xor32_sum(xor16_sum(lpart[nt]));
    const int n = wave * RPW + nt * 16 + l16;
    if (tl.nsplit > 1) {
      // Unnormalised state of this split for the merge (invalid rows too: they are never stored).
      float* slot = partial + (((size_t)tile_id * max_splits + split) * num_kv_heads + kvh) * pf_slot_floats(D);
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt)
        *reinterpret_cast<floatx4_t*>(slot + (size_t)n * D + 16 * dt + 4 * blk) = o[nt][dt];
      if (blk == 0) {
        slot[(size_t)kPfRows * D + n] = m[nt] * scale_log2;  // log2 units for the merge
        slot[(size_t)kPfRows * D + kPfRows + n] = lt;
      }
      continue;
    }
    if (pos_of[nt] < 0) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int g = n % G;
    uint16_t* op = out + ((size_t)(tl.qstart + pos_of[nt]) * num_q_heads + kvh * G + g) * D + 4 * blk;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const floatx4_t v = o[nt][dt] * inv;
      *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(MM::pack2(v[0], v[1]), MM::pack2(v[2], v[3]));
    }
  }
}

// Merge the splits of every query tile that has more than one: per q-row,
// M = max_s m_s, w_s = exp2(m_s - M), out = sum_s w_s O_s / sum_s w_s l_s.
// One workgroup per (query tile, KV head, group of rows); D/8 threads per
// q-row, each owning one 16-byte output piece (8 dims), so every partial row is
// read as whole 16-byte pieces, and the split loop is unrolled so several
// splits' loads are in flight at once.  (Measured against eight threads per
// row with D/8 dims each: 8-14 % faster on the mixed step's merges, from twice
// the workgroups and half the dependent loads per thread.)
template <int D>
struct MgGeom {
  static constexpr int TPR = D / 8;              // threads per q-row
  static constexpr int ROWS = kPfThreads / TPR;  // q-rows per merge workgroup
  static_assert(kPfThreads % TPR == 0 && kPfRows % ROWS == 0, "merge geometry");
};

template <typename T, int D, int G>
__global__ void __launch_bounds__(kPfThreads)
paged_prefill_merge_kernel(const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start_loc,
                           int32_t num_seqs, int32_t num_kv_heads, int32_t split_keys, int32_t max_splits,
                           const float* __restrict__ partial, uint16_t* __restrict__ out) {
  constexpr int BQ = kPfRows / G;
  constexpr int kMgThreadsPerRow = MgGeom<D>::TPR;
  constexpr int kMgRows = MgGeom<D>::ROWS;
  constexpr int DPT = D / kMgThreadsPerRow;  // dims per thread
  constexpr int F4 = DPT / 4;
  constexpr int UNROLL = 4;
  static_assert(DPT % 8 == 0, "whole 16-byte output pieces");
  const int kvh = blockIdx.x;
  PfTile tl;
  if (!pf_tile(query_start_loc, context_lens, num_seqs, BQ, split_keys, blockIdx.y, &tl)) return;
  if (tl.nsplit <= 1 || tl.nsplit > max_splits) return;
  const int n = blockIdx.z * kMgRows + threadIdx.x / kMgThreadsPerRow;  // q-row in the tile
  const int d0 = (threadIdx.x % kMgThreadsPerRow) * DPT;
  const int pos = tl.q0 + n / G;
  if (pos >= tl.qlen) return;
  const int num_q_heads = num_kv_heads * G;
  const size_t slot_stride = (size_t)num_kv_heads * pf_slot_floats(D);
  const float* base = partial + ((size_t)blockIdx.y * max_splits * num_kv_heads + kvh) * pf_slot_floats(D);
  const float* mrow = base + (size_t)kPfRows * D + n;  // m of split s at mrow[s * slot_stride]
  const float* lrow = mrow + kPfRows;
  const int ns = tl.nsplit;

  // One pass over the splits, UNROLL at a time with all their loads in
  // flight: a running maximum rescales what has been accumulated, so the
  // maxima need no round trip of their own.
  float mm = kNegBig, lt = 0.f;
  floatx4_t acc[F4];
#pragma unroll
  for (int c = 0; c < F4; ++c) acc[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += UNROLL) {
    floatx4_t o[UNROLL][F4];
    float mu[UNROLL], lu[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int s = min(s0 + u, ns - 1);  // past the last split: reloads it, weighted 0 below
      const float* sl = base + (size_t)s * slot_stride;
      mu[u] = mrow[s * slot_stride];
      lu[u] = lrow[s * slot_stride];
#pragma unroll
      for (int c = 0; c < F4; ++c) o[u][c] = *reinterpret_cast<const floatx4_t*>(sl + (size_t)n * D + d0 + 4 * c);
    }
    float mnew = mm;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) mnew = fmaxf(mnew, mu[u]);
    const float sc = fast_exp2(mm - mnew);
    lt *= sc;
#pragma unroll
    for (int c = 0; c < F4; ++c) acc[c] *= sc;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const float wu = s0 + u < ns ? fast_exp2(mu[u] - mnew) : 0.f;
      lt += wu * lu[u];
#pragma unroll
      for (int c = 0; c < F4; ++c) acc[c] += wu * o[u][c];
    }
    mm = mnew;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* op = out + ((size_t)(tl.qstart + pos) * num_q_heads + kvh * G + n % G) * D + d0;
#pragma unroll
  for (int c = 0; c < F4 / 2; ++c) {
    const floatx4_t a = acc[2 * c] * inv, b = acc[2 * c + 1] * inv;
    *reinterpret_cast<uint4*>(op + 8 * c) = make_uint4(Mfma<T>::pack2(a[0], a[1]), Mfma<T>::pack2(a[2], a[3]),
                                                       Mfma<T>::pack2(b[0], b[1]), Mfma<T>::pack2(b[2], b[3]));
  }
}

size_t prefill_tiles_upper_bound(int num_q_tokens, int num_seqs, int group) {
  const int bq = kPfRows / group;
  return (size_t)(num_q_tokens + bq - 1) / bq + num_seqs;
}

// Keys per split.  Splitting a query tile's key range buys parallelism at
// the price of writing and merging a partial state per split, so it is used
// only to fill the GPU: the number of (query tile, KV head) work items is
// multiplied by the smallest split count that gives about two rounds of
// resident workgroups per compute unit (four items up to 128 dims, two at 256
// dims, whose workgroups take a whole compute unit's LDS), and no split is
// shorter than kPfMinSplitKeys keys.  Batches with enough query tiles are not split at all.
// The host sees only the longest context, not how the work spreads over the
// chunks: when one long chunk shares a batch with short ones, its splits set
// the critical path, so splits are held to kPfCapSplitKeys keys unless that
// would more than double the work-item target (a batch of uniformly long
// chunks, where longer splits cost less than the extra partial states).
int prefill_split_keys(int num_q_tokens, int num_seqs, int num_kv_heads, int group, int head_dim,
                       int max_context_len, int num_cus) {
  const size_t items = prefill_tiles_upper_bound(num_q_tokens, num_seqs, group) * (size_t)num_kv_heads;
  const size_t per_cu = head_dim > 128 ? 2 : 4;  // two rounds of the workgroups one compute unit holds
  const size_t target = per_cu * (size_t)(num_cus > 0 ? num_cus : 256);
  size_t s = items >= target ? 1 : (target + items - 1) / items;
  s = std::min(s, (size_t)std::max(1, (max_context_len + kPfMinSplitKeys - 1) / kPfMinSplitKeys));
  int keys = (int)(((size_t)max_context_len + s - 1) / s);
  const size_t capped_splits = ((size_t)max_context_len + kPfCapSplitKeys - 1) / kPfCapSplitKeys;
  if (s > 1 && keys > kPfCapSplitKeys && items * capped_splits <= 2 * target) keys = kPfCapSplitKeys;
  return std::max(kPfKeys, (keys + kPfKeys - 1) / kPfKeys * kPfKeys);
}

size_t prefill_workspace_floats(int num_q_tokens, int num_seqs, int num_kv_heads, int group, int head_dim,
                                int max_context_len, int split_keys) {
  const size_t splits = (size_t)(max_context_len + split_keys - 1) / split_keys;
  if (splits <= 1) return 0;
  return prefill_tiles_upper_bound(num_q_tokens, num_seqs, group) * splits * num_kv_heads * pf_slot_floats(head_dim);
}

template <typename T, int D, int G, int BS>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  const size_t tiles = prefill_tiles_upper_bound(a.num_q_tokens, a.num_seqs, G);
  if (a.split_keys <= 0 || a.split_keys % kPfKeys) return hipErrorInvalidValue;
  const int splits = (a.max_context_len + a.split_keys - 1) / a.split_keys;
  if (tiles > 65535 || splits > 65535) return hipErrorInvalidValue;
  // One grid row per (query tile, split) item slot; rows past the batch's
  // items exit at once.
  if (tiles * (size_t)splits > 65535) return hipErrorInvalidValue;
  dim3 grid(a.num_kv_heads, (unsigned)(tiles * splits));
  hipLaunchKernelGGL((paged_prefill_kernel<T, D, G, BS>), grid, dim3(PfGeom<D>::THREADS), 0, stream, a.q, a.k_cache, a.v_cache,
                     a.block_tables, a.context_lens, a.query_start_loc, a.num_seqs, a.max_blocks_per_seq,
                     a.num_kv_heads, a.split_keys, splits, a.scale * kLog2e, a.out, a.workspace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits <= 1) return e;
  hipLaunchKernelGGL((paged_prefill_merge_kernel<T, D, G>), dim3(a.num_kv_heads, (unsigned)tiles, kPfRows / MgGeom<D>::ROWS),
                     dim3(kPfThreads),
                     0, stream, a.context_lens, a.query_start_loc, a.num_seqs, a.num_kv_heads, a.split_keys, splits,
                     a.workspace, a.out);
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t launch_prefill_b(const PrefillArgs& a, hipStream_t stream) {
  switch (a.block_size) {
    case 8: return launch_prefill_t<T, D, G, 8>(a, stream);
    case 16: return launch_prefill_t<T, D, G, 16>(a, stream);
    case 32: return launch_prefill_t<T, D, G, 32>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t stream) {
  switch (a.group) {
    case 1: return launch_prefill_b<T, D, 1>(a, stream);
    case 2: return launch_prefill_b<T, D, 2>(a, stream);
    case 4: return launch_prefill_b<T, D, 4>(a, stream);
    case 8: return launch_prefill_b<T, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

bool prefill_supported(bool bf16, int head_dim, int group, int block_size) {
  return (head_dim == 64 || head_dim == 128 || head_dim == 256) && (group == 1 || group == 2 || group == 4 || group == 8) &&
         (block_size == 8 || block_size == 16 || block_size == 32);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.bf16) {
    if (a.head_dim == 64) return launch_prefill_g<BF16, 64>(a, stream);
    if (a.head_dim == 128) return launch_prefill_g<BF16, 128>(a, stream);
    if (a.head_dim == 256) return launch_prefill_g<BF16, 256>(a, stream);
  } else {
    if (a.head_dim == 64) return launch_prefill_g<F16, 64>(a, stream);
    if (a.head_dim == 128) return launch_prefill_g<F16, 128>(a, stream);
    if (a.head_dim == 256) return launch_prefill_g<F16, 256>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pka
