// C ABI of the paged-attention library: argument checks (host only, before
// any launch), the decode dispatcher, and the launches on the caller's stream.
// The operations are defined in include/pka.h.

#include "pka.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <climits>
#include <cstdint>
#include <mutex>

#include "launch.h"

// Library-owned scratch of the allocation-free decode entry point
// (pka_paged_attn_decode_noalloc): the split-K counter header and partition
// states live here instead of in a caller's workspace.  Every device the
// library runs on holds its own copy until the process ends.  It starts
// zeroed, so the counter header starts at zero, and every call leaves the
// counters at zero.  Host code never passes the array's name to a kernel (on
// the host it only stands in for the symbol): its device address is looked up
// per device below.
static __device__ __align__(256) unsigned char scratch[PKA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_cu_count[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int32_t elem_size(int32_t dtype) { return 2; }

// Shape checks common to every call that reads the pool.
int32_t check_cache(const pka_cache_desc& c) {
  if (c.num_blocks <= 0 || c.block_size <= 0 || c.num_kv_heads <= 0 || c.head_dim <= 0) return PKA_ERR_SHAPE;
  if (c.dtype != PKA_F16 && c.dtype != PKA_BF16) return PKA_ERR_UNSUPPORTED;
  if (c.block_size != 8 && c.block_size != 16 && c.block_size != 32) return PKA_ERR_UNSUPPORTED;
  if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256) return PKA_ERR_UNSUPPORTED;
  return PKA_OK;
}

int32_t check_group(int32_t num_q_heads, int32_t num_kv_heads, int32_t* group) {
  if (num_q_heads <= 0) return PKA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads) return PKA_ERR_SHAPE;
  const int32_t g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return PKA_ERR_UNSUPPORTED;
  *group = g;
  return PKA_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? PKA_OK : PKA_ERR_HIP; }

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int32_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKA_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKA_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKA_OK;
}

int32_t num_partitions(int32_t max_context_len) {
  return (max_context_len + pka::kPartitionSize - 1) / pka::kPartitionSize;
}

// Shared checks of the decode entry points; fills `a` on success.
int32_t prepare_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_blocks_per_seq, float scale, const pka_cache_desc& cache,
                       pka::DecodeArgs* a) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PKA_ERR_NULL;
  int32_t st = check_cache(cache);
  if (st) return st;
  int32_t group = 0;
  st = check_group(num_q_heads, cache.num_kv_heads, &group);
  if (st) return st;
  if (max_blocks_per_seq <= 0) return PKA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKA_ERR_ALIGN;
  *a = pka::DecodeArgs{};
  a->q = static_cast<const uint16_t*>(q);
  a->k_cache = static_cast<const uint16_t*>(k_cache);
  a->v_cache = static_cast<const uint16_t*>(v_cache);
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->num_seqs = num_seqs;
  a->num_kv_heads = cache.num_kv_heads;
  a->group = group;
  a->head_dim = cache.head_dim;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->block_size = cache.block_size;
  // The single-pass kernel runs sequences longest first, bucketed against an
  // upper bound of the context length (the table width unless the caller
  // gives a tighter one).
  a->order_max_ctx = (int32_t)std::min<int64_t>((int64_t)max_blocks_per_seq * cache.block_size, INT32_MAX);
  a->scale = scale;
  a->bf16 = cache.dtype == PKA_BF16;
  a->num_cus = std::max<int32_t>(0, pka_device_cu_count());
  return PKA_OK;
}

int32_t splitk_into(pka::DecodeArgs& a, int32_t P, char* workspace, hipStream_t s);

// Dispatched decode (single pass, or split-K + reduce); new_k / new_v non-null
// append one token per sequence (pka_paged_attn_decode_append).
int32_t decode_dispatch(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                        int32_t max_blocks_per_seq, int32_t max_context_len, float scale, void* out,
                        const pka_cache_desc& cache, void* workspace, size_t workspace_bytes, void* stream,
                        const void* new_k, const void* new_v) {
  if (num_seqs < 0 || max_context_len < 0) return PKA_ERR_SHAPE;
  if (num_seqs == 0) return PKA_OK;
  if (max_context_len == 0) return PKA_ERR_SHAPE;
  pka::DecodeArgs a;
  int32_t st = prepare_decode(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                              max_blocks_per_seq, scale, cache, &a);
  if (st) return st;
  if (!out) return PKA_ERR_NULL;
  if (!aligned16(out)) return PKA_ERR_ALIGN;
  if (num_seqs > 65535) return PKA_ERR_UNSUPPORTED;
  a.out = static_cast<uint16_t*>(out);
  a.order_max_ctx = max_context_len;
  a.max_context_len = max_context_len;
  if (new_k) {
    a.new_k = static_cast<const uint16_t*>(new_k);
    a.new_v = static_cast<const uint16_t*>(new_v);
    a.k_store = static_cast<uint16_t*>(const_cast<void*>(k_cache));
    a.v_store = static_cast<uint16_t*>(const_cast<void*>(v_cache));
  }
  const int32_t cus = pka_device_cu_count();
  const int32_t variant = pka_decode_choose_variant(num_seqs, cache.num_kv_heads, max_context_len, cus);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (variant == 1) return hip_status(pka::launch_decode(a, pka::kLaunchSingle, s));

  const int32_t P = num_partitions(max_context_len);
  if (P > 65535) return PKA_ERR_UNSUPPORTED;
  const size_t need = pka_splitk_workspace_bytes(num_seqs, num_q_heads, cache.head_dim, max_context_len);
  if (!workspace || workspace_bytes < need) return PKA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PKA_ERR_ALIGN;
  return splitk_into(a, P, static_cast<char*>(workspace), s);
}

int32_t splitk_into(pka::DecodeArgs& a, int32_t P, char* w, hipStream_t s) {
  // Workspace: the counter header, then tmp_out, max_logits, exp_sums.
  const size_t rows = (size_t)a.num_seqs * a.num_kv_heads * a.group * P;
  a.max_num_partitions = P;
  a.counters = reinterpret_cast<uint32_t*>(w);
  w += pka::kSplitCounterBytes;
  a.tmp_out = reinterpret_cast<float*>(w);
  a.max_logits = reinterpret_cast<float*>(w + align256(rows * a.head_dim * sizeof(float)));
  a.exp_sums = reinterpret_cast<float*>(w + align256(rows * a.head_dim * sizeof(float)) +
                                        align256(rows * sizeof(float)));
  // One launch when the counters fit the header; else partitions + reduce.
  if ((int64_t)a.num_seqs * a.num_kv_heads <= pka::kSplitCounterSlots)
    return hip_status(pka::launch_decode(a, pka::kLaunchSplitFused, s));
  hipError_t e = pka::launch_decode(a, pka::kLaunchSplit, s);
  if (e != hipSuccess) return PKA_ERR_HIP;
  pka::ReduceArgs r{};
  r.tmp_out = a.tmp_out;
  r.max_logits = a.max_logits;
  r.exp_sums = a.exp_sums;
  r.context_lens = a.context_lens;
  r.num_seqs = a.num_seqs;
  r.num_q_heads = a.num_kv_heads * a.group;
  r.head_dim = a.head_dim;
  r.partition_size = pka::kPartitionSize;
  r.max_num_partitions = P;
  r.bf16 = a.bf16;
  r.out = a.out;
  return hip_status(pka::launch_splitk_reduce(r, s));
}


}  // namespace

extern "C" {

const char* pka_status_str(int32_t status) {
  switch (status) {
    case PKA_OK: return "ok";
    case PKA_ERR_NULL: return "null pointer argument";
    case PKA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case PKA_ERR_UNSUPPORTED: return "shape or dtype not supported by this library";
    case PKA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case PKA_ERR_WORKSPACE: return "split-K workspace missing or too small";
    case PKA_ERR_HIP: return "HIP runtime error";
    case PKA_ERR_SCRATCH: return "request needs more split-K scratch than the library's built-in array holds";
  }
  return "unknown status";
}

int32_t pka_version(void) { return 100; }

int32_t pka_device_cu_count(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev < 0 || dev >= kMaxDevices) return -1;
  int32_t n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return -1;
  g_cu_count[dev].store(v, std::memory_order_relaxed);
  return v;
}

int32_t pka_kv_cache_write(const void* key, const void* value, const int64_t* slot_mapping, int32_t num_tokens,
                           void* k_cache, void* v_cache, pka_cache_desc cache, void* stream) {
  if (num_tokens < 0) return PKA_ERR_SHAPE;
  int32_t st = check_cache(cache);
  if (st) return st;
  if (num_tokens == 0) return PKA_OK;
  if (!key || !value || !slot_mapping || !k_cache || !v_cache) return PKA_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache)) return PKA_ERR_ALIGN;
  pka::KvWriteArgs a{};
  a.key = key;
  a.value = value;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.row_bytes = cache.num_kv_heads * cache.head_dim * elem_size(cache.dtype);
  a.num_slots = (int64_t)cache.num_blocks * cache.block_size;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  return hip_status(pka::launch_kv_write(a, static_cast<hipStream_t>(stream)));
}

int32_t pka_rope_table(float* table, int32_t max_position, int32_t head_dim, double theta, void* stream) {
  if (max_position < 0 || head_dim <= 0 || head_dim % 16) return PKA_ERR_SHAPE;
  if (!(theta > 1.0) || !std::isfinite(theta)) return PKA_ERR_SHAPE;
  if (max_position == 0) return PKA_OK;
  if (!table) return PKA_ERR_NULL;
  if (!aligned16(table)) return PKA_ERR_ALIGN;
  return hip_status(pka::launch_rope_table(table, max_position, head_dim, theta, static_cast<hipStream_t>(stream)));
}

size_t pka_rope_table_bytes(int32_t max_position, int32_t head_dim) {
  if (max_position <= 0 || head_dim <= 0) return 0;
  return (size_t)max_position * (size_t)head_dim * sizeof(float);
}

int32_t pka_fused_rope_kv_write(const void* qkv, int64_t qkv_row_stride, const int64_t* positions,
                                const int64_t* slot_mapping, int32_t num_tokens, int32_t num_q_heads,
                                const float* rope_table, int32_t max_position, void* q_out, void* k_cache,
                                void* v_cache, pka_cache_desc cache, void* stream) {
  if (num_tokens < 0 || max_position <= 0) return PKA_ERR_SHAPE;
  int32_t st = check_cache(cache);
  if (st) return st;
  if (cache.head_dim % 16) return PKA_ERR_UNSUPPORTED;
  if (num_q_heads <= 0) return PKA_ERR_SHAPE;
  const int64_t row = (int64_t)(num_q_heads + 2 * cache.num_kv_heads) * cache.head_dim;
  if (qkv_row_stride < row || (qkv_row_stride * elem_size(cache.dtype)) % 16) return PKA_ERR_SHAPE;
  if (num_tokens == 0) return PKA_OK;
  if (!qkv || !positions || !slot_mapping || !rope_table || !q_out || !k_cache || !v_cache) return PKA_ERR_NULL;
  if (!aligned16(qkv) || !aligned16(rope_table) || !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKA_ERR_ALIGN;
  pka::RopeKvArgs a{};
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.row_stride = qkv_row_stride;
  a.positions = positions;
  a.slot_mapping = slot_mapping;
  a.table = rope_table;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache.num_kv_heads;
  a.head_dim = cache.head_dim;
  a.max_position = max_position;
  a.num_slots = (int64_t)cache.num_blocks * cache.block_size;
  a.bf16 = cache.dtype == PKA_BF16;
  a.q_out = static_cast<uint16_t*>(q_out);
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  return hip_status(pka::launch_rope_kv_write(a, static_cast<hipStream_t>(stream)));
}

int32_t pka_paged_attn_decode_v1(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_blocks_per_seq, float scale, void* out,
                                 pka_cache_desc cache, void* stream) {
  if (num_seqs < 0) return PKA_ERR_SHAPE;
  if (num_seqs == 0) return PKA_OK;
  pka::DecodeArgs a;
  int32_t st = prepare_decode(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                              max_blocks_per_seq, scale, cache, &a);
  if (st) return st;
  if (!out) return PKA_ERR_NULL;
  if (!aligned16(out)) return PKA_ERR_ALIGN;
  if (num_seqs > 65535) return PKA_ERR_UNSUPPORTED;
  a.out = static_cast<uint16_t*>(out);
  return hip_status(pka::launch_decode(a, pka::kLaunchSingle, static_cast<hipStream_t>(stream)));
}

int32_t pka_paged_attn_decode_splitk(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t max_blocks_per_seq, float scale,
                                     int32_t partition_size, int32_t max_num_partitions, float* tmp_out,
                                     float* max_logits, float* exp_sums, pka_cache_desc cache, void* stream) {
  if (num_seqs < 0 || max_num_partitions < 0) return PKA_ERR_SHAPE;
  if (num_seqs == 0) return PKA_OK;
  if (partition_size != pka::kPartitionSize) return PKA_ERR_UNSUPPORTED;
  pka::DecodeArgs a;
  int32_t st = prepare_decode(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                              max_blocks_per_seq, scale, cache, &a);
  if (st) return st;
  if (max_num_partitions == 0) return PKA_ERR_SHAPE;
  if (!tmp_out || !max_logits || !exp_sums) return PKA_ERR_WORKSPACE;
  if (num_seqs > 65535 || max_num_partitions > 65535) return PKA_ERR_UNSUPPORTED;
  a.max_num_partitions = max_num_partitions;
  a.tmp_out = tmp_out;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  return hip_status(pka::launch_decode(a, pka::kLaunchSplit, static_cast<hipStream_t>(stream)));
}

int32_t pka_paged_attn_splitk_reduce(const float* tmp_out, const float* max_logits, const float* exp_sums,
                                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t head_dim, int32_t partition_size, int32_t max_num_partitions,
                                     void* out, int32_t dtype, void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || max_num_partitions <= 0) return PKA_ERR_SHAPE;
  if (num_seqs == 0) return PKA_OK;
  if (!tmp_out || !max_logits || !exp_sums || !context_lens || !out) return PKA_ERR_NULL;
  if (dtype != PKA_F16 && dtype != PKA_BF16) return PKA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PKA_ERR_UNSUPPORTED;
  if (partition_size != pka::kPartitionSize) return PKA_ERR_UNSUPPORTED;
  if (num_seqs > 65535) return PKA_ERR_UNSUPPORTED;
  pka::ReduceArgs a{};
  a.tmp_out = tmp_out;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.head_dim = head_dim;
  a.partition_size = partition_size;
  a.max_num_partitions = max_num_partitions;
  a.bf16 = dtype == PKA_BF16;
  a.out = static_cast<uint16_t*>(out);
  return hip_status(pka::launch_splitk_reduce(a, static_cast<hipStream_t>(stream)));
}

size_t pka_splitk_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const size_t rows = (size_t)num_seqs * num_q_heads * num_partitions(max_context_len);
  return pka::kSplitCounterBytes + align256(rows * head_dim * sizeof(float)) + 2 * align256(rows * sizeof(float));
}

int32_t pka_decode_choose_variant(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                  int32_t num_cus) {
  // Nothing to split in a single partition.
  if (max_context_len <= pka::kPartitionSize) return 1;
  if (num_cus <= 0) num_cus = 256;
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  // At least two (sequence, KV head) workgroups per CU, and no context so long
  // that one workgroup's tail dominates: single pass.  (Measured on 256 CUs:
  // 64 x 8 workgroups with contexts up to 2,048 run about as fast single-pass
  // as split, without the partial-result traffic and the reduce launch.)
  if (units >= 2 * (int64_t)num_cus && max_context_len <= 4096) return 1;
  return 2;
}

int32_t pka_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_blocks_per_seq, int32_t max_context_len, float scale, void* out,
                              pka_cache_desc cache, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_dispatch(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, max_blocks_per_seq,
                         max_context_len, scale, out, cache, workspace, workspace_bytes, stream, nullptr, nullptr);
}

int32_t pka_paged_attn_decode_append(const void* q, const void* key, const void* value, void* k_cache,
                                     void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                     int32_t max_context_len, float scale, void* out, pka_cache_desc cache,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!key || !value)) return PKA_ERR_NULL;
  if (num_seqs > 0 && (!aligned16(key) || !aligned16(value))) return PKA_ERR_ALIGN;
  return decode_dispatch(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, max_blocks_per_seq,
                         max_context_len, scale, out, cache, workspace, workspace_bytes, stream, key, value);
}

int32_t pka_paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, void* out, pka_cache_desc cache, void* stream) {
  if (num_seqs < 0 || max_context_len < 0) return PKA_ERR_SHAPE;
  if (num_seqs == 0) return PKA_OK;
  if (max_context_len == 0 || cache.num_kv_heads <= 0) return PKA_ERR_SHAPE;
  const int32_t variant = pka_decode_choose_variant(num_seqs, cache.num_kv_heads, max_context_len,
                                                    pka_device_cu_count());
  void* ws = nullptr;
  if (variant == 2) {
    if (pka_splitk_workspace_bytes(num_seqs, num_q_heads, cache.head_dim, max_context_len) >
        (size_t)PKA_NOALLOC_SCRATCH_BYTES)
      return PKA_ERR_SCRATCH;
    const int32_t st = scratch_address(&ws);
    if (st) return st;
  }
  return decode_dispatch(q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, max_blocks_per_seq,
                         max_context_len, scale, out, cache, ws, ws ? (size_t)PKA_NOALLOC_SCRATCH_BYTES : 0, stream,
                         nullptr, nullptr);
}

size_t pka_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_tokens, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len <= 0 || num_q_heads % num_kv_heads)
    return 0;
  const int group = num_q_heads / num_kv_heads;
  const int keys = pka::prefill_split_keys(num_q_tokens, num_seqs, num_kv_heads, group, head_dim, max_context_len,
                                           pka_device_cu_count());
  return pka::prefill_workspace_floats(num_q_tokens, num_seqs, num_kv_heads, group, head_dim, max_context_len, keys) *
         sizeof(float);
}

int32_t pka_prefill_split_keys(int32_t num_seqs, int32_t num_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len <= 0 || num_q_heads % num_kv_heads)
    return -1;
  return pka::prefill_split_keys(num_q_tokens, num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim,
                                 max_context_len, pka_device_cu_count());
}

int32_t pka_paged_attn_prefill(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_seqs,
                               int32_t num_q_tokens, int32_t max_query_len, int32_t max_context_len,
                               int32_t num_q_heads, int32_t max_blocks_per_seq, float scale, void* out,
                               pka_cache_desc cache, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || num_q_tokens < 0 || max_query_len < 0 || max_context_len < 0) return PKA_ERR_SHAPE;
  if (num_seqs == 0 || num_q_tokens == 0) return PKA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc || !out)
    return PKA_ERR_NULL;
  int32_t st = check_cache(cache);
  if (st) return st;
  int32_t group = 0;
  st = check_group(num_q_heads, cache.num_kv_heads, &group);
  if (st) return st;
  if (max_blocks_per_seq <= 0 || max_query_len == 0 || max_query_len > num_q_tokens) return PKA_ERR_SHAPE;
  if (max_context_len < max_query_len) return PKA_ERR_SHAPE;
  if (!pka::prefill_supported(cache.dtype == PKA_BF16, cache.head_dim, group, cache.block_size))
    return PKA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return PKA_ERR_UNSUPPORTED;  // the running max assumes scale > 0
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PKA_ERR_ALIGN;
  const size_t need = pka_prefill_workspace_bytes(num_seqs, num_q_tokens, num_q_heads, cache.num_kv_heads,
                                                  cache.head_dim, max_context_len);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return PKA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PKA_ERR_ALIGN;
  }
  pka::PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = num_seqs;
  a.num_q_tokens = num_q_tokens;
  a.max_query_len = max_query_len;
  a.max_context_len = max_context_len;
  a.num_kv_heads = cache.num_kv_heads;
  a.group = group;
  a.head_dim = cache.head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = cache.block_size;
  a.scale = scale;
  a.bf16 = cache.dtype == PKA_BF16;
  a.out = static_cast<uint16_t*>(out);
  a.split_keys = pka::prefill_split_keys(num_q_tokens, num_seqs, cache.num_kv_heads, group, cache.head_dim,
                                         max_context_len, pka_device_cu_count());
  a.workspace = need > 0 ? static_cast<float*>(workspace) : nullptr;
  return hip_status(pka::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
