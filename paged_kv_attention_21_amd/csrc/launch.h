// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pka {

// Split-K partition length in tokens (one partition = 16 KV blocks).
constexpr int kPartitionSize = 256;

// The dispatched split-K decode runs as one launch: the partitions of each
// (sequence, KV head) are counted as they finish, and the last one merges
// them.  The counters sit in a fixed header at the start of the workspace
// (so partial results of a call with other sizes never land on them); every
// call leaves them at zero.  Batches with more (sequence, KV head) pairs than
// the header holds take the two-launch path (partitions, then the reduce).
constexpr int kSplitCounterSlots = 16384;
constexpr size_t kSplitCounterBytes = kSplitCounterSlots * sizeof(uint32_t);

// Launch forms of the decode kernels (see decode_impl.h).
constexpr int kLaunchSingle = 0;
constexpr int kLaunchSplit = 1;
constexpr int kLaunchSplitFused = 2;

// Keys per prefill split: a query tile that sees more keys is spread over
// several workgroups whose states are merged afterwards.
// Shortest key range a prefill split is given (four 64-key tiles), and the
// split length held to in mixed batches (see prefill_split_keys).
constexpr int kPfMinSplitKeys = 256;
constexpr int kPfCapSplitKeys = 1024;

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t group;  // query heads per KV head
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t block_size;          // tokens per KV block: 8, 16 or 32
  int32_t max_num_partitions;  // split-K only
  int32_t max_context_len;     // upper bound of context_lens (0 if unknown)
  int32_t order_max_ctx;       // single pass: > 0 runs sequences longest first (bucketed by this bound)
  int32_t num_cus;             // compute units of the device (0 if unknown)
  float scale;
  bool bf16;
  uint16_t* out;     // single pass only
  float* tmp_out;    // split-K only
  float* max_logits;
  float* exp_sums;
  uint32_t* counters;  // single-launch split-K: one per (sequence, KV head), zero before the launch
  // Appended token (pka_paged_attn_decode_append): rows [num_seqs][kv heads][D]
  // stored at position context_lens[s] - 1 and attended from registers; null otherwise.
  const uint16_t* new_k;
  const uint16_t* new_v;
  uint16_t* k_store;  // the caches again, writable
  uint16_t* v_store;
};

struct ReduceArgs {
  const float* tmp_out;
  const float* max_logits;
  const float* exp_sums;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t partition_size;
  int32_t max_num_partitions;
  bool bf16;
  uint16_t* out;
};

struct KvWriteArgs {
  const void* key;
  const void* value;
  const int64_t* slot_mapping;
  int32_t num_tokens;
  int32_t row_bytes;  // num_kv_heads * head_dim * element size, a multiple of 16
  int64_t num_slots;  // num_blocks * block_size: slots at or past it are skipped like padding
  void* k_cache;
  void* v_cache;
};

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  int32_t num_seqs;
  int32_t num_q_tokens;
  int32_t max_query_len;
  int32_t max_context_len;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t block_size;  // tokens per KV block: 8, 16 or 32
  float scale;
  bool bf16;
  uint16_t* out;
  int32_t split_keys;  // keys per split (multiple of 32), from prefill_split_keys
  float* workspace;  // split states; may be null when no tile needs more than one split
};

hipError_t launch_decode(const DecodeArgs& a, int mode, hipStream_t stream);
hipError_t launch_splitk_reduce(const ReduceArgs& a, hipStream_t stream);
struct RopeKvArgs {
  const uint16_t* qkv;       // [T, row_stride] rows: q heads, k heads, v heads
  int64_t row_stride;        // elements between consecutive token rows
  const int64_t* positions;  // [T]
  const int64_t* slot_mapping;
  const float* table;        // [max_position][head_dim / 2] (cos, sin) pairs
  int32_t num_tokens, num_q_heads, num_kv_heads, head_dim;
  int32_t max_position;      // rows of the table; positions are clamped into [0, max_position)
  int64_t num_slots;         // num_blocks * block_size: slots at or past it are skipped like padding
  bool bf16;
  uint16_t* q_out;           // [T, Hq, D]
  uint16_t* k_cache;
  uint16_t* v_cache;
};

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);
hipError_t launch_rope_table(float* table, int max_position, int head_dim, double theta, hipStream_t stream);
hipError_t launch_rope_kv_write(const RopeKvArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
bool prefill_supported(bool bf16, int head_dim, int group, int block_size);
int prefill_split_keys(int num_q_tokens, int num_seqs, int num_kv_heads, int group, int head_dim, int max_context_len,
                       int num_cus);
size_t prefill_workspace_floats(int num_q_tokens, int num_seqs, int num_kv_heads, int group, int head_dim,
                                int max_context_len, int split_keys);

}  // namespace pka
