// Internal interface between the C-ABI host layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace duo {

constexpr int kMaxKvHeads = 64;
constexpr float kLog2e = 1.4426950408889634f;  // scores are kept in the log2 domain

struct AppendParams {
  void* k_pool;
  void* v_pool;
  const int32_t* table;
  const void* k_new;
  const void* v_new;
  const int32_t* lens_before;
  int32_t* lens_after;
  int32_t num_blocks, log2_bs, max_blocks_per_head;
  int32_t batch, t_new, num_kv_heads, head_dim;
  int32_t sink, sink_blocks, ring_slots;
  uint64_t retrieval_bits;  // bit h set = kv head h is a retrieval head
  // int8 cache: one fp32 scale per slot ([num_blocks][block_size]) for K and for V (written);
  // 4-bit cache: one per kv head and channel ([num_kv_heads][head_dim], read). Also the dtype of
  // k_new / v_new.
  float* k_scale;
  float* v_scale;
  int32_t dtype;
};

struct DecodeParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  void* out;
  const float* k_scale;   // int8 cache: [num_blocks][block_size] per-slot scales of K;
  const float* v_scale;   // and of V; 4-bit cache: [num_kv_heads][head_dim] per-channel scales
  // merge records and tickets per row = (sequence, kv head, chunk of up to 16 q heads); a record
  // is [min(group, 16)][head_dim + 2] floats
  float* partial;     // [batch][num_kv_heads][gchunks][n_split] records
  int32_t* counter;   // [batch][num_kv_heads][gchunks]
  float* gpartial;    // [batch][num_kv_heads][gchunks][n_group] records (n_group > 0)
  int32_t* gcounter;  // [batch][num_kv_heads][gchunks][n_group]
  int32_t n_group;    // groups of kMergeGroup splits merged first; 0: one-level merge
  int32_t num_blocks, log2_bs, max_blocks_per_head;
  int32_t batch, num_q_heads, num_kv_heads, group;
  int32_t gchunks;   // ceil(group / 16): chunks of q heads taken one per item
  // a streaming head's window for the query at position p: keys from (p & win_mask) - win_back
  int32_t sink, win_mask, win_back, sink_blocks, ring_slots;
  int32_t split_tokens, n_split, n_ret, n_str;
  // 1: streaming items first in the grid and the retrieval rows' last splits last (the host then
  // shortens the last splits); 0: retrieval items (split fastest), then streaming items
  int32_t str_first;
  float scale_log2;  // softmax_scale * log2(e)
  uint8_t ret_heads[kMaxKvHeads];
  uint8_t str_heads[kMaxKvHeads];
  // Dual Chunk Attention only: the succ / inter query vectors (laid out like q), one fp32 mscale
  // per sequence (its query row), and the chunk length in tokens (a multiple of 64)
  const void* q_succ;
  const void* q_inter;
  const float* mscale;
  int32_t chunk_len;
  // packed batches (decode items inside the packed-batch prefill launch): sequence b's rows of q
  // and out are [q_start[b], q_start[b+1]) clamped into [0, total_q); its items run only when it
  // has exactly one row, which then takes the place of row b. null: row b.
  const int32_t* q_start;
  int32_t total_q;
  // fused append (decode_append_kernel only): the token of each (sequence, kv head) that sits at
  // position seq_lens[b], laid out [batch][num_kv_heads][head_dim] (one step of kv_append_circular's
  // input); the items then attend over seq_lens[b] + 1 keys, and seq_lens_after[b] (may be null)
  // receives that length
  const void* k_new;
  const void* v_new;
  int32_t* seq_lens_after;
};

struct PrefillParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  void* out;
  int32_t* counter;   // [retrieval items] arrival tickets (zero between calls)
  float* partial;     // [retrieval items][n_split] partial (m, l, O^T) of every row
  // packed (varlen) batches: rows [q_start[b], q_start[b+1]) of q / out belong to sequence b
  // (at most q_len of them, clamped into [0, total_q)); null: b * q_len .. + q_len. Packed, the
  // live row tiles of all sequences form one list of at most n_qtiles tiles.
  const int32_t* q_start;
  int32_t total_q;
  // packed batches in one launch with decode items: a sequence with exactly one row is left to them
  int32_t skip_single_rows;
  int32_t num_blocks, log2_bs, max_blocks_per_head;
  int32_t batch, q_len, num_q_heads, num_kv_heads, group;
  // a streaming head's window for the query at position p: keys from (p & win_mask) - win_back
  int32_t sink, win_mask, win_back, sink_blocks, ring_slots;
  int32_t n_qtiles, n_ret, n_str, n_split;
  float scale_log2;
  uint8_t ret_heads[kMaxKvHeads];
  uint8_t str_heads[kMaxKvHeads];
  // Dual Chunk Attention only: the query vectors for keys of the preceding chunk (q_succ) and of
  // earlier chunks (q_inter), laid out like q; one fp32 mscale per query row; the chunk length in
  // 64-key tiles
  const void* q_succ;
  const void* q_inter;
  const float* mscale;
  int32_t chunk_tiles;
};

// Events the attention kernel launched by the current C-ABI call records at its start and its end
// (null when the caller set none; see duo_profile_next_launch).
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
LaunchEvents current_launch_events();

// Launchers (return the HIP launch status). dtype: 0 f32, 1 f16, 2 bf16.
hipError_t launch_append(const AppendParams& p, int elem_bytes, hipStream_t stream);
hipError_t launch_append_int8(const AppendParams& p, hipStream_t stream);
hipError_t launch_append_int4(const AppendParams& p, hipStream_t stream);
// quant: 0 = 16-bit / fp32 cache, 8 = int8 cache, 4 = 4-bit cache (dtype 1 or 2 only)
hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, int quant, int grid,
                         hipStream_t stream);
hipError_t launch_decode_dca(const DecodeParams& p, int dtype, int head_dim, int grid,
                             hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, int grid,
                          hipStream_t stream);
hipError_t launch_prefill_dca(const PrefillParams& p, int dtype, int head_dim, int grid,
                              hipStream_t stream);
// The packed-batch prefill with split-K decode items for single-row sequences: blocks
// [0, n_prefill) run prefill items, the rest decode items of dp.
hipError_t launch_prefill_mixed(const PrefillParams& p, const DecodeParams& dp, int n_prefill,
                                int dtype, int head_dim, int grid, hipStream_t stream);

// The decode scratch of duo_attn_decode_noalloc: a device array of kNoAllocScratchBytes in the
// library's code object (one copy per GPU). noalloc_scratch gives the current device's address of
// it (looked up once per device); launch_zero_words clears n_words 32-bit words with a fill kernel.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_zero_words(uint32_t* p, size_t n_words, hipStream_t stream);
constexpr int kPrefillKeyTile = 64;   // keys per prefill K/V tile (Dual Chunk lengths are multiples)

// Decode split merge in two levels when a (sequence, kv head) has more than kMergeGroup splits
// (and at most kMergeGroup * kMaxMergeGroups): groups of kMergeGroup splits, then the groups.
constexpr int32_t kMergeGroup = 16;
constexpr int32_t kMaxMergeGroups = 256;
inline int32_t decode_merge_groups(int32_t n_split) {
  return (n_split > kMergeGroup && n_split <= kMergeGroup * kMaxMergeGroups)
             ? (n_split + kMergeGroup - 1) / kMergeGroup : 0;
}
// Up to this many splits per (sequence, kv head) the fused merge takes its two-phase fast path.
constexpr int32_t kFastMergeSplits = 256;
// Decode split size (keys per retrieval item) from static sizes. rows = (sequence, retrieval kv
// head) pairs; stretch_keys > 0: the call puts its streaming items first (see below). Shared by the
// workspace-size query (no stretch: the smallest split) and the call.
//
// About one retrieval item per CU (256 on MI355X): n = 256 / rows splits per row (at least 1, at
// most kFastMergeSplits, so that the fused merge takes its fast path), S = capacity / n rounded up
// to 64 keys, at least 256. With stretch_keys > 0 the streaming items come first in the grid and
// the last split of every row comes last, so those last splits start on the CUs the streaming
// items free: S grows by stretch_keys (about as many keys as a streaming item's time would stream)
// spread over the row's splits, so that each last split is that much shorter and ends with the
// others.
inline int32_t decode_split_tokens(int32_t rows, int32_t capacity_tokens, int32_t requested,
                                   int32_t stretch_keys = 0) {
  if (requested > 0) return requested;
  const int64_t r = rows > 0 ? rows : 1;
  const int64_t cap = capacity_tokens > 0 ? capacity_tokens : 1;
  int64_t n = 256 / r;
  n = n < 1 ? 1 : n > kFastMergeSplits ? kFastMergeSplits : n;
  int64_t s = ((cap + n - 1) / n + 63) / 64 * 64;
  if (s < 256) s = 256;
  if (stretch_keys > 0 && n > 1) {
    // nearest multiple of 64; kept only while every split still holds keys
    const int64_t st = ((cap + stretch_keys + n - 1) / n + 32) / 64 * 64;
    if (st > s && (n - 1) * st < cap) s = st;
  }
  return (int32_t)(s < (int64_t)(INT32_MAX / 64) * 64 ? s : (int64_t)(INT32_MAX / 64) * 64);
}

// Prefill workgroup shape: eight waves (two per SIMD, 32 query rows each) while one 64-key K+V tile
// takes at most 32 KiB, so that four tile stages fit in LDS; four waves otherwise.
constexpr int prefill_waves(int elem_bytes, int head_dim) {
  return 64 * head_dim * elem_bytes * 2 <= 32768 ? 8 : 4;
}
constexpr int prefill_rows(int elem_bytes, int head_dim) { return 32 * prefill_waves(elem_bytes, head_dim); }
constexpr int kPrefillSplits = 2;   // key-range splits of a retrieval item (merged in the launch)
// Workspace floats of one split's partial: per wave and lane, m, l and the D / 2 O^T accumulators.
constexpr int64_t prefill_partial_floats(int elem_bytes, int head_dim) {
  return (int64_t)prefill_waves(elem_bytes, head_dim) * 64 * (2 + head_dim / 2);
}
constexpr int kDecodeStep = 32;     // keys per wave step (two 16-key runs)

}  // namespace duo
