// C ABI of libduoattn: argument validation, static work planning and kernel launches.
// Every check runs before any HIP call, so invalid calls return an error without touching a device.
#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "../../include/duo_attn.h"
#include "duo_kernels.h"

static_assert(DUO_NOALLOC_SCRATCH_BYTES == duo::kNoAllocScratchBytes,
              "the header states the scratch size of duo_attn_decode_noalloc");

namespace {

using namespace duo;

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int32_t x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool head_dim_ok(int32_t d) { return d == 64 || d == 128 || d == 256; }
bool dtype_ok(int32_t t) { return t == DUO_F32 || t == DUO_F16 || t == DUO_BF16; }
int elem_bytes(int32_t t) { return t == DUO_F32 ? 4 : 2; }
int32_t sink_blocks(int32_t sink, int32_t bs) { return (sink + bs - 1) / bs; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Mask -> lists of retrieval / streaming kv heads. Returns false on a value other than 0/1.
bool split_heads(const uint8_t* mask, int32_t hkv, uint8_t* ret, int32_t* n_ret, uint8_t* str,
                 int32_t* n_str) {
  *n_ret = *n_str = 0;
  for (int32_t h = 0; h < hkv; ++h) {
    if (mask[h] > 1) return false;
    if (mask[h]) ret[(*n_ret)++] = (uint8_t)h;
    else str[(*n_str)++] = (uint8_t)h;
  }
  return true;
}

// Checks common to the two attention calls (everything except q/out/workspace/q_len specifics).
int32_t check_cache(const void* k_pool, const void* v_pool, const int32_t* table, int32_t num_blocks,
                    int32_t bs, int32_t mbph, const int32_t* seq_lens, int32_t batch, int32_t hq,
                    int32_t hkv, int32_t head_dim, int32_t dtype, const uint8_t* mask) {
  if (!k_pool || !v_pool || !table || !seq_lens || !mask) return DUO_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(table, 4) || !aligned(seq_lens, 4))
    return DUO_ERR_INVALID_ARG;
  if (batch < 1 || hq < 1 || hkv < 1 || num_blocks < 1 || mbph < 1) return DUO_ERR_INVALID_ARG;
  if (batch > 65535) return DUO_ERR_UNSUPPORTED;
  if (hq % hkv != 0) return DUO_ERR_INVALID_ARG;
  if (hkv > kMaxKvHeads) return DUO_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype) || !head_dim_ok(head_dim)) return DUO_ERR_UNSUPPORTED;
  if (!is_pow2(bs) || bs < 16 || bs > 256) return DUO_ERR_UNSUPPORTED;
  if ((int64_t)mbph * bs > INT32_MAX) return DUO_ERR_INVALID_ARG;
  return DUO_OK;
}

// A streaming head's recent window, as the kernels take it: for a query at position p it starts at
// (p & mask) - back and ends at p.
//   recent > 0: the recent newest positions (mask keeps every bit, back = recent - 1);
//   recent < 0: the -recent newest blocks of bs positions, the query's own block counting as one
//               however few of its positions exist (mask clears the offset inside the block,
//               back = (blocks - 1) * bs). This is the block-granular policy of the vLLM
//               attention-sink issue (ChuanhongLi's comment): the oldest middle block is dropped
//               when a new block starts.
// span is the most positions one window holds.
struct Window {
  int32_t mask, back;
  int64_t span;
};
Window window_of(int32_t n_str, int32_t recent, int32_t bs) {
  if (n_str == 0 || recent == 0) return Window{-1, 0, 0};
  if (recent > 0) return Window{-1, recent - 1, recent};
  const int64_t blocks = -(int64_t)recent;
  return Window{-bs, (int32_t)std::min<int64_t>((blocks - 1) * bs, INT32_MAX), blocks * bs};
}

int32_t check_stream_geometry(int32_t n_str, int32_t sink, int32_t recent, int32_t ring_blocks,
                              int32_t bs, int32_t mbph, int32_t q_len) {
  if (sink < 0) return DUO_ERR_INVALID_ARG;
  if (n_str == 0) return DUO_OK;
  if (recent == 0 || ring_blocks < 1) return DUO_ERR_INVALID_ARG;
  if ((int64_t)sink_blocks(sink, bs) + ring_blocks > mbph) return DUO_ERR_CAPACITY;
  // the oldest key of the first row's window and the newest row's key share the ring
  if ((int64_t)ring_blocks * bs < window_of(n_str, recent, bs).span + q_len - 1)
    return DUO_ERR_CAPACITY;
  return DUO_OK;
}

// Decode rows: a kv head's q heads ride in the 16 MFMA columns, so a group of more than 16 is taken
// in chunks of 16 q heads, each chunk its own row of items; a merge record holds min(group, 16)
// q heads.
int32_t decode_group_chunks(int32_t hq, int32_t hkv) { return (hq / hkv + 15) / 16; }
int32_t decode_record_heads(int32_t hq, int32_t hkv) { return std::min(hq / hkv, 16); }

// The decode workspace starts with its tickets: one per row (sequence, kv head, chunk of q heads),
// then one per merge group for as many groups as any split of this capacity can have (splits are
// >= 128 tokens). The region depends on the shapes only, so a workspace reused with other split
// sizes or masks still finds every ticket at zero.
size_t decode_counter_bytes(int32_t batch, int32_t hkv, int32_t cap, int32_t gch = 1) {
  const int32_t most_splits = (int32_t)(((int64_t)cap + 127) / 128);
  const int32_t groups = most_splits <= kMergeGroup
                             ? 0 : std::min<int32_t>(kMaxMergeGroups, (most_splits + kMergeGroup - 1) / kMergeGroup);
  return align256((size_t)batch * hkv * gch * (1 + (size_t)groups) * sizeof(int32_t));
}

// rows: (sequence, retrieval kv head) pairs the split is sized for (times the chunks of q heads);
// stretch_keys: see decode_split_tokens (0 unless the streaming items go first). The workspace-size
// queries pass rows = batch and no stretch (one retrieval head per sequence: the smallest split and
// the most partials any mask needs).
int32_t decode_plan(int32_t batch, int32_t hq, int32_t hkv, int32_t head_dim, int32_t mbph,
                    int32_t bs, int32_t rows, int32_t split_req, int32_t* split_tokens,
                    int32_t* n_split, size_t* ws_bytes, int32_t stretch_keys = 0) {
  if (split_req < 0 || (split_req % 128) != 0) return DUO_ERR_INVALID_ARG;
  const int32_t cap = mbph * bs;
  const int32_t gch = decode_group_chunks(hq, hkv);
  const int32_t S = decode_split_tokens((int32_t)std::min<int64_t>((int64_t)rows * gch, INT32_MAX),
                                        cap, split_req, stretch_keys);
  const int32_t ns = (cap + S - 1) / S;
  *split_tokens = S;
  *n_split = ns;
  *ws_bytes = decode_counter_bytes(batch, hkv, cap, gch) +
              (size_t)batch * hkv * gch * (ns + decode_merge_groups(ns)) *
                  decode_record_heads(hq, hkv) * (head_dim + 2) * sizeof(float);
  return DUO_OK;
}

// Prefill work layout: row tiles of prefill_rows() rows; retrieval items split their keys in
// kPrefillSplits workgroups that merge through the workspace (tickets, then partials). Fixed-length
// calls: n_qtiles tiles per sequence. Packed batches (total_q > 0): one list of the live tiles of
// all sequences, at most ceil(total_q / rows) + batch - 1 long (each sequence leaves at most one
// tile partly empty) and at most batch * ceil(q_len / rows).
void prefill_plan(int32_t batch, int32_t q_len, int32_t hq, int32_t n_ret_kv, int32_t hkv,
                  int32_t head_dim, int32_t dtype, int32_t* n_qtiles, int64_t* ret_items,
                  size_t* ws_bytes, int32_t total_q = 0) {
  const int eb = elem_bytes(dtype);
  const int rows = prefill_rows(eb, head_dim);
  const int64_t per_seq = (q_len + rows - 1) / rows;
  if (total_q > 0) {
    const int64_t bound = std::min<int64_t>((int64_t)batch * per_seq,
                                            ((int64_t)total_q + rows - 1) / rows + batch - 1);
    *n_qtiles = (int32_t)std::min<int64_t>(bound, INT32_MAX);
    *ret_items = (int64_t)n_ret_kv * (hq / hkv) * *n_qtiles;
  } else {
    *n_qtiles = (int32_t)per_seq;
    *ret_items = (int64_t)batch * n_ret_kv * (hq / hkv) * *n_qtiles;
  }
  *ws_bytes = *ret_items == 0 ? 0
              : align256((size_t)*ret_items * sizeof(int32_t)) +
                (size_t)*ret_items * kPrefillSplits * prefill_partial_floats(eb, head_dim) * sizeof(float);
}

// The profiling hook: events set by duo_profile_next_launch wait here until the next attention call
// on this thread takes them; that call's launch sees them through current_launch_events().
thread_local LaunchEvents t_pending_events{nullptr, nullptr};
thread_local LaunchEvents t_call_events{nullptr, nullptr};
struct CallEvents {   // one attention call: take the pending events, drop them when the call returns
  CallEvents() {
    t_call_events = t_pending_events;
    t_pending_events = LaunchEvents{nullptr, nullptr};
  }
  ~CallEvents() { t_call_events = LaunchEvents{nullptr, nullptr}; }
};

}  // namespace

namespace duo {
LaunchEvents current_launch_events() { return t_call_events; }
}  // namespace duo

extern "C" {

int32_t duo_profile_next_launch(void* start_event, void* stop_event) {
  t_pending_events = LaunchEvents{static_cast<hipEvent_t>(start_event),
                                  static_cast<hipEvent_t>(stop_event)};
  return DUO_OK;
}

int32_t duo_abi_version(void) { return DUO_ATTN_ABI_VERSION; }

const char* duo_status_string(int32_t s) {
  switch (s) {
    case DUO_OK: return "ok";
    case DUO_ERR_INVALID_ARG: return "invalid argument";
    case DUO_ERR_UNSUPPORTED: return "unsupported configuration";
    case DUO_ERR_CAPACITY: return "cache capacity too small for the request";
    case DUO_ERR_WORKSPACE: return "decode workspace missing or too small";
    case DUO_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

// The append behind the three caches. quant 8: each new row quantized into int8 codes + one scale
// per slot (written); quant 4: 4-bit codes with the caller's per-(kv head, channel) scales (read).
static int32_t append_impl(int quant, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                           const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                           int32_t max_blocks_per_head, const void* k_new, const void* v_new,
                           const int32_t* seq_lens_before, int32_t* seq_lens_after, int32_t batch,
                           int32_t t_new, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                           const uint8_t* head_is_retrieval, int32_t sink_size, int32_t recent_size,
                           int32_t ring_blocks, void* stream) {
  (void)recent_size;  // the append keeps every ring slot; the window is applied when attending
  if (!k_pool || !v_pool || !block_table || !k_new || !v_new || !seq_lens_before ||
      !head_is_retrieval)
    return DUO_ERR_INVALID_ARG;
  if (quant != 0 && (!k_scale || !v_scale || !aligned(k_scale, 16) || !aligned(v_scale, 16) ||
                     (quant == 8 && k_scale == v_scale)))
    return DUO_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens_before, 4) ||
      (seq_lens_after && !aligned(seq_lens_after, 4)))
    return DUO_ERR_INVALID_ARG;
  if (seq_lens_after == seq_lens_before) return DUO_ERR_INVALID_ARG;
  if (batch < 1 || t_new < 1 || num_kv_heads < 1 || num_blocks < 1 || max_blocks_per_head < 1)
    return DUO_ERR_INVALID_ARG;
  if (batch > 65535 || num_kv_heads > kMaxKvHeads) return DUO_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype) || !head_dim_ok(head_dim)) return DUO_ERR_UNSUPPORTED;
  if (!is_pow2(block_size) || block_size > 256) return DUO_ERR_UNSUPPORTED;
  // a 4-bit V page row packs 8 slots to a word, and a run of 16 slots must sit in one page
  if (quant == 4 && (block_size < 16 || dtype == DUO_F32)) return DUO_ERR_UNSUPPORTED;
  if ((int64_t)max_blocks_per_head * block_size > INT32_MAX) return DUO_ERR_INVALID_ARG;
  if (t_new > INT32_MAX - 64 * 16) return DUO_ERR_INVALID_ARG;
  uint8_t ret[kMaxKvHeads], str[kMaxKvHeads];
  int32_t n_ret, n_str;
  if (!split_heads(head_is_retrieval, num_kv_heads, ret, &n_ret, str, &n_str))
    return DUO_ERR_INVALID_ARG;
  if (sink_size < 0) return DUO_ERR_INVALID_ARG;
  if (n_str > 0) {
    if (ring_blocks < 1) return DUO_ERR_INVALID_ARG;
    if ((int64_t)sink_blocks(sink_size, block_size) + ring_blocks > max_blocks_per_head)
      return DUO_ERR_CAPACITY;
  }
  AppendParams p{};
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.table = block_table;
  p.k_new = k_new;
  p.v_new = v_new;
  p.lens_before = seq_lens_before;
  p.lens_after = seq_lens_after;
  p.num_blocks = num_blocks;
  p.log2_bs = log2i(block_size);
  p.max_blocks_per_head = max_blocks_per_head;
  p.batch = batch;
  p.t_new = t_new;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.sink = sink_size;
  p.sink_blocks = sink_blocks(sink_size, block_size);
  p.ring_slots = n_str > 0 ? ring_blocks * block_size : 1;
  p.retrieval_bits = 0;
  for (int32_t i = 0; i < n_ret; ++i) p.retrieval_bits |= 1ull << ret[i];
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.dtype = dtype;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = quant == 8 ? launch_append_int8(p, st)
                       : quant == 4 ? launch_append_int4(p, st)
                                    : launch_append(p, elem_bytes(dtype), st);
  return e == hipSuccess ? DUO_OK : DUO_ERR_HIP;
}

int32_t kv_append_circular(void* k_pool, void* v_pool, const int32_t* block_table,
                           int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_head,
                           const void* k_new, const void* v_new, const int32_t* seq_lens_before,
                           int32_t* seq_lens_after, int32_t batch, int32_t t_new,
                           int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                           const uint8_t* head_is_retrieval, int32_t sink_size, int32_t recent_size,
                           int32_t ring_blocks, void* stream) {
  return append_impl(0, k_pool, v_pool, nullptr, nullptr, block_table, num_blocks, block_size,
                     max_blocks_per_head, k_new, v_new, seq_lens_before, seq_lens_after, batch,
                     t_new, num_kv_heads, head_dim, dtype, head_is_retrieval, sink_size,
                     recent_size, ring_blocks, stream);
}

int32_t kv_append_circular_int8(int8_t* k_pool, int8_t* v_pool, float* k_scale, float* v_scale,
                                const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_head, const void* k_new, const void* v_new,
                                const int32_t* seq_lens_before, int32_t* seq_lens_after,
                                int32_t batch, int32_t t_new, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                                int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                                void* stream) {
  return append_impl(8, k_pool, v_pool, k_scale, v_scale, block_table, num_blocks, block_size,
                     max_blocks_per_head, k_new, v_new, seq_lens_before, seq_lens_after, batch,
                     t_new, num_kv_heads, head_dim, dtype, head_is_retrieval, sink_size,
                     recent_size, ring_blocks, stream);
}

int32_t kv_append_circular_int4(uint8_t* k_pool, uint8_t* v_pool, const float* k_scale,
                                const float* v_scale, const int32_t* block_table,
                                int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_head, const void* k_new, const void* v_new,
                                const int32_t* seq_lens_before, int32_t* seq_lens_after,
                                int32_t batch, int32_t t_new, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                                int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                                void* stream) {
  return append_impl(4, k_pool, v_pool, const_cast<float*>(k_scale), const_cast<float*>(v_scale),
                     block_table, num_blocks, block_size, max_blocks_per_head, k_new, v_new,
                     seq_lens_before, seq_lens_after, batch, t_new, num_kv_heads, head_dim, dtype,
                     head_is_retrieval, sink_size, recent_size, ring_blocks, stream);
}

size_t duo_attn_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_blocks_per_head,
                                      int32_t block_size, int32_t split_tokens) {
  if (batch < 1 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 ||
      !head_dim_ok(head_dim) || max_blocks_per_head < 1 || !is_pow2(block_size) ||
      (int64_t)max_blocks_per_head * block_size > INT32_MAX)
    return 0;
  int32_t S, ns;
  size_t bytes;
  if (decode_plan(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_head, block_size,
                  batch, split_tokens, &S, &ns, &bytes) != DUO_OK)
    return 0;
  return bytes;
}

// The decode behind both caches: int8 = codes in the pools plus one scale per slot for K and V.
// The extra inputs of Dual Chunk Attention (checked by the dca_* entry points).
struct DcaArgs {
  const void* q_succ;
  const void* q_inter;
  const float* mscale;
  int32_t chunk_len;
};

// The fused append of duo_attn_append_decode: one token per (sequence, kv head) and the lengths
// after it.
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  int32_t* seq_lens_after;
};

// The decode behind the three caches (quant 0: 16-bit or fp32, 8: int8 codes + per-slot scales,
// 4: 4-bit codes + per-(kv head, channel) scales); dca != nullptr: Dual Chunk Attention (16-bit
// cache, full heads); app != nullptr: the token at position seq_lens[b] is appended first (no dca).
static int32_t decode_impl(int quant, const void* q, const void* k_pool, const void* v_pool,
                           const float* k_scale, const float* v_scale, const int32_t* block_table,
                           int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_head,
                           const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                           const uint8_t* head_is_retrieval, int32_t sink_size, int32_t recent_size,
                           int32_t ring_blocks, float softmax_scale, void* out, void* workspace,
                           size_t workspace_bytes, int32_t split_tokens, void* stream,
                           const DcaArgs* dca = nullptr, bool noalloc = false,
                           const AppendArgs* app = nullptr) {
  const CallEvents events;
  int32_t st = check_cache(k_pool, v_pool, block_table, num_blocks, block_size, max_blocks_per_head,
                           seq_lens, batch, num_q_heads, num_kv_heads, head_dim, dtype,
                           head_is_retrieval);
  if (st != DUO_OK) return st;
  if (quant != 0 && (!k_scale || !v_scale || !aligned(k_scale, 16) || !aligned(v_scale, 16)))
    return DUO_ERR_INVALID_ARG;
  if (quant == 4 && dtype == DUO_F32) return DUO_ERR_UNSUPPORTED;
  if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return DUO_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale > 3.0e38f) return DUO_ERR_INVALID_ARG;
  if (app != nullptr) {
    if (dca != nullptr) return DUO_ERR_UNSUPPORTED;
    if (!app->k_new || !app->v_new || !aligned(app->k_new, 16) || !aligned(app->v_new, 16))
      return DUO_ERR_INVALID_ARG;
    // the lengths are read by every work item while one item per sequence writes the new ones
    if (app->seq_lens_after &&
        (!aligned(app->seq_lens_after, 4) || app->seq_lens_after == seq_lens))
      return DUO_ERR_INVALID_ARG;
  }
  uint8_t ret[kMaxKvHeads], str[kMaxKvHeads];
  int32_t n_ret, n_str;
  if (!split_heads(head_is_retrieval, num_kv_heads, ret, &n_ret, str, &n_str))
    return DUO_ERR_INVALID_ARG;
  st = check_stream_geometry(n_str, sink_size, recent_size, ring_blocks, block_size,
                             max_blocks_per_head, 1);
  if (st != DUO_OK) return st;
  int32_t S, ns;
  size_t need;
  // With streaming heads and the library's split: streaming items first, and the retrieval rows'
  // last splits shortened by the keys a streaming item's time would stream. A streaming item is
  // bound by latency, so its time is about that of (sink + window + 256) keys of a 16-bit cache
  // whatever the cache: in keys of this cache, that many times 16-bit bytes per key over this
  // cache's (2 D + 8 per key for int8 with its two scales, D for 4 bits, 8 D for fp32).
  const bool str_first = n_str > 0 && split_tokens == 0;
  int32_t stretch = 0;
  if (str_first) {
    const int64_t bpk16 = 4LL * head_dim;
    const int64_t bpk = quant == 8 ? 2LL * head_dim + 8 : quant == 4 ? head_dim
                                                        : 2LL * head_dim * elem_bytes(dtype);
    const int64_t span = window_of(n_str, recent_size, block_size).span;
    stretch = (int32_t)std::min<int64_t>(((int64_t)sink_size + span + 256) * bpk16 / bpk,
                                         INT32_MAX / 2);
  }
  st = decode_plan(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_head, block_size,
                   batch * (n_ret > 0 ? n_ret : 1), split_tokens, &S, &ns, &need, stretch);
  if (st != DUO_OK) return st;
  if (noalloc) {
    if (need > kNoAllocScratchBytes) return DUO_ERR_WORKSPACE;
  } else if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) {
    return DUO_ERR_WORKSPACE;
  }
  const int32_t gch = decode_group_chunks(num_q_heads, num_kv_heads);
  const int64_t grid = ((int64_t)batch * n_ret * ns + (int64_t)batch * n_str) * gch;
  if (grid > INT32_MAX) return DUO_ERR_UNSUPPORTED;
  const size_t ticket_bytes =
      decode_counter_bytes(batch, num_kv_heads, max_blocks_per_head * block_size, gch);
  if (noalloc) {
    // every check has passed: take this device's scratch and clear its tickets (a fill kernel on
    // the call's stream, ahead of the decode)
    if (noalloc_scratch(&workspace) != hipSuccess) return DUO_ERR_HIP;
    workspace_bytes = kNoAllocScratchBytes;
    if (launch_zero_words(static_cast<uint32_t*>(workspace), ticket_bytes / 4,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
      return DUO_ERR_HIP;
  }

  DecodeParams p{};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.table = block_table;
  p.seq_lens = seq_lens;
  p.k_new = app ? app->k_new : nullptr;
  p.v_new = app ? app->v_new : nullptr;
  p.seq_lens_after = app ? app->seq_lens_after : nullptr;
  p.out = out;
  p.counter = static_cast<int32_t*>(workspace);
  p.gcounter = p.counter + (size_t)batch * num_kv_heads * gch;
  p.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + ticket_bytes);
  p.n_group = decode_merge_groups(ns);
  p.gpartial = p.partial + (size_t)batch * num_kv_heads * gch * ns *
                               decode_record_heads(num_q_heads, num_kv_heads) * (head_dim + 2);
  p.gchunks = gch;
  p.num_blocks = num_blocks;
  p.log2_bs = log2i(block_size);
  p.max_blocks_per_head = max_blocks_per_head;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.sink = sink_size;
  const Window win = window_of(n_str, recent_size, block_size);
  p.win_mask = win.mask;
  p.win_back = win.back;
  p.sink_blocks = sink_blocks(sink_size, block_size);
  p.ring_slots = n_str > 0 ? ring_blocks * block_size : block_size;
  p.split_tokens = S;
  p.n_split = ns;
  p.n_ret = n_ret;
  p.n_str = n_str;
  p.str_first = str_first ? 1 : 0;
  p.scale_log2 = softmax_scale * kLog2e;
  for (int32_t i = 0; i < n_ret; ++i) p.ret_heads[i] = ret[i];
  for (int32_t i = 0; i < n_str; ++i) p.str_heads[i] = str[i];
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  if (dca) {
    p.q_succ = dca->q_succ;
    p.q_inter = dca->q_inter;
    p.mscale = dca->mscale;
    p.chunk_len = dca->chunk_len;
    if (launch_decode_dca(p, dtype, head_dim, (int)grid, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
      return DUO_ERR_HIP;
    return DUO_OK;
  }
  if (launch_decode(p, dtype, head_dim, quant, (int)grid, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return DUO_ERR_HIP;
  return DUO_OK;
}

int32_t duo_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                        int32_t max_blocks_per_head, const int32_t* seq_lens, int32_t batch,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                        const uint8_t* head_is_retrieval, int32_t sink_size, int32_t recent_size,
                        int32_t ring_blocks, float softmax_scale, void* out, void* workspace,
                        size_t workspace_bytes, int32_t split_tokens, void* stream) {
  return decode_impl(0, q, k_pool, v_pool, nullptr, nullptr, block_table, num_blocks,
                     block_size, max_blocks_per_head, seq_lens, batch, num_q_heads, num_kv_heads,
                     head_dim, dtype, head_is_retrieval, sink_size, recent_size, ring_blocks,
                     softmax_scale, out, workspace, workspace_bytes, split_tokens, stream);
}

int32_t duo_attn_append_decode(const void* q, const void* k_new, const void* v_new, void* k_pool,
                               void* v_pool, const int32_t* block_table, int32_t num_blocks,
                               int32_t block_size, int32_t max_blocks_per_head,
                               const int32_t* seq_lens_before, int32_t* seq_lens_after,
                               int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                               int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                               float softmax_scale, void* out, void* workspace,
                               size_t workspace_bytes, int32_t split_tokens, void* stream) {
  const AppendArgs app{k_new, v_new, seq_lens_after};
  return decode_impl(0, q, k_pool, v_pool, nullptr, nullptr, block_table, num_blocks, block_size,
                     max_blocks_per_head, seq_lens_before, batch, num_q_heads, num_kv_heads,
                     head_dim, dtype, head_is_retrieval, sink_size, recent_size, ring_blocks,
                     softmax_scale, out, workspace, workspace_bytes, split_tokens, stream, nullptr,
                     false, &app);
}

int32_t duo_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_head, const int32_t* seq_lens,
                                int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                                int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                                float softmax_scale, void* out, int32_t split_tokens,
                                void* stream) {
  return decode_impl(0, q, k_pool, v_pool, nullptr, nullptr, block_table, num_blocks,
                     block_size, max_blocks_per_head, seq_lens, batch, num_q_heads, num_kv_heads,
                     head_dim, dtype, head_is_retrieval, sink_size, recent_size, ring_blocks,
                     softmax_scale, out, nullptr, 0, split_tokens, stream, nullptr, true);
}

int32_t duo_attn_append_decode_int8(const void* q, const void* k_new, const void* v_new,
                                    int8_t* k_pool, int8_t* v_pool, float* k_scale, float* v_scale,
                                    const int32_t* block_table, int32_t num_blocks,
                                    int32_t block_size, int32_t max_blocks_per_head,
                                    const int32_t* seq_lens_before, int32_t* seq_lens_after,
                                    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t dtype,
                                    const uint8_t* head_is_retrieval, int32_t sink_size,
                                    int32_t recent_size, int32_t ring_blocks, float softmax_scale,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    int32_t split_tokens, void* stream) {
  const AppendArgs app{k_new, v_new, seq_lens_after};
  return decode_impl(8, q, k_pool, v_pool, k_scale, v_scale, block_table, num_blocks, block_size,
                     max_blocks_per_head, seq_lens_before, batch, num_q_heads, num_kv_heads,
                     head_dim, dtype, head_is_retrieval, sink_size, recent_size, ring_blocks,
                     softmax_scale, out, workspace, workspace_bytes, split_tokens, stream, nullptr,
                     false, &app);
}

int32_t duo_attn_decode_int8(const void* q, const int8_t* k_pool, const int8_t* v_pool,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                             int32_t max_blocks_per_head, const int32_t* seq_lens, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t dtype, const uint8_t* head_is_retrieval, int32_t sink_size,
                             int32_t recent_size, int32_t ring_blocks, float softmax_scale,
                             void* out, void* workspace, size_t workspace_bytes,
                             int32_t split_tokens, void* stream) {
  return decode_impl(8, q, k_pool, v_pool, k_scale, v_scale, block_table, num_blocks,
                     block_size, max_blocks_per_head, seq_lens, batch, num_q_heads, num_kv_heads,
                     head_dim, dtype, head_is_retrieval, sink_size, recent_size, ring_blocks,
                     softmax_scale, out, workspace, workspace_bytes, split_tokens, stream);
}

int32_t duo_attn_append_decode_int4(const void* q, const void* k_new, const void* v_new,
                                    uint8_t* k_pool, uint8_t* v_pool, const float* k_scale,
                                    const float* v_scale, const int32_t* block_table,
                                    int32_t num_blocks, int32_t block_size,
                                    int32_t max_blocks_per_head, const int32_t* seq_lens_before,
                                    int32_t* seq_lens_after, int32_t batch, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                    const uint8_t* head_is_retrieval, int32_t sink_size,
                                    int32_t recent_size, int32_t ring_blocks, float softmax_scale,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    int32_t split_tokens, void* stream) {
  const AppendArgs app{k_new, v_new, seq_lens_after};
  return decode_impl(4, q, k_pool, v_pool, k_scale, v_scale, block_table, num_blocks, block_size,
                     max_blocks_per_head, seq_lens_before, batch, num_q_heads, num_kv_heads,
                     head_dim, dtype, head_is_retrieval, sink_size, recent_size, ring_blocks,
                     softmax_scale, out, workspace, workspace_bytes, split_tokens, stream, nullptr,
                     false, &app);
}

int32_t duo_attn_decode_int4(const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                             int32_t max_blocks_per_head, const int32_t* seq_lens, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t dtype, const uint8_t* head_is_retrieval, int32_t sink_size,
                             int32_t recent_size, int32_t ring_blocks, float softmax_scale,
                             void* out, void* workspace, size_t workspace_bytes,
                             int32_t split_tokens, void* stream) {
  return decode_impl(4, q, k_pool, v_pool, k_scale, v_scale, block_table, num_blocks,
                     block_size, max_blocks_per_head, seq_lens, batch, num_q_heads, num_kv_heads,
                     head_dim, dtype, head_is_retrieval, sink_size, recent_size, ring_blocks,
                     softmax_scale, out, workspace, workspace_bytes, split_tokens, stream);
}

size_t duo_attn_prefill_workspace_size(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                       const uint8_t* head_is_retrieval) {
  if (batch < 1 || q_len < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_kv_heads > kMaxKvHeads || num_q_heads % num_kv_heads != 0 || !head_dim_ok(head_dim) ||
      !dtype_ok(dtype) || !head_is_retrieval)
    return 0;
  uint8_t ret[kMaxKvHeads], str[kMaxKvHeads];
  int32_t n_ret, n_str;
  if (!split_heads(head_is_retrieval, num_kv_heads, ret, &n_ret, str, &n_str)) return 0;
  int32_t n_qt;
  int64_t ret_items;
  size_t bytes;
  prefill_plan(batch, q_len, num_q_heads, n_ret, num_kv_heads, head_dim, dtype, &n_qt, &ret_items,
               &bytes);
  return bytes > 0 ? bytes : 256;   // 0 means invalid arguments
}

// The prefill behind both layouts of the queries: q_start == nullptr: [batch][q_len] rows;
// otherwise packed rows, sequence b's at [q_start[b], q_start[b+1]) of total_q, at most q_len each.
// dca != nullptr: Dual Chunk Attention over full heads (the mask is all ones).
static int32_t prefill_impl(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                            int32_t max_blocks_per_head, const int32_t* seq_lens,
                            const int32_t* q_start, int32_t total_q, int32_t batch, int32_t q_len,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t dtype, const uint8_t* head_is_retrieval, int32_t sink_size,
                            int32_t recent_size, int32_t ring_blocks, float softmax_scale,
                            void* out, void* workspace, size_t workspace_bytes, void* stream,
                            const DcaArgs* dca = nullptr) {
  const CallEvents events;
  int32_t st = check_cache(k_pool, v_pool, block_table, num_blocks, block_size, max_blocks_per_head,
                           seq_lens, batch, num_q_heads, num_kv_heads, head_dim, dtype,
                           head_is_retrieval);
  if (st != DUO_OK) return st;
  if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return DUO_ERR_INVALID_ARG;
  if (q_len < 1) return DUO_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale > 3.0e38f) return DUO_ERR_INVALID_ARG;
  if (dtype == DUO_F32 && head_dim > 128) return DUO_ERR_UNSUPPORTED;
  uint8_t ret[kMaxKvHeads], str[kMaxKvHeads];
  int32_t n_ret, n_str;
  if (!split_heads(head_is_retrieval, num_kv_heads, ret, &n_ret, str, &n_str))
    return DUO_ERR_INVALID_ARG;
  st = check_stream_geometry(n_str, sink_size, recent_size, ring_blocks, block_size,
                             max_blocks_per_head, q_len);
  if (st != DUO_OK) return st;
  const bool packed = q_start != nullptr;
  int32_t n_qt;
  int64_t ret_items;
  size_t need;
  prefill_plan(batch, q_len, num_q_heads, n_ret, num_kv_heads, head_dim, dtype, &n_qt, &ret_items,
               &need, packed ? total_q : 0);
  // Packed batches run their single-row sequences as split-K decode items in the same launch;
  // their workspace follows the prefill's.
  const bool mixed = packed;
  const int32_t gch = decode_group_chunks(num_q_heads, num_kv_heads);
  int32_t dS = 0, dns = 0;
  size_t dneed = 0;
  if (mixed) {
    const int32_t st2 = decode_plan(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_head,
                                    block_size, batch * (n_ret > 0 ? n_ret : 1), 0, &dS, &dns, &dneed);
    if (st2 != DUO_OK) return st2;
  }
  const size_t pneed = mixed ? align256(need) : need;
  if (pneed + dneed > 0 &&
      (!workspace || workspace_bytes < pneed + dneed || !aligned(workspace, 16)))
    return DUO_ERR_WORKSPACE;
  const int64_t seqs = packed ? 1 : batch;
  const int64_t n_prefill = ret_items * kPrefillSplits +
                            seqs * n_str * (num_q_heads / num_kv_heads) * n_qt;
  const int64_t n_decode = mixed ? ((int64_t)batch * n_ret * dns + (int64_t)batch * n_str) * gch : 0;
  const int64_t grid = n_prefill + n_decode;
  if (grid > INT32_MAX) return DUO_ERR_UNSUPPORTED;

  PrefillParams p{};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.table = block_table;
  p.seq_lens = seq_lens;
  p.out = out;
  p.q_start = q_start;
  p.total_q = total_q;
  p.skip_single_rows = mixed ? 1 : 0;
  p.counter = need > 0 ? static_cast<int32_t*>(workspace) : nullptr;
  p.partial = need > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                  align256((size_t)ret_items * sizeof(int32_t)))
                       : nullptr;
  p.num_blocks = num_blocks;
  p.log2_bs = log2i(block_size);
  p.max_blocks_per_head = max_blocks_per_head;
  p.batch = batch;
  p.q_len = q_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.sink = sink_size;
  const Window win = window_of(n_str, recent_size, block_size);
  p.win_mask = win.mask;
  p.win_back = win.back;
  p.sink_blocks = sink_blocks(sink_size, block_size);
  p.ring_slots = n_str > 0 ? ring_blocks * block_size : block_size;
  p.n_qtiles = n_qt;
  p.n_ret = n_ret;
  p.n_str = n_str;
  p.n_split = kPrefillSplits;
  p.scale_log2 = softmax_scale * kLog2e;
  for (int32_t i = 0; i < n_ret; ++i) p.ret_heads[i] = ret[i];
  for (int32_t i = 0; i < n_str; ++i) p.str_heads[i] = str[i];
  if (dca) {
    p.q_succ = dca->q_succ;
    p.q_inter = dca->q_inter;
    p.mscale = dca->mscale;
    p.chunk_tiles = dca->chunk_len / kPrefillKeyTile;
    if (launch_prefill_dca(p, dtype, head_dim, (int)grid, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
      return DUO_ERR_HIP;
    return DUO_OK;
  }
  if (mixed) {
    DecodeParams d{};
    d.q = q;
    d.k_pool = k_pool;
    d.v_pool = v_pool;
    d.table = block_table;
    d.seq_lens = seq_lens;
    d.out = out;
    d.q_start = q_start;
    d.total_q = total_q;
    char* dws = static_cast<char*>(workspace) + pneed;
    const size_t ticket_bytes =
        decode_counter_bytes(batch, num_kv_heads, max_blocks_per_head * block_size, gch);
    d.counter = reinterpret_cast<int32_t*>(dws);
    d.gcounter = d.counter + (size_t)batch * num_kv_heads * gch;
    d.partial = reinterpret_cast<float*>(dws + ticket_bytes);
    d.n_group = decode_merge_groups(dns);
    d.gpartial = d.partial + (size_t)batch * num_kv_heads * gch * dns *
                                 decode_record_heads(num_q_heads, num_kv_heads) * (head_dim + 2);
    d.num_blocks = num_blocks;
    d.log2_bs = p.log2_bs;
    d.max_blocks_per_head = max_blocks_per_head;
    d.batch = batch;
    d.num_q_heads = num_q_heads;
    d.num_kv_heads = num_kv_heads;
    d.group = num_q_heads / num_kv_heads;
    d.gchunks = gch;
    d.sink = sink_size;
    d.win_mask = win.mask;
    d.win_back = win.back;
    d.sink_blocks = p.sink_blocks;
    d.ring_slots = p.ring_slots;
    d.split_tokens = dS;
    d.n_split = dns;
    d.n_ret = n_ret;
    d.n_str = n_str;
    d.scale_log2 = p.scale_log2;
    for (int32_t i = 0; i < n_ret; ++i) d.ret_heads[i] = ret[i];
    for (int32_t i = 0; i < n_str; ++i) d.str_heads[i] = str[i];
    if (launch_prefill_mixed(p, d, (int)n_prefill, dtype, head_dim, (int)grid,
                             static_cast<hipStream_t>(stream)) != hipSuccess)
      return DUO_ERR_HIP;
    return DUO_OK;
  }
  if (launch_prefill(p, dtype, head_dim, (int)grid, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DUO_ERR_HIP;
  return DUO_OK;
}

int32_t duo_attn_prefill(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_head, const int32_t* seq_lens, int32_t batch,
                         int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                         int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                         float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (q_len < 1 || (int64_t)batch * q_len > INT32_MAX) return DUO_ERR_INVALID_ARG;
  return prefill_impl(q, k_pool, v_pool, block_table, num_blocks, block_size, max_blocks_per_head,
                      seq_lens, nullptr, batch * q_len, batch, q_len, num_q_heads, num_kv_heads,
                      head_dim, dtype, head_is_retrieval, sink_size, recent_size, ring_blocks,
                      softmax_scale, out, workspace, workspace_bytes, stream);
}

int32_t duo_attn_prefill_varlen(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, int32_t num_blocks, int32_t block_size,
                                int32_t max_blocks_per_head, const int32_t* seq_lens,
                                const int32_t* q_start, int32_t batch, int32_t total_q,
                                int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t dtype, const uint8_t* head_is_retrieval,
                                int32_t sink_size, int32_t recent_size, int32_t ring_blocks,
                                float softmax_scale, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!q_start || !aligned(q_start, 4) || total_q < 1 || max_q_len < 1)
    return DUO_ERR_INVALID_ARG;
  return prefill_impl(q, k_pool, v_pool, block_table, num_blocks, block_size, max_blocks_per_head,
                      seq_lens, q_start, total_q, batch, max_q_len, num_q_heads, num_kv_heads,
                      head_dim, dtype, head_is_retrieval, sink_size, recent_size, ring_blocks,
                      softmax_scale, out, workspace, workspace_bytes, stream);
}

size_t duo_attn_prefill_varlen_workspace_size(int32_t batch, int32_t total_q, int32_t max_q_len,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t dtype,
                                              int32_t max_blocks_per_head, int32_t block_size,
                                              const uint8_t* head_is_retrieval) {
  if (batch < 1 || total_q < 1 || max_q_len < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_kv_heads > kMaxKvHeads || num_q_heads % num_kv_heads != 0 || !head_dim_ok(head_dim) ||
      !dtype_ok(dtype) || !head_is_retrieval || max_blocks_per_head < 1 || !is_pow2(block_size) ||
      (int64_t)max_blocks_per_head * block_size > INT32_MAX)
    return 0;
  uint8_t ret[kMaxKvHeads], str[kMaxKvHeads];
  int32_t n_ret, n_str;
  if (!split_heads(head_is_retrieval, num_kv_heads, ret, &n_ret, str, &n_str)) return 0;
  int32_t n_qt;
  int64_t ret_items;
  size_t bytes;
  prefill_plan(batch, max_q_len, num_q_heads, n_ret, num_kv_heads, head_dim, dtype, &n_qt,
               &ret_items, &bytes, total_q);
  {
    int32_t S, ns;
    size_t dbytes;
    if (decode_plan(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_head, block_size,
                    batch * (n_ret > 0 ? n_ret : 1), 0, &S, &ns, &dbytes) != DUO_OK)
      return 0;
    bytes = align256(bytes) + dbytes;
  }
  return bytes > 0 ? bytes : 256;   // 0 means invalid arguments
}

size_t dca_attn_prefill_workspace_size(int32_t batch, int32_t q_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
  if (num_kv_heads < 1 || num_kv_heads > kMaxKvHeads) return 0;
  uint8_t all[kMaxKvHeads];
  for (int32_t h = 0; h < num_kv_heads; ++h) all[h] = 1;
  return duo_attn_prefill_workspace_size(batch, q_len, num_q_heads, num_kv_heads, head_dim, dtype,
                                         all);
}

// Checks shared by the two Dual Chunk Attention calls (before the common ones).
static int32_t check_dca(const void* q_succ, const void* q_inter, const float* mscale,
                         int32_t chunk_len, int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
  if (!q_succ || !q_inter || !mscale || !aligned(q_succ, 16) || !aligned(q_inter, 16) ||
      !aligned(mscale, 4))
    return DUO_ERR_INVALID_ARG;
  if (chunk_len < 1) return DUO_ERR_INVALID_ARG;
  if (chunk_len % kPrefillKeyTile != 0) return DUO_ERR_UNSUPPORTED;
  if (dtype != DUO_F16 && dtype != DUO_BF16) return DUO_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return DUO_ERR_UNSUPPORTED;
  if (num_kv_heads < 1) return DUO_ERR_INVALID_ARG;
  if (num_kv_heads > kMaxKvHeads) return DUO_ERR_UNSUPPORTED;
  return DUO_OK;
}

int32_t dca_attn_decode(const void* q, const void* q_succ, const void* q_inter,
                        const float* mscale, int32_t chunk_len, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, int32_t num_blocks,
                        int32_t block_size, int32_t max_blocks_per_head, const int32_t* seq_lens,
                        int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t dtype, float softmax_scale, void* out, void* workspace,
                        size_t workspace_bytes, int32_t split_tokens, void* stream) {
  const int32_t st = check_dca(q_succ, q_inter, mscale, chunk_len, num_kv_heads, head_dim, dtype);
  if (st != DUO_OK) return st;
  uint8_t all[kMaxKvHeads];
  for (int32_t h = 0; h < num_kv_heads; ++h) all[h] = 1;
  const DcaArgs dca{q_succ, q_inter, mscale, chunk_len};
  return decode_impl(0, q, k_pool, v_pool, nullptr, nullptr, block_table, num_blocks,
                     block_size, max_blocks_per_head, seq_lens, batch, num_q_heads, num_kv_heads,
                     head_dim, dtype, all, 0, 1, 0, softmax_scale, out, workspace, workspace_bytes,
                     split_tokens, stream, &dca);
}

int32_t dca_attn_prefill(const void* q, const void* q_succ, const void* q_inter,
                         const float* mscale, int32_t chunk_len, const void* k_pool,
                         const void* v_pool, const int32_t* block_table, int32_t num_blocks,
                         int32_t block_size, int32_t max_blocks_per_head, const int32_t* seq_lens,
                         int32_t batch, int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, float softmax_scale, void* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (q_len < 1 || (int64_t)batch * q_len > INT32_MAX) return DUO_ERR_INVALID_ARG;
  const int32_t st = check_dca(q_succ, q_inter, mscale, chunk_len, num_kv_heads, head_dim, dtype);
  if (st != DUO_OK) return st;
  uint8_t all[kMaxKvHeads];
  for (int32_t h = 0; h < num_kv_heads; ++h) all[h] = 1;
  const DcaArgs dca{q_succ, q_inter, mscale, chunk_len};
  return prefill_impl(q, k_pool, v_pool, block_table, num_blocks, block_size, max_blocks_per_head,
                      seq_lens, nullptr, batch * q_len, batch, q_len, num_q_heads, num_kv_heads,
                      head_dim, dtype, all, 0, 1, 0, softmax_scale, out, workspace,
                      workspace_bytes, stream, &dca);
}

}  // extern "C"
