// Host-side checks of the C ABI layer (api.hip) under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// api.hip is compiled for the host only and linked against the stubs below in place of the kernel
// launchers: each stub records what the layer would launch and returns success, so every entry
// point runs its argument checks and launch planning on the CPU with no GPU and no device memory.
// Device pointers are fake addresses that nothing dereferences; host inputs (the retrieval masks)
// are heap arrays of exactly num_kv_heads bytes, so a read past one is reported.
//
// Exit status 0 and no sanitizer report: every case returned the documented status, and every
// accepted call planned the launch the layer documents.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/duo_attn.h"
#include "../../kv_cache_sparsity_amd/csrc/duo_kernels.h"

namespace {

struct Launch {
  int kind = 0;           // 0 none, 1 append, 2 append int8, 3 decode, 4 decode dca, 5 prefill,
                          // 6 prefill dca, 7 zero words, 8 append int4, 9 prefill + decode
  int grid = 0, dtype = -1, head_dim = 0;
  int quant = 0;
  duo::AppendParams ap{};
  duo::DecodeParams dp{};
  duo::PrefillParams pp{};
  duo::LaunchEvents ev{nullptr, nullptr};
  size_t zero_words = 0;
  int n_prefill = 0;
};
std::vector<Launch> g_launches;
int g_failures = 0;

void record(Launch l) {
  l.ev = duo::current_launch_events();
  g_launches.push_back(l);
}

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                              \
    }                                                                            \
  } while (0)

}  // namespace

// ---- stubs of the kernel side ------------------------------------------------------------------
namespace duo {
hipError_t launch_append(const AppendParams& p, int elem_bytes, hipStream_t) {
  Launch l; l.kind = 1; l.ap = p; l.dtype = elem_bytes; record(l); return hipSuccess;
}
hipError_t launch_append_int8(const AppendParams& p, hipStream_t) {
  Launch l; l.kind = 2; l.ap = p; record(l); return hipSuccess;
}
hipError_t launch_append_int4(const AppendParams& p, hipStream_t) {
  Launch l; l.kind = 8; l.ap = p; record(l); return hipSuccess;
}
hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, int quant, int grid,
                         hipStream_t) {
  Launch l; l.kind = 3; l.dp = p; l.dtype = dtype; l.head_dim = head_dim; l.quant = quant;
  l.grid = grid; record(l); return hipSuccess;
}
hipError_t launch_decode_dca(const DecodeParams& p, int dtype, int head_dim, int grid, hipStream_t) {
  Launch l; l.kind = 4; l.dp = p; l.dtype = dtype; l.head_dim = head_dim; l.grid = grid;
  record(l); return hipSuccess;
}
hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, int grid, hipStream_t) {
  Launch l; l.kind = 5; l.pp = p; l.dtype = dtype; l.head_dim = head_dim; l.grid = grid;
  record(l); return hipSuccess;
}
hipError_t launch_prefill_mixed(const PrefillParams& p, const DecodeParams& dp, int n_prefill,
                                int dtype, int head_dim, int grid, hipStream_t) {
  Launch l; l.kind = 9; l.pp = p; l.dp = dp; l.dtype = dtype; l.head_dim = head_dim; l.grid = grid;
  l.n_prefill = n_prefill; record(l); return hipSuccess;
}
hipError_t launch_prefill_dca(const PrefillParams& p, int dtype, int head_dim, int grid,
                              hipStream_t) {
  Launch l; l.kind = 6; l.pp = p; l.dtype = dtype; l.head_dim = head_dim; l.grid = grid;
  record(l); return hipSuccess;
}
hipError_t noalloc_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t(0x7f0000000000));
  return hipSuccess;
}
hipError_t launch_zero_words(uint32_t*, size_t n_words, hipStream_t) {
  Launch l; l.kind = 7; l.zero_words = n_words; record(l); return hipSuccess;
}
}  // namespace duo

namespace {

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t(0x100000) + off); }

struct Mask {   // exactly n host bytes
  explicit Mask(int n, int ret_every = 2) : n(n), p(new uint8_t[n]) {
    for (int i = 0; i < n; ++i) p[i] = (i % ret_every == 0) ? 1 : 0;
  }
  ~Mask() { delete[] p; }
  int n;
  uint8_t* p;
};

size_t launches_of(int kind) {
  size_t c = 0;
  for (const Launch& l : g_launches) c += l.kind == kind;
  return c;
}

// ---- kv_append_circular -------------------------------------------------------------------------
void append_cases() {
  for (int hkv : {1, 2, 7, 64}) {
    Mask m(hkv);
    g_launches.clear();
    const int32_t st = kv_append_circular(fake(), fake(), (const int32_t*)fake(), 1000, 16, 40,
                                          fake(), fake(), (const int32_t*)fake(),
                                          (int32_t*)fake(256), 3, 70, hkv, 128, DUO_BF16, m.p, 4,
                                          16, 2, nullptr);
    CHECK(st == DUO_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].kind == 1);
    if (!g_launches.empty()) {
      const duo::AppendParams& p = g_launches[0].ap;
      uint64_t bits = 0;
      for (int h = 0; h < hkv; ++h) bits |= (uint64_t)m.p[h] << h;
      CHECK(p.retrieval_bits == bits);
      const bool streaming = hkv > 1;   // heads 1, 3, ... are streaming heads
      CHECK(p.sink_blocks == 1 && p.log2_bs == 4 && p.ring_slots == (streaming ? 32 : 1));
    }
  }
  Mask m(2);
  g_launches.clear();
  CHECK(kv_append_circular(nullptr, fake(), (const int32_t*)fake(), 64, 16, 8, fake(), fake(),
                           (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_BF16, m.p, 4, 16, 2,
                           nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(kv_append_circular(fake(), fake(), (const int32_t*)fake(), 64, 16, 8, fake(8), fake(),
                           (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_BF16, m.p, 4, 16, 2,
                           nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(kv_append_circular(fake(), fake(), (const int32_t*)fake(), 64, 12, 8, fake(), fake(),
                           (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_BF16, m.p, 4, 16, 2,
                           nullptr) == DUO_ERR_UNSUPPORTED);
  CHECK(kv_append_circular(fake(), fake(), (const int32_t*)fake(), 64, 16, 8, fake(), fake(),
                           (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_BF16, m.p, 4, 16, 8,
                           nullptr) == DUO_ERR_CAPACITY);
  // sizes at the edges of int32 arithmetic
  CHECK(kv_append_circular(fake(), fake(), (const int32_t*)fake(), 64, 256, INT32_MAX, fake(),
                           fake(), (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_BF16, m.p, 4,
                           16, 2, nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(kv_append_circular(fake(), fake(), (const int32_t*)fake(), 64, 16, 8, fake(), fake(),
                           (const int32_t*)fake(), nullptr, 2, INT32_MAX, 2, 128, DUO_BF16, m.p, 4,
                           16, 2, nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(kv_append_circular(fake(), fake(), (const int32_t*)fake(), 64, 16, 8, fake(), fake(),
                           (const int32_t*)fake(), nullptr, 65536, 5, 2, 128, DUO_BF16, m.p, 4, 16,
                           2, nullptr) == DUO_ERR_UNSUPPORTED);
  CHECK(launches_of(1) == 0);
  // int8: scale pools required and distinct
  CHECK(kv_append_circular_int8((int8_t*)fake(), (int8_t*)fake(), (float*)fake(), (float*)fake(),
                                (const int32_t*)fake(), 64, 16, 8, fake(), fake(),
                                (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_F16, m.p, 4, 16,
                                2, nullptr) == DUO_ERR_INVALID_ARG);
  CHECK(kv_append_circular_int8((int8_t*)fake(), (int8_t*)fake(), (float*)fake(), (float*)fake(4096),
                                (const int32_t*)fake(), 64, 16, 8, fake(), fake(),
                                (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_F16, m.p, 4, 16,
                                2, nullptr) == DUO_OK);
  CHECK(launches_of(2) == 1);
  // 4-bit append: bf16/fp16 rows, pages of at least 16 slots
  CHECK(kv_append_circular_int4((uint8_t*)fake(), (uint8_t*)fake(), (const float*)fake(),
                                (const float*)fake(4096), (const int32_t*)fake(), 64, 16, 8, fake(),
                                fake(), (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_BF16,
                                m.p, 4, 16, 2, nullptr) == DUO_OK);
  CHECK(launches_of(8) == 1);
  CHECK(kv_append_circular_int4((uint8_t*)fake(), (uint8_t*)fake(), (const float*)fake(),
                                (const float*)fake(4096), (const int32_t*)fake(), 64, 8, 16, fake(),
                                fake(), (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_BF16,
                                m.p, 4, 16, 2, nullptr) == DUO_ERR_UNSUPPORTED);
  CHECK(kv_append_circular_int4((uint8_t*)fake(), (uint8_t*)fake(), (const float*)fake(),
                                (const float*)fake(4096), (const int32_t*)fake(), 64, 16, 8, fake(),
                                fake(), (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_F32,
                                m.p, 4, 16, 2, nullptr) == DUO_ERR_UNSUPPORTED);
  CHECK(kv_append_circular_int4((uint8_t*)fake(), (uint8_t*)fake(), nullptr, (const float*)fake(),
                                (const int32_t*)fake(), 64, 16, 8, fake(), fake(),
                                (const int32_t*)fake(), nullptr, 2, 5, 2, 128, DUO_BF16, m.p, 4, 16,
                                2, nullptr) == DUO_ERR_INVALID_ARG);
}

// ---- decode ---------------------------------------------------------------------------------------
int32_t decode(const Mask& m, int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t mbph,
               size_t ws_bytes, int32_t split, int32_t dtype = DUO_BF16, int32_t bs = 16) {
  return duo_attn_decode(fake(), fake(), fake(), (const int32_t*)fake(), 100000, bs, mbph,
                         (const int32_t*)fake(), batch, hq, hkv, d, dtype, m.p, 64, 256, 16,
                         0.088f, fake(), fake(), ws_bytes, split, nullptr);
}

void decode_cases() {
  // the Llama-3-8B decode shape: 4 of 8 kv heads retrieval
  Mask m(8);
  const size_t ws = duo_attn_decode_workspace_size(8, 32, 8, 128, 2048, 16, 0);
  CHECK(ws > 0);
  g_launches.clear();
  CHECK(decode(m, 8, 32, 8, 128, 2048, ws, 0) == DUO_OK);
  CHECK(g_launches.size() == 1);
  if (g_launches.size() == 1) {
    const Launch& l = g_launches[0];
    const duo::DecodeParams& p = l.dp;
    CHECK(l.kind == 3 && l.quant == 0 && l.head_dim == 128 && l.dtype == DUO_BF16);
    CHECK(p.n_ret == 4 && p.n_str == 4 && p.group == 4);
    // 8 splits per row; with streaming heads each split grows by (64 + 256 + 256) / 8 keys, to the
    // nearest 64, so that the last splits (dispatched last) are shorter: 7 x 4160 + 3648
    CHECK(p.split_tokens == 4160 && p.n_split == 8 && p.str_first == 1);
    CHECK(l.grid == 8 * 4 * 8 + 8 * 4);
    for (int i = 0; i < p.n_ret; ++i) CHECK(m.p[p.ret_heads[i]] == 1);
    for (int i = 0; i < p.n_str; ++i) CHECK(m.p[p.str_heads[i]] == 0);
    // partials sit past the tickets and inside the workspace
    const size_t part_off = (const char*)p.partial - (const char*)fake();
    const size_t part_bytes = (size_t)8 * 8 * (p.n_split + p.n_group) * 4 * (128 + 2) * 4;
    CHECK(part_off > 0 && part_off % 256 == 0 && part_off + part_bytes <= ws);
  }
  // the size query without a mask covers the smallest split any mask gives; with the split given,
  // it is exactly what the call needs
  const size_t ws4096 = duo_attn_decode_workspace_size(8, 32, 8, 128, 2048, 16, 4096);
  CHECK(ws4096 > 0 && ws4096 <= ws);
  g_launches.clear();
  CHECK(decode(m, 8, 32, 8, 128, 2048, ws4096, 4096) == DUO_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].dp.str_first == 0 && g_launches[0].dp.split_tokens == 4096);
  CHECK(decode(m, 8, 32, 8, 128, 2048, ws4096 - 1, 4096) == DUO_ERR_WORKSPACE);
  CHECK(decode(m, 8, 32, 8, 128, 2048, 0, 0) == DUO_ERR_WORKSPACE);
  // a group of 40 q heads per kv head: three chunks of up to 16 q heads, each its own row of items
  {
    Mask m2(2, 2);   // kv head 0 retrieval, kv head 1 streaming
    const size_t w40 = duo_attn_decode_workspace_size(4, 80, 2, 128, 2048, 16, 0);
    CHECK(w40 > 0);
    g_launches.clear();
    CHECK(decode(m2, 4, 80, 2, 128, 2048, w40, 0) == DUO_OK);
    CHECK(g_launches.size() == 1);
    if (g_launches.size() == 1) {
      const duo::DecodeParams& p = g_launches[0].dp;
      CHECK(p.group == 40 && p.gchunks == 3);
      // rows: 4 sequences x 1 retrieval head x 3 chunks = 12 -> 256 / 12 = 21 splits of 1600 keys
      // (with the streaming stretch: (32768 + 576) / 21 to the nearest 64 = 1600)
      CHECK(p.n_split == 21 && p.split_tokens == 1600);
      CHECK(g_launches[0].grid == (4 * 1 * 21 + 4 * 1) * 3);
      // tickets: 4 x 2 x 3 rows, then their group tickets; records of 16 q heads
      CHECK(p.gcounter == p.counter + 4 * 2 * 3);
      const size_t rec = (size_t)16 * (128 + 2) * 4;
      CHECK((const char*)p.gpartial == (const char*)p.partial + (size_t)4 * 2 * 3 * 21 * rec);
      CHECK((const char*)p.gpartial + (size_t)4 * 2 * 3 * p.n_group * rec <= (const char*)fake() + w40);
    }
  }
  CHECK(decode(m, 8, 32, 8, 96, 2048, ws, 0) == DUO_ERR_UNSUPPORTED);
  CHECK(decode(m, 8, 32, 8, 128, 2048, ws, 100) == DUO_ERR_INVALID_ARG);  // not a multiple of 128
  CHECK(decode(m, 8, 32, 8, 128, 2048, ws, 0, 9) == DUO_ERR_UNSUPPORTED);
  CHECK(decode(m, 8, 32, 8, 128, 2048, ws, 0, DUO_BF16, 8) == DUO_ERR_UNSUPPORTED);
  // every split size a caller may ask for fits the workspace sized for it
  for (int32_t split : {128, 256, 1024, 4096, 16384, 65536}) {
    const size_t w2 = duo_attn_decode_workspace_size(8, 32, 8, 128, 65540, 16, split);
    CHECK(w2 > 0);
    CHECK(decode(m, 8, 32, 8, 128, 65540, w2, split) == DUO_OK);
  }
  // 64 kv heads, all streaming but one
  Mask m64(64, 64);
  const size_t w64 = duo_attn_decode_workspace_size(2, 64, 64, 64, 100, 16, 0);
  CHECK(decode(m64, 2, 64, 64, 64, 100, w64, 0) == DUO_OK);
  // the profiling hook applies to the next call only
  g_launches.clear();
  duo_profile_next_launch(fake(1), fake(2));
  CHECK(decode(m, 8, 32, 8, 128, 2048, ws, 0) == DUO_OK);
  CHECK(decode(m, 8, 32, 8, 128, 2048, ws, 0) == DUO_OK);
  CHECK(g_launches.size() == 2);
  if (g_launches.size() == 2) {
    CHECK(g_launches[0].ev.start == (hipEvent_t)fake(1) && g_launches[0].ev.stop == (hipEvent_t)fake(2));
    CHECK(g_launches[1].ev.start == nullptr && g_launches[1].ev.stop == nullptr);
  }
  // workspace-size queries reject sizes whose products would overflow
  CHECK(duo_attn_decode_workspace_size(8, 32, 8, 128, INT32_MAX, 16, 0) == 0);
  CHECK(duo_attn_decode_workspace_size(0, 32, 8, 128, 2048, 16, 0) == 0);
  // int8 decode needs its scale pools
  CHECK(duo_attn_decode_int8(fake(), (const int8_t*)fake(), (const int8_t*)fake(), nullptr,
                             (const float*)fake(), (const int32_t*)fake(), 100000, 16, 2048,
                             (const int32_t*)fake(), 8, 32, 8, 128, DUO_BF16, m.p, 64, 256, 16,
                             0.088f, fake(), fake(), ws, 0, nullptr) == DUO_ERR_INVALID_ARG);
  g_launches.clear();
  CHECK(duo_attn_decode_int8(fake(), (const int8_t*)fake(), (const int8_t*)fake(),
                             (const float*)fake(), (const float*)fake(), (const int32_t*)fake(),
                             100000, 16, 2048, (const int32_t*)fake(), 8, 32, 8, 128, DUO_BF16,
                             m.p, 64, 256, 16, 0.088f, fake(), fake(), ws, 0, nullptr) == DUO_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].quant == 8);
  // streaming items first; a streaming item's time is worth (64 + 256 + 256) x 512 / 264 = 1117
  // keys of the int8 cache (2 x 128 code bytes + 2 scales per key against 512 bytes of bf16):
  // (32768 + 1117) / 8 to the nearest 64 = 4224
  if (g_launches.size() == 1)
    CHECK(g_launches[0].dp.str_first == 1 && g_launches[0].dp.split_tokens == 4224);
  // 4-bit: per-channel scales required; 16-bit calls only
  g_launches.clear();
  CHECK(duo_attn_decode_int4(fake(), (const uint8_t*)fake(), (const uint8_t*)fake(),
                             (const float*)fake(), (const float*)fake(4096), (const int32_t*)fake(),
                             100000, 16, 2048, (const int32_t*)fake(), 8, 32, 8, 128, DUO_BF16,
                             m.p, 64, 256, 16, 0.088f, fake(), fake(), ws, 0, nullptr) == DUO_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].quant == 4);
  CHECK(duo_attn_decode_int4(fake(), (const uint8_t*)fake(), (const uint8_t*)fake(),
                             (const float*)fake(), (const float*)fake(4096), (const int32_t*)fake(),
                             100000, 16, 2048, (const int32_t*)fake(), 8, 32, 8, 128, DUO_F32,
                             m.p, 64, 256, 16, 0.088f, fake(), fake(), ws, 0, nullptr) == DUO_ERR_UNSUPPORTED);
  CHECK(duo_attn_decode_int4(fake(), (const uint8_t*)fake(), (const uint8_t*)fake(), nullptr,
                             (const float*)fake(4096), (const int32_t*)fake(), 100000, 16, 2048,
                             (const int32_t*)fake(), 8, 32, 8, 128, DUO_BF16, m.p, 64, 256, 16,
                             0.088f, fake(), fake(), ws, 0, nullptr) == DUO_ERR_INVALID_ARG);
}

void noalloc_cases() {
  Mask m(8);
  g_launches.clear();
  CHECK(duo_attn_decode_noalloc(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                                (const int32_t*)fake(), 8, 32, 8, 128, DUO_BF16, m.p, 64, 256, 16,
                                0.088f, fake(), 0, nullptr) == DUO_OK);
  CHECK(g_launches.size() == 2 && g_launches[0].kind == 7 && g_launches[1].kind == 3);
  if (g_launches.size() == 2) {
    const size_t tickets = (const char*)g_launches[1].dp.partial - (const char*)g_launches[1].dp.counter;
    CHECK(g_launches[0].zero_words * 4 == tickets);
  }
  // shapes whose workspace passes the scratch: refused before anything is launched
  Mask m64(64);
  g_launches.clear();
  CHECK(duo_attn_decode_noalloc(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 65540,
                                (const int32_t*)fake(), 64, 256, 64, 256, DUO_BF16, m64.p, 64, 256,
                                16, 0.0625f, fake(), 128, nullptr) == DUO_ERR_WORKSPACE);
  CHECK(g_launches.empty());
}

// ---- prefill ----------------------------------------------------------------------------------------
void prefill_cases() {
  Mask m(32, 4);   // 8 of 32 heads retrieval (the Llama-2-7B shape)
  const size_t ws = duo_attn_prefill_workspace_size(1, 4096, 32, 32, 128, DUO_BF16, m.p);
  CHECK(ws > 0);
  g_launches.clear();
  CHECK(duo_attn_prefill(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                         (const int32_t*)fake(), 1, 4096, 32, 32, 128, DUO_BF16, m.p, 128, 1024,
                         320, 0.088f, fake(), fake(), ws, nullptr) == DUO_OK);
  CHECK(g_launches.size() == 1);
  if (g_launches.size() == 1) {
    const Launch& l = g_launches[0];
    CHECK(l.kind == 5 && l.pp.n_ret == 8 && l.pp.n_str == 24 && l.pp.n_qtiles == 16);
    CHECK(l.grid == 8 * 16 * 2 + 24 * 16);
  }
  CHECK(duo_attn_prefill(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                         (const int32_t*)fake(), 1, 4096, 32, 32, 128, DUO_BF16, m.p, 128, 1024,
                         300, 0.088f, fake(), fake(), ws, nullptr) == DUO_ERR_CAPACITY);
  CHECK(duo_attn_prefill(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                         (const int32_t*)fake(), 1, 4096, 32, 32, 128, DUO_BF16, m.p, 128, 1024,
                         320, 0.088f, fake(), fake(), ws - 1, nullptr) == DUO_ERR_WORKSPACE);
  CHECK(duo_attn_prefill(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                         (const int32_t*)fake(), 1, 4096, 32, 32, 256, DUO_F32, m.p, 128, 1024,
                         320, 0.088f, fake(), fake(), ws, nullptr) == DUO_ERR_UNSUPPORTED);
  CHECK(duo_attn_prefill(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                         (const int32_t*)fake(), 2, INT32_MAX / 2 + 1, 32, 32, 128, DUO_BF16, m.p,
                         128, 1024, 320, 0.088f, fake(), fake(), ws, nullptr) == DUO_ERR_INVALID_ARG);
  // varlen: needs its offsets
  CHECK(duo_attn_prefill_varlen(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                                (const int32_t*)fake(), nullptr, 4, 5000, 4096, 32, 32, 128,
                                DUO_BF16, m.p, 128, 1024, 320, 0.088f, fake(), fake(), ws,
                                nullptr) == DUO_ERR_INVALID_ARG);
  // a continuous-batching step: one 4096-row chunk and 31 single rows, Llama-3-8B shape, one launch
  Mask m8(8);
  const size_t wv = duo_attn_prefill_varlen_workspace_size(32, 4127, 4096, 32, 8, 128, DUO_BF16, 2048,
                                                           16, m8.p);
  CHECK(wv > 0);
  g_launches.clear();
  CHECK(duo_attn_prefill_varlen(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                                (const int32_t*)fake(), (const int32_t*)fake(), 32, 4127, 4096, 32,
                                8, 128, DUO_BF16, m8.p, 64, 256, 272, 0.088f, fake(), fake(), wv,
                                nullptr) == DUO_OK);
  CHECK(g_launches.size() == 1);
  if (g_launches.size() == 1) {
    const Launch& l = g_launches[0];
    // 48 live row tiles at most (17 for 4127 rows + 31); per tile 16 retrieval q heads x 2 splits
    // and 16 streaming q heads; decode items: 32 sequences x 4 retrieval heads x 2 splits + 32 x 4
    CHECK(l.kind == 9 && l.pp.n_qtiles == 48 && l.pp.skip_single_rows == 1);
    CHECK(l.n_prefill == 48 * (16 * 2 + 16));
    CHECK(l.grid == l.n_prefill + 32 * 4 * 2 + 32 * 4);
    CHECK(l.dp.q_start == l.pp.q_start && l.dp.n_split == 2 && l.dp.split_tokens == 16384);
    const size_t dec_off = (const char*)l.dp.counter - (const char*)fake();
    CHECK(dec_off > 0 && dec_off % 256 == 0 && dec_off < wv);
  }
  CHECK(duo_attn_prefill_varlen(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                                (const int32_t*)fake(), (const int32_t*)fake(), 32, 4127, 4096, 32,
                                8, 128, DUO_BF16, m8.p, 64, 256, 272, 0.088f, fake(), fake(), wv - 1,
                                nullptr) == DUO_ERR_WORKSPACE);
  CHECK(duo_attn_prefill_varlen_workspace_size(32, 0, 4096, 32, 8, 128, DUO_BF16, 2048, 16, m8.p) == 0);
  // all streaming: no workspace needed
  Mask none(32, 1000);
  none.p[0] = 0;
  CHECK(duo_attn_prefill_workspace_size(1, 4096, 32, 32, 128, DUO_BF16, none.p) == 256);
  CHECK(duo_attn_prefill(fake(), fake(), fake(), (const int32_t*)fake(), 100000, 16, 2048,
                         (const int32_t*)fake(), 1, 4096, 32, 32, 128, DUO_BF16, none.p, 128, 1024,
                         320, 0.088f, fake(), nullptr, 0, nullptr) == DUO_OK);
}

// ---- Dual Chunk Attention -------------------------------------------------------------------------
void dca_cases() {
  const size_t ws = dca_attn_prefill_workspace_size(1, 32768, 16, 2, 128, DUO_BF16);
  CHECK(ws > 0);
  g_launches.clear();
  CHECK(dca_attn_prefill(fake(), fake(), fake(), (const float*)fake(), 32768, fake(), fake(),
                         (const int32_t*)fake(), 100000, 16, 8192, (const int32_t*)fake(), 1, 32768,
                         16, 2, 128, DUO_BF16, 0.088f, fake(), fake(), ws, nullptr) == DUO_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].kind == 6 && g_launches[0].pp.chunk_tiles == 512);
  CHECK(dca_attn_prefill(fake(), fake(), fake(), (const float*)fake(), 100, fake(), fake(),
                         (const int32_t*)fake(), 100000, 16, 8192, (const int32_t*)fake(), 1, 32768,
                         16, 2, 128, DUO_BF16, 0.088f, fake(), fake(), ws, nullptr) == DUO_ERR_UNSUPPORTED);
  CHECK(dca_attn_prefill(fake(), nullptr, fake(), (const float*)fake(), 32768, fake(), fake(),
                         (const int32_t*)fake(), 100000, 16, 8192, (const int32_t*)fake(), 1, 32768,
                         16, 2, 128, DUO_BF16, 0.088f, fake(), fake(), ws, nullptr) == DUO_ERR_INVALID_ARG);
  const size_t wd = duo_attn_decode_workspace_size(1, 16, 2, 128, 8192, 16, 0);
  g_launches.clear();
  CHECK(dca_attn_decode(fake(), fake(), fake(), (const float*)fake(), 32768, fake(), fake(),
                        (const int32_t*)fake(), 100000, 16, 8192, (const int32_t*)fake(), 1, 16, 2,
                        128, DUO_BF16, 0.088f, fake(), fake(), wd, 0, nullptr) == DUO_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].kind == 4 && g_launches[0].dp.n_ret == 2);
  CHECK(dca_attn_decode(fake(), fake(), fake(), (const float*)fake(), 32768, fake(), fake(),
                        (const int32_t*)fake(), 100000, 16, 8192, (const int32_t*)fake(), 1, 16, 2,
                        128, DUO_F32, 0.088f, fake(), fake(), wd, 0, nullptr) == DUO_ERR_UNSUPPORTED);
}

}  // namespace

int main() {
  CHECK(duo_abi_version() == DUO_ATTN_ABI_VERSION);
  for (int s = 0; s <= 6; ++s) CHECK(std::strlen(duo_status_string(s)) > 0);
  append_cases();
  decode_cases();
  noalloc_cases();
  prefill_cases();
  dca_cases();
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host ABI checks passed\n");
  return 0;
}
