// kv_append_circular kernel: copy new K/V tokens into their head's pages.
//
// Slot rule (vLLM issue "Could you support Attention Sink?", sh1ng's comment, option 3 and the
// circular-buffer tables): a retrieval head stores position t at slot t; a streaming head stores
// sinks (t < sink) at slot t and every later position in a ring of ring_slots slots after the sink
// pages, at ring index (t - sink) mod ring_slots.
//
// One workgroup copies one 16-position run of one (sequence, kv head). Within one call only the
// newest ring_slots streamed positions of a head are written; older ones would be overwritten by a
// newer position of the same call, so the final cache equals writing every token in order.
// K rows are copied 16 bytes per lane into the token-major K page; V rows go through LDS and are
// written channel-major (16 consecutive lanes fill one channel's 16 rows).
#include "duo_common.h"
#include "duo_kernels.h"

namespace duo {

namespace {

constexpr int kAppendThreads = 256;
constexpr int kMaxHeadDim = 256;

// The positions [t_lo, t_hi) of this workgroup's 16-position run (blockIdx.x) of sequence b, kv
// head h, and where they go. Also writes the sequence's new length (once per sequence).
struct AppendRun {
  int32_t L0, t_lo, t_hi;
  bool ret;
  const int32_t* trow;
  __device__ __forceinline__ int32_t slot_of(const AppendParams& p, int32_t t) const {
    if (ret || t < p.sink) return t;
    return (p.sink_blocks << p.log2_bs) + (int32_t)((int64_t)(t - p.sink) % p.ring_slots);
  }
  __device__ __forceinline__ int64_t page_of(const AppendParams& p, int32_t s) const {
    return clamp_page(trow[s >> p.log2_bs], p.num_blocks);
  }
};

__device__ __forceinline__ AppendRun append_run(const AppendParams& p, int vg, int h, int b) {
  AppendRun a;
  const int32_t L0 = min(max(p.lens_before[b], 0), INT32_MAX - p.t_new);  // no position overflow
  const int32_t L1 = L0 + p.t_new;
  if (vg == 0 && h == 0 && threadIdx.x == 0 && p.lens_after != nullptr) p.lens_after[b] = L1;
  const bool ret = (p.retrieval_bits >> h) & 1ull;
  int32_t t_lo, t_hi;
  if (ret) {
    const int32_t end = min(L1, p.max_blocks_per_head << p.log2_bs);
    const int32_t g = L0 / 16 + vg;
    t_lo = max(g * 16, L0);
    t_hi = min(g * 16 + 16, end);
  } else {
    const int32_t s_end = min(L1, p.sink);
    const int32_t ns = (L0 < s_end) ? ((s_end - 1) / 16 - L0 / 16 + 1) : 0;
    if (vg < ns) {
      const int32_t g = L0 / 16 + vg;
      t_lo = max(g * 16, L0);
      t_hi = min(g * 16 + 16, s_end);
    } else {
      // ring positions that survive this call: the newest ring_slots of them
      const int32_t r_start = max(max(p.sink, L0), L1 - p.ring_slots);
      const int32_t k = (r_start - p.sink) / 16 + (vg - ns);
      t_lo = max(p.sink + k * 16, r_start);
      t_hi = min(p.sink + k * 16 + 16, L1);
    }
  }
  a.L0 = L0;
  a.t_lo = t_lo;
  a.t_hi = t_hi;
  a.ret = ret;
  a.trow = p.table + ((int64_t)b * p.num_kv_heads + h) * p.max_blocks_per_head;
  return a;
}

template <typename E>  // raw element bits: uint16_t or uint32_t
__global__ void __launch_bounds__(kAppendThreads) append_kernel(const AppendParams p) {
  __shared__ E vstage[16][kMaxHeadDim];
  const int h = blockIdx.y, b = blockIdx.z;
  const int D = p.head_dim;
  const AppendRun run = append_run(p, blockIdx.x, h, b);
  const int32_t L0 = run.L0, t_lo = run.t_lo, t_hi = run.t_hi;
  if (t_lo >= t_hi) return;
  const int n_tok = t_hi - t_lo;
  const int32_t bs_mask = (1 << p.log2_bs) - 1;
  const int32_t* trow = run.trow;
  auto slot_of = [&](int32_t t) -> int32_t { return run.slot_of(p, t); };

  constexpr int kVec = 16 / sizeof(E);  // elements per 16-byte chunk
  const int chunks = D / kVec;
  const E* kn = static_cast<const E*>(p.k_new);
  const E* vn = static_cast<const E*>(p.v_new);
  E* kp = static_cast<E*>(p.k_pool);
  E* vp = static_cast<E*>(p.v_pool);
  const int64_t tok_stride = (int64_t)p.num_kv_heads * D;            // elements between tokens
  const int64_t src0 = ((int64_t)b * p.t_new) * tok_stride + (int64_t)h * D;

  for (int idx = threadIdx.x; idx < n_tok * chunks; idx += kAppendThreads) {
    const int r = idx / chunks, c = idx % chunks;
    const int32_t t = t_lo + r;
    const int64_t src = src0 + (int64_t)(t - L0) * tok_stride + c * kVec;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(kn + src);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(vn + src);
    const int32_t s = slot_of(t);
    const int64_t page = clamp_page(trow[s >> p.log2_bs], p.num_blocks);
    const int64_t dst = ((page << p.log2_bs) + (s & bs_mask)) * D + c * kVec;
    *reinterpret_cast<u32x4*>(kp + dst) = kv;
    *reinterpret_cast<u32x4*>(&vstage[r][c * kVec]) = vv;
  }
  __syncthreads();
  // V page is [D][block_size]: element (d, row) at page * D * bs + d * bs + row.
  const int32_t s0 = slot_of(t_lo);
  if (n_tok == 16 && (s0 & 15) == 0 && p.log2_bs >= 4) {
    // A whole run of 16 consecutive slots in one page (pages of >= 16 slots; ring size a
    // multiple of the page size): each thread writes 8 (16-bit) or 4 (32-bit) consecutive slots of
    // one channel as one 16-byte store.
    const int64_t page = clamp_page(trow[s0 >> p.log2_bs], p.num_blocks);
    E* vrow = vp + page * D * ((int64_t)1 << p.log2_bs) + (s0 & bs_mask);
    constexpr int kPer = 16 / sizeof(E);                 // slots per 16-byte store
    for (int idx = threadIdx.x; idx < D * (16 / kPer); idx += kAppendThreads) {
      const int d = idx / (16 / kPer), r0 = (idx % (16 / kPer)) * kPer;
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(E) == 2)
          w[j] = (uint32_t)vstage[r0 + 2 * j][d] | ((uint32_t)vstage[r0 + 2 * j + 1][d] << 16);
        else
          w[j] = vstage[r0 + j][d];
      }
      *reinterpret_cast<u32x4*>(vrow + (int64_t)d * ((int64_t)1 << p.log2_bs) + r0) = w;
    }
    return;
  }
  for (int idx = threadIdx.x; idx < 16 * D; idx += kAppendThreads) {
    const int r = idx & 15, d = idx >> 4;
    if (r >= n_tok) continue;
    const int32_t s = slot_of(t_lo + r);
    const int64_t page = clamp_page(trow[s >> p.log2_bs], p.num_blocks);
    vp[(page * D + d) * ((int64_t)1 << p.log2_bs) + (s & bs_mask)] = vstage[r][d];
  }
}

// Element bits of the new rows as fp32 (exact): bf16, fp16 or fp32.
template <typename E>
__device__ __forceinline__ float elem_to_f32(uint32_t bits, int dtype) {
  if constexpr (sizeof(E) == 4) {
    return __uint_as_float(bits);
  } else {
    if (dtype == 2) return __uint_as_float(bits << 16);                       // bf16
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);                // fp16
  }
}

// int8 cache: every new K and V row is quantized with one fp32 scale, amax / 127 (0 for an all-zero
// row, whose codes are 0), and its codes and scale go to the row's slot: codes into the pages (K
// token-major, V channel-major, one byte per element) and the scale into k_scale / v_scale at
// [page][row]. The lanes of one row (D / elements-per-16-bytes of them, a divisor of the wave)
// reduce its amax with xor shuffles.
template <typename E>  // raw element bits of the new rows: uint16_t or uint32_t
__global__ void __launch_bounds__(kAppendThreads) append_int8_kernel(const AppendParams p) {
  __shared__ uint8_t vstage[16][kMaxHeadDim];
  const int h = blockIdx.y, b = blockIdx.z;
  const int D = p.head_dim;
  const AppendRun run = append_run(p, blockIdx.x, h, b);
  const int32_t L0 = run.L0, t_lo = run.t_lo, t_hi = run.t_hi;
  if (t_lo >= t_hi) return;
  const int n_tok = t_hi - t_lo;
  const int32_t bs_mask = (1 << p.log2_bs) - 1;

  constexpr int kVec = 16 / sizeof(E);  // elements per 16-byte chunk
  const int chunks = D / kVec;          // lanes per row: 8, 16, 32 or 64
  const E* kn = static_cast<const E*>(p.k_new);
  const E* vn = static_cast<const E*>(p.v_new);
  int8_t* kq = static_cast<int8_t*>(p.k_pool);
  int8_t* vq = static_cast<int8_t*>(p.v_pool);
  const int64_t tok_stride = (int64_t)p.num_kv_heads * D;            // elements between tokens
  const int64_t src0 = ((int64_t)b * p.t_new) * tok_stride + (int64_t)h * D;

  // Whole rows per pass (256 threads hold 256 / chunks rows), so a row's lanes are all active.
  for (int idx = threadIdx.x; idx < n_tok * chunks; idx += kAppendThreads) {
    const int r = idx / chunks, c = idx % chunks;
    const int32_t t = t_lo + r;
    const int64_t src = src0 + (int64_t)(t - L0) * tok_stride + c * kVec;
    const u32x4 kw = *reinterpret_cast<const u32x4*>(kn + src);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(vn + src);
    float xk[kVec], xv[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      const int word = i / (kVec / 4), sh = 32 / (kVec / 4) * (i % (kVec / 4));
      const uint32_t mask = sizeof(E) == 4 ? 0xffffffffu : 0xffffu;
      xk[i] = elem_to_f32<E>((kw[word] >> sh) & mask, p.dtype);
      xv[i] = elem_to_f32<E>((vw[word] >> sh) & mask, p.dtype);
    }
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      ak = fmaxf(ak, fabsf(xk[i]));
      av = fmaxf(av, fabsf(xv[i]));
    }
    for (int m = 1; m < chunks; m <<= 1) {   // the row's lanes are aligned in the wave
      ak = fmaxf(ak, __shfl_xor(ak, m, kWave));
      av = fmaxf(av, __shfl_xor(av, m, kWave));
    }
    const float inv_k = ak > 0.f ? __fdiv_rn(127.f, ak) : 0.f;
    const float inv_v = av > 0.f ? __fdiv_rn(127.f, av) : 0.f;
    const int32_t s = run.slot_of(p, t);
    const int64_t page = run.page_of(p, s);
    const int64_t row = (page << p.log2_bs) + (s & bs_mask);
    // K codes: kVec consecutive bytes of the token-major row, one store
    uint32_t kb[kVec / 4];
#pragma unroll
    for (int w = 0; w < kVec / 4; ++w) {
      kb[w] = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kb[w] |= ((uint32_t)quant_code(xk[4 * w + i], inv_k) & 0xffu) << (8 * i);
    }
    int8_t* kdst = kq + row * D + c * kVec;
    if constexpr (kVec == 8)
      *reinterpret_cast<u32x2*>(kdst) = u32x2{kb[0], kb[1]};
    else
      *reinterpret_cast<uint32_t*>(kdst) = kb[0];
#pragma unroll
    for (int i = 0; i < kVec; ++i) vstage[r][c * kVec + i] = (uint8_t)quant_code(xv[i], inv_v);
    if (c == 0) {
      p.k_scale[row] = ak > 0.f ? __fdiv_rn(ak, 127.f) : 0.f;
      p.v_scale[row] = av > 0.f ? __fdiv_rn(av, 127.f) : 0.f;
    }
  }
  __syncthreads();
  // V codes, channel-major: element (d, row) at page * D * bs + d * bs + row.
  const int32_t s0 = run.slot_of(p, t_lo);
  if (n_tok == 16 && (s0 & 15) == 0 && p.log2_bs >= 4) {
    // a whole run of 16 consecutive slots in one page: one 16-byte store per channel
    const int64_t page = run.page_of(p, s0);
    int8_t* vrow = vq + page * D * ((int64_t)1 << p.log2_bs) + (s0 & bs_mask);
    for (int d = threadIdx.x; d < D; d += kAppendThreads) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)vstage[4 * j][d] | ((uint32_t)vstage[4 * j + 1][d] << 8) |
               ((uint32_t)vstage[4 * j + 2][d] << 16) | ((uint32_t)vstage[4 * j + 3][d] << 24);
      *reinterpret_cast<u32x4*>(vrow + (int64_t)d * ((int64_t)1 << p.log2_bs)) = w;
    }
    return;
  }
  for (int idx = threadIdx.x; idx < 16 * D; idx += kAppendThreads) {
    const int r = idx & 15, d = idx >> 4;
    if (r >= n_tok) continue;
    const int32_t s = run.slot_of(p, t_lo + r);
    const int64_t page = run.page_of(p, s);
    vq[(page * D + d) * ((int64_t)1 << p.log2_bs) + (s & bs_mask)] = (int8_t)vstage[r][d];
  }
}

// 4-bit cache: every new K and V row is quantized with the static scales of its kv head
// (k_scale, v_scale [num_kv_heads][head_dim]). K rows (head_dim / 8 words, token-major) are written
// whole. A V page row holds the block_size codes of one channel, 8 tokens to a word, so a token
// changes half a byte of each channel's row: the run's codes are staged in LDS, and each word of
// the run is written whole when this workgroup owns all 8 of its tokens, else merged with atomic
// AND / OR on its own fields only (the other tokens of the word may belong to an earlier call, or
// to another workgroup of this call when the ring window starts inside the run).
__global__ void __launch_bounds__(kAppendThreads) append_int4_kernel(const AppendParams p) {
  __shared__ uint8_t vstage[16][kMaxHeadDim];
  const int h = blockIdx.y, b = blockIdx.z;
  const int D = p.head_dim;
  const AppendRun run = append_run(p, blockIdx.x, h, b);
  const int32_t L0 = run.L0, t_lo = run.t_lo, t_hi = run.t_hi;
  if (t_lo >= t_hi) return;
  const int n_tok = t_hi - t_lo;
  const int32_t bs_mask = (1 << p.log2_bs) - 1;
  const int words = D / 8;   // words of a K row; one thread per word and token
  const uint16_t* kn = static_cast<const uint16_t*>(p.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(p.v_new);
  uint8_t* kq = static_cast<uint8_t*>(p.k_pool);
  uint32_t* vq = static_cast<uint32_t*>(p.v_pool);
  const float* ks = p.k_scale + (int64_t)h * D;
  const float* vs = p.v_scale + (int64_t)h * D;
  const int64_t tok_stride = (int64_t)p.num_kv_heads * D;
  const int64_t src0 = ((int64_t)b * p.t_new) * tok_stride + (int64_t)h * D;

  for (int idx = threadIdx.x; idx < n_tok * words; idx += kAppendThreads) {
    const int r = idx / words, j = idx % words;
    const int32_t t = t_lo + r;
    const int64_t src = src0 + (int64_t)(t - L0) * tok_stride + j * 8;
    const u32x4 kw = *reinterpret_cast<const u32x4*>(kn + src);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(vn + src);
    const f32x4 ks0 = *reinterpret_cast<const f32x4*>(ks + j * 8);
    const f32x4 ks1 = *reinterpret_cast<const f32x4*>(ks + j * 8 + 4);
    const f32x4 vs0 = *reinterpret_cast<const f32x4*>(vs + j * 8);
    const f32x4 vs1 = *reinterpret_cast<const f32x4*>(vs + j * 8 + 4);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t kb = (kw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const uint32_t vb = (vw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const float sk = e < 4 ? ks0[e] : ks1[e - 4];
      const float sv = e < 4 ? vs0[e] : vs1[e - 4];
      word |= quant4_u(elem_to_f32<uint16_t>(kb, p.dtype), sk) << nibble_shift(e);
      vstage[r][j * 8 + e] = (uint8_t)quant4_u(elem_to_f32<uint16_t>(vb, p.dtype), sv);
    }
    const int32_t slot = run.slot_of(p, t);
    const int64_t row = (run.page_of(p, slot) << p.log2_bs) + (slot & bs_mask);
    *reinterpret_cast<uint32_t*>(kq + row * (D / 2) + j * 4) = word;
  }
  __syncthreads();
  // V: the run's slots are consecutive inside one 16-slot-aligned run of one page (pages hold >= 16
  // slots); this workgroup owns offsets [o_lo, o_lo + n_tok) of it.
  const int32_t s_first = run.slot_of(p, t_lo);
  const int32_t sr = s_first & ~15;
  const int o_lo = s_first - sr;
  const int64_t page = run.page_of(p, sr);
  // channel d's row of the page: bs / 8 words; the run's two words start at word (sr % bs) / 8
  uint32_t* vrow0 = vq + page * D * ((int64_t)1 << p.log2_bs) / 8 + (sr & bs_mask) / 8;
  for (int idx = threadIdx.x; idx < 2 * D; idx += kAppendThreads) {
    const int d = idx >> 1, w = idx & 1;
    uint32_t val = 0, mask = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int o = 8 * w + e;
      if (o >= o_lo && o < o_lo + n_tok) {
        val |= (uint32_t)vstage[o - o_lo][d] << nibble_shift(e);
        mask |= 0xFu << nibble_shift(e);
      }
    }
    if (mask == 0) continue;
    uint32_t* dst = vrow0 + (int64_t)d * ((int64_t)1 << p.log2_bs) / 8 + w;
    if (mask == 0xffffffffu) {
      *dst = val;
    } else {
      atomicAnd(dst, ~mask);
      atomicOr(dst, val);
    }
  }
}

}  // namespace

hipError_t launch_append_int4(const AppendParams& p, hipStream_t stream) {
  const int groups = p.t_new == 1 ? 1 : (p.t_new + 15) / 16 + 3;
  const dim3 grid(groups, p.num_kv_heads, p.batch);
  (void)hipGetLastError();  // report only this launch's status
  hipLaunchKernelGGL(append_int4_kernel, grid, dim3(kAppendThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_append_int8(const AppendParams& p, hipStream_t stream) {
  const int groups = p.t_new == 1 ? 1 : (p.t_new + 15) / 16 + 3;
  const dim3 grid(groups, p.num_kv_heads, p.batch);
  (void)hipGetLastError();  // report only this launch's status
  if (p.dtype == 0)
    hipLaunchKernelGGL(append_int8_kernel<uint32_t>, grid, dim3(kAppendThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(append_int8_kernel<uint16_t>, grid, dim3(kAppendThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, int elem_bytes, hipStream_t stream) {
  // Runs of 16 positions a (sequence, kv head) can touch: a single new token is one run; longer
  // appends may start mid-run and split at the sink / ring boundary.
  const int groups = p.t_new == 1 ? 1 : (p.t_new + 15) / 16 + 3;
  const dim3 grid(groups, p.num_kv_heads, p.batch);
  (void)hipGetLastError();  // report only this launch's status
  if (elem_bytes == 2)
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, dim3(kAppendThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(append_kernel<uint32_t>, grid, dim3(kAppendThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace duo
