// Device-side building blocks shared by the append, decode and prefill kernels (gfx950 only).
//
// Element types: float, _Float16, __bf16. An "8-vector" is the per-lane operand of one MFMA
// k-step: 8 consecutive elements of the contraction dimension (16 bytes for 16-bit types, 32 bytes
// for fp32). For fp32 one k-step of 8 is issued as eight k=4 (16x16) or k=2 (32x32) fp32 MFMAs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace duo {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

template <typename T> struct V8;
template <> struct V8<__bf16> { using type = bf16x8; };
template <> struct V8<_Float16> { using type = f16x8; };
template <> struct V8<float> { using type = f32x8; };
template <typename T> using v8 = typename V8<T>::type;

// 16-byte-aligned loads of 8 elements.
template <typename T>
__device__ __forceinline__ v8<T> load8(const T* p) {
  return *reinterpret_cast<const v8<T>*>(p);
}

// The same load marked non-temporal: data read once (streamed K/V) should not displace reused
// lines in the caches.
template <typename T>
__device__ __forceinline__ v8<T> load8_stream(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(v8<T>, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  } else {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
    return v8<T>{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

template <typename T>
__device__ __forceinline__ v8<T> zero8() {
  v8<T> z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = T(0.0f);
  return z;
}

// fp32 -> element, round to nearest even (hardware conversions on gfx950).
template <typename T> __device__ __forceinline__ T from_f32(float x) { return T(x); }

// Symmetric int8 code of x for a row whose largest magnitude is amax > 0, with inv = 127 / amax
// (correctly rounded): x * inv correctly rounded fp32, rounded half to even and clamped to
// [-127, 127]. The row's scale is amax / 127, correctly rounded (0 and codes 0 for an all-zero
// row). Shared by the int8 append and the decode's fused append, which must store the same bits.
__device__ __forceinline__ int32_t quant_code(float x, float inv) {
  const float c = rintf(__fmul_rn(x, inv));
  return (int32_t)fminf(fmaxf(c, -127.f), 127.f);
}

// 4-bit code of x with a per-channel scale s (0 -> code 0): x / s correctly rounded, rounded half
// to even and clamped to [-7, 7]; stored as u = code + 8. Shared by the 4-bit append and the
// decode's fused append.
__device__ __forceinline__ uint32_t quant4_u(float x, float s) {
  if (!(s > 0.f)) return 8u;
  const float c = fminf(fmaxf(rintf(__fdiv_rn(x, s)), -7.f), 7.f);
  return (uint32_t)((int32_t)c + 8);
}

// Position of element e (0..7) of a run of 8 codes in its 32-bit word: even elements in the low
// half, odd ones in the high half, 4 bits each, the first lowest.
__device__ __forceinline__ int nibble_shift(int e) { return (e & 1) * 16 + (e >> 1) * 4; }

// Eight int8 codes (8 consecutive bytes, 8-byte aligned) streamed past the caches, as two words.
__device__ __forceinline__ u32x2 load_codes8_stream(const int8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// Eight int8 codes (byte i of the two words is code i) as an MFMA operand: every code in
// [-127, 127] is exact in bf16, fp16 and fp32.
template <typename T>
__device__ __forceinline__ v8<T> codes_to_v8(u32x2 w) {
  v8<T> r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int32_t c = (int32_t)(w[i >> 2] << (24 - 8 * (i & 3))) >> 24;   // sign-extended byte
    r[i] = from_f32<T>((float)c);
  }
  return r;
}

// Eight 4-bit codes (one word of a 4-bit cache row: element 2i at bits 4i..4i+3, element 2i+1 at
// bits 16+4i..16+4i+3, stored as u = code + 8) as an MFMA operand holding 16 + u = 24 + code for
// every element, exactly: the bf16 with bits 0x4180 | (u << 3), the fp16 with bits 0x4C00 | (u << 6).
// Whoever multiplies the operand removes the offset 24. The mask and the exponent bits come in
// registers (Nib4Consts, set once), so each pair is one shift and one fused AND-OR: a VOP3
// instruction on gfx9 cannot carry the two 32-bit literals itself.
struct Nib4Consts {
  uint32_t mask, bits;
};
template <typename T>
__device__ __forceinline__ Nib4Consts nib4_consts() {
  Nib4Consts k;
  if constexpr (__is_same(T, __bf16)) {
    __asm__("v_mov_b32 %0, 0x00780078" : "=v"(k.mask));
    __asm__("v_mov_b32 %0, 0x41804180" : "=v"(k.bits));
  } else {
    __asm__("v_mov_b32 %0, 0x03C003C0" : "=v"(k.mask));
    __asm__("v_mov_b32 %0, 0x4C004C00" : "=v"(k.bits));
  }
  return k;
}
template <typename T>
__device__ __forceinline__ v8<T> nib8_plus24(uint32_t w, Nib4Consts k) {
  u32x4 r;
  if constexpr (__is_same(T, __bf16)) {
    r[0] = ((w << 3) & k.mask) | k.bits;
    r[1] = ((w >> 1) & k.mask) | k.bits;
    r[2] = ((w >> 5) & k.mask) | k.bits;
    r[3] = ((w >> 9) & k.mask) | k.bits;
  } else {
    r[0] = ((w << 6) & k.mask) | k.bits;
    r[1] = ((w << 2) & k.mask) | k.bits;
    r[2] = ((w >> 2) & k.mask) | k.bits;
    r[3] = ((w >> 6) & k.mask) | k.bits;
  }
  return __builtin_bit_cast(v8<T>, r);
}

template <typename T>
__device__ __forceinline__ v8<T> pack8(const float* x) {
  v8<T> r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = from_f32<T>(x[i]);
  return r;
}

// acc + the sum of the 8 elements of `p` (paired dot products with ones for 16-bit types, so that
// a softmax normaliser sums exactly the rounded weights the MFMA multiplies).
__device__ __forceinline__ float sum8(bf16x8 p, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {__bf16(1.0f), __bf16(1.0f)};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
}
__device__ __forceinline__ float sum8(f16x8 p, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 one = {_Float16(1.0f), _Float16(1.0f)};
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
}
__device__ __forceinline__ float sum8(f32x8 p, float acc) {
  return acc + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
}

// Keep element i of `v` where bit i of `keep` is set, else 0. Works on the raw bits so that NaN or
// Inf garbage is replaced, never multiplied.
template <typename T>
__device__ __forceinline__ v8<T> select8(v8<T> v, uint32_t keep) {
  v8<T> r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = ((keep >> i) & 1u) ? v[i] : T(0.0f);
  return r;
}

// Zero the elements of a 16-byte chunk whose keys t0 + i fall outside [lo, hi), on the raw
// 32-bit words (so NaN or Inf garbage is replaced, never multiplied). Element i of a chunk of
// 16-bit values is half (i & 1) of word i / 2; a chunk of fp32 values holds one element per word.
template <int kElemBytes>
__device__ __forceinline__ u32x4 zero_absent(u32x4 v, int32_t t0, int32_t lo, int32_t hi) {
  constexpr int kPerWord = 4 / kElemBytes;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < kPerWord; ++e) {
      const int32_t t = t0 + w * kPerWord + e;
      const uint32_t lane_bits = kPerWord == 2 ? (0xFFFFu << (16 * e)) : 0xFFFFFFFFu;
      m |= (t >= lo && t < hi) ? lane_bits : 0u;
    }
    v[w] &= m;
  }
  return v;
}

// ---- MFMA: C[16x16] += A[16 x 8k] * B[8k x 16] over one 8-element k-step per lane ---------------
// Lane layout (16x16 family): A row = lane % 16, B col = lane % 16, the lane's 8 k-elements belong
// to k-group lane / 16; C: col = lane % 16, rows 4 * (lane / 16) + [0..3].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

// ---- MFMA: C[32x32] += A[32 x 8k] * B[8k x 32] -------------------------------------------------
// Lane layout (32x32 family): A row = lane % 32, B col = lane % 32, k-group lane / 32;
// C: col = lane % 32, rows 8 * i + 4 * (lane / 32) + j for register 4 * i + j.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f32x8 a, f32x8 b, f32x16 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A value combined with the same value of lane (lane ^ 32) by one v_permlane32_swap, which trades
// the upper 32 lanes of its first operand for the lower 32 of its second: given v twice, every lane
// gets back its own v and its partner's, one in each result. (A shuffle would go through LDS.)
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same with lane (lane ^ 16): v_permlane16_swap trades the odd rows (16 lanes) of its first
// operand for the even rows of its second.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum / sum over the 64 lanes of a wave, in every lane, without LDS: DPP moves combine lane
// pairs inside quads (lane ^ 1, lane ^ 2), then the two quads of each 8 (row_half_mirror) and the
// two 8s of each row (row_mirror); the row swaps above finish it. Each step combines two values
// that are equal within their group, commutatively, so every lane ends with the same bits.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i within each 8
constexpr int kDppMirror = 0x140;       // lane i <-> 15 - i within each row
__device__ __forceinline__ float wave_max(float v) {
  v = __builtin_elementwise_maximum(v, dpp_move<kDppXor1>(v));
  v = __builtin_elementwise_maximum(v, dpp_move<kDppXor2>(v));
  v = __builtin_elementwise_maximum(v, dpp_move<kDppHalfMirror>(v));
  v = __builtin_elementwise_maximum(v, dpp_move<kDppMirror>(v));
  return max_xor32(max_xor16(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<kDppXor1>(v);
  v += dpp_move<kDppXor2>(v);
  v += dpp_move<kDppHalfMirror>(v);
  v += dpp_move<kDppMirror>(v);
  return add_xor32(add_xor16(v));
}

// Device-scope coherent store / load (write-through / read-through the XCD-local L2): used for
// the few bytes that one workgroup hands to another within a launch.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's outstanding memory operations have completed.
__device__ __forceinline__ void wait_stores_complete() {
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ int clamp_page(int32_t phys, int32_t num_blocks) {
  return min(max(phys, 0), num_blocks - 1);
}

// A 16-position run of one head's logical positions: t0 is the first position and `slot` the
// slot holding it (pages hold >= 16 slots and runs start at multiples of 16 slots, so a run never
// spans pages). Keys t in [lo, hi) are present and may be attended; `windowed` marks a streaming
// head's ring run, whose keys are further limited to the recent window of each query.
struct Run {
  int32_t t0, slot, lo, hi;
  bool windowed;
};

// Which 16-position runs a head exposes:
//   retrieval: runs at t0 = 16 g, g = 0, 1, ...   (slot t0)
//   streaming: sink runs at t0 = 16 j while 16 j < sink (slot t0);
//              ring runs at t0 = sink + 16 k       (slot SB*bs + (16 k mod ring_slots))
// Run positions are pure arithmetic; the page of a slot is one block-table read (page_of).
struct HeadGeom {
  const int32_t* row;     // this (sequence, kv head)'s block-table row
  int32_t num_blocks, log2_bs, sink, sink_blocks, ring_slots;
  __device__ __forceinline__ int32_t page_of(int32_t slot) const {
    return clamp_page(row[slot >> log2_bs], num_blocks);
  }
  __device__ __forceinline__ int32_t row0(int32_t slot) const {
    return slot & ((1 << log2_bs) - 1);
  }
  __device__ __forceinline__ Run retrieval_run(int32_t g, int32_t L) const {
    return Run{g * 16, g * 16, 0, L, false};
  }
  __device__ __forceinline__ Run sink_run(int32_t j, int32_t L) const {
    return Run{j * 16, j * 16, 0, min(sink, L), false};
  }
  __device__ __forceinline__ Run ring_run(int32_t k, int32_t lo, int32_t L) const {
    const int32_t off = (int32_t)(((int64_t)k * 16) % ring_slots);
    return Run{sink + k * 16, (sink_blocks << log2_bs) + off, lo, L, true};
  }
  __device__ __forceinline__ Run empty_run() const { return Run{0, 0, 0, 0, false}; }
};

// Runs of one work item, enumerated 0 .. n-1: a retrieval key range, or a streaming head's sink
// runs followed by the ring runs meeting a window.
struct RunList {
  bool ret;
  int32_t n, first, n_sink, k_lo, ring_lo, L;
  // Positions only (no slot): what masks and visibility need, no division.
  __device__ __forceinline__ Run pos(const HeadGeom& g, int32_t v) const {
    if (v >= n) return Run{0, 0, 0, 0, false};
    if (ret) return Run{(first + v) * 16, 0, 0, L, false};
    if (v < n_sink) return Run{v * 16, 0, 0, min(g.sink, L), false};
    return Run{g.sink + (k_lo + v - n_sink) * 16, 0, ring_lo, L, true};
  }
  __device__ __forceinline__ Run at(const HeadGeom& g, int32_t v) const {
    if (v >= n) return g.empty_run();
    if (ret) return g.retrieval_run(first + v, L);
    if (v < n_sink) return g.sink_run(v, L);
    return g.ring_run(k_lo + (v - n_sink), ring_lo, L);
  }
};

// Where a segment of runs lives, staged in LDS so that no K/V load waits on a block-table read:
// packed = page * 16 + row0 / 16 (row0 is a multiple of 16 below block_size <= 256).
constexpr int kRunSeg = 512;

__device__ __forceinline__ int32_t pack_run(int32_t page, int32_t row0) { return page * 16 + (row0 >> 4); }
__device__ __forceinline__ int32_t packed_page(int32_t packed) { return packed >> 4; }
__device__ __forceinline__ int32_t packed_row0(int32_t packed) { return (packed & 15) << 4; }

template <int kThreads>
__device__ __forceinline__ void load_pages(int32_t* sm_run, const HeadGeom& g, const RunList& rl,
                                           int32_t seg0, int32_t nseg) {
  for (int i = threadIdx.x; i < nseg; i += kThreads) {
    const int32_t slot = rl.at(g, seg0 + i).slot;
    sm_run[i] = pack_run(g.page_of(slot), g.row0(slot));
  }
}

}  // namespace duo
