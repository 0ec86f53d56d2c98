// duo_attn_decode kernel: split-K flash-decode over the paged, per-head circular cache with the
// split merge fused into the same launch.
//
// What is computed (DuoAttention README, abstract; transformers PR "[WIP] Dynamic length in static
// cache", description): the query of sequence b at position p = L - 1 attends, per kv head h, to
//   retrieval head: positions [0, L)
//   streaming head: positions [0, min(sink, L)) and [max(sink, W(L - 1)), L)
// where the recent window of a query at p starts at W(p) = (p & win_mask) - win_back: p - recent + 1
// for a window of the recent newest positions, or the first position of the -recent newest blocks
// for the block-granular window (vLLM issue "Could you support Attention Sink?", ChuanhongLi's
// comment: keep the first block, drop middle blocks, keep the recent blocks), with scores softmax_scale * (q . k) formed in fp32 (vLLM DualChunkAttention PR, review thread on
// the fp32 scale). Partial results over disjoint key ranges are merged through their log-sum-exp
// (same review thread).
//
// Work decomposition. One workgroup (eight waves up to D = 128, four at D = 256) = one work item:
//   retrieval head: (b, h, split s) over keys [s*S, (s+1)*S), S = split_tokens;
//   streaming head: (b, h) over its sink runs and the ring runs that meet the recent window.
// The grid comes from static capacities only (no host read of the lengths); items past the valid
// length exit at once. Streaming items come first in the grid and the last split of every
// retrieval row last: with one workgroup per CU the streaming items run beside the first retrieval
// splits, and the last splits, which the host makes shorter, start on the CUs they free. A wave
// processes steps of two 16-key runs (32 keys; four runs for the 4-bit cache); wave w starts with
// step w and then claims the next unclaimed step, and the waves are merged in LDS at the end.
//
// MFMA formulation (16x16x32, one k-step = 8 elements per lane). All q heads of a kv head (the GQA
// group, G <= 16) ride in the 16 columns, so K and V are read once per kv head:
//   S^T[key, g] = sum_d K[key, d] Q[g, d]       A = K rows (from the token-major K page),
//                                               B = Q^T (registers for the whole item)
//   O^T[d, g]  += sum_key V^T[d, key] P^T[key, g] A = V^T (from the channel-major V page),
//                                               B = P^T straight from the S^T accumulators.
// The K rows of each 16-row MFMA are permuted so that the S^T accumulator a lane holds covers the
// same 8 consecutive keys that the lane loads as its V^T operand: no LDS, no cross-lane moves.
//
// K and V are streamed with non-temporal loads: each byte is read once per launch.
//
// Split merge: each retrieval item writes (m, l, O) for its G q heads to the workspace, then takes a
// ticket on the (b, h) counter; the last item merges the partials, writes the output and resets the
// counter to zero for the next call. Up to 256 splits it merges in two phases (per q head the
// merged max, denominator and each split's weight, then the weighted partial outputs with many
// loads in flight), since each of its loads is a round trip to another XCD's writes.
//
// Dual Chunk Attention (vLLM PR "[Model] Implement DualChunkAttention for Qwen2 Models": the paged
// decode beside the prefill; review thread on the query swap and on mscale): every kv head is a full
// head, and the query vector that meets a key depends on the chunk (t / chunk_len) of the key
// against the chunk of the decoded position: q in the same chunk, q_succ in the one before, q_inter
// further back. A wave step (32 keys) lies in one chunk (chunk_len is a multiple of 64), and every
// lane of an item shares the query position, so the choice is uniform per step; the Q^T registers
// are reloaded when it changes, at most twice per item. The scale is softmax_scale times the
// sequence's fp32 mscale.
#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "decode_body.h"
#include "duo_common.h"
#include "duo_kernels.h"

namespace duo {

namespace {

template <typename T, int D>
__global__ void __launch_bounds__((decode_waves<D>() * kWave), 1) decode_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds[DecodeLds<decode_waves<D>(), D>::kBytes];
  decode_body<T, D, false>(p, blockIdx.x, lds);
}

// Decode with the fused append of one token per (sequence, kv head) (DecodeParams::k_new).
template <typename T, int D>
__global__ void __launch_bounds__((decode_waves<D>() * kWave), 1) decode_append_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds[DecodeLds<decode_waves<D>(), D>::kBytes];
  decode_body<T, D, false, false, false, decode_waves<D>(), true>(p, blockIdx.x, lds);
}

// Decode over the int8 cache with the fused append: the token is quantized as the int8 append does.
template <typename T, int D>
__global__ void __launch_bounds__((decode_waves<D>() * kWave), 1) decode_int8_append_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds[DecodeLds<decode_waves<D>(), D>::kBytes];
  decode_body<T, D, true, false, false, decode_waves<D>(), true>(p, blockIdx.x, lds);
}

// Decode over the 4-bit cache with the fused append (the 4-bit append's codes).
template <typename T, int D>
__global__ void __launch_bounds__((decode_waves<D>() * kWave), 1) decode_int4_append_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds[DecodeLds<decode_waves<D>(), D>::kBytes];
  decode_body<T, D, false, false, true, decode_waves<D>(), true>(p, blockIdx.x, lds);
}

// Decode over the int8 cache (one fp32 scale per slot for K and for V).
template <typename T, int D>
__global__ void __launch_bounds__((decode_waves<D>() * kWave), 1) decode_int8_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds[DecodeLds<decode_waves<D>(), D>::kBytes];
  decode_body<T, D, true>(p, blockIdx.x, lds);
}

// Decode over the 4-bit cache (one fp32 scale per kv head and channel for K and for V).
template <typename T, int D>
__global__ void __launch_bounds__((decode_waves<D>() * kWave), 1) decode_int4_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds[DecodeLds<decode_waves<D>(), D>::kBytes];
  decode_body<T, D, false, false, true>(p, blockIdx.x, lds);
}

// Dual Chunk Attention decode (16-bit cache, every kv head a full head).
template <typename T, int D>
__global__ void __launch_bounds__((decode_waves<D>() * kWave), 1) decode_dca_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds[DecodeLds<decode_waves<D>(), D>::kBytes];
  decode_body<T, D, false, true>(p, blockIdx.x, lds);
}

template <typename T, int D>
void launch_d(const DecodeParams& p, int quant, int grid, hipStream_t stream) {
  const LaunchEvents ev = current_launch_events();
  if constexpr (!std::is_same<T, float>::value) {
    if (quant == 4) {
      if (p.k_new != nullptr)
        hipExtLaunchKernelGGL((decode_int4_append_kernel<T, D>), dim3(grid),
                              dim3(decode_waves<D>() * kWave), 0, stream, ev.start, ev.stop, 0, p);
      else
        hipExtLaunchKernelGGL((decode_int4_kernel<T, D>), dim3(grid),
                              dim3(decode_waves<D>() * kWave), 0, stream, ev.start, ev.stop, 0, p);
      return;
    }
  }
  if (quant == 8 && p.k_new != nullptr)
    hipExtLaunchKernelGGL((decode_int8_append_kernel<T, D>), dim3(grid),
                          dim3(decode_waves<D>() * kWave), 0, stream, ev.start, ev.stop, 0, p);
  else if (quant == 8)
    hipExtLaunchKernelGGL((decode_int8_kernel<T, D>), dim3(grid), dim3(decode_waves<D>() * kWave), 0,
                          stream, ev.start, ev.stop, 0, p);
  else if (p.k_new != nullptr)
    hipExtLaunchKernelGGL((decode_append_kernel<T, D>), dim3(grid), dim3(decode_waves<D>() * kWave),
                          0, stream, ev.start, ev.stop, 0, p);
  else
    hipExtLaunchKernelGGL((decode_kernel<T, D>), dim3(grid), dim3(decode_waves<D>() * kWave), 0,
                          stream, ev.start, ev.stop, 0, p);
}

template <typename T, int D>
void launch_dca_d(const DecodeParams& p, int grid, hipStream_t stream) {
  const LaunchEvents ev = current_launch_events();
  hipExtLaunchKernelGGL((decode_dca_kernel<T, D>), dim3(grid), dim3(decode_waves<D>() * kWave), 0,
                        stream, ev.start, ev.stop, 0, p);
}

template <typename T>
hipError_t launch_t(const DecodeParams& p, int head_dim, int quant, int grid, hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's status
  if (quant == 4 && std::is_same<T, float>::value) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: launch_d<T, 64>(p, quant, grid, stream); break;
    case 128: launch_d<T, 128>(p, quant, grid, stream); break;
    case 256: launch_d<T, 256>(p, quant, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

// ---- scratch of the no-alloc decode ------------------------------------------------------------
// Callers that cannot allocate device memory (graph capture, serving loops, harnesses that forbid
// it) get the decode workspace from this array instead. Every GPU the library runs on holds its own
// copy until the process ends; calls on one GPU share it.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  // The symbol's address differs per device: look it up once per device, with that device
  // current, and keep it. The array's name in host code is only a stand-in for the symbol.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_zero_words(uint32_t* p, size_t n_words, hipStream_t stream) {
  (void)hipGetLastError();
  const size_t blocks = std::min<size_t>((n_words + 255) / 256, 1024);
  if (blocks > 0) hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n_words);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, int quant, int grid,
                         hipStream_t stream) {
  if (dtype == 0) return launch_t<float>(p, head_dim, quant, grid, stream);
  if (dtype == 1) return launch_t<_Float16>(p, head_dim, quant, grid, stream);
  return launch_t<__bf16>(p, head_dim, quant, grid, stream);
}

hipError_t launch_decode_dca(const DecodeParams& p, int dtype, int head_dim, int grid,
                             hipStream_t stream) {
  (void)hipGetLastError();
  if (dtype != 1 && dtype != 2) return hipErrorInvalidValue;
  if (head_dim == 64) {
    if (dtype == 1) launch_dca_d<_Float16, 64>(p, grid, stream);
    else launch_dca_d<__bf16, 64>(p, grid, stream);
  } else if (head_dim == 128) {
    if (dtype == 1) launch_dca_d<_Float16, 128>(p, grid, stream);
    else launch_dca_d<__bf16, 128>(p, grid, stream);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace duo
