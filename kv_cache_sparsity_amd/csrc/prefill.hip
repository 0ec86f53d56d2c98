// duo_attn_prefill kernel: tiled flash attention of a prompt chunk over the paged cache.
//
// What is computed (DuoAttention README, abstract and efficiency section; transformers PR
// "[WIP] Dynamic length in static cache"): query row i of sequence b sits at position
// p = L - q_len + i and attends causally (keys j <= p); a streaming head further keeps only the sink
// positions j < sink and its recent window j >= W(p) = (p & win_mask) - win_back (p - recent + 1, or
// the first position of the newest blocks for the block-granular window; see the decode kernel).
// Scores are softmax_scale * (q . k) in fp32 (vLLM DualChunkAttention PR, review thread).
//
// Work decomposition. A work item is (b, q head, tile of R query rows); R = 32 x waves (256 with
// eight waves, 128 with four). The item walks only the 16-key runs that can be visible to its rows:
//   retrieval head: runs 0 .. p_hi / 16;
//   streaming head: the sink runs, then the ring runs covering [W(p_lo), p_hi].
// So a streaming item costs about (sink + window + R) keys whatever the context length. A retrieval
// item's key tiles are split in n_split contiguous ranges, one workgroup each; the workgroups write
// partial softmax states (m, l, O) to the workspace and the last to arrive merges them through
// their log-sum-exp (vLLM DualChunkAttention PR, review thread) and writes the output. Retrieval
// items come first in the grid, latest rows first (they scan the most keys); within a row tile the
// kv head varies fastest, so that a GQA group's workgroups share XCDs.
//
// Inside a workgroup every wave owns 32 rows and all waves work on the same 64-key tile, so each
// K/V byte brought into LDS serves all R rows: copy traffic per MFMA is what the L2 -> LDS path
// (and the chip's power) pays for, and it halves from 128 to 256 rows.
//
// Data movement: four runs (64 keys) form one K/V tile, copied straight from the pages into LDS by
// 16-byte global->LDS loads (no staging registers); run r of a tile is copied by the waves w with
// w mod 4 = r. Tiles rotate through a ring of stages: with four stages the copies run two tiles
// ahead of the math, and the second half of the waves works half a tile behind the first (the PV
// of its previous tile, whose V is still in its stage, comes first), so that on each SIMD one wave's
// softmax overlaps the other's MFMAs; with two stages (64 KiB tiles) the copies run one tile ahead.
// Rows are XOR-swizzled in 16-byte units instead of padded, so both the copies and the MFMA operand
// reads are free of LDS bank conflicts. V channels of absent keys (past the valid length, unwritten
// sink slots) are read from a zero chunk, or zeroed in LDS when a chunk is only partly absent;
// absent K rows are masked by position. Where each run lives (page, row) and how each tile is
// classified for each wave are resolved once per segment of 512 runs; a tile's classification is
// taken when its copies are issued. One barrier per tile: each wave waits for its own copies of the
// tile (later tiles' copies stay in flight), then the barrier makes all of them visible.
//
// MFMA formulation (32x32x16, k-step of 8 elements per lane), per 32-key block:
//   S^T[key, row] = sum_d K[key, d] Q[row, d]       A = K rows (LDS), B = Q^T (registers)
//   O^T[d, row]  += sum_key V^T[d, key] P^T[key, row] A = V^T (LDS, channel-major like the V page),
//                                                     B = P^T taken from the S^T accumulators.
// K rows sit in LDS in a permuted order so that the eight S^T accumulators a lane holds per
// 16-key chunk are the chunk's keys 8*(lane/32) .. +7, the k-group of its P^T operand.
//
// Dual Chunk Attention (vLLM PR "[Model] Implement DualChunkAttention for Qwen2 Models", review
// thread on the brute-force prefill and on mscale) is the same walk over a cache of full heads with
// two changes. The query vector that meets a key depends on the chunks (chunk(t) = t / chunk_len)
// of the two: the row's own q within its chunk, q_succ in the chunk before, q_inter further back.
// Chunk lengths are multiples of the 64-key tile, so a tile lies in one chunk and each lane (one
// query row of the B operand) picks its vector per tile; a lane reloads its Q^T registers only when
// its kind changes, at most twice along the ascending walk. The scores scale is softmax_scale times
// the row's fp32 mscale, applied to the fp32 accumulators.
#include <hip/hip_ext.h>

#include "decode_body.h"
#include "duo_common.h"
#include "duo_kernels.h"

namespace duo {

// Sixteen zero bytes: the source of V chunks whose keys are all absent.
__device__ __attribute__((aligned(64))) uint32_t g_prefill_zero_chunk[16];

namespace {

constexpr int kKeys = kPrefillKeyTile;   // keys per K/V tile (four 16-key runs)
constexpr int kLdsAhead = 4;   // LDS operand reads kept in flight ahead of the MFMAs

// Row of the 32-key block that holds key r of the block (an involution: swaps the middle two
// groups of four in each half).
__device__ __forceinline__ int perm32(int r) {
  const int a = (r >> 2) & 3;
  const int off = (a == 1) ? 8 : (a == 2) ? 4 : (a == 3) ? 12 : 0;
  return (r & 16) + off + (r & 3);
}

template <typename T, int D>
struct TileGeo {
  static constexpr int kChunk = 16 / sizeof(T);              // elements per 16-byte chunk
  // K tile: [64 keys][D], rows permuted (perm32) and 16-byte chunks XOR-swizzled by row
  static constexpr int kKRowBytes = D * sizeof(T);
  static constexpr int kKRowChunks = D / kChunk;             // chunks per K row
  static constexpr int kKSwz = kKRowChunks < 16 ? kKRowChunks : 16;
  static constexpr int kKRunBytes = 16 * kKRowBytes;         // one 16-key run
  static constexpr int kKBytes = 4 * kKRunBytes;
  // V tile: [4 runs][D channels][16 keys], as in the page; the 16-byte chunks of a channel row are
  // XOR-swizzled by (d / rows per 256 bytes) so that 32 lanes reading one chunk each of 32
  // consecutive channels hit distinct banks
  static constexpr int kVRowBytes = 16 * sizeof(T);          // one channel of one run
  static constexpr int kVRowChunks = kVRowBytes / 16;
  static constexpr int kVRowsPer256 = 256 / kVRowBytes;
  static constexpr int kVRunBytes = D * kVRowBytes;
  static constexpr int kVBytes = 4 * kVRunBytes;
  // workgroup shape
  static constexpr int kWaves = prefill_waves(sizeof(T), D);
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRows = 32 * kWaves;
  static constexpr int kStages = 4 * (kKBytes + kVBytes) <= 128 * 1024 ? 4 : 2;
  static constexpr int kAhead = kStages == 4 ? 2 : 1;        // tiles in flight ahead of the math
  static constexpr bool kLag = kStages == 4 && kWaves == 8;  // second half of the waves lags
  // run r of a tile is copied by the waves w = r (mod 4), 1 KiB per instruction
  static constexpr int kCopyWaves = kWaves / 4;
  static constexpr int kKLoadsPerWave = kKRunBytes / 1024 / kCopyWaves;
  static constexpr int kVLoadsPerWave = kVRunBytes / 1024 / kCopyWaves;
  static constexpr int kCopiesPerTile = kKLoadsPerWave + kVLoadsPerWave;
  __device__ static __forceinline__ int vswz(int d) { return (d / kVRowsPer256) & (kVRowChunks - 1); }
};

template <typename V>
__device__ __forceinline__ V sel4(const V (&a)[4], int i) {
  return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3];
}

// 8-element MFMA operand from a swizzled LDS row: logical chunk `chunk` sits at chunk ^ swz.
template <typename T>
__device__ __forceinline__ v8<T> lds_operand(const char* row, int chunk, int swz) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const v8<T>*>(row + ((chunk ^ swz) << 4));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + ((chunk ^ swz) << 4));
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + (((chunk + 1) ^ swz) << 4));
    return v8<T>{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// Byte address of a location in LDS (what M0 and ds instructions take).
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// 16 bytes per lane from global memory straight into LDS: global_load_lds_dwordx4 writes lane i's
// bytes at M0 + 16 i (M0 = lds_base, wave-uniform; one wait state after M0 is written). It is
// issued as inline assembly so that the compiler does not track it: it cannot tell which stage an
// LDS read touches, so it would make every operand read wait for all copies in flight, the
// look-ahead ones included. The kernel orders copies and reads itself, by vmcnt and barrier
// (wait_older_then_barrier).
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

// Wait until at most `n` of this wave's vector memory operations are outstanding (they complete in
// order, so every older one has landed) and its LDS operations have completed, then meet the other
// waves at the barrier. Unlike __syncthreads() this leaves younger copies in flight.
// s_waitcnt immediate: vmcnt(0), other counters not waited on.
constexpr int kWaitVmcnt0 = (0 & 15) | (7 << 4) | (15 << 8) | ((0 >> 4) << 14);

template <int n>
__device__ __forceinline__ void wait_older_then_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  constexpr int kImm = (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14);   // vmcnt(n) expcnt(7) lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kImm);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Scheduling hint for a run of `n` MFMAs whose A operands are `n` LDS reads issued in the same
// region: keep `ahead` reads in flight (reads first, then one MFMA per further read), so that each
// MFMA waits for a read issued `ahead` operands earlier instead of the one just before it.
template <int n, int ahead>
__device__ __forceinline__ void pipeline_lds_mfma() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
#pragma unroll
  for (int i = 0; i < ahead; ++i) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
#pragma unroll
  for (int i = 0; i < n - ahead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < ahead; ++i) __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
}

template <int bytes, bool used>
struct StageBytes { static constexpr int value = used ? bytes : 16; };

// Packed batches: the sequence and row tile of global row tile gt, where the live row tiles of the
// sequences are numbered one after the other (sequence b owns ceil(n_b / rows) of them, or none
// when its single row goes to a decode item). Every thread of the workgroup calls this; it returns
// false when gt lies past the last live tile. The sequences are scanned kScan at a time (an
// inclusive prefix sum in LDS); `scratch` holds kScan + 2 ints of LDS.
template <int kThreads>
__device__ __forceinline__ bool find_packed_tile(const PrefillParams& p, int rows, int gt, int* scratch,
                                                 int* b_out, int* qt_out) {
  constexpr int kScan = kThreads < 256 ? kThreads : 256;
  const int tid = threadIdx.x;
  int base = 0;   // live tiles of the sequences before this chunk
  if (tid == 0) scratch[kScan] = -1;
  for (int c0 = 0; c0 < p.batch; c0 += kScan) {
    const int b = c0 + tid;
    int tiles = 0;
    if (tid < kScan && b < p.batch) {
      const int32_t s0 = min(max(p.q_start[b], 0), p.total_q);
      const int32_t s1 = min(max(p.q_start[b + 1], s0), p.total_q);
      const int32_t n = min(s1 - s0, p.q_len);
      tiles = (p.skip_single_rows && n == 1) ? 0 : (n + rows - 1) / rows;
    }
    __syncthreads();
    if (tid < kScan) scratch[tid] = tiles;
    __syncthreads();
    for (int o = 1; o < kScan; o <<= 1) {
      const int v = (tid < kScan && tid >= o) ? scratch[tid - o] : 0;
      __syncthreads();
      if (tid < kScan) scratch[tid] += v;
      __syncthreads();
    }
    if (tid < kScan && tiles > 0) {
      const int incl = base + scratch[tid];
      if (gt < incl && gt >= incl - tiles) {
        scratch[kScan] = b;
        scratch[kScan + 1] = gt - (incl - tiles);
      }
    }
    base += scratch[kScan - 1];
    __syncthreads();
    if (scratch[kScan] >= 0) break;
  }
  const int found = scratch[kScan];
  *b_out = found;
  *qt_out = scratch[kScan + 1];
  __syncthreads();   // the scratch is the page list's: everybody has read it
  return found >= 0;
}

// The stage ring as one block of LDS (the mixed kernel, whose decode items use its start).
template <typename T, int D>
struct PrefillLdsLayout {
  using TG = TileGeo<T, D>;
  static constexpr int kK23 = StageBytes<TG::kKBytes, TG::kStages == 4>::value;
  static constexpr int kV23 = StageBytes<TG::kVBytes, TG::kStages == 4>::value;
  static constexpr int kOffK0 = 0;
  static constexpr int kOffV0 = TG::kKBytes;
  static constexpr int kOffK1 = TG::kKBytes + TG::kVBytes;
  static constexpr int kOffV1 = kOffK1 + TG::kKBytes;
  static constexpr int kOffK2 = 2 * (TG::kKBytes + TG::kVBytes);
  static constexpr int kOffV2 = kOffK2 + kK23;
  static constexpr int kOffK3 = kOffV2 + kV23;
  static constexpr int kOffV3 = kOffK3 + kK23;
  static constexpr int kBytes = kOffV3 + kV23;
};

// MIX: a packed batch of prompt chunks and single decode rows in one launch. Blocks below
// n_prefill are prefill items of the sequences with more than one row; the others are split-K
// decode items (decode_body, the decode kernels' work item, over dp) that run for the sequences
// with exactly one row. The stage ring is then one block of LDS, whose start the decode items use.
template <typename T, int D, bool DCA, bool MIX>
__global__ void __launch_bounds__((TileGeo<T, D>::kThreads), 1) prefill_kernel(
    const PrefillParams p, const DecodeParams dp, int n_prefill) {
  using TG = TileGeo<T, D>;
  constexpr int kThreads = TG::kThreads;
  constexpr int kWaves = TG::kWaves;
  constexpr int kRows = TG::kRows;
  constexpr int kStages = TG::kStages;
  constexpr int kAhead = TG::kAhead;
  constexpr bool kLag = TG::kLag;
  constexpr int DC = D / 16;  // k-steps over the head dim (16 channels per 32x32 MFMA step)
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  // the stage ring (stages 2 and 3 only with four stages)
  constexpr int kK23 = StageBytes<TG::kKBytes, kStages == 4>::value;
  constexpr int kV23 = StageBytes<TG::kVBytes, kStages == 4>::value;
  using LL = PrefillLdsLayout<T, D>;
  constexpr int kSep = MIX ? 16 : 1;   // separate stage arrays (their size when unused: 16 bytes)
  __shared__ __attribute__((aligned(1024))) char k_lds0[MIX ? 16 : TG::kKBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds0[MIX ? 16 : TG::kVBytes];
  __shared__ __attribute__((aligned(1024))) char k_lds1[MIX ? 16 : TG::kKBytes];
  __shared__ __attribute__((aligned(1024))) char v_lds1[MIX ? 16 : TG::kVBytes];
  __shared__ __attribute__((aligned(1024))) char k_lds2[MIX ? 16 : kK23];
  __shared__ __attribute__((aligned(1024))) char v_lds2[MIX ? 16 : kV23];
  __shared__ __attribute__((aligned(1024))) char k_lds3[MIX ? 16 : kK23];
  __shared__ __attribute__((aligned(1024))) char v_lds3[MIX ? 16 : kV23];
  __shared__ __attribute__((aligned(1024))) char ring[MIX ? LL::kBytes : 16];
  __shared__ int32_t sm_run[kRunSeg];
  __shared__ int32_t sm_flags[kRunSeg / 4];   // per tile of the segment: see tile_flags
  __shared__ int sm_ticket;
  (void)kSep;
  if constexpr (MIX) {
    static_assert(DecodeLds<TG::kWaves, D>::kBytes <= LL::kBytes, "decode items fit the ring");
    if ((int)blockIdx.x >= n_prefill) {
      decode_body<T, D, false, false, false, TG::kWaves>(dp, (int)blockIdx.x - n_prefill, ring);
      return;
    }
  }
  auto kst = [&](auto C) -> char* {
    constexpr int c = decltype(C)::value;
    if constexpr (MIX) {
      if constexpr (c == 0) return ring + LL::kOffK0;
      else if constexpr (c == 1) return ring + LL::kOffK1;
      else if constexpr (c == 2) return ring + LL::kOffK2;
      else return ring + LL::kOffK3;
    } else {
      if constexpr (c == 0) return k_lds0;
      else if constexpr (c == 1) return k_lds1;
      else if constexpr (c == 2) return k_lds2;
      else return k_lds3;
    }
  };
  auto vst = [&](auto C) -> char* {
    constexpr int c = decltype(C)::value;
    if constexpr (MIX) {
      if constexpr (c == 0) return ring + LL::kOffV0;
      else if constexpr (c == 1) return ring + LL::kOffV1;
      else if constexpr (c == 2) return ring + LL::kOffV2;
      else return ring + LL::kOffV3;
    } else {
      if constexpr (c == 0) return v_lds0;
      else if constexpr (c == 1) return v_lds1;
      else if constexpr (c == 2) return v_lds2;
      else return v_lds3;
    }
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int rcol = lane & 31;  // MFMA column = query row within the wave
  const int half = lane >> 5;  // k-group of the lane
  const int G = p.group;

  // ---- which item -------------------------------------------------------------------------------
  // Row tiles come per sequence (fixed-length calls: sequence b's n_qtiles tiles), or, in a packed
  // batch, as one list of the live tiles of all sequences (n_qtiles bounds its length), found on
  // the device from q_start.
  const bool packed = !DCA && p.q_start != nullptr;
  const int n_split = p.n_split;
  const int seqs = packed ? 1 : p.batch;
  const int per_tile_r = seqs * p.n_ret * G;
  const int ret_items = per_tile_r * p.n_qtiles;
  int b, hq, qt, split = 0, item = 0;
  bool ret;
  if ((int)blockIdx.x < ret_items * n_split) {
    // split-major, so that the workgroups of one head and split (same keys) share an XCD's L2
    split = blockIdx.x / ret_items;
    item = blockIdx.x % ret_items;
    qt = p.n_qtiles - 1 - item / per_tile_r;
    int r = item % per_tile_r;
    b = r / (p.n_ret * G);
    r %= p.n_ret * G;
    // kv head fastest: workgroup i runs on XCD i mod 8, so the q heads that read one kv head's
    // keys gather on the same XCDs (and L2s) instead of every XCD reading every kv head
    hq = p.ret_heads[r % p.n_ret] * G + r / p.n_ret;
    ret = true;
  } else {
    const int per_tile_s = seqs * p.n_str * G;
    const int it = blockIdx.x - ret_items * n_split;
    qt = p.n_qtiles - 1 - it / per_tile_s;
    int r = it % per_tile_s;
    b = r / (p.n_str * G);
    r %= p.n_str * G;
    hq = p.str_heads[r % p.n_str] * G + r / p.n_str;
    ret = false;
  }
  if constexpr (!DCA) {   // (Dual Chunk Attention takes no packed batches)
    if (packed) {   // qt is the global live tile: which sequence and tile (the same for every split)
      if (!find_packed_tile<kThreads>(p, kRows, qt, sm_run, &b, &qt)) return;
    }
  }
  const int h = hq / G;
  int32_t L = max(p.seq_lens[b], 0);
  if (ret) L = min(L, p.max_blocks_per_head << p.log2_bs);
  // The sequence's query rows: rows [q0, q0 + qn) of q and out.
  int64_t q0;
  int32_t qn;
  if (packed) {   // packed batch: bounds from the device, clamped into [0, total_q)
    const int32_t s0 = min(max(p.q_start[b], 0), p.total_q);
    const int32_t s1 = min(max(p.q_start[b + 1], s0), p.total_q);
    q0 = s0;
    qn = min(s1 - s0, p.q_len);
  } else {
    q0 = (int64_t)b * p.q_len;
    qn = p.q_len;
  }
  const int row0 = qt * kRows;
  const int n_rows = min(kRows, qn - row0);
  // A row tile past the sequence's rows has nothing to do; every split of its item sees the same,
  // so none of them takes a ticket.
  if (n_rows <= 0) return;
  const int32_t p_lo = L - qn + row0;            // position of the tile's first row
  const int32_t p_hi = p_lo + n_rows - 1;

  HeadGeom geo;
  geo.row = p.table + ((int64_t)b * p.num_kv_heads + h) * p.max_blocks_per_head;
  geo.num_blocks = p.num_blocks;
  geo.log2_bs = p.log2_bs;
  geo.sink = p.sink;
  geo.sink_blocks = p.sink_blocks;
  geo.ring_slots = p.ring_slots;

  RunList rl;
  rl.ret = ret;
  rl.L = L;
  rl.n = rl.first = rl.n_sink = rl.k_lo = 0;
  rl.ring_lo = p.sink;   // ring keys are present from the sink on; the window is per row
  if (p_hi >= 0) {
    if (ret) {
      rl.n = p_hi / 16 + 1;
    } else {
      rl.n_sink = (min(p.sink, p_hi + 1) + 15) / 16;
      int32_t n_ring = 0;
      if (p_hi >= p.sink) {
        rl.k_lo = (max(p.sink, (p_lo & p.win_mask) - p.win_back) - p.sink) / 16;
        n_ring = (p_hi - p.sink) / 16 - rl.k_lo + 1;
      }
      rl.n = rl.n_sink + n_ring;
    }
  }
  const int32_t n_runs = rl.n;

  const T* kpool = static_cast<const T*>(p.k_pool);
  const T* vpool = static_cast<const T*>(p.v_pool);
  const int64_t page_elems = (int64_t)D << p.log2_bs;
  const int bs = 1 << p.log2_bs;
  int32_t seg0 = 0;   // first run whose location sits in sm_run[0]

  // ---- the wave's query rows: Q^T operand (B of S^T) ----------------------------------------
  const int wrow0 = wave * 32;                       // first row of this wave inside the tile
  const int qrow = row0 + wrow0 + rcol;              // chunk row of this lane's column
  const bool wave_live = wrow0 < n_rows;
  v8<T> qT[DC];
  {
    const bool ok = qrow < qn;
    const T* src = static_cast<const T*>(p.q) + ((q0 + (ok ? qrow : 0)) * p.num_q_heads + hq) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qT[dc] = ok ? load8(src + dc * 16 + half * 8) : zero8<T>();
  }
  f32x16 oT[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) oT[i][j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int32_t my_p = p_lo + wrow0 + rcol;          // this lane's query position
  // Scores scale (log2 domain) of this lane's row, and for Dual Chunk Attention the first tiles of
  // the row's own chunk and of the chunk before it (tiles below t_succ take q_inter). Rows before
  // the sequence start (p < 0) see no key; they keep kind 0.
  float sl2 = p.scale_log2;
  int32_t t_intra = 0, t_succ = 0;
  int q_kind = 0;                                    // the vector held in qT: 0 q, 1 q_succ, 2 q_inter
  if constexpr (DCA) {
    if (qrow < qn) sl2 *= p.mscale[q0 + qrow];
    const int32_t cq = my_p >= 0 ? my_p / (p.chunk_tiles * kKeys) : -1;
    t_intra = cq * p.chunk_tiles;
    t_succ = t_intra - p.chunk_tiles;
  }

  // Loop-invariant per-lane copy offsets (elements): this wave copies part (wave / 4) of run
  // (wave mod 4) of every tile.
  const int crun = wave & 3, cpart = wave >> 2;
  int32_t k_lane[TG::kKLoadsPerWave], v_lane[TG::kVLoadsPerWave], v_key[TG::kVLoadsPerWave];
#pragma unroll
  for (int i = 0; i < TG::kKLoadsPerWave; ++i) {
    const int idx = (cpart * TG::kKLoadsPerWave + i) * 64 + lane;
    const int rl_ = idx / TG::kKRowChunks, pos = idx % TG::kKRowChunks;   // LDS row in the run
    const int j = pos ^ (rl_ & (TG::kKSwz - 1));                           // logical chunk
    k_lane[i] = perm32(rl_) * D + j * TG::kChunk;                          // key perm32(row)
  }
#pragma unroll
  for (int i = 0; i < TG::kVLoadsPerWave; ++i) {
    const int idx = (cpart * TG::kVLoadsPerWave + i) * 64 + lane;
    const int d = idx / TG::kVRowChunks, pos = idx % TG::kVRowChunks;
    const int c = pos ^ TG::vswz(d);
    v_key[i] = c * TG::kChunk;
    v_lane[i] = d * bs + c * TG::kChunk;
  }

  // The tile loop, specialised for retrieval / streaming heads.
  auto body = [&](auto RET_C) {
    constexpr bool RET = decltype(RET_C)::value;
    auto run_pos = [&](int32_t v) -> Run {
      if constexpr (RET) {
        return Run{v * 16, 0, 0, v < n_runs ? L : 0, false};
      } else {
        return rl.pos(geo, v);
      }
    };
    // Does any 16-byte V chunk of `tile` mix present and absent keys? (position arithmetic only)
    auto partial_chunks = [&](int tile) -> bool {
      bool any = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const Run r = run_pos(tile * 4 + i);
        const int32_t a = max(r.t0, r.lo) - r.t0;
        const int32_t e = min(r.t0 + 16, r.hi) - r.t0;
        if (a < e) any = any || (a % TG::kChunk) != 0 || (e % TG::kChunk) != 0;
      }
      return any;
    };
    // Copy this wave's part of run (wave mod 4) of `tile` into the stage: a scalar page base plus
    // the lane's loop-invariant offsets.
    auto issue = [&](int tile, char* k_st, char* v_st) {
      const int v = tile * 4 + crun;
      const Run r = run_pos(v);
      const int32_t pr = sm_run[min(max(v - seg0, 0), kRunSeg - 1)];
      const int32_t page = v < n_runs ? packed_page(pr) : 0;   // absent runs: page 0, masked
      const int32_t r0 = v < n_runs ? packed_row0(pr) : 0;
      const int64_t pe = (int64_t)page * page_elems;
      const T* kbase = kpool + pe + (int64_t)r0 * D;
      const T* vbase = vpool + pe + r0;
      const uint32_t kdst = lds_addr(k_st) + crun * TG::kKRunBytes + cpart * TG::kKLoadsPerWave * 1024;
      const uint32_t vdst = lds_addr(v_st) + crun * TG::kVRunBytes + cpart * TG::kVLoadsPerWave * 1024;
#pragma unroll
      for (int i = 0; i < TG::kKLoadsPerWave; ++i)   // absent keys' rows are masked by position
        copy16_to_lds(kbase + k_lane[i], kdst + i * 1024);
#pragma unroll
      for (int i = 0; i < TG::kVLoadsPerWave; ++i) {
        const int32_t t = r.t0 + v_key[i];
        const bool absent = t + TG::kChunk <= r.lo || t >= r.hi;
        const void* src = absent ? static_cast<const void*>(g_prefill_zero_chunk)
                                 : static_cast<const void*>(vbase + v_lane[i]);
        copy16_to_lds(src, vdst + i * 1024);
      }
    };
    // Zero, in LDS, the V channels of absent keys inside partly present chunks of `tile` (rare).
    auto fixup = [&](int tile, char* v_st) {
      int32_t t0[4], lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const Run r = run_pos(tile * 4 + i);
        t0[i] = r.t0;
        lo[i] = r.lo;
        hi[i] = r.hi;
      }
      for (int idx = tid; idx < kKeys * D; idx += kThreads) {
        const int k = idx & (kKeys - 1), d = idx / kKeys;
        const int run = k >> 4;
        const int32_t t = sel4(t0, run) + (k & 15);
        if (t < sel4(lo, run) || t >= sel4(hi, run)) {
          const int c = (k & 15) / TG::kChunk;
          const int pos = c ^ TG::vswz(d);
          *reinterpret_cast<T*>(v_st + run * TG::kVRunBytes + d * TG::kVRowBytes + pos * 16 +
                                (k % TG::kChunk) * (int)sizeof(T)) = T(0.0f);
        }
      }
    };
    // The weights of one tile: S^T, the element mask when `mask`, online softmax; the tile's P^T
    // operands (one per 16-key chunk) go to `P`. (One body for both cases: two inlined copies
    // would each hoist their own LDS addresses out of the loop and run out of registers.)
    auto scores = [&](int tile, bool mask, const Run* runs, const char* k_st, v8<T> (&P)[4]) {
      if constexpr (DCA) {
        const int need = tile >= t_intra ? 0 : tile >= t_succ ? 1 : 2;
        if (__any(need != q_kind)) {
          if (need != q_kind && qrow < qn) {
            const void* base = need == 0 ? p.q : need == 1 ? p.q_succ : p.q_inter;
            const T* src = static_cast<const T*>(base) + ((q0 + qrow) * p.num_q_heads + hq) * D;
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) qT[dc] = load8(src + dc * 16 + half * 8);
          }
          q_kind = need;
        }
      }
      // All K operands of the tile are read first, then the MFMAs run back to back: the LDS
      // latency is paid once per tile instead of once per MFMA.
      v8<T> ka[2][DC];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
        const int R = b2 * 32 + rcol;
        const char* row = k_st + R * TG::kKRowBytes;
        const int swz = R & (TG::kKSwz - 1);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) ka[b2][dc] = lds_operand<T>(row, (dc * 16 + half * 8) / TG::kChunk, swz);
      }
      f32x16 s[2];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
        for (int j = 0; j < 16; ++j) s[b2][j] = 0.f;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) s[b2] = mfma32(ka[b2][dc], qT[dc], s[b2]);
      }
      if constexpr (sizeof(T) == 2) pipeline_lds_mfma<2 * DC, kLdsAhead>();
      // accumulator 4*i + j of block b2 is key 8*half + 4*(i&1) + j of run 2*b2 + (i>>1)
      if (mask) {
        // The keys of run k that this lane's row may see form one interval [lo, hi): present
        // keys [r.lo, r.hi), causal t <= my_p and, in a ring run, the window that starts at
        // (my_p & win_mask) - win_back.
        // Key t is kept iff t - lo, taken unsigned, is below hi - lo: one compare per score.
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const Run& r = runs[k];
          const int32_t lo = r.windowed ? max(r.lo, (my_p & p.win_mask) - p.win_back) : r.lo;
          const int32_t hi = min(r.hi, my_p + 1);
          const uint32_t width = (uint32_t)max(hi - lo, 0);
          const int32_t d0 = r.t0 + 8 * half - lo;   // the lane's first key of the run, from lo
          const int b2 = k >> 1;
#pragma unroll
          for (int i = 2 * (k & 1); i < 2 * (k & 1) + 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bool ok = (uint32_t)(d0 + 4 * (i & 1) + j) < width;
              s[b2][4 * i + j] = ok ? s[b2][4 * i + j] : -INFINITY;
            }
        }
      }
      // Row max of the raw scores (softmax_scale > 0, so scaling after the max is exact). The
      // scores are finite or -inf here (absent keys were masked), so the NaN-propagating maximum
      // equals fmaxf and needs no input canonicalisation; a balanced tree keeps it short.
      float t16[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) t16[k] = __builtin_elementwise_maximum(s[0][k], s[1][k]);
#pragma unroll
      for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int k = 0; k < w; ++k) t16[k] = __builtin_elementwise_maximum(t16[k], t16[k + w]);
      float mx = t16[0];
      mx = max_xor32(mx) * (DCA ? sl2 : p.scale_log2);
      // Lazy reference max: it moves only when some row of the wave exceeds it by more than 8
      // (log2 units), so p <= 256 and O / l are rescaled on few tiles. The final O / l is exact
      // whatever reference was used. O holds every earlier tile's PV at this point.
      if (__any(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oT[db] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          x[k] = fast_exp2(fmaf(s[c >> 1][8 * (c & 1) + k], DCA ? sl2 : p.scale_log2, -m_use));
        P[c] = pack8<T>(x);
        l_run = sum8(P[c], l_run);
      }
    };
    // O^T += V^T P^T over the tile's four 16-key chunks.
    auto pv = [&](const v8<T> (&P)[4], const char* v_st) {
      v8<T> va[4][DB];   // operands first, as for S
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = db * 32 + rcol;
          va[c][db] = lds_operand<T>(v_st + c * TG::kVRunBytes + d * TG::kVRowBytes,
                                     (half * 8) / TG::kChunk, TG::vswz(d));
        }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db) oT[db] = mfma32(va[c][db], P[c], oT[db]);
      if constexpr (sizeof(T) == 2) pipeline_lds_mfma<4 * DB, kLdsAhead>();
    };
    // Classification of a tile for the row blocks, computed once per segment of runs: bit w: some
    // key of the tile is visible to some row of wave w; bit 8 + w: every key is present and visible
    // to every row of wave w (no mask); bit 16: some 16-byte V chunk mixes present and absent keys
    // (zeroed in LDS before use).
    auto tile_flags = [&](int tile) -> int32_t {
      Run runs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) runs[i] = run_pos(tile * 4 + i);
      int32_t f = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (w * 32 >= n_rows) continue;   // the wave has no rows
        const int32_t lo = p_lo + w * 32, hi = min(lo + 31, p_hi);
        bool all_full = true, any_vis = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const Run& r = runs[i];
          const int32_t a = max(r.t0, r.lo), e = min(r.t0 + 16, r.hi);   // present keys [a, e)
          // some key visible to some row: the closest pair is key min(e-1, hi) seen from row
          // max(lo, that key) (a window starts at or before its query and never moves back as the
          // query moves on, so row lo has the lowest start)
          const bool vis = a < e && a <= hi &&
                           (!r.windowed || min(e - 1, hi) >= (lo & p.win_mask) - p.win_back);
          const bool full = r.lo <= r.t0 && r.t0 + 16 <= r.hi && r.t0 + 15 <= lo &&
                            (!r.windowed || r.t0 >= (hi & p.win_mask) - p.win_back);
          all_full = all_full && full;
          any_vis = any_vis || vis;
        }
        f |= (any_vis ? 1 : 0) << w;
        f |= (all_full ? 1 : 0) << (8 + w);
      }
      return f | (partial_chunks(tile) ? 1 << 16 : 0);
    };
    auto load_flags = [&](int32_t tile0, int32_t ntiles) {
      for (int i = tid; i < ntiles; i += kThreads) sm_flags[i] = tile_flags(tile0 + i);
    };
    auto compute = [&](int tile, int32_t flags, const char* k_st, v8<T> (&P)[4]) -> bool {
      if (!((flags >> wave) & 1)) return false;
      const bool all_full = (flags >> (8 + wave)) & 1;
      Run runs[4];
      if (!all_full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) runs[i] = run_pos(tile * 4 + i);
      }
      scores(tile, !all_full, runs, k_st, P);
      return true;
    };

    // This workgroup's tiles: all of a streaming item, a contiguous share of a retrieval item's.
    // The shares are cut at the same key tiles for every row tile of the sequence (those of its
    // last rows, which see all L keys), so that the workgroups of one head and share, which run
    // side by side on one XCD, walk the same keys together through its L2.
    const int n_all = (n_runs + 3) / 4;
    const int per = RET ? ((L + kKeys - 1) / kKeys + n_split - 1) / n_split : n_all;
    const int t_begin = min(n_all, split * per);
    const int n_tiles = min(n_all, t_begin + per) - t_begin;
    if (n_tiles <= 0) return;
    seg0 = ((t_begin * 4) / kRunSeg) * kRunSeg;
    load_pages<kThreads>(sm_run, geo, rl, seg0, min(kRunSeg, n_runs - seg0));
    load_flags(seg0 / 4, min(kRunSeg / 4, n_all - seg0 / 4));
    __syncthreads();
    // Retire the Q loads (issued before the page staging, whose latency they share) before the
    // first copy. Left pending, the compiler would wait for them at their first use inside the
    // tile loop, by a full vmcnt wait that every step would then pay for the copies in flight.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    // retrieval tiles below the workgroup's first row are fully visible to every live wave
    const int n_full = RET ? max(0, (p_lo + 1) / kKeys) : 0;
    const int32_t live = (1 << min(kWaves, (n_rows + 31) / 32)) - 1;
    const int32_t lean_flags = live | (live << 8);
    auto flags_of = [&](int t) -> int32_t {
      return t < n_full ? lean_flags : sm_flags[t - seg0 / 4];
    };
    // Tile tn is about to be copied: when it starts a new segment of runs (it always lies past
    // the current one's start), stage that segment once nobody reads the current one any more.
    auto enter = [&](int tn) {
      if (((tn * 4) % kRunSeg) != 0 || tn * 4 == seg0) return;
      __syncthreads();
      seg0 = tn * 4;
      load_pages<kThreads>(sm_run, geo, rl, seg0, min(kRunSeg, n_runs - seg0));
      load_flags(tn, min(kRunSeg / 4, n_all - tn));
      __syncthreads();
    };
    // a tile's classification, taken when its copies are issued (a later segment refill cannot
    // overwrite it), indexed by stage
    int32_t fq[kStages];
#pragma unroll
    for (int c = 0; c < kStages; ++c) fq[c] = 0;
    // prologue: the first kAhead tiles (the first lies in the staged segment)
    issue(t_begin, kst(std::integral_constant<int, 0>{}), vst(std::integral_constant<int, 0>{}));
    fq[0] = flags_of(t_begin);
    if constexpr (kAhead == 2) {
      if (n_tiles > 1) {
        enter(t_begin + 1);
        issue(t_begin + 1, kst(std::integral_constant<int, 1>{}), vst(std::integral_constant<int, 1>{}));
        fq[1] = flags_of(t_begin + 1);
      }
    }
    v8<T> P[4];
    bool pend = false;        // lagging waves: P holds a tile whose PV is still to be done
    const char* pend_v = nullptr;
    // Step s (tile t_begin + s) on stage c = s mod kStages: copies of tile s + kAhead go to stage
    // (c + kAhead) mod kStages, which holds no tile still in use (with four stages: tile s - 1 is in
    // stage c - 1 for the lagging waves' PV, tiles s and s + 1 in c and c + 1).
    auto step = [&](auto C, int s) {
      constexpr int c = decltype(C)::value;
      constexpr int cn = (c + kAhead) % kStages;
      const int t = t_begin + s;
      if (kAhead == 2 && s + 1 < n_tiles) wait_older_then_barrier<TG::kCopiesPerTile>();
      else wait_older_then_barrier<0>();
      if (kLag && pend) {   // the lagging waves finish the previous tile first
        pv(P, pend_v);
        pend = false;
      }
      const int32_t flags = fq[c];
      if (s + kAhead < n_tiles) {
        const int tn = t + kAhead;
        enter(tn);
        issue(tn, kst(std::integral_constant<int, cn>{}), vst(std::integral_constant<int, cn>{}));
        fq[cn] = flags_of(tn);
      }
      if ((flags >> 16) & 1) {   // uniform: the same word for every wave
        fixup(t, vst(C));
        __syncthreads();
      }
      if (compute(t, flags, kst(C), P)) {
        pend_v = vst(C);
        if (kLag && wave >= kWaves / 2) pend = true;
        else pv(P, pend_v);
      }
    };
    for (int s = 0; s < n_tiles; s += kStages) {
      step(std::integral_constant<int, 0>{}, s);
      if (s + 1 < n_tiles) step(std::integral_constant<int, 1>{}, s + 1);
      if constexpr (kStages == 4) {
        if (s + 2 < n_tiles) step(std::integral_constant<int, 2 % kStages>{}, s + 2);
        if (s + 3 < n_tiles) step(std::integral_constant<int, 3 % kStages>{}, s + 3);
      }
    }
    if (pend) pv(P, pend_v);   // the lagging waves' last tile (no copies follow)
  };
  if (ret) body(std::integral_constant<bool, true>{});
  else body(std::integral_constant<bool, false>{});

  // ---- split merge: the last workgroup of a retrieval item to arrive reduces the partials ---
  // Partials go out with device-coherent (write-through) stores; waiting for them to complete
  // before the ticket makes them visible to whichever workgroup, on any XCD, draws the last
  // ticket, which reads them back with device-coherent loads.
  if (ret && n_split > 1) {
    constexpr int64_t kPart = prefill_partial_floats(sizeof(T), D);
    constexpr int kWavePart = 64 * (2 + DB * 16);
    float* mine = p.partial + ((int64_t)item * n_split + split) * kPart + wave * kWavePart;
    store_coherent(mine + lane, m_run);
    store_coherent(mine + 64 + lane, l_run);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) store_coherent(mine + 128 + (db * 16 + j) * 64 + lane, oT[db][j]);
    wait_stores_complete();
    __syncthreads();
    int32_t* ctr = p.counter + item;
    if (tid == 0) sm_ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (sm_ticket != n_split - 1) return;
    for (int sp = 0; sp < n_split; ++sp) {
      if (sp == split) continue;
      const float* other = p.partial + ((int64_t)item * n_split + sp) * kPart + wave * kWavePart;
      const float m_o = load_coherent(other + lane), l_o = load_coherent(other + 64 + lane);
      const float m_new = fmaxf(m_run, m_o);
      const float f_me = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      const float f_o = (m_o == -INFINITY) ? 0.f : fast_exp2(m_o - m_new);
      m_run = m_new;
      l_run = l_run * f_me + l_o * f_o;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          oT[db][j] = oT[db][j] * f_me + load_coherent(other + 128 + (db * 16 + j) * 64 + lane) * f_o;
    }
    if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- normalise and store -----------------------------------------------------------------
  l_run = add_xor32(l_run);
  if (qrow < qn && wave_live) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    T* dst = static_cast<T*>(p.out) + ((q0 + qrow) * p.num_q_heads + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[db * 32 + 8 * i + 4 * half + j] = from_f32<T>(oT[db][4 * i + j] * inv);
  }
}

template <typename T, int D, bool DCA, bool MIX = false>
void launch_d(const PrefillParams& p, int grid, hipStream_t stream, const DecodeParams* dp = nullptr,
              int n_prefill = 0) {
  const LaunchEvents ev = current_launch_events();
  const DecodeParams none{};
  hipExtLaunchKernelGGL((prefill_kernel<T, D, DCA, MIX>), dim3(grid), dim3(TileGeo<T, D>::kThreads),
                        0, stream, ev.start, ev.stop, 0, p, dp ? *dp : none, n_prefill);
}

template <typename T>
hipError_t launch_mixed_t(const PrefillParams& p, const DecodeParams& dp, int n_prefill,
                          int head_dim, int grid, hipStream_t stream) {
  (void)hipGetLastError();
  switch (head_dim) {
    case 64: launch_d<T, 64, false, true>(p, grid, stream, &dp, n_prefill); break;
    case 128: launch_d<T, 128, false, true>(p, grid, stream, &dp, n_prefill); break;
    case 256:
      if constexpr (sizeof(T) == 2) {
        launch_d<T, 256, false, true>(p, grid, stream, &dp, n_prefill);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const PrefillParams& p, int head_dim, int grid, hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's status
  switch (head_dim) {
    case 64: launch_d<T, 64, false>(p, grid, stream); break;
    case 128: launch_d<T, 128, false>(p, grid, stream); break;
    case 256:
      if constexpr (sizeof(T) == 2) {
        launch_d<T, 256, false>(p, grid, stream);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Dual Chunk Attention: 16-bit queries and caches, head dims 64 and 128.
template <typename T>
hipError_t launch_dca_t(const PrefillParams& p, int head_dim, int grid, hipStream_t stream) {
  (void)hipGetLastError();
  switch (head_dim) {
    case 64: launch_d<T, 64, true>(p, grid, stream); break;
    case 128: launch_d<T, 128, true>(p, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_dim, int grid,
                          hipStream_t stream) {
  if (dtype == 0) return launch_t<float>(p, head_dim, grid, stream);
  if (dtype == 1) return launch_t<_Float16>(p, head_dim, grid, stream);
  return launch_t<__bf16>(p, head_dim, grid, stream);
}

hipError_t launch_prefill_mixed(const PrefillParams& p, const DecodeParams& dp, int n_prefill,
                                int dtype, int head_dim, int grid, hipStream_t stream) {
  if (dtype == 0) return launch_mixed_t<float>(p, dp, n_prefill, head_dim, grid, stream);
  if (dtype == 1) return launch_mixed_t<_Float16>(p, dp, n_prefill, head_dim, grid, stream);
  return launch_mixed_t<__bf16>(p, dp, n_prefill, head_dim, grid, stream);
}

hipError_t launch_prefill_dca(const PrefillParams& p, int dtype, int head_dim, int grid,
                              hipStream_t stream) {
  if (dtype == 1) return launch_dca_t<_Float16>(p, head_dim, grid, stream);
  if (dtype == 2) return launch_dca_t<__bf16>(p, head_dim, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace duo
