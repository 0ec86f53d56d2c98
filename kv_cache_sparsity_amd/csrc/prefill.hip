// duo_attn_prefill kernel: tiled flash attention of a prompt chunk over the paged cache.
//
// What is computed (DuoAttention README, abstract and efficiency section; transformers PR
// "[WIP] Dynamic length in static cache"): query row i of sequence b sits at position
// p = L - q_len + i and attends causally (keys j <= p); a streaming head further keeps only the sink
// positions j < sink and its recent window p - j < recent. Scores are softmax_scale * (q . k) in
// fp32 (vLLM DualChunkAttention PR, review thread).
//
// Work decomposition: one workgroup (4 waves, 128 query rows, 32 per wave) per (b, q head, row
// tile); retrieval heads' tiles come first, latest rows first (they scan the most keys). The
// workgroup walks only the 16-key runs that can be visible to its rows:
//   retrieval head: runs 0 .. p_hi / 16;
//   streaming head: the sink runs, then the ring runs covering [p_lo - recent + 1, p_hi].
// So a streaming tile costs about (sink + recent + 128) keys whatever the context length. Four
// runs (64 keys) form one K/V tile, staged into LDS (double-buffered, next tile's global loads in
// flight during this tile's math). Where each run lives (page, row) is resolved once per segment
// of 512 runs into LDS; inside the tile loop a run is a base pointer plus per-thread constant
// offsets. Per wave and tile, each run is classified as fully visible, invisible or partial for
// the wave's 32 rows: fully invisible tiles are skipped, fully visible tiles skip the element mask.
//
// MFMA formulation (32x32x16, k-step of 8 elements per lane), per 32-key block:
//   S^T[key, row] = sum_d K[key, d] Q[row, d]       A = K rows (LDS), B = Q^T (registers)
//   O^T[d, row]  += sum_key V^T[d, key] P^T[key, row] A = V^T (LDS, channel-major like the V page),
//                                                     B = P^T taken from the S^T accumulators.
// K rows are staged into LDS in a permuted order so that the eight S^T accumulators a lane holds
// per 16-key chunk are the chunk's keys 8*(lane/32) .. +7, the k-group of its P^T operand.
#include "duo_common.h"
#include "duo_kernels.h"

namespace duo {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = kPrefillRows;  // 128 query rows per workgroup
constexpr int kKeys = 64;            // keys per K/V tile (four 16-key runs)

// Row of the 32-key block that holds key r of the block (an involution: swaps the middle two
// groups of four in each half).
__device__ __forceinline__ int perm32(int r) {
  const int a = (r >> 2) & 3;
  const int off = (a == 1) ? 8 : (a == 2) ? 4 : (a == 3) ? 12 : 0;
  return (r & 16) + off + (r & 3);
}

template <typename T, int D>
struct Tile {
  static constexpr int kPad = 8;                   // row padding: one 8-element operand
  static constexpr int kKStride = D + kPad;        // K tile: [64 keys][D]
  static constexpr int kVStride = kKeys + kPad;    // V tile: [D][64 keys]
  static constexpr int kChunk = 16 / sizeof(T);    // elements per 16-byte chunk
  static constexpr int kRowChunks = D / kChunk;    // 16-byte chunks per K row
  static constexpr int kRunChunks = 16 / kChunk;   // 16-byte chunks per V channel per run
  static constexpr int kKPer = kKeys * kRowChunks / kThreads;
  static constexpr int kVPer = D * 4 * kRunChunks / kThreads;
};

// Element offsets and key ranges of the four runs of a tile (uniform values).
struct TileRuns {
  int64_t kofs[4];   // K rows of run i: k_pool + kofs[i] + row * D
  int64_t vofs[4];   // V channels of run i: v_pool + vofs[i] + d * block_size
  int32_t t0[4], lo[4], hi[4];
};

template <typename V>
__device__ __forceinline__ V sel4(const V (&a)[4], int i) {
  return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3];
}

template <typename T, int D>
__global__ void __launch_bounds__(kThreads, 2) prefill_kernel(const PrefillParams p) {
  using TL = Tile<T, D>;
  constexpr int DC = D / 16;  // k-steps over the head dim (16 channels per 32x32 MFMA step)
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) T k_lds[2][kKeys * TL::kKStride];
  __shared__ __attribute__((aligned(16))) T v_lds[2][D * TL::kVStride];
  __shared__ int32_t sm_run[kRunSeg];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int rcol = lane & 31;  // MFMA column = query row within the wave
  const int half = lane >> 5;  // k-group of the lane
  const int G = p.group;

  // ---- which item ---------------------------------------------------------------------------
  const int per_tile_r = p.batch * p.n_ret * G;
  const int ret_items = per_tile_r * p.n_qtiles;
  int b, hq, qt;
  bool ret;
  if ((int)blockIdx.x < ret_items) {
    qt = p.n_qtiles - 1 - blockIdx.x / per_tile_r;
    int r = blockIdx.x % per_tile_r;
    b = r / (p.n_ret * G);
    r %= p.n_ret * G;
    hq = p.ret_heads[r / G] * G + r % G;
    ret = true;
  } else {
    const int per_tile_s = p.batch * p.n_str * G;
    const int it = blockIdx.x - ret_items;
    qt = p.n_qtiles - 1 - it / per_tile_s;
    int r = it % per_tile_s;
    b = r / (p.n_str * G);
    r %= p.n_str * G;
    hq = p.str_heads[r / G] * G + r % G;
    ret = false;
  }
  const int h = hq / G;
  int32_t L = max(p.seq_lens[b], 0);
  if (ret) L = min(L, p.max_blocks_per_head << p.log2_bs);
  const int row0 = qt * kRows;
  const int n_rows = min(kRows, p.q_len - row0);
  const int32_t p_lo = L - p.q_len + row0;       // position of the tile's first row
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
        rl.k_lo = (max(p.sink, p_lo - p.recent + 1) - p.sink) / 16;
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

  auto tile_runs = [&](int tile, TileRuns& tr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tile * 4 + i;
      const Run r = rl.pos(geo, v);
      const int32_t pr = sm_run[min(max(v - seg0, 0), kRunSeg - 1)];
      const int32_t page = v < n_runs ? packed_page(pr) : 0;      // absent runs read page 0
      const int32_t r0 = v < n_runs ? packed_row0(pr) : 0;        // (their keys are masked)
      const int64_t pe = (int64_t)page * page_elems;
      tr.kofs[i] = pe + (int64_t)r0 * D;
      tr.vofs[i] = pe + r0;
      tr.t0[i] = r.t0;
      tr.lo[i] = r.lo;
      tr.hi[i] = r.hi;
    }
  };

  // ---- staging of one tile: global -> registers -> LDS --------------------------------------
  u32x4 k_stage[TL::kKPer], v_stage[TL::kVPer];
  auto stage_load = [&](const TileRuns& tr) {
#pragma unroll
    for (int it = 0; it < TL::kKPer; ++it) {
      const int idx = it * kThreads + tid;
      const int kt = idx / TL::kRowChunks, c = idx % TL::kRowChunks;
      // rows of absent keys may hold anything: their scores are masked by position
      k_stage[it] = *reinterpret_cast<const u32x4*>(kpool + sel4(tr.kofs, kt >> 4) + (kt & 15) * D +
                                                    c * TL::kChunk);
    }
#pragma unroll
    for (int it = 0; it < TL::kVPer; ++it) {
      const int idx = it * kThreads + tid;
      const int run = idx / (D * TL::kRunChunks);
      const int rem = idx % (D * TL::kRunChunks);
      const int d = rem / TL::kRunChunks, c = rem % TL::kRunChunks;
      u32x4 val = *reinterpret_cast<const u32x4*>(vpool + sel4(tr.vofs, run) + (int64_t)d * bs +
                                                  c * TL::kChunk);
      const int32_t t0 = sel4(tr.t0, run) + c * TL::kChunk;
      const int32_t lo = sel4(tr.lo, run), hi = sel4(tr.hi, run);
      // the channel values of absent keys may be NaN or Inf: zero them
      if (t0 < lo || t0 + TL::kChunk > hi) val = zero_absent<sizeof(T)>(val, t0, lo, hi);
      v_stage[it] = val;
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int it = 0; it < TL::kKPer; ++it) {
      const int idx = it * kThreads + tid;
      const int kt = idx / TL::kRowChunks, c = idx % TL::kRowChunks;
      const int lrow = (kt & 32) + perm32(kt & 31);
      *reinterpret_cast<u32x4*>(&k_lds[buf][lrow * TL::kKStride + c * TL::kChunk]) = k_stage[it];
    }
#pragma unroll
    for (int it = 0; it < TL::kVPer; ++it) {
      const int idx = it * kThreads + tid;
      const int run = idx / (D * TL::kRunChunks);
      const int rem = idx % (D * TL::kRunChunks);
      const int d = rem / TL::kRunChunks, c = rem % TL::kRunChunks;
      *reinterpret_cast<u32x4*>(&v_lds[buf][d * TL::kVStride + run * 16 + c * TL::kChunk]) = v_stage[it];
    }
  };

  // ---- the wave's query rows: Q^T operand (B of S^T) ----------------------------------------
  const int wrow0 = wave * 32;                       // first row of this wave inside the tile
  const int qrow = row0 + wrow0 + rcol;              // chunk row of this lane's column
  const int32_t pw_lo = p_lo + wrow0;
  const int32_t pw_hi = min(pw_lo + 31, p_hi);
  const bool wave_live = wrow0 < n_rows;
  v8<T> qT[DC];
  {
    const bool ok = qrow < p.q_len;
    const T* src = static_cast<const T*>(p.q) + (((int64_t)b * p.q_len + (ok ? qrow : 0)) * p.num_q_heads + hq) * D;
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

  const int n_tiles = (n_runs + 3) / 4;
  TileRuns tr_next;
  if (n_tiles > 0) {
    load_pages<kThreads>(sm_run, geo, rl, 0, min(kRunSeg, n_runs));
    __syncthreads();
    tile_runs(0, tr_next);
    stage_load(tr_next);
    stage_store(0);
  }
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < n_tiles) {
      if ((((tile + 1) * 4) % kRunSeg) == 0) {   // next tile starts a new segment of runs
        seg0 = (tile + 1) * 4;
        load_pages<kThreads>(sm_run, geo, rl, seg0, min(kRunSeg, n_runs - seg0));
        __syncthreads();
      }
      tile_runs(tile + 1, tr_next);
      stage_load(tr_next);
    }

    // classify this tile's runs for the wave's rows
    Run runs[4];
    bool all_full = true, any_vis = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      runs[i] = rl.pos(geo, tile * 4 + i);
      const Run& r = runs[i];
      const int32_t a = max(r.t0, r.lo), e = min(r.t0 + 16, r.hi);   // present keys [a, e)
      const bool present = a < e;
      // Some key visible to some row: the closest (key, row) pair is key t = min(e-1, pw_hi) seen
      // from row max(pw_lo, t).
      const bool vis = present && a <= pw_hi &&
                       (!r.windowed || pw_lo - min(e - 1, pw_hi) < p.recent);
      const bool full = r.lo <= r.t0 && r.t0 + 16 <= r.hi && r.t0 + 15 <= pw_lo &&
                        (!r.windowed || pw_hi - r.t0 < p.recent);
      all_full = all_full && full;
      any_vis = any_vis || vis;
    }

    if (wave_live && any_vis) {
      const T* kl = k_lds[buf];
      const T* vl = v_lds[buf];
      f32x16 s[2];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
#pragma unroll
        for (int j = 0; j < 16; ++j) s[b2][j] = 0.f;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const v8<T> a = load8(kl + (b2 * 32 + rcol) * TL::kKStride + dc * 16 + half * 8);
          s[b2] = mfma32(a, qT[dc], s[b2]);
        }
      }
      // accumulator 4*i + j of block b2 is key 8*half + 4*(i&1) + j of run 2*b2 + (i>>1)
      if (!all_full) {
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const Run& r = runs[2 * b2 + (i >> 1)];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int32_t t = r.t0 + 8 * half + 4 * (i & 1) + j;
              const bool ok = t >= r.lo && t < r.hi && t <= my_p &&
                              (!r.windowed || my_p - t < p.recent);
              s[b2][4 * i + j] = ok ? s[b2][4 * i + j] : -INFINITY;
            }
          }
      }
      // Row max of the raw scores (softmax_scale > 0, so scaling after the max is exact).
      float mx = -INFINITY;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int k = 0; k < 16; ++k) mx = fmaxf(mx, s[b2][k]);
      mx = fmaxf(mx, shfl_xor(mx, 32)) * p.scale_log2;
      // Lazy reference max: it moves only when some row of the wave exceeds it by more than 8
      // (log2 units), so p <= 256 and O / l are rescaled on few tiles. The final O / l is exact
      // whatever reference was used.
      if (__any(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oT[db] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float x[2][16];
      float psum = 0.f;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          x[b2][k] = fast_exp2(fmaf(s[b2][k], p.scale_log2, -m_use));
          psum += x[b2][k];
        }
      l_run += psum;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const v8<T> pB = pack8<T>(&x[b2][8 * kc]);
          const int chunk = 2 * b2 + kc;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const v8<T> a = load8(vl + (db * 32 + rcol) * TL::kVStride + chunk * 16 + half * 8);
            oT[db] = mfma32(a, pB, oT[db]);
          }
        }
    }
    if (tile + 1 < n_tiles) stage_store(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store -----------------------------------------------------------------
  l_run += shfl_xor(l_run, 32);
  if (qrow < p.q_len && wave_live) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    T* dst = static_cast<T*>(p.out) + (((int64_t)b * p.q_len + qrow) * p.num_q_heads + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[db * 32 + 8 * i + 4 * half + j] = from_f32<T>(oT[db][4 * i + j] * inv);
  }
}

template <typename T>
hipError_t launch_t(const PrefillParams& p, int head_dim, int grid, hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's status
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((prefill_kernel<T, 64>), dim3(grid), dim3(kThreads), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((prefill_kernel<T, 128>), dim3(grid), dim3(kThreads), 0, stream, p); break;
    case 256:
      if constexpr (sizeof(T) == 2) {
        hipLaunchKernelGGL((prefill_kernel<T, 256>), dim3(grid), dim3(kThreads), 0, stream, p);
        break;
      }
      return hipErrorInvalidValue;
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

}  // namespace duo
