// The split-K decode work item, shared by the decode kernels (decode.hip) and the packed-batch
// prefill kernel (prefill.hip), which runs decode items for its single-row sequences in the same
// launch. What is computed, the work decomposition and the merge are described in decode.hip.
#pragma once

#include <type_traits>

#include "duo_common.h"
#include "duo_kernels.h"

namespace duo {

namespace {


// Waves per workgroup: eight up to D = 128 (more loads in flight per CU); four at D = 256, where
// eight waves' merge buffers would not fit in LDS next to a second workgroup.
template <int D> constexpr int decode_waves() { return D <= 128 ? 8 : 4; }

// Split merge: up to kFastMergeSplits splits per (sequence, kv head) take the two-phase merge
// (weights in LDS, then the partial outputs with merge_loads 8-byte loads in flight per thread:
// 32 with eight waves per workgroup (256 registers a lane), 64 with four (512 registers), so that
// the 16 records of a D = 256 row come in one round).
template <int kWaves> constexpr int merge_loads() { return kWaves <= 4 ? 64 : 32; }

// Two consecutive floats (8-byte aligned) read or written at device coherence, as the single
// floats are.
__device__ __forceinline__ uint64_t load_coherent_pair(const float* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent_pair(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The decode body. Q4: the cache holds 4-bit codes (two per byte, in words of 8) with one fp32
// scale per kv head and channel for K and for V ([num_kv_heads][head_dim]); the K scales multiply q
// once per item, each code enters its MFMA as 24 + code (nib8_plus24), the 24 of a score is the same
// for every key of a q head (softmax ignores it), and the output of a wave is
// (O - 24 l) * v_scale per channel, with l the sum of the rounded weights PV multiplied.
// Q8: the cache holds int8 codes with one fp32 scale per slot and per K / V
// (k_scale, v_scale [num_blocks][block_size]); a score is (codes . q) * k_scale of its key, and a
// key's weight enters PV as p * v_scale of the key (the row sum l takes p itself). Otherwise the row
// sum l adds the weights as rounded for PV.
// LDS of one decode work item (decode_body's `lds`): per wave and q head the partial O, the max and
// the row sum, then the staged page list, the merge ticket and the step counter.
template <int kWaves, int D>
struct DecodeLds {
  static constexpr int kO = kWaves * 16 * D * 4;
  static constexpr int kM = kWaves * 16 * 4;
  static constexpr int kPage = (kRunSeg + 8) * 4;
  static constexpr int kBytes = kO + 2 * kM + kPage + 16;
};

// One decode work item `blk` of the grid the host planned (see decode.hip), with `lds` pointing at
// DecodeLds<kWavesT, D>::kBytes of LDS. kWavesT waves per workgroup.
// APPEND: the fused append of decode_append_kernel (see DecodeParams::k_new).
template <typename T, int D, bool Q8, bool DCA = false, bool Q4 = false, int kWavesT = decode_waves<D>(),
          bool APPEND = false>
__device__ __forceinline__ void decode_body(const DecodeParams& p, int blk, char* lds) {
  constexpr int kDecodeWaves = kWavesT;
  constexpr int kThreads = kDecodeWaves * kWave;
  constexpr int KC = D / 32;  // k-steps of S^T over the head dim
  constexpr int DT = D / 16;  // 16-row tiles of O^T
  // PV operand type. An fp16 call over the int8 cache takes PV in bf16: a weight (up to 2^8 under
  // the lazy max) times a V scale (up to 65504 / 127) can pass fp16's range, and every code is
  // exact in bf16 as well.
  using PT = typename std::conditional<Q8 && std::is_same<T, _Float16>::value, __bf16, T>::type;
  using LB = DecodeLds<kDecodeWaves, D>;
  float (*const sm_o)[16][D] = reinterpret_cast<float (*)[16][D]>(lds);
  float (*const sm_m)[16] = reinterpret_cast<float (*)[16]>(lds + LB::kO);
  float (*const sm_l)[16] = reinterpret_cast<float (*)[16]>(lds + LB::kO + LB::kM);
  int32_t* const sm_page = reinterpret_cast<int32_t*>(lds + LB::kO + 2 * LB::kM);
  int& sm_ticket = *reinterpret_cast<int*>(lds + LB::kO + 2 * LB::kM + LB::kPage);
  int& sm_next_step = *reinterpret_cast<int*>(lds + LB::kO + 2 * LB::kM + LB::kPage + 4);  // the
                                                         // segment's next unclaimed wave step

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int col = lane & 15;   // MFMA column = q head within the group
  const int quad = lane >> 4;  // k-group of the lane
  // ---- which item -------------------------------------------------------------------------
  // A kv head's group of q heads rides in the 16 MFMA columns; a group of more than 16 is taken in
  // gchunks chunks of 16 q heads (the last may be short), each its own row of items. The chunk is
  // the fastest index of a row.
  // str_first: streaming items first, then the retrieval splits of every (sequence, retrieval
  // head) row but its last, then the rows' last splits. With one workgroup per CU, the workgroups
  // dispatched last start on the CUs that the short streaming items free, and the last splits are
  // the shortest (the host sizes the splits for that). Otherwise the retrieval items (split
  // fastest), then the streaming items, which start on the CUs of the first retrieval items done.
  const int gch = p.gchunks;
  const int n_str_items = p.str_first ? p.batch * p.n_str * gch : 0;
  const int n_rows = p.batch * p.n_ret * gch;
  const int n_ret_items = n_rows * p.n_split;
  int b, h, split, gc;
  bool ret;
  if (blk < n_str_items || blk >= n_str_items + n_ret_items) {
    const int it = blk < n_str_items ? blk : blk - n_ret_items;
    b = it / (p.n_str * gch);
    const int r = it % (p.n_str * gch);
    h = p.str_heads[r / gch];
    gc = r % gch;
    split = 0;
    ret = false;
  } else {
    const int r = blk - n_str_items;
    int row;
    if (!p.str_first) {
      split = r % p.n_split;
      row = r / p.n_split;
    } else if (r < n_rows * (p.n_split - 1)) {
      split = r % (p.n_split - 1);
      row = r / (p.n_split - 1);
    } else {
      split = p.n_split - 1;
      row = r - n_rows * (p.n_split - 1);
    }
    b = row / (p.n_ret * gch);
    const int rr = row % (p.n_ret * gch);
    h = p.ret_heads[rr / gch];
    gc = rr % gch;
    ret = true;
  }
  const int G = min(16, p.group - gc * 16);   // q heads (MFMA columns) of this chunk
  const int Gs = min(16, p.group);            // q heads a merge record has room for
  const int qh0 = h * p.group + gc * 16;      // the chunk's first q head
  // The row of q and out: b, or in a packed batch the sequence's row when it has exactly one
  // (a sequence with more rows is the prefill tiles' work: every item of it returns here, before
  // any ticket).
  int64_t qb = b;
  if (p.q_start != nullptr) {
    const int32_t s0 = min(max(p.q_start[b], 0), p.total_q);
    const int32_t s1 = min(max(p.q_start[b + 1], s0), p.total_q);
    if (s1 - s0 != 1) return;
    qb = s0;
  }
  HeadGeom geo;
  geo.row = p.table + ((int64_t)b * p.num_kv_heads + h) * p.max_blocks_per_head;
  geo.num_blocks = p.num_blocks;
  geo.log2_bs = p.log2_bs;
  geo.sink = p.sink;
  geo.sink_blocks = p.sink_blocks;
  geo.ring_slots = p.ring_slots;

  // A retrieval split's first segment of block-table entries does not depend on the sequence's
  // length: they are read before it, so that the two reads' round trips overlap (entries of runs
  // past the length are read and not used; page_of clamps every entry into the pool).
  constexpr int kPre = (kRunSeg + kThreads - 1) / kThreads;
  int32_t pre[kPre];
  if (ret) {
    const int32_t cap = p.max_blocks_per_head << p.log2_bs;
    const int32_t t0 = split * p.split_tokens;
    const int32_t nr = min((min(p.split_tokens, max(cap - t0, 0)) + 15) / 16, kRunSeg);
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const int32_t v = (int32_t)threadIdx.x + j * kThreads;
      const int32_t slot = t0 + v * 16;
      pre[j] = v < nr ? pack_run(geo.page_of(slot), geo.row0(slot)) : 0;
    }
  }
  // APPEND: the call's token of (b, h) does not depend on the length either: its elements (and the
  // 4-bit channel scales) are loaded before it, into the registers the writing item stores from.
  // One element per thread (D <= kThreads); the int8 quantizer takes the K row in wave 0 and the V
  // row in wave 1, D / kWave elements a lane; the 4-bit K words take 8 elements a thread.
  [[maybe_unused]] T tok_k = T(), tok_v = T();
  [[maybe_unused]] T tok_k8[8];
  [[maybe_unused]] float tok_x[D / kWave];
  [[maybe_unused]] float tok_ks[8], tok_vs = 0.f;
  if constexpr (APPEND) {
    static_assert(D <= kThreads, "one token element per thread");
    const int64_t src = ((int64_t)b * p.num_kv_heads + h) * D;
    const T* kn = static_cast<const T*>(p.k_new) + src;
    const T* vn = static_cast<const T*>(p.v_new) + src;
    const int d = (int)threadIdx.x;
    if constexpr (Q8) {
      if (wave < 2) {
        const T* x_row = wave == 0 ? kn : vn;
#pragma unroll
        for (int i = 0; i < D / kWave; ++i) tok_x[i] = (float)x_row[lane + kWave * i];
      }
    } else if constexpr (Q4) {
      if (d < D / 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          tok_k8[e] = kn[8 * d + e];
          tok_ks[e] = p.k_scale[(int64_t)h * D + 8 * d + e];
        }
      }
      if (d < D) {
        tok_v = vn[d];
        tok_vs = p.v_scale[(int64_t)h * D + d];
      }
    } else {
      if (d < D) {
        tok_k = kn[d];
        tok_v = vn[d];
      }
    }
  }
  [[maybe_unused]] bool wrote = false;   // APPEND: this item stored the token
  int32_t L = max(p.seq_lens[b], 0);
  if constexpr (APPEND) {
    // The call's token of (b, h) goes to position t = L (the length before it), and every item of
    // the sequence attends over L + 1 keys. The item whose keys hold position t writes the token
    // into its slot before reading any key, as kv_append_circular would (a retrieval head: slot t,
    // unless t is past the row's capacity; a streaming head: its sink or ring slot); the q-head
    // chunks of a kv head each write the same bits. No other item reads that slot: a retrieval
    // split reads only its own keys, and the ring slot the token takes held a position older than
    // any window (the ring holds at least the window's span). One item per sequence stores the
    // new length.
    const int32_t t = L;
    L = t + 1;
    const bool writer_of_len = gc == 0 && split == 0 &&
                               (p.n_ret > 0 ? ret && h == p.ret_heads[0] : h == p.str_heads[0]);
    if (p.seq_lens_after != nullptr && writer_of_len && threadIdx.x == 0) p.seq_lens_after[b] = L;
    const int32_t cap = p.max_blocks_per_head << p.log2_bs;
    if (ret ? (t < cap && t / p.split_tokens == split) : true) {
      const int32_t slot = (ret || t < p.sink) ? t : (p.sink_blocks << p.log2_bs) + (t - p.sink) % p.ring_slots;
      int64_t page;
      int32_t row;
      // a retrieval split read its token run's table entry before the length (pre): the thread
      // holding it passes it on through that run's cell of the page staging, which stores the
      // same value there again (runs start at multiples of 16 slots, so the row is the run's
      // first row plus t mod 16)
      const int32_t vt = ret ? (t - split * p.split_tokens) >> 4 : kRunSeg;
      if (vt < kRunSeg) {
        if ((int)threadIdx.x == vt % kThreads) {
#pragma unroll
          for (int j = 0; j < kPre; ++j)
            if (j == vt / kThreads) sm_page[vt] = pre[j];
        }
        __syncthreads();
        const int32_t pr = sm_page[vt];
        page = packed_page(pr);
        row = packed_row0(pr) + (t & 15);
      } else {
        page = geo.page_of(slot);
        row = geo.row0(slot);
      }
      const int d = (int)threadIdx.x;
      if constexpr (Q8) {
        // the int8 append's arithmetic (quant_code): wave 0 quantizes the K row, wave 1 the V row;
        // codes into the pages (K token-major, V channel-major), the row's scale amax / 127 into
        // k_scale / v_scale at [page][row]
        if (wave < 2) {
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < D / kWave; ++i) amax = fmaxf(amax, fabsf(tok_x[i]));
          amax = wave_max(amax);
          const float inv = amax > 0.f ? __fdiv_rn(127.f, amax) : 0.f;
          int8_t* codes = static_cast<int8_t*>(const_cast<void*>(wave == 0 ? p.k_pool : p.v_pool));
#pragma unroll
          for (int i = 0; i < D / kWave; ++i) {
            const int dd = lane + kWave * i;
            const int64_t at = wave == 0 ? ((page << p.log2_bs) + row) * D + dd
                                         : ((page * D + dd) << p.log2_bs) + row;
            codes[at] = (int8_t)quant_code(tok_x[i], inv);
          }
          if (lane == 0)
            const_cast<float*>(wave == 0 ? p.k_scale : p.v_scale)[(page << p.log2_bs) + row] =
                amax > 0.f ? __fdiv_rn(amax, 127.f) : 0.f;
        }
      } else if constexpr (Q4) {
        // the 4-bit append's arithmetic (quant4_u, the kv head's channel scales): the K row's
        // D / 8 words whole; for V, each channel's nibble of the token's slot merged into its word
        // by a plain read-modify-write (in this launch no other item changes the word's other
        // nibbles, and every item that writes the token writes the same bits)
        if (d < D / 8) {
          uint32_t word = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            word |= quant4_u((float)tok_k8[e], tok_ks[e]) << nibble_shift(e);
          reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(const_cast<void*>(p.k_pool)) +
                                      ((page << p.log2_bs) + row) * (D / 2))[d] = word;
        }
        if (d < D) {
          const int sh = nibble_shift(row & 7);
          uint32_t* w = static_cast<uint32_t*>(const_cast<void*>(p.v_pool)) +
                        ((((page * D + d) << p.log2_bs) + row) >> 3);
          *w = (*w & ~(0xFu << sh)) | (quant4_u((float)tok_v, tok_vs) << sh);
        }
      } else {
        if (d < D) {
          T* kdst = static_cast<T*>(const_cast<void*>(p.k_pool)) + ((page << p.log2_bs) + row) * D;
          T* vdst = static_cast<T*>(const_cast<void*>(p.v_pool)) + ((page * D) << p.log2_bs) + row;
          kdst[d] = tok_k;
          vdst[(int64_t)d << p.log2_bs] = tok_v;
        }
      }
      // the stores complete at the first page staging below, before any wave reads a key
      wrote = true;
    }
  }
  if (ret) L = min(L, p.max_blocks_per_head << p.log2_bs);

  // ---- the item's runs ----------------------------------------------------------------------
  RunList rl;
  rl.ret = ret;
  rl.L = L;
  rl.first = rl.n_sink = rl.k_lo = rl.ring_lo = 0;
  if (ret) {
    const int32_t t0 = split * p.split_tokens;
    const int32_t end = min(L, t0 + p.split_tokens);
    rl.first = t0 / 16;
    rl.n = end > t0 ? (end - t0 + 15) / 16 : 0;
  } else {
    rl.n_sink = (min(p.sink, L) + 15) / 16;
    rl.ring_lo = max(p.sink, ((L - 1) & p.win_mask) - p.win_back);
    int32_t n_ring = 0;
    if (L > p.sink) {
      rl.k_lo = (rl.ring_lo - p.sink) / 16;
      n_ring = (L - 1 - p.sink) / 16 - rl.k_lo + 1;
    }
    rl.n = rl.n_sink + n_ring;
  }
  const int32_t n_runs = rl.n;

  const T* kpool = static_cast<const T*>(p.k_pool);
  const T* vpool = static_cast<const T*>(p.v_pool);
  const int8_t* kq = static_cast<const int8_t*>(p.k_pool);   // the int8 cache's codes (Q8)
  const uint8_t* k4 = static_cast<const uint8_t*>(p.k_pool);  // the 4-bit cache's codes (Q4)
  const uint8_t* v4 = static_cast<const uint8_t*>(p.v_pool);
  const int8_t* vq = static_cast<const int8_t*>(p.v_pool);
  const int64_t page_elems = (int64_t)D << p.log2_bs;
  const int bs = 1 << p.log2_bs;

  if (n_runs > 0) {
    // ---- Q^T operand (B of S^T): column = q head, k = head-dim chunk ------------------------
    v8<T> qT[KC];
    {
      const T* qrow = static_cast<const T*>(p.q) + (qb * p.num_q_heads + qh0 + col) * D;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        // Q8 takes each lane's K codes 16 at a time, so its k-step c pairs lane quad with head
        // dims (c / 2) * 64 + 16 * quad + 8 * (c % 2) .. +7; q must follow the same order
        // Q4 takes a lane's K codes D / 8 bytes at a time: k-step c pairs lane quad with head dims
        // quad * D / 4 + 8 c .. +7, and q is taken times those channels' K scales
        const int d0 = Q8 ? (c >> 1) * 64 + quad * 16 + (c & 1) * 8
                          : Q4 ? quad * (D / 4) + c * 8 : c * 32 + quad * 8;
        if constexpr (Q4) {
          const T* qq = qrow + d0;
          const float* ksc = p.k_scale + (int64_t)h * D + d0;
          float qs[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) qs[i] = (col < G) ? (float)qq[i] * ksc[i] : 0.f;
          qT[c] = pack8<T>(qs);
        } else {
          qT[c] = (col < G) ? load8(qrow + d0) : zero8<T>();
        }
      }
    }
    f32x4 oT[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) oT[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    // Dual Chunk Attention: the chunk of the decoded position, the vector held in qT (0 q,
    // 1 q_succ, 2 q_inter) and the scale with the sequence's mscale
    int32_t cq = 0;
    int q_kind = 0;
    float sl2 = p.scale_log2;
    // the three query bases as values (selecting among the parameter fields themselves would take
    // their addresses and copy the parameter block to scratch)
    const void* const q_intra = p.q;
    const void* const q_succ = p.q_succ;
    const void* const q_inter = p.q_inter;
    if constexpr (DCA) {
      cq = (L - 1) / p.chunk_len;
      sl2 *= p.mscale[b];
    }

    // A wave step covers kChunks 32-key chunks (2 runs of 16 keys each). In chunk c, K tile t' (two
    // per chunk) puts key 8*(r/4) + 4*t' + r%4 of the chunk in MFMA row r, so the S^T accumulator
    // a lane holds for chunk c is keys 8*quad .. 8*quad+7 of the chunk: exactly the keys of its
    // V^T operand (channel dt*16 + col) and of its P^T operand.
    // Q4 (two chunks, four runs per step) orders the keys so that a lane owns one run: chunk c's
    // K tile t' puts slot 8c + 4t' + r%4 of run r/4 in MFMA row r, so lane (col, quad) holds slots
    // 8c .. 8c+7 of run quad in chunk c, and its V codes of a channel for the whole step are the
    // run's 16 slots: one 8-byte load per channel tile instead of one 4-byte load per chunk.
    const Nib4Consts n4 = Q4 ? nib4_consts<T>() : Nib4Consts{0u, 0u};
    // One 32-key chunk per step for 16-bit and int8 caches (measured best: two waves per SIMD).
    // A 4-bit step moves a quarter of the bytes, so it takes two chunks (measured on the
    // Llama-3-8B shape: 36.0 us against 38.6 us with four chunks).
    constexpr int kChunks = Q4 ? 2 : 1;
    constexpr int kRunsPerStep = 2 * kChunks;
    v8<T> kA[kChunks][2][KC], vA[kChunks][DT];
    // Q8: the raw code words, converted only where the MFMAs take them, so that the look-ahead
    // loads are waited for at their use and not at their issue
    u32x2 kR[kChunks][2][KC], vR[kChunks][DT];
    uint32_t kW[kChunks][2][KC], vW[kChunks][DT];   // Q4: the code words
    f32x4 kS[kChunks][2], vS[kChunks][2];   // Q8: scales of the lane's 8 keys (S^T / P^T slots)
    // With four waves (D = 256) and for the int8 cache the look-ahead loads are issued whether or
    // not the wave has a next step (`live`); a dead one reads page 0 (valid memory, its values
    // unused). Loads that are always issued keep the loop free of branches around them, so that
    // the compiler waits at each use for just the loads that use needs: behind a branch it waited
    // for every load in flight, the step's V included, at the top of each step. Keeping V in
    // flight across the S MFMAs pays where a CU has four waves' loads in flight (Gemma-2b static
    // decode 31.6 -> 30.7 us) and for int8, whose steps spend longer converting codes (Llama-3-8B
    // shape 58.4 -> 57.8 us); the 16-bit and 4-bit D <= 128 shapes stream at the chip's paged-read
    // rate and the extra overlap made them slower (Llama-3-8B 90.9 -> 94.4 us), so they keep the
    // branch.
    constexpr bool kAlwaysLoad = kDecodeWaves <= 4 || Q8;
    // 16-bit K and V: non-temporal loads (not kept in the caches) with eight waves, plain loads
    // with four (D = 256). Measured with a 1 GiB read before each launch: plain loads take the
    // Gemma-2b static decode from 32.2 to 29.5 us, and the eight-wave shapes from 92.5 to 100.7 us
    // (Llama-3-8B) and 337 to 367 us (1M context).
    auto load_kv8 = [&](const T* ptr) {
      if constexpr (kDecodeWaves <= 4 && sizeof(T) == 2) return load8(ptr);
      else return load8_stream(ptr);
    };
    // Scales of keys 8*(quad&1) .. +7 of run 2c + quad/2 of the step: the keys of the lane's
    // S^T accumulators and of its P^T operand.
    auto load_scales = [&](const float* pool, int step, bool live, f32x4 (&dst)[kChunks][2]) {
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int v = kRunsPerStep * step + 2 * c + (quad >> 1);
        const int32_t pr = live ? sm_page[min(v, kRunSeg + kRunsPerStep - 1)] : 0;
        const f32x4* sp = reinterpret_cast<const f32x4*>(
            pool + ((int64_t)packed_page(pr) << p.log2_bs) + packed_row0(pr) + (quad & 1) * 8);
        dst[c][0] = __builtin_nontemporal_load(sp);
        dst[c][1] = __builtin_nontemporal_load(sp + 1);
      }
    };
    auto load_k = [&](int32_t seg0, int step, bool live) {
      const int r = col;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int v = kRunsPerStep * step + (Q4 ? (r >> 2) : 2 * c + (r >> 3));
        const int32_t pr = live ? sm_page[min(v, kRunSeg + kRunsPerStep - 1)] : 0;
        const int64_t base = packed_page(pr) * page_elems + (int64_t)packed_row0(pr) * D;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int krow = (Q4 ? 8 * c : ((r >> 2) & 1) * 8) + 4 * t + (r & 3);
          if constexpr (Q4) {
            // the lane's D / 8 bytes of the row: KC words, one per k-step
            const uint8_t* src = k4 + (packed_page(pr) * page_elems + ((int64_t)packed_row0(pr) + krow) * D) / 2 +
                                 quad * (D / 8);
            if constexpr (KC == 2) {
              const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
              kW[c][t][0] = w[0];
              kW[c][t][1] = w[1];
            } else {
#pragma unroll
              for (int i = 0; i < KC / 4; ++i) {
                const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) kW[c][t][4 * i + e] = w[e];
              }
            }
          } else if constexpr (Q8) {
            // 16 codes per load: head dims 64 i + 16 quad .. +15, the lane's slots of k-steps
            // 2i and 2i + 1
#pragma unroll
            for (int i = 0; i < KC / 2; ++i) {
              const u32x4 w = __builtin_nontemporal_load(
                  reinterpret_cast<const u32x4*>(kq + base + krow * D + i * 64 + quad * 16));
              kR[c][t][2 * i] = u32x2{w[0], w[1]};
              kR[c][t][2 * i + 1] = u32x2{w[2], w[3]};
            }
          } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
              kA[c][t][kc] = load_kv8(kpool + base + krow * D + kc * 32 + quad * 8);
          }
        }
      }
      if constexpr (Q8) load_scales(p.k_scale, step, live, kS);
    };
    auto load_v = [&](int32_t seg0, int step, bool live) {
      if constexpr (Q4) {
        // the lane's run (quad) of the step: slots 0 .. 15 of channel dt * 16 + col in one word
        // pair, slots 8c .. 8c+7 for chunk c
        const int32_t pr = live ? sm_page[min(kRunsPerStep * step + quad, kRunSeg + kRunsPerStep - 1)] : 0;
        const int64_t base = packed_page(pr) * page_elems + packed_row0(pr);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x2 w = __builtin_nontemporal_load(
              reinterpret_cast<const u32x2*>(v4 + (base + (int64_t)(dt * 16 + col) * bs) / 2));
#pragma unroll
          for (int c = 0; c < kChunks; ++c) vW[c][dt] = w[c];
        }
        return;
      }
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int v = kRunsPerStep * step + 2 * c + (quad >> 1);
        const int32_t pr = live ? sm_page[min(v, kRunSeg + kRunsPerStep - 1)] : 0;
        const int64_t base = packed_page(pr) * page_elems + packed_row0(pr) + (quad & 1) * 8;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          if constexpr (Q8)
            vR[c][dt] = load_codes8_stream(vq + base + (int64_t)(dt * 16 + col) * bs);
          else
            vA[c][dt] = load_kv8(vpool + base + (int64_t)(dt * 16 + col) * bs);
        }
      }
      if constexpr (Q8) load_scales(p.v_scale, step, live, vS);
    };

    for (int32_t seg0 = 0; seg0 < n_runs; seg0 += kRunSeg) {
      const int32_t nseg = min(kRunSeg, n_runs - seg0);
      if (seg0 > 0) __syncthreads();   // everyone is done with the previous segment's pages
      if (ret && seg0 == 0) {
#pragma unroll
        for (int j = 0; j < kPre; ++j) {
          const int32_t v = (int32_t)threadIdx.x + j * kThreads;
          if (v < nseg) sm_page[v] = pre[j];
        }
      } else {
        load_pages<kThreads>(sm_page, geo, rl, seg0, nseg);
      }
      // runs past the end of the list read page 0 (valid memory, fully masked)
      for (int i = nseg + (int)threadIdx.x; i < nseg + kRunsPerStep; i += kThreads) sm_page[i] = 0;
      if (threadIdx.x == 0) sm_next_step = kDecodeWaves;
      if constexpr (APPEND) {
        // the token stored above is in place before any key of the item is read
        if (seg0 == 0 && wrote) wait_stores_complete();
      }
      __syncthreads();
      const int n_steps = (nseg + kRunsPerStep - 1) / kRunsPerStep;
      int step = wave;
      if (kAlwaysLoad || step < n_steps) {
        load_k(seg0, step, step < n_steps);
        load_v(seg0, step, step < n_steps);
      }
      // Wave w starts with step w; after that each wave claims the next unclaimed step, so waves
      // that run ahead take more steps and all of them finish together.
      while (step < n_steps) {
        int nxt = 0;
        if (lane == 0) nxt = atomicAdd(&sm_next_step, 1);
        nxt = __builtin_amdgcn_readfirstlane(nxt);
        const bool has_next = nxt < n_steps;
        if constexpr (DCA) {
          // all keys of the step share one chunk: choose the query vector for it (uniform)
          const int32_t ck = (rl.first + seg0 + kRunsPerStep * step) * 16 / p.chunk_len;
          const int need = ck == cq ? 0 : ck == cq - 1 ? 1 : 2;
          if (need != q_kind) {
            q_kind = need;
            const void* base = need == 0 ? q_intra : need == 1 ? q_succ : q_inter;
            const T* qrow = static_cast<const T*>(base) + (qb * p.num_q_heads + qh0 + col) * D;
#pragma unroll
            for (int c = 0; c < KC; ++c) qT[c] = (col < G) ? load8(qrow + c * 32 + quad * 8) : zero8<T>();
          }
        }
        f32x4 s[kChunks][2];
#pragma unroll
        for (int c = 0; c < kChunks; ++c)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            s[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
              if constexpr (Q4) s[c][t] = mfma16(nib8_plus24<T>(kW[c][t][kc], n4), qT[kc], s[c][t]);
              else if constexpr (Q8) s[c][t] = mfma16(codes_to_v8<T>(kR[c][t][kc]), qT[kc], s[c][t]);
              else s[c][t] = mfma16(kA[c][t][kc], qT[kc], s[c][t]);
            }
          }
        f32x4 kS_cur[kChunks][2];   // this step's K scales (the next step's load replaces kS)
        if constexpr (Q8) {
#pragma unroll
          for (int c = 0; c < kChunks; ++c) {
            kS_cur[c][0] = kS[c][0];
            kS_cur[c][1] = kS[c][1];
          }
        }
        // next step's K streams in during this step's math
        if (kAlwaysLoad || has_next) load_k(seg0, nxt, has_next);
        if constexpr (Q8) {   // scores of the int8 cache: (codes . q) * the key's K scale
#pragma unroll
          for (int c = 0; c < kChunks; ++c)
#pragma unroll
            for (int t = 0; t < 2; ++t) s[c][t] *= kS_cur[c][t];
        }

        // Lane holds keys t0 + 8*(quad&1) + i of run 2c + quad/2, i = 4*t + j (Q4: keys t0 + 8c + i
        // of run quad).
        uint32_t keep[kChunks];
        bool full = true;
        float mloc = -INFINITY;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          const Run rv = rl.at(geo, seg0 + kRunsPerStep * step + (Q4 ? quad : 2 * c + (quad >> 1)));
          const int32_t key0 = rv.t0 + (Q4 ? 8 * c : (quad & 1) * 8);
          keep[c] = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int32_t t = key0 + i;
            keep[c] |= (uint32_t)((t >= rv.lo) && (t < rv.hi)) << i;
          }
          full = full && keep[c] == 0xFFu;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float e = ((keep[c] >> i) & 1u) ? s[c][i >> 2][i & 3] : -INFINITY;
            s[c][i >> 2][i & 3] = e;
            mloc = fmaxf(mloc, e);
          }
        }
        mloc *= DCA ? sl2 : p.scale_log2;   // softmax_scale > 0: max commutes with the scale
        // Lazy reference max, shared by the four lanes of a column: it moves only when a score
        // exceeds it by more than 8 (log2 units), so the cross-lane max and the O rescale run on
        // few steps; p = 2^(x - m_run) <= 256 in between.
        if (__any(mloc > m_run + 8.f)) {
          const float mx = max_xor32(max_xor16(mloc));
          const float m_new = fmaxf(m_run, mx);
          const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oT[dt] *= alpha;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            x[i] = fast_exp2(fmaf(s[c][i >> 2][i & 3], DCA ? sl2 : p.scale_log2, -m_use));
          if constexpr (Q8) {
            // weights times the keys' V scales; absent keys (whose scale may be anything) give 0.
            // The row sum takes the fp32 weights: PV multiplies each one by its key's scale first.
            float xv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              l_run += x[i];
              xv[i] = ((keep[c] >> i) & 1u) ? x[i] * vS[c][i >> 2][i & 3] : 0.f;
            }
            const v8<PT> pB = pack8<PT>(xv);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oT[dt] = mfma16(codes_to_v8<PT>(vR[c][dt]), pB, oT[dt]);
          } else if constexpr (Q4) {
            // codes are always finite and absent keys weigh 0: no selection needed
            const v8<T> pB = pack8<T>(x);
            l_run = sum8(pB, l_run);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oT[dt] = mfma16(nib8_plus24<T>(vW[c][dt], n4), pB, oT[dt]);
          } else {
            // the row sum adds exactly the rounded weights that PV multiplies
            const v8<T> pB = pack8<T>(x);
            l_run = sum8(pB, l_run);
            if (!full) {
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) vA[c][dt] = select8<T>(vA[c][dt], keep[c]);
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oT[dt] = mfma16(vA[c][dt], pB, oT[dt]);
          }
        }
        // V registers are free once the PV MFMAs issued
        if (kAlwaysLoad || has_next) load_v(seg0, nxt, has_next);
        step = nxt;
      }
    }
    // lanes sharing a column hold partial sums over disjoint keys
    l_run = add_xor32(add_xor16(l_run));
    if constexpr (Q4) {
      // every V operand was 24 + code: take 24 times the weights back out, then the channel scale
      const float* vsc = p.v_scale + (int64_t)h * D + quad * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 sc = *reinterpret_cast<const f32x4*>(vsc + dt * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) oT[dt][j] = (oT[dt][j] - 24.f * l_run) * sc[j];
      }
    }
    if (quad == 0) {
      sm_m[wave][col] = m_run;
      sm_l[wave][col] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm_o[wave][col][dt * 16 + quad * 4 + j] = oT[dt][j];
    __syncthreads();

    // ---- merge the waves; write the output (single item) or a partial -----------------------
    // Two channels per thread and pass: a record takes one 8-byte store per pair.
    const bool direct = !ret || p.n_split == 1;
    float* part = p.partial + ((((int64_t)b * p.num_kv_heads + h) * gch + gc) * p.n_split + split) *
                                  Gs * (D + 2);
    for (int idx = tid; idx < G * D / 2; idx += kThreads) {
      const int g = idx / (D / 2), d = (idx % (D / 2)) * 2;
      float M = sm_m[0][g];
#pragma unroll
      for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, sm_m[w][g]);
      const float Mu = (M == -INFINITY) ? 0.f : M;
      float num0 = 0.f, num1 = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float c = fast_exp2(sm_m[w][g] - Mu);
        num0 += c * sm_o[w][g][d];
        num1 += c * sm_o[w][g][d + 1];
        den += c * sm_l[w][g];
      }
      if (direct) {
        T* o = static_cast<T*>(p.out) + (qb * p.num_q_heads + qh0 + g) * D;
        o[d] = from_f32<T>(den > 0.f ? num0 / den : 0.f);
        o[d + 1] = from_f32<T>(den > 0.f ? num1 / den : 0.f);
      } else {
        store_coherent_pair(part + g * (D + 2) + d, num0, num1);
        if (d == 0) store_coherent_pair(part + g * (D + 2) + D, M, den);
      }
    }
    if (direct) return;
  } else if (!ret || p.n_split == 1) {
    // nothing visible (L == 0): zero output row(s)
    for (int idx = tid; idx < G * D; idx += kThreads) {
      T* o = static_cast<T*>(p.out) + (qb * p.num_q_heads + qh0) * D;
      o[idx] = from_f32<T>(0.f);
    }
    return;
  }

  // ---- split merge ----------------------------------------------------------------------------
  // Partials were written with device-coherent (write-through) stores; waiting for them to
  // complete before a ticket makes them visible to whichever workgroup, on any XCD, draws the
  // last ticket, which reads them back with device-coherent loads. No cache-wide write-back or
  // invalidate is needed, so other workgroups' cached K/V lines are left alone.
  //
  // Up to kMergeGroup splits per (b, h): the last item to arrive folds all partials into the
  // output. More (n_group > 0): the last item of each group of kMergeGroup splits folds the
  // group's partials into one record of the same form (unnormalised O, max, denominator), and the
  // last group to finish folds the records into the output, so no single workgroup reads more than
  // kMergeGroup partials per q head.
  wait_stores_complete();
  __syncthreads();
  const int64_t row = ((int64_t)b * p.num_kv_heads + h) * gch + gc;
  const int n_act = (L + p.split_tokens - 1) / p.split_tokens;
  T* const obase = static_cast<T*>(p.out) + (qb * p.num_q_heads + qh0) * D;
  const int64_t rec_floats = (int64_t)Gs * (D + 2);   // record stride

  // Fold n_in records at src (rec_floats apart; heads 0 .. G - 1 of each used; all complete) into
  // the output (rec == nullptr) or into the record rec: (1) per q head g, one wave reduces the
  // records' (m, l) into the merged max and denominator and leaves each record's weight in LDS
  // (the wave buffers are free by now); (2) out[g][d] = sum_s w[g][s] O_s[g][d], two channels per
  // 8-byte load, each thread keeping merge_loads loads in flight across its outputs and the
  // records, and reading its weights four at a time.
  auto fold_records = [&](const float* src, int n_in, float* rec) {
    constexpr int kR = kFastMergeSplits / kWave;
    constexpr int kWStride = kR * kWave;   // weights of one q head; zero past n_in
    float* sm_w = &sm_o[0][0][0];          // [G][kWStride]
    // q heads per wave in the weights phase: the (m, l) loads of all of them go out first
    constexpr int kGW = (16 + kDecodeWaves - 1) / kDecodeWaves;
    auto weights = [&]() {
      uint64_t ml[kGW][kR];
#pragma unroll
      for (int j = 0; j < kGW; ++j) {
        const int g = wave + j * kDecodeWaves;
#pragma unroll
        for (int i = 0; i < kR; ++i) {
          const int sp = lane + i * kWave;
          ml[j][i] = (g < G && sp < n_in) ? load_coherent_pair(src + sp * rec_floats + g * (D + 2) + D) : 0;
        }
      }
#pragma unroll
      for (int j = 0; j < kGW; ++j) {
        const int g = wave + j * kDecodeWaves;
        if (g >= G) break;
        float mv[kR], lv[kR];
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < kR; ++i) {
          const bool in = lane + i * kWave < n_in;
          mv[i] = in ? __uint_as_float((uint32_t)ml[j][i]) : -INFINITY;
          lv[i] = in ? __uint_as_float((uint32_t)(ml[j][i] >> 32)) : 0.f;
          M = fmaxf(M, mv[i]);
        }
        M = wave_max(M);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float den = 0.f;
#pragma unroll
        for (int i = 0; i < kR; ++i) den += (mv[i] == -INFINITY) ? 0.f : fast_exp2(mv[i] - Mu) * lv[i];
        den = wave_sum(den);
        // the output is normalised; a record keeps its max and denominator
        const float inv = rec ? 1.f : (den > 0.f ? 1.f / den : 0.f);
        if (rec && lane == 0) {
          store_coherent(rec + g * (D + 2) + D, M);
          store_coherent(rec + g * (D + 2) + D + 1, den);
        }
#pragma unroll
        for (int i = 0; i < kR; ++i)
          sm_w[g * kWStride + lane + i * kWave] = (mv[i] == -INFINITY) ? 0.f : fast_exp2(mv[i] - Mu) * inv;
      }
      __syncthreads();
    };
    const int pairs = G * D / 2;
    // The first round of partial outputs is loaded before the weights, so that both round trips
    // to the records (written from other XCDs) overlap.
    auto fold = [&](auto KP) {
      constexpr int kP = decltype(KP)::value;        // channel pairs per thread
      constexpr int kCS = merge_loads<kDecodeWaves>() / kP;   // records per round
      float acc0[kP], acc1[kP];
      int gk[kP];
      int64_t off[kP];
#pragma unroll
      for (int k = 0; k < kP; ++k) {
        const int pr = min(tid + k * kThreads, pairs - 1);
        gk[k] = pr / (D / 2);
        off[k] = (int64_t)gk[k] * (D + 2) + (pr % (D / 2)) * 2;
        acc0[k] = acc1[k] = 0.f;
      }
      uint64_t v[kP][kCS];
      auto load_round = [&](int s0) {
#pragma unroll
        for (int k = 0; k < kP; ++k)
#pragma unroll
          for (int i = 0; i < kCS; ++i)
            v[k][i] = load_coherent_pair(src + (int64_t)min(s0 + i, n_in - 1) * rec_floats + off[k]);
      };
      if (n_in > 0) load_round(0);
      weights();
      static_assert(kCS % 4 == 0 && kWStride % kCS == 0, "weights are read four at a time");
      for (int s0 = 0; s0 < n_in; s0 += kCS) {
        if (s0 > 0) load_round(s0);
#pragma unroll
        for (int k = 0; k < kP; ++k) {
          // records past n_in were loaded from the last one (finite) and weigh 0
          const f32x4* w4 = reinterpret_cast<const f32x4*>(sm_w + gk[k] * kWStride + s0);
#pragma unroll
          for (int i4 = 0; i4 < kCS / 4; ++i4) {
            const f32x4 w = w4[i4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc0[k] += w[e] * __uint_as_float((uint32_t)v[k][4 * i4 + e]);
              acc1[k] += w[e] * __uint_as_float((uint32_t)(v[k][4 * i4 + e] >> 32));
            }
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kP; ++k) {
        const int pr = tid + k * kThreads;
        if (pr < pairs) {
          const int d = (pr % (D / 2)) * 2;
          if (rec) {
            store_coherent(rec + off[k], acc0[k]);
            store_coherent(rec + off[k] + 1, acc1[k]);
          } else {
            obase[gk[k] * D + d] = from_f32<T>(acc0[k]);
            obase[gk[k] * D + d + 1] = from_f32<T>(acc1[k]);
          }
        }
      }
    };
    const int ppt = (pairs + kThreads - 1) / kThreads;
    if (ppt <= 1) fold(std::integral_constant<int, 1>{});
    else if (ppt <= 2) fold(std::integral_constant<int, 2>{});
    else if (ppt <= 4) fold(std::integral_constant<int, 4>{});
    else fold(std::integral_constant<int, 8>{});
  };

  int32_t* ctr = p.counter + row;
  if (p.n_group > 0) {
    const int grp = split / kMergeGroup;
    const int first = grp * kMergeGroup;
    const int members = min(kMergeGroup, p.n_split - first);
    int32_t* gctr = p.gcounter + row * p.n_group + grp;
    if (tid == 0) sm_ticket = __hip_atomic_fetch_add(gctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (sm_ticket != members - 1) return;
    float* rec = p.gpartial + (row * p.n_group + grp) * rec_floats;
    fold_records(p.partial + (row * p.n_split + first) * rec_floats,
                 min(max(n_act - first, 0), kMergeGroup), rec);
    if (tid == 0) __hip_atomic_store(gctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_stores_complete();
    __syncthreads();
    if (tid == 0) sm_ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (sm_ticket != p.n_group - 1) return;
    // records of groups past the valid length hold max -inf and weigh nothing
    fold_records(p.gpartial + row * p.n_group * rec_floats, (n_act + kMergeGroup - 1) / kMergeGroup,
                 nullptr);
    if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (tid == 0) sm_ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (sm_ticket != p.n_split - 1) return;
  const float* base = p.partial + row * p.n_split * rec_floats;
  if (n_act <= kFastMergeSplits) {
    fold_records(base, n_act, nullptr);
  } else {
    // Many splits (a small split_tokens on a long context): one pass over the partials, online;
    // a chunk of kMergeChunk splits is loaded at once, then folded into the running (M, num, den)
    // of each (q head, channel).
    constexpr int kMergeChunk = 16;
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int g = idx / D, d = idx % D;
      float M = -INFINITY, num = 0.f, den = 0.f;
      for (int s0 = 0; s0 < n_act; s0 += kMergeChunk) {
        float mv[kMergeChunk], lv[kMergeChunk], ov[kMergeChunk];
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) {
          const float* rec = base + min(s0 + i, n_act - 1) * rec_floats + g * (D + 2);
          mv[i] = load_coherent(rec + D);
          lv[i] = load_coherent(rec + D + 1);
          ov[i] = load_coherent(rec + d);
        }
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) {
          if (s0 + i < n_act) {
            const float mn = fmaxf(M, mv[i]);
            const float keep = (M == -INFINITY) ? 0.f : fast_exp2(M - mn);
            const float c = fast_exp2(mv[i] - mn);
            num = num * keep + c * ov[i];
            den = den * keep + c * lv[i];
            M = mn;
          }
        }
      }
      obase[g * D + d] = from_f32<T>(den > 0.f ? num / den : 0.f);
    }
  }
  if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


}  // namespace

}  // namespace duo
