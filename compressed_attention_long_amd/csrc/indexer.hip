// Lightning indexer scores and top-k selection.
//
// Score of compressed entry j for one query token: a weighted sum over the indexer
// heads of the ReLU of the head's query dotted with the entry's key; the k best
// visible entries are kept (DeepSeek-V4-Pro vs Inkling, Component-by-component
// table, CSA row; atlas Raw config fields index_n_heads / index_head_dim /
// index_topk).
//
// Scores: the contraction is q_idx [heads x Di] times keys [Di x entries], run on
// bf16 MFMA 16x16x32 with heads as M, entries as N and Di as K.  Each lane then owns
// one entry and 4 heads per 16-head block, so the ReLU and the per-head weights are
// applied in registers and only two cross-lane adds finish the head sum.  Keys
// stream from HBM straight into registers (no LDS): lane (entry n, group g) reads the
// contiguous channels [32g, 32g+32) of key n, so a wave reads 16 whole key rows per
// tile; the query fragments follow the same channel permutation.  fp8 keys are
// widened to bf16 in registers (exact: E4M3 values fit bf16) and the per-key scale
// multiplies the finished score (scales are >= 0, so they commute with the ReLU).
//
// Top-k: one 1024-lane block per query row.  Scores map to order-preserving uint32
// keys.  A 2048-bin histogram over a linear scale of the current key range finds the
// bin holding the k-th largest key; that bin's own key range becomes the next range
// (at most three passes reach a single key) until the candidates fit in LDS, where
// they are ranked exactly by (score descending, index ascending).  The k-th candidate
// (T, I) is a threshold in that total order; a final pass writes every j with key > T,
// or key == T and j <= I, in ascending index order.  Bins that are linear in the key
// (uniform in value within a binade) keep LDS atomics spread out even when all scores
// crowd into one binade.
#include "compress_dev.hpp"

namespace csa {

// Number of entries of a cache visible to a query at position qp (see csa.h).
__device__ __forceinline__ int visible_rows(int64_t qp, int64_t pos0, int window, int stride,
                                            int n_valid, int cap) {
  int nv = min(max(n_valid, 0), cap);
  int64_t num = qp - pos0 - (window - 1);
  if (num < 0) return 0;
  int64_t jmax = num / stride;             // last visible row
  return (int)min((int64_t)nv, jmax + 1);
}

// ReLU as an integer max on the bit pattern: negative floats are negative integers.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// x[l] + x[l ^ 16] + x[l ^ 32] + x[l ^ 48] for every lane, with the gfx950 lane-swap
// permutes (row pairs, then wave halves) instead of LDS-routed shuffles.
__device__ __forceinline__ float sum_lane_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------- scores

constexpr int kIdxBlockTiles = 128;      // tiles of 16 entries per block (2,048 entries)
constexpr int kIdxWaves = 4;             // waves per block of the fused scores + compress launch
// Score-tile loads in flight per wave (the register ring's depth): 8 when the scores grid has
// at most kDeepRingBlocks blocks (about one per CU, so each wave must keep more loads in flight:
// 65K decode fused call 32.8 -> 32.1 us), else 4 (grids of 512 and more, as at 1M, lose with 8).
constexpr int kDeepRingBlocks = 256;

// Tiles of 16 entries in a decode scores block's chunk: 128 for one query row per block; 64 when
// a block holds a sequence's 2 or 4 rows (each wave then scores a whole row's share of the chunk,
// and twice the blocks run two per CU).
constexpr int scores_chunk_tiles(int tq) { return tq == 1 ? kIdxBlockTiles : kIdxBlockTiles / 2; }

// One block of the decode scores grid: entries from chunk * 16 scores_chunk_tiles(TQ) for TQ query rows
// row0 .. row0 + TQ - 1.  TQ = 1: the block's waves split the chunk for one row.  TQ = Tq > 1
// (several query tokens per sequence): the block holds all of a sequence's rows, NW / TQ waves
// per row, so its waves read the same key tiles at about the same time and the keys cross
// from memory once per sequence instead of once per row (the other waves' loads hit the cache).
template <int HB, bool FP8, int DEPTH, int NW, int TQ = 1>
__device__ __forceinline__ void index_scores_block(const IndexArgs& a, int row0, int chunk) {
  static_assert(NW % TQ == 0, "whole waves per row");
  constexpr int WPR = NW / TQ;                               // waves per row
  constexpr int CT = scores_chunk_tiles(TQ);                 // tiles of the block's chunk
  constexpr int kIdxTilesPerWave = CT / WPR;
  static_assert(kIdxTilesPerWave % DEPTH == 0, "whole ring rounds stay inside a wave's tiles");
  __shared__ float sbuf[NW][kIdxTilesPerWave * 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, in an SGPR
  const int row = row0 + wave / WPR;
  const int b = row / a.Tq;
  const int n = lane & 15, g = lane >> 4;
  const int64_t qp = a.q_pos[row];
  const int nvis = visible_rows(qp, a.pos0[b], a.window, a.stride, a.n_valid[b], a.cap);
  float* srow = a.scores + (int64_t)row * a.cap;
  const int base = chunk * (CT * 16) + (wave % WPR) * (kIdxTilesPerWave * 16);

  // query fragments: A operand, row = head (hb*16 + n), k = 8g + i <-> channel 32g + 8s + i
  bf16x8 qf[HB][4];
  float wv[HB][4];
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q_idx) + (int64_t)row * a.Hi * a.Di;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hb * 16 + n;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(q + (int64_t)min(h, a.Hi - 1) * a.Di + 32 * g + 8 * s);
      if (h >= a.Hi) v = u32x4{0u, 0u, 0u, 0u};
      qf[hb][s] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = hb * 16 + 4 * g + i;
      const float wl = a.w[(int64_t)row * a.Hi + min(hh, a.Hi - 1)];
      wv[hb][i] = hh < a.Hi ? wl : 0.f;
    }
  }

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.keys) +
                         (int64_t)b * a.cap * (FP8 ? a.Di : 2 * a.Di);
  // per tile and lane: KW dwords of key channels, plus (fp8) one dword holding the key's scale
  constexpr int KW = FP8 ? 8 : 16;
  constexpr int KR = FP8 ? KW + 1 : KW;
  const float* sbase = FP8 ? a.key_scales + (int64_t)b * a.cap : nullptr;
  // Branch-free loads (row index clamped into the visible range; results past nvis are
  // masked when the score is written) so the compiler can keep DEPTH tiles in flight.
  const int jlast = max(nvis - 1, 0);
  auto load_tile = [&](int t0, uint32_t (&r)[KR]) {
    const int j = min(t0 + n, jlast);
    const uint8_t* p = kbase + (int64_t)j * (FP8 ? 128 : 256) + (FP8 ? 32 : 64) * g;
#pragma unroll
    for (int c = 0; c < KW / 4; ++c) {
      u32x4 v = *reinterpret_cast<const u32x4*>(p + 16 * c);
      r[4 * c] = v[0]; r[4 * c + 1] = v[1]; r[4 * c + 2] = v[2]; r[4 * c + 3] = v[3];
    }
    if constexpr (FP8) r[KW] = __float_as_uint(sbase[j]);
  };

  // DEPTH tiles in flight per wave: the loads of tile t + DEPTH are issued as tile t is
  // consumed, from a ring of register buffers indexed at compile time.  The loop is software
  // pipelined by one tile: tile t's products are issued before tile t - 1's ReLU-weighted head
  // sum, which does not depend on them, so the matrix cores run while the vector ALU works.
  uint32_t ring[DEPTH][KR];
  int ntile = 0;
  if (base < nvis) ntile = min(kIdxTilesPerWave, (nvis - base + 15) / 16);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    load_tile(base + 16 * min(d, max(ntile - 1, 0)), ring[d]);
  // Straight-line body: the loop runs whole ring rounds (tiles past ntile recompute the last
  // tile's rows and land in sbuf slots whose entries are not visible), and the first round's
  // head sum of "tile -1" lands in tile 0's slots, rewritten a step later.
  f32x4 prev[HB];            // products of the previous tile, awaiting their head sum
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) prev[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float prev_scale = 1.f;
  int tprev = 0;
  auto finish = [&](const f32x4 (&acc)[HB], float kscale, int t) {
    float sc = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc += wv[hb][i] * relu(acc[hb][i]);
    sc = sum_lane_groups(sc);
    if (FP8) sc *= kscale;
    // staged in LDS: global stores inside the loop would count against vmcnt and stall the ring
    if (g == 0) sbuf[wave][16 * t + n] = sc;
  };
  // The tile loop always runs its full compile-time count (tiles past ntile recompute the last
  // tile), fully unrolled: with a back edge the compiler waits for every load in flight at the
  // loop header, which drains the ring once per round.
  if (ntile > 0) {
#pragma unroll
  for (int t0 = 0; t0 < kIdxTilesPerWave; t0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int t = t0 + d;
      uint32_t (&cur)[KR] = ring[d];
      f32x4 acc[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 kb;
        if (FP8) {
          // 8 codes (channels 32g + 8s .. +8) -> 8 bf16, exactly: gfx950's scaled converter with
          // scale 1 takes two E4M3FN codes straight to a bf16 pair (every E4M3 value is a bf16
          // value; checked bit for bit against the fp32 converter over all finite code pairs)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const uint32_t w = cur[2 * s + h2];
            kb[2 * h2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
            kb[2 * h2 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
          }
        } else {
          kb[0] = cur[4 * s]; kb[1] = cur[4 * s + 1]; kb[2] = cur[4 * s + 2]; kb[3] = cur[4 * s + 3];
        }
        const bf16x8 kf = __builtin_bit_cast(bf16x8, kb);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[hb][s], kf, acc[hb], 0, 0, 0);
      }
      const float kscale = FP8 ? __uint_as_float(cur[KW]) : 1.f;
      // next load for this ring slot (past the last tile it re-reads that tile: an L2 hit)
      load_tile(base + 16 * min(t + DEPTH, ntile - 1), ring[d]);
      finish(prev, prev_scale, tprev);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) prev[hb] = acc[hb];
      prev_scale = kscale;
      tprev = t;
    }
  }
  finish(prev, prev_scale, tprev);
  }
  // write this wave's scores, coalesced; entries past the visible count score -inf
#pragma unroll
  for (int i = lane; i < kIdxTilesPerWave * 16; i += 64) {
    const int j = base + i;
    if (j < a.cap) srow[j] = j < nvis ? sbuf[wave][i] : -INFINITY;
  }
}

// grid (rows / TQ, chunks): block x takes rows TQ x .. TQ x + TQ - 1
template <int HB, bool FP8, int DEPTH, int NW, int TQ>
__global__ void __launch_bounds__(64 * NW) k_index_scores(IndexArgs a) {
  index_scores_block<HB, FP8, DEPTH, NW, TQ>(a, TQ * blockIdx.x, blockIdx.y);
}

// The same grid with a decode step's compress blocks after it (csa_index_topk_compress): the
// compressor writes only the KV and window caches, which the scores do not read, so its
// short, latency-bound blocks run beside the scores blocks instead of in a launch of their
// own.  Blocks [0, n_idx) are the scores grid in launch order (row fastest).
template <int HB, bool FP8, int DEPTH, int TQ>
__global__ void __launch_bounds__(256) k_index_scores_compress(IndexArgs a, CompressBatch cb, int n_idx) {
  const int L = blockIdx.x;
  const int units = a.B * a.Tq / TQ;
  if (L < n_idx) index_scores_block<HB, FP8, DEPTH, kIdxWaves, TQ>(a, TQ * (L % units), L / units);
  else compress_batch_block(cb, L - n_idx);
}

// Query rows per scores block: a sequence's Tq rows when Tq is 2 or 4 (whole waves per row),
// else one.
static inline int scores_rows_per_block(int Tq) { return (Tq == 2 || Tq == 4) ? Tq : 1; }

// ---------------------------------------------------------------- scores, many query rows

// Prefill chunks (many query rows per sequence): every query row scores the same keys, so a
// block takes 16 consecutive query rows of one sequence (two per wave, eight waves) and
// streams the sequence's keys once through LDS, 128 keys per double-buffered chunk, instead
// of once per query row.  Each key fragment read from LDS then feeds 2 rows x HB head
// blocks of MFMAs, and the contraction is MFMA-bound rather than bound by key traffic.
// Keys are staged with the 16-byte segments of key r rotated by r (slot = segment ^ (r & 15)),
// so that the 16 keys of an MFMA tile read one segment each from 16 different bank groups.
// bf16 keys; the query and channel permutation are those of k_index_scores.
constexpr int kMqWaves = 8;
constexpr int kMqRows = 2 * kMqWaves;     // query rows per block
constexpr int kMqChunk = 128;             // keys per LDS chunk (32 KB of bf16 keys)

template <int HB>
__global__ void __launch_bounds__(kMqWaves * 64, 1) k_index_scores_mq(IndexArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kb0[kMqChunk * 256];
  __shared__ __attribute__((aligned(16))) uint8_t kb1[kMqChunk * 256];
  const int groups = (a.Tq + kMqRows - 1) / kMqRows;
  const int b = blockIdx.x / groups;
  const int t0 = (blockIdx.x % groups) * kMqRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;

  // visible entries: of every row of the block (the loop runs to the largest), and of this
  // wave's two rows
  const int64_t pos0 = a.pos0[b];
  const int nv = a.n_valid[b];
  int nvis_max = 0;
  for (int r = 0; r < kMqRows; ++r) {
    const int t = t0 + r;
    if (t < a.Tq) nvis_max = max(nvis_max, visible_rows(a.q_pos[(int64_t)b * a.Tq + t], pos0, a.window, a.stride, nv, a.cap));
  }
  int row[2], nvis[2];
  bool rok[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = t0 + 2 * wave + r;
    rok[r] = t < a.Tq;
    row[r] = b * a.Tq + min(t, a.Tq - 1);
    nvis[r] = rok[r] ? visible_rows(a.q_pos[row[r]], pos0, a.window, a.stride, nv, a.cap) : 0;
  }

  // query fragments (A operand): row r, head hb*16 + n, channels 32g + 8s + [0, 8)
  bf16x8 qf[2][HB][4];
  float wv[2][HB][4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q_idx) + (int64_t)row[r] * a.Hi * a.Di;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = hb * 16 + n;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 v = *reinterpret_cast<const u32x4*>(q + (int64_t)min(h, a.Hi - 1) * a.Di + 32 * g + 8 * s);
        if (h >= a.Hi) v = u32x4{0u, 0u, 0u, 0u};
        qf[r][hb][s] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = hb * 16 + 4 * g + i;
        const float wl = a.w[(int64_t)row[r] * a.Hi + min(hh, a.Hi - 1)];
        wv[r][hb][i] = hh < a.Hi ? wl : 0.f;
      }
    }
  }

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.keys) + (int64_t)b * a.cap * 256;
  const int jlast = max(nvis_max - 1, 0);
  const int nchunk = (nvis_max + kMqChunk - 1) / kMqChunk;
  // chunk c: 32 loads of 1 KB (4 keys each), four per wave
  auto issue_chunk = [&](int c, uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int blk = wave * 4 + i;
      const int kl = blk * 4 + (lane >> 4);          // key within the chunk
      const int j = min(c * kMqChunk + kl, jlast);
      const int seg = (lane & 15) ^ (kl & 15);       // this lane's slot holds segment seg
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kbase + (int64_t)j * 256 + 16 * seg),
                                       (__attribute__((address_space(3))) void*)&buf[blk * 1024], 16, 0, 0);
    }
  };
  auto chunk_step = [&](int c, const uint8_t* cur, uint8_t* nxt) {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0): this wave's part of chunk c
    __syncthreads();                                    // all parts; everyone is done with c - 1
    if (c + 1 < nchunk) issue_chunk(c + 1, nxt);
#pragma unroll 4
    for (int tt = 0; tt < kMqChunk / 16; ++tt) {
      const int kl = 16 * tt + n;
      bf16x8 kf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[s] = *reinterpret_cast<const bf16x8*>(&cur[kl * 256 + 16 * ((4 * g + s) ^ n)]);
      f32x4 acc[2][HB];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          acc[r][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc[r][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[r][hb][s], kf[s], acc[r][hb], 0, 0, 0);
        }
      const int j = c * kMqChunk + kl;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        float sc = 0.f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc += wv[r][hb][i] * relu(acc[r][hb][i]);
        sc = sum_lane_groups(sc);
        if (g == 0 && rok[r] && j < a.cap) a.scores[(int64_t)row[r] * a.cap + j] = j < nvis[r] ? sc : -INFINITY;
      }
    }
  };
  if (nchunk > 0) issue_chunk(0, kb0);
  for (int c = 0; c < nchunk; c += 2) {
    chunk_step(c, kb0, kb1);
    if (c + 1 < nchunk) chunk_step(c + 1, kb1, kb0);
  }
  // entries past the last chunk score -inf
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (rok[r])
      for (int j = nchunk * kMqChunk + lane; j < a.cap; j += 64) a.scores[(int64_t)row[r] * a.cap + j] = -INFINITY;
}

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s) {
  const int rows = a.B * a.Tq;
  const int tq = scores_rows_per_block(a.Tq);
  const int cent = 16 * scores_chunk_tiles(tq);
  dim3 grid(rows / tq, (a.cap + cent - 1) / cent);
  const int HB = (a.Hi + 15) / 16;
  const bool f8 = a.key_dtype == CSA_FP8_E4M3;
  const bool deep = (long long)grid.x * grid.y <= kDeepRingBlocks;
  // 8 waves (two per SIMD at one block per CU) measured slower: 17.9 against 16.7 us at 65K
#define CSA_IDX_LAUNCH_TQ(hb, TQ)                                                                              \
  if (HB == hb && tq == TQ) {                                                                                 \
    if (f8 && deep) hipLaunchKernelGGL((k_index_scores<hb, true, 8, kIdxWaves, TQ>), grid, dim3(256), 0, s, a); \
    else if (f8) hipLaunchKernelGGL((k_index_scores<hb, true, 4, kIdxWaves, TQ>), grid, dim3(256), 0, s, a);    \
    else if (deep) hipLaunchKernelGGL((k_index_scores<hb, false, 8, kIdxWaves, TQ>), grid, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((k_index_scores<hb, false, 4, kIdxWaves, TQ>), grid, dim3(256), 0, s, a);          \
  }
#define CSA_IDX_LAUNCH(hb) CSA_IDX_LAUNCH_TQ(hb, 1) CSA_IDX_LAUNCH_TQ(hb, 2) CSA_IDX_LAUNCH_TQ(hb, 4)
  if (!f8 && a.Tq >= kMqRows && a.Di == 128) {
    const dim3 gmq(a.B * ((a.Tq + kMqRows - 1) / kMqRows));
#define CSA_IDX_MQ(hb) \
    if (HB == hb) hipLaunchKernelGGL((k_index_scores_mq<hb>), gmq, dim3(kMqWaves * 64), 0, s, a);
    CSA_IDX_MQ(1) CSA_IDX_MQ(2) CSA_IDX_MQ(3) CSA_IDX_MQ(4)
#undef CSA_IDX_MQ
    return hipGetLastError();
  }
  CSA_IDX_LAUNCH(1) CSA_IDX_LAUNCH(2) CSA_IDX_LAUNCH(3) CSA_IDX_LAUNCH(4)
#undef CSA_IDX_LAUNCH
#undef CSA_IDX_LAUNCH_TQ
  return hipGetLastError();
}

hipError_t launch_index_scores_compress(const IndexArgs& a, const CompressArgs* calls, int n, hipStream_t s) {
  const int rows = a.B * a.Tq;
  const int HB = (a.Hi + 15) / 16;
  const bool f8 = a.key_dtype == CSA_FP8_E4M3;
  const bool mq = !f8 && a.Tq >= kMqRows && a.Di == 128;
  CompressBatch cb;
  long long total = 0;
  if (mq || !make_compress_batch(calls, n, cb, total) || cb.n == 0) {
    if (n > 0) {
      const hipError_t e = launch_compress_batch(calls, n, s);
      if (e != hipSuccess) return e;
    }
    return launch_index_scores(a, s);
  }
  const int tq = scores_rows_per_block(a.Tq);
  const int cent = 16 * scores_chunk_tiles(tq);
  const long long n_idx = (long long)(rows / tq) * ((a.cap + cent - 1) / cent);
  const dim3 grid((unsigned)(n_idx + total));
  const bool deep = n_idx <= kDeepRingBlocks;
#define CSA_IDX_FUSED_TQ(hb, TQ)                                                                                        \
  if (HB == hb && tq == TQ) {                                                                                         \
    if (f8 && deep) hipLaunchKernelGGL((k_index_scores_compress<hb, true, 8, TQ>), grid, dim3(256), 0, s, a, cb, (int)n_idx); \
    else if (f8) hipLaunchKernelGGL((k_index_scores_compress<hb, true, 4, TQ>), grid, dim3(256), 0, s, a, cb, (int)n_idx);    \
    else if (deep) hipLaunchKernelGGL((k_index_scores_compress<hb, false, 8, TQ>), grid, dim3(256), 0, s, a, cb, (int)n_idx); \
    else hipLaunchKernelGGL((k_index_scores_compress<hb, false, 4, TQ>), grid, dim3(256), 0, s, a, cb, (int)n_idx);          \
  }
#define CSA_IDX_FUSED(hb) CSA_IDX_FUSED_TQ(hb, 1) CSA_IDX_FUSED_TQ(hb, 2) CSA_IDX_FUSED_TQ(hb, 4)
  CSA_IDX_FUSED(1) CSA_IDX_FUSED(2) CSA_IDX_FUSED(3) CSA_IDX_FUSED(4)
#undef CSA_IDX_FUSED
#undef CSA_IDX_FUSED_TQ
  return hipGetLastError();
}

// ---------------------------------------------------------------- top-k

constexpr int kTopkThreads = 1024;
constexpr int kTopkBins = 2048;
constexpr int kCandMax = 512;

// Order-preserving map of fp32 bit patterns onto uint32.
__device__ __forceinline__ uint32_t okey(float v) {
  const uint32_t u = __float_as_uint(v);
  // negative: all bits flipped; otherwise the sign bit set (branch-free: three operations)
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// The selection holds a row (or a chunk of one) in registers, read once with coalesced loads:
// thread t owns entries j = i * T + t (i < NPT).  Order-dependent steps (ascending output, the
// smallest index among tied keys) number the selected entries in index order.
// ---- wave-wide reductions without LDS: DPP within rows of 16 lanes (quad swaps, half-row
// and row mirrors), then the gfx950 lane-swap permutes across rows and wave halves.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xf, 0xf, false);
}
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x) {
  auto op = [](uint32_t p, uint32_t q) { return MAX ? max(p, q) : min(p, q); };
  x = op(x, dpp_u32<0xB1>(x));    // quad_perm [1,0,3,2]
  x = op(x, dpp_u32<0x4E>(x));    // quad_perm [2,3,0,1]
  x = op(x, dpp_u32<0x141>(x));   // row_half_mirror
  x = op(x, dpp_u32<0x140>(x));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(b[0], b[1]);
}
// inclusive prefix sum across the 64 lanes
// DPP only: shifts by 1, 2, 4, 8 within each row of 16 lanes (lanes without a source add 0),
// then lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add_src(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xf, true);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_add_src<0x111, 0xf>(x);   // row_shr:1
  x += dpp_add_src<0x112, 0xf>(x);   // row_shr:2
  x += dpp_add_src<0x114, 0xf>(x);   // row_shr:4
  x += dpp_add_src<0x118, 0xf>(x);   // row_shr:8
  x += dpp_add_src<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_add_src<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// f(Ic<I>{}) for I = B .. E - 1, each I a compile-time constant
template <int V>
struct Ic {
  static constexpr int value = V;
};
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Ic<B>{});
    static_for<B + 1, E>(f);
  }
}

// Shared state of one selection by a block of T lanes holding NPT keys each.
template <int T, int NPT>
struct SelShared {
  static constexpr int W = T / 64;
  alignas(16) uint32_t hist[kTopkBins];
  alignas(16) uint32_t ckey[kCandMax + 4];   // + 4: padding for 16-byte reads of the tail
  alignas(16) int cidx[kCandMax + 4];
  alignas(16) uint8_t flag[64 % NPT == 0 ? 16 : T * NPT];   // selection flags by entry (byte path)
  uint64_t flagw[64 % NPT == 0 ? NPT * (T / 64) : 1];        // the same as the waves' ballots
  int cnt[NPT * W];
  uint32_t red[3 * W];
  int ccount, bstar, above, bcnt, total;
  uint32_t TK;
  int I;
};

// Number the flagged entries (i, t) -- entry j = i * T + t, flag = bit i of `bits` -- in
// ascending j: per-(i, wave) counts, one in-order exclusive scan of them by wave 0, then each
// lane's offset within its wave; emit(i, number) for every flagged entry.  Two barriers.
// Returns the total.  (Flags live as bits of one 64-bit value per lane: an array of bools
// would occupy a 64-bit lane mask per element.)
template <int T, int NPT, class Emit>
__device__ __forceinline__ int sel_ranks(SelShared<T, NPT>& sh, uint64_t bits, Emit&& emit) {
  constexpr int W = T / 64, N = NPT * W, PER = (N + 63) / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const uint64_t m = __ballot((bits >> i) & 1);
    if (lane == 0) sh.cnt[i * W + wave] = __popcll(m);
  }
  __syncthreads();
  if (wave == 0) {
    int v[PER], sum = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = lane * PER + e;
      v[e] = idx < N ? sh.cnt[idx] : 0;
      sum += v[e];
    }
    const int incl = wave_incl_scan(sum);
    int run = incl - sum;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int idx = lane * PER + e;
      if (idx < N) sh.cnt[idx] = run;
      run += v[e];
    }
    if (lane == 63) sh.total = incl;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const bool on = (bits >> i) & 1;
    const uint64_t m = __ballot(on);
    if (on)
      emit(i, sh.cnt[i * W + wave] +
                  (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)));
  }
  return sh.total;
}

// The same numbering through LDS, thread-contiguous, of the selected entries (sel(i): the wave's
// lane mask of its entries i * T + t that are selected): the flags go to LDS, thread t reads back
// those of entries [t NPT, (t + 1) NPT), the per-thread counts are scanned across the block (a
// wave scan plus the wave totals), and each thread numbers its own entries in order:
// emit(j, number) with j the entry.  Two barriers and no per-index ballot rounds.  Returns the
// total.  When NPT divides 64 the flags are the waves' ballots, one 64-bit word per (index i,
// wave): entries [t NPT, (t + 1) NPT) are NPT consecutive bits of one word.  Otherwise they are
// stored as one byte per entry and read back 4 or 16 at a time.
template <int T, int NPT, class Sel, class Emit>
__device__ __forceinline__ int sel_ranks_contig(SelShared<T, NPT>& sh, Sel&& sel, Emit&& emit) {
  constexpr int W = T / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t m = 0;
  auto take4 = [](uint32_t w) -> uint32_t {   // four 0/1 bytes -> four bits
    return (w & 1u) | ((w >> 7) & 2u) | ((w >> 14) & 4u) | ((w >> 21) & 8u);
  };
  if constexpr (64 % NPT == 0) {
    uint32_t mlo = 0u, mhi = 0u;   // lane i < NPT: the wave's ballot of index i
    static_for<0, NPT>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint64_t bl = sel(i);
      // v_writelane: the wave-uniform word into lane i (a lane-select compare and two
      // conditional moves per index otherwise); the lane is an inline constant
      uint32_t lo = mlo, hi = mhi;
      asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(lo) : "s"((uint32_t)bl), "i"(i));
      asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(hi) : "s"((uint32_t)(bl >> 32)), "i"(i));
      mlo = lo;
      mhi = hi;
    });
    if (lane < NPT) sh.flagw[lane * W + wave] = ((uint64_t)mhi << 32) | mlo;
    __syncthreads();
    const int j0 = tid * NPT;             // entry j0 = i T + t0: lanes t0 .. t0 + NPT - 1 of index i
    const int t0 = j0 % T;
    const uint64_t wd = sh.flagw[(j0 / T) * W + (t0 >> 6)];
    m = NPT == 64 ? wd : (wd >> (t0 & 63)) & ((1ull << (NPT & 63)) - 1ull);
  } else if constexpr (NPT % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) sh.flag[i * T + tid] = (uint8_t)((sel(i) >> lane) & 1u);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NPT / 16; ++q) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(&sh.flag[tid * NPT + 16 * q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) m |= (uint64_t)take4(w[e]) << (16 * q + 4 * e);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NPT; ++i) sh.flag[i * T + tid] = (uint8_t)((sel(i) >> lane) & 1u);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NPT / 4; ++q)
      m |= (uint64_t)take4(*reinterpret_cast<const uint32_t*>(&sh.flag[tid * NPT + 4 * q])) << (4 * q);
  }
  const int c = __popcll(m);
  const int incl = wave_incl_scan(c);
  if (lane == 63) sh.red[wave] = (uint32_t)incl;
  __syncthreads();
  int pos = incl - c, total = 0;
#pragma unroll
  for (int w2 = 0; w2 < W; ++w2) {
    const int v = (int)sh.red[w2];
    pos += w2 < wave ? v : 0;
    total += v;
  }
  while (m) {
    emit(tid * NPT + __builtin_ctzll(m), pos++);
    m &= m - 1;
  }
  return total;
}

// The selection shared by all top-k kernels.  Lane t of the block holds entries
// j = i * T + t (i < NPT) of a key array in key[i]; key 0 marks "no entry" (keys of finite
// scores are never 0).  Selects the min(k, nvalid) entries with the largest keys, the
// smaller j winning a tie, numbers them in ascending j and calls emit(i, number) for each.
// Returns the number selected.
//
// emit(j, number) receives the entry j itself (not the register index).
// Keys are counted in 2048 equal-width bins over the current key range [klo, khi]; the bin
// holding the k-th largest key becomes the next range.  Widths shrink from < 2^32 to
// < 2^21, < 2^10 and 1, so after at most three rounds the range is a single key; the
// rounds stop early once the bin holds <= kCandMax keys, which are then ranked exactly.
template <int T, int NPT, class Emit>
__device__ __forceinline__ int select_keys(SelShared<T, NPT>& sh, const uint32_t (&key)[NPT], int nvalid,
                                           int k, Emit&& emit) {
  constexpr int W = T / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto jof = [&](int i) { return i * T + tid; };
  auto ok = [&](int i) { return key[i] != 0u; };
  uint32_t TK = 0xffffffffu;
  int I = -1;
  const bool take_all = nvalid <= k;
  if (!take_all) {
    uint32_t klo = 0xffffffffu, khi = 0u;
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      { klo = min(klo, key[i] - 1u); khi = max(khi, key[i]); }   // key 0 (no entry): -1 wraps to the top
    // A lower bound of the k-th largest key: split the lanes into aligned groups of G lanes,
    // G the largest power of two (<= 64) with G k <= T, so that there are at least k groups.
    // Each group's largest key is a different entry, so at least k entries hold a key >= the
    // smallest of those maxima, and keys below it can be left out of every round (a group
    // without an entry has maximum 0: no bound).  For k > T there is no bound.
    uint32_t lb = 0u;
    if (k <= T) {
      uint32_t gm = khi;   // this lane's largest key (0 without an entry)
      for (int m = 1; m < 64 && 2 * m * k <= T; m <<= 1) gm = max(gm, (uint32_t)__shfl_xor((int)gm, m, 64));
      lb = wave_reduce_u32<false>(gm);
    }
    klo = wave_reduce_u32<false>(klo);
    khi = wave_reduce_u32<true>(khi);
    if (lane == 0) { sh.red[wave] = klo; sh.red[W + wave] = khi; sh.red[2 * W + wave] = lb; }
    for (int b = tid; b < kTopkBins; b += T) sh.hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) {
      klo = min(klo, sh.red[w2]);
      khi = max(khi, sh.red[W + w2]);
      lb = min(lb, sh.red[2 * W + w2]);
    }
    klo = max(klo + 1u, lb);   // the smallest key (see the minimum above)
    int above = 0, cnt = 0;
    for (int round = 0; round < 3 && klo < khi; ++round) {
      const uint32_t range = khi - klo;
      const int shift = max(0, 32 - __clz((int)range) - 11);
      // keys in [klo, khi] (klo > 0: no entry's key 0 is in range), as one unsigned compare
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const uint32_t d = key[i] - klo;
        if (d <= range) atomicAdd(&sh.hist[d >> shift], 1u);
      }
      __syncthreads();
      {
        // thread t owns bins 2047 - BPT t - e (e < BPT): the bins in descending key order.
        // Every wave scans its bins; the wave totals give each thread its prefix.
        constexpr int BPT = kTopkBins / T;
        int c[BPT], sum = 0;
#pragma unroll
        for (int e = 0; e < BPT; ++e) {
          c[e] = (int)sh.hist[kTopkBins - 1 - (BPT * tid + e)];
          sum += c[e];
        }
        const int incl = wave_incl_scan(sum);
        if (lane == 63) sh.red[wave] = (uint32_t)incl;   // the min/max scratch is free by now
#pragma unroll
        for (int e = 0; e < BPT; ++e) sh.hist[kTopkBins - 1 - (BPT * tid + e)] = 0;   // next round
        __syncthreads();
        if (tid == 0) sh.ccount = 0;   // for the candidate collection below; unused within rounds
        int pre = incl - sum;
#pragma unroll
        for (int w2 = 0; w2 < W; ++w2) pre += w2 < wave ? (int)sh.red[w2] : 0;
        const int need = k - above;
        if (pre < need && need <= pre + sum) {
          int run = pre;
#pragma unroll
          for (int e = 0; e < BPT; ++e) {
            if (run < need && run + c[e] >= need) {
              sh.bstar = kTopkBins - 1 - (BPT * tid + e);
              sh.above = run;
              sh.bcnt = c[e];
            }
            run += c[e];
          }
        }
      }
      __syncthreads();
      const int bstar = sh.bstar;
      above += sh.above;
      cnt = sh.bcnt;
      const uint32_t nlo = klo + ((uint32_t)bstar << shift);
      khi = min(khi, nlo + ((1u << shift) - 1u));
      klo = nlo;
      if (cnt <= kCandMax) break;
    }
    const int need = k - above;
    if (klo == khi) {
      // one key value left: the need-th smallest index among the entries holding it
      TK = klo;
      uint64_t g = 0;
#pragma unroll
      for (int i = 0; i < NPT; ++i) g |= (uint64_t)(ok(i) && key[i] == klo) << i;
      sel_ranks<T, NPT>(sh, g, [&](int i, int r) {
        if (r == need - 1) sh.I = jof(i);
      });
      __syncthreads();
      I = sh.I;
    } else {
      // at most kCandMax keys in [klo, khi]: collect them (one slot reservation per wave and
      // index i), then rank each among all by (key desc, index asc).  The count was zeroed in
      // the last histogram round, between its barriers.
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const bool c = key[i] - klo <= khi - klo;   // klo > 0: keys of entries only
        const uint64_t m = __ballot(c);
        if (m == 0) continue;
        int base = 0;
        if (lane == 0) base = atomicAdd(&sh.ccount, __popcll(m));
        base = __builtin_amdgcn_readlane(base, 0);   // every lane is active here
        const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (c && slot < kCandMax) { sh.ckey[slot] = key[i]; sh.cidx[slot] = jof(i); }
      }
      __syncthreads();
      const int c = min(sh.ccount, kCandMax);
      const int c4 = (c + 3) >> 2;   // the last group of four reads past c: masked below
      for (int ci = tid; ci < c; ci += T) {
        const uint32_t v = sh.ckey[ci];
        const int ji = sh.cidx[ci];
        int rank = 0;
#pragma unroll 4
        for (int o4 = 0; o4 < c4; ++o4) {
          const u32x4 vo = *reinterpret_cast<const u32x4*>(&sh.ckey[4 * o4]);
          const u32x4 jo = *reinterpret_cast<const u32x4*>(&sh.cidx[4 * o4]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            rank += (4 * o4 + e < c && (vo[e] > v || (vo[e] == v && (int)jo[e] < ji))) ? 1 : 0;
        }
        if (rank == need - 1) { sh.TK = v; sh.I = ji; }
      }
      __syncthreads();
      TK = sh.TK;
      I = sh.I;
    }
  }
  // ascending compaction: selected entries numbered in index order.  The test is taken on the
  // compares' lane masks, without branches (every vector operation per key here costs the block
  // a wave instruction per 64 keys).
  if (take_all) { TK = 0u; I = -1; }   // then key > 0, i.e. every entry, is selected
  auto sel = [&](int i) -> uint64_t {
    return __builtin_amdgcn_ballot_w64(key[i] > TK) |
           (__builtin_amdgcn_ballot_w64(key[i] == TK) & __builtin_amdgcn_ballot_w64(jof(i) <= I));
  };
  return sel_ranks_contig<T, NPT>(sh, sel, emit);
}

// Scores of entries j < lim starting at s, read once with coalesced loads (index clamped
// into the range).  The loads go out before the visible count is known (lim is the row's
// allocation), so their latency overlaps that of the count's inputs.
template <int T, int NPT>
__device__ __forceinline__ void load_scores(const float* s, int lim, float (&v)[NPT]) {
  const int last = max(lim - 1, 0);
#pragma unroll
  for (int i = 0; i < NPT; ++i) v[i] = s[min(i * T + (int)threadIdx.x, last)];
}
// their keys, entries j >= n (not visible) key 0
template <int T, int NPT>
__device__ __forceinline__ void score_keys(const float (&v)[NPT], int n, uint32_t (&key)[NPT]) {
#pragma unroll
  for (int i = 0; i < NPT; ++i) key[i] = i * T + (int)threadIdx.x < n ? okey(v[i]) : 0u;
}

// One block per query row holding the whole row in registers (rows of <= T * NPT entries).
template <int T, int NPT>
__global__ void __launch_bounds__(T) k_topk_reg(IndexArgs a) {
  __shared__ SelShared<T, NPT> sh;
  const int row = blockIdx.x;
  const int b = row / a.Tq;
  const int k = a.topk;
  float v[NPT];
  load_scores<T, NPT>(a.scores + (int64_t)row * a.cap, min(a.cap, T * NPT), v);   // cap <= T NPT here
  const int nvis = visible_rows(a.q_pos[row], a.pos0[b], a.window, a.stride, a.n_valid[b], a.cap);
  int32_t* out = a.idx_out + (int64_t)row * k;
  uint32_t key[NPT];
  score_keys<T, NPT>(v, nvis, key);
  const int tot = select_keys<T, NPT>(sh, key, nvis, k, [&](int j, int pos) {
    if (pos < k) out[pos] = j;
  });
  for (int p2 = min(tot, k) + threadIdx.x; p2 < k; p2 += T) out[p2] = -1;
}

// Chunked top-k for long rows.  Stage 1: block (row, p) selects the top k of entries
// [p * chunk, (p + 1) * chunk) of the row and writes them (key, row index) in ascending index
// order to candidate slots [p * k, (p + 1) * k), padded with key 0 / index -1, and its count.
// Every entry of the row's top k is in the top k of its own chunk (same order restricted to
// the chunk), so the union of the chunks' selections holds the answer.
template <int T, int NPT>
__global__ void __launch_bounds__(T) k_topk_chunk(IndexArgs a) {
  __shared__ SelShared<T, NPT> sh;
  const int row = blockIdx.x, pch = blockIdx.y, P = gridDim.y;
  const int b = row / a.Tq;
  const int k = a.topk;
  const int base = pch * a.chunk;
  float v[NPT];
  load_scores<T, NPT>(a.scores + (int64_t)row * a.cap + base, min(a.cap - base, a.chunk), v);
  const int nvis = visible_rows(a.q_pos[row], a.pos0[b], a.window, a.stride, a.n_valid[b], a.cap);
  const int n = min(max(nvis - base, 0), a.chunk);
  uint32_t key[NPT];
  score_keys<T, NPT>(v, n, key);
  const int64_t slot0 = ((int64_t)row * P + pch) * k;
  const float* srow = a.scores + (int64_t)row * a.cap + base;
  const int tot = select_keys<T, NPT>(sh, key, n, k, [&](int j, int pos) {
    if (pos < k) {
      a.cand_key[slot0 + pos] = okey(srow[j]);   // the selected entry's key, read again
      a.cand_idx[slot0 + pos] = base + j;
    }
  });
  for (int p2 = min(tot, k) + threadIdx.x; p2 < k; p2 += T) {
    a.cand_key[slot0 + p2] = 0u;
    a.cand_idx[slot0 + p2] = -1;
  }
  if (threadIdx.x == 0) a.cand_count[(int64_t)row * P + pch] = min(tot, k);
}

// Later stages: block (row, q) takes candidate chunks [q * group, (q + 1) * group) of the
// previous stage (chunk c of a row holds its top k in slots [c * k, (c + 1) * k), in
// ascending row index, padded with key 0) and selects their top k, either as one chunk of
// the next stage (same layout) or, in the last stage (one block per row), as the output.
// Slot order is row-index order among real entries, so ties by slot are ties by row index.
template <int T, int NPT, bool FINAL>
__global__ void __launch_bounds__(T) k_topk_merge(IndexArgs a, const uint32_t* in_key, const int32_t* in_idx,
                                                  const int* in_count, int in_chunks, int group,
                                                  uint32_t* out_key, int32_t* out_idx, int* out_count) {
  __shared__ SelShared<T, NPT> sh;
  const int row = blockIdx.x, q = blockIdx.y, out_chunks = gridDim.y;
  const int k = a.topk;
  const int c0 = q * group, c1 = min(in_chunks, c0 + group);
  const int n = (c1 - c0) * k;
  int nvalid = 0;
  for (int c = c0; c < c1; ++c) nvalid += in_count[(int64_t)row * in_chunks + c];
  const int64_t base = ((int64_t)row * in_chunks + c0) * k;
  uint32_t key[NPT];
  {
    const int last = max(n - 1, 0);
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int j = i * T + (int)threadIdx.x;
      const uint32_t v = in_key[base + min(j, last)];
      key[i] = j < n ? v : 0u;
    }
  }
  int32_t* out = a.idx_out + (int64_t)row * k;
  const int64_t ob = ((int64_t)row * out_chunks + q) * k;
  const int tot = select_keys<T, NPT>(sh, key, nvalid, k, [&](int j, int pos) {
    if (pos >= k) return;
    const int32_t gi = in_idx[base + j];
    if (FINAL) {
      out[pos] = gi;
    } else {
      out_key[ob + pos] = in_key[base + j];
      out_idx[ob + pos] = gi;
    }
  });
  if (FINAL) {
    for (int p2 = min(tot, k) + threadIdx.x; p2 < k; p2 += T) out[p2] = -1;
  } else {
    for (int p2 = min(tot, k) + threadIdx.x; p2 < k; p2 += T) {
      out_key[ob + p2] = 0u;
      out_idx[ob + p2] = -1;
    }
    if (threadIdx.x == 0) out_count[(int64_t)row * out_chunks + q] = min(tot, k);
  }
}

static void launch_merge(int n, bool final_stage, dim3 grid, hipStream_t s, const IndexArgs& a,
                         const uint32_t* in_key, const int32_t* in_idx, const int* in_count, int chunks,
                         int group, uint32_t* out_key, int32_t* out_idx, int* out_count) {
  const dim3 block(1024);
#define CSA_TOPK_MERGE(NPT, FIN)                                                                          \
  hipLaunchKernelGGL((k_topk_merge<1024, NPT, FIN>), grid, block, 0, s, a, in_key, in_idx, in_count, chunks, \
                     group, out_key, out_idx, out_count)
  if (final_stage) {
    if (n <= 4096) CSA_TOPK_MERGE(4, true);
    else if (n <= 8192) CSA_TOPK_MERGE(8, true);
    else CSA_TOPK_MERGE(16, true);
  } else {
    if (n <= 4096) CSA_TOPK_MERGE(4, false);
    else if (n <= 8192) CSA_TOPK_MERGE(8, false);
    else CSA_TOPK_MERGE(16, false);
  }
#undef CSA_TOPK_MERGE
}

hipError_t launch_topk(const IndexArgs& a0, hipStream_t s) {
  IndexArgs a = a0;
  const int rows = a.B * a.Tq;
  const int k = a.topk;
  const TopkPlan pl = topk_plan(rows, a.cap, k);
  if (pl.mode == 0) {
    const dim3 grid(rows);
    if (a.cap <= 4096) hipLaunchKernelGGL((k_topk_reg<1024, 4>), grid, dim3(1024), 0, s, a);
    else if (a.cap <= 8192) hipLaunchKernelGGL((k_topk_reg<1024, 8>), grid, dim3(1024), 0, s, a);
#ifndef CSA_TOPK16K_T
#define CSA_TOPK16K_T 1024
#endif
    else if (a.cap <= 16384)
      hipLaunchKernelGGL((k_topk_reg<CSA_TOPK16K_T, 16384 / CSA_TOPK16K_T>), grid, dim3(CSA_TOPK16K_T), 0, s, a);
    else if (a.cap <= 32768) hipLaunchKernelGGL((k_topk_reg<1024, 32>), grid, dim3(1024), 0, s, a);
    // a 131K-token prefix plus a 4,096-token chunk: 33,791 entries
    else if (a.cap <= 36864) hipLaunchKernelGGL((k_topk_reg<1024, 36>), grid, dim3(1024), 0, s, a);
    else if (a.cap <= 49152) hipLaunchKernelGGL((k_topk_reg<1024, 48>), grid, dim3(1024), 0, s, a);
    else hipLaunchKernelGGL((k_topk_reg<1024, 64>), grid, dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  // candidate areas A (stage-1 chunks) and B (first merge stage): offsets from the candidate
  // area's start (the workspace part the C ABI points cand_key at, 256-byte aligned)
  const TopkCarve cv = topk_carve(rows, pl, k);
  uint8_t* w = reinterpret_cast<uint8_t*>(a.cand_key);
  uint32_t* keyA = reinterpret_cast<uint32_t*>(w + cv.keyA);
  int32_t* idxA = reinterpret_cast<int32_t*>(w + cv.idxA);
  int* cntA = reinterpret_cast<int*>(w + cv.cntA);
  uint32_t* keyB = reinterpret_cast<uint32_t*>(w + cv.keyB);
  int32_t* idxB = reinterpret_cast<int32_t*>(w + cv.idxB);
  int* cntB = reinterpret_cast<int*>(w + cv.cntB);
  a.cand_key = keyA;
  a.cand_idx = idxA;
  a.cand_count = cntA;
  a.chunk = pl.chunk;
  a.nchunk = pl.nchunk;
  hipLaunchKernelGGL((k_topk_chunk<1024, kTopkChunk / 1024>), dim3(rows, pl.nchunk), dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t* in_key = keyA;
  const int32_t* in_idx = idxA;
  const int* in_count = cntA;
  int chunks = pl.nchunk;
  bool in_A = true;
  for (;;) {
    if (chunks <= pl.group) {
      launch_merge(chunks * k, true, dim3(rows, 1), s, a, in_key, in_idx, in_count, chunks, chunks, nullptr,
                   nullptr, nullptr);
      return hipGetLastError();
    }
    const int out_chunks = (chunks + pl.group - 1) / pl.group;
    uint32_t* ok_ = in_A ? keyB : keyA;
    int32_t* oi = in_A ? idxB : idxA;
    int* oc = in_A ? cntB : cntA;
    launch_merge(pl.group * k, false, dim3(rows, out_chunks), s, a, in_key, in_idx, in_count, chunks,
                 pl.group, ok_, oi, oc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    in_key = ok_;
    in_idx = oi;
    in_count = oc;
    chunks = out_chunks;
    in_A = !in_A;
  }
}

}  // namespace csa
