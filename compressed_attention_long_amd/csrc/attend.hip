// Shared-KV multi-query attention with sink and inverse output rotation (CSA and HCA).
//
// Every query head attends to the same rows, each row being key and value at once:
// the selected compressed entries (CSA) or every visible entry (HCA), plus the raw
// tokens of the sliding window.  Each head's sink logit adds its exponential to the
// softmax denominator only.  Queries are rotated at their position on the last
// rope_dim channels, and the same channels of each head's output are rotated back by
// that position (DeepSeek-V4-Pro vs Inkling, Component-by-component table: CSA, HCA,
// sink and partial-RoPE rows; atlas Raw config fields head_dim 512, one KV head).
//
// Kernel design (gfx950, wave64, bf16 MFMA 16x16x32, fp32 accumulation):
//  * a block = 8 waves in tile groups: two groups of 4 waves holding 64 heads (32-row tiles),
//    or four groups of 2 waves holding 32 heads (16-row tiles), 16 heads per wave, for one
//    query row and one split of its row set.  Tiles are staged in LDS and used by all waves
//    of a group for both contractions (K = V); the groups take alternate tiles and merge
//    their softmax states through LDS at the end, so each SIMD runs two waves whose load,
//    softmax and MFMA phases overlap;
//  * scores are computed transposed, S^T = K Q^T (M = rows, N = heads, K = channels),
//    and the output as O^T = V^T P^T (M = channels, N = heads, K = rows): every
//    accumulator lane then belongs to one head, so the online-softmax statistics,
//    the rescaling and the final normalisation stay in the lane, and the P tile
//    leaves the score accumulators already in the B-operand layout of the second
//    contraction;
//  * the V^T operand is read from the same row-major LDS tile with the gfx950
//    transposing LDS load (ds_read_b64_tr_b16), so no transposed copy is stored;
//  * the block's query rows reach LDS by DMA once (both tile groups read their fragments
//    there), issued at entry together with the first top-k indices, ahead of the scalar
//    loads that size the row set;
//  * the sink joins the denominator once, in the epilogue (one split) or the split merge;
//  * lazy rescaling: the reference maximum moves only when a tile exceeds it by 2^8;
//  * several splits of the row set run in parallel when the query rows alone cannot
//    fill the GPU; their (max, sums, normalised fp16 output) partials are merged by
//    k_attend_combine.  With one split the kernel normalises, rotates and stores.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

constexpr int kAttWaves = 8;
constexpr int kAttThreads = kAttWaves * 64;
constexpr int kD = 512;             // channels (head dim)
// bf16 per LDS row: 1056 B, so consecutive rows start 8 banks apart.  Measured with the LDS
// bank-conflict counter at the 65K decode shape: no conflicts at this pitch (for the scores'
// 16-byte row reads and the transposing reads of P V alike), against 2.4 M conflict cycles per
// launch at 1040, 1072, 1088 or 1104 bytes.
constexpr int kPitch = 528;
constexpr int kStepRows = 64;       // rows staged per step (one tile per group); two steps in LDS
constexpr int kTargetBlocks = 256;  // split until the grid has about this many blocks
constexpr float kRescale = 8.f;     // lazy-rescale threshold (log2 units)

// Block shapes.  HPB = heads per block: 64 (two groups of 4 waves, 32-row tiles) or 32 (four
// groups of 2 waves, 16-row tiles).  Both stage 64 rows per step; each row read from LDS
// serves 16 heads per wave either way.  The 32-head shape gives twice the blocks for the same
// splits, for calls too small to fill the GPU with the 64-head shape; its 16-row tiles take
// the 16x16x16 MFMA for P V (half the work per instruction), so it is slower per row.
template <int HPB>
struct AttCfg {
  static constexpr int GW = HPB / 16;            // waves per tile group
  static constexpr int NG = kAttWaves / GW;      // tile groups
  static constexpr int T = kStepRows / NG;       // rows per tile
  static constexpr int RPT = T / 8;              // rows of each tile a wave moves per step
};

__device__ __forceinline__ int visible_rows_att(int64_t qp, int64_t pos0, int window, int stride,
                                                int n_valid, int cap) {
  int nv = min(max(n_valid, 0), cap);
  int64_t num = qp - pos0 - (window - 1);
  if (num < 0) return 0;
  return (int)min((int64_t)nv, num / stride + 1);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Reductions over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups holding one head) with
// the gfx950 lane-swap permutes, no LDS round trip.
__device__ __forceinline__ float max_lane_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_lane_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Hardware exp2 (v_exp_f32): results below 2^-126 flush to zero, which softmax weights tolerate.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N vector-memory loads of this wave are outstanding (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima = no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// KVF: the compressed cache's storage (CSA_BF16, CSA_FP8_E4M3 or CSA_FP4_E2M1); HPB: the
// block shape (AttCfg).
template <bool CSA, int KVF, int HPB>
__global__ void __launch_bounds__(kAttThreads, 2) k_attend(AttendArgs a) {
  constexpr bool QKV = KVF != CSA_BF16;   // quantized entry rows take the register path
  constexpr int kRowB = KVF == CSA_FP8_E4M3 ? kD : (KVF == CSA_FP4_E2M1 ? kD / 2 : 2 * kD);
  constexpr int GW = AttCfg<HPB>::GW, NG = AttCfg<HPB>::NG, T = AttCfg<HPB>::T, RPT = AttCfg<HPB>::RPT;
  // Two halves of tile buffers as two objects: one step's tiles are read from one half while
  // the next step's stream into the other, and separate objects let the compiler see that the
  // LDS reads never touch the half in flight (it then does not wait for those loads).  Group
  // g's tile of a step is rows [g T, (g + 1) T) of the half.
  __shared__ __attribute__((aligned(16))) uint16_t tbA[kStepRows * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t tbB[kStepRows * kPitch];
  __shared__ __attribute__((aligned(4))) uint8_t tvalid[2 * NG][T];
  __shared__ f32x2 rtab[kD / 2];                // (cos, sin) of q_pos * inv_freq[i], fp64-evaluated
  __shared__ f32x4 mrg_ml[kAttWaves / 2][kWave];  // merging waves' (max, sum, normaliser) per lane

  const int HG = (a.H + HPB - 1) / HPB;
  const uint32_t total = gridDim.x;
  const uint32_t logical = xcd_remap(blockIdx.x, total);
  const int hg = logical % HG;
  const int split = (logical / HG) % a.nsplit;
  const int row = logical / (HG * a.nsplit);
  const int b = row / a.Tq;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int grp = wave / GW, hw = wave % GW;                    // tile group, head block
  const int n = lane & 15, g = lane >> 4;
  const int head = hg * HPB + hw * 16 + n;
  const bool head_ok = head < a.H;

  // ---- loads that need only the block's coordinates go out first, ahead of the row set's
  // scalars: the first two steps' top-k indices (for CSA the split and topk bound them), the
  // block's query rows and the rotation frequencies
  const int s0 = split * a.slots_per_split;
  const int32_t* idxrow = CSA ? a.idx + (int64_t)row * a.topk : nullptr;
  // the raw top-k index behind lane k's row (CSA entries only), loaded a step ahead; turning
  // it into a row waits until the step is issued, so the load's latency stays hidden
  auto pair_idx = [&](int pr) -> int {
    const int k = lane & 7;
    const int t = NG * pr + k / RPT;
    const int slot = s0 + t * T + wave + 8 * (k % RPT);
    int j = -1;
    if (CSA && lane < 8 && slot < s0 + a.slots_per_split && slot < a.topk) j = idxrow[slot];
    return j;
  };
  const int idx0 = pair_idx(0);
  int idx_next = pair_idx(1);
  // the block's HPB query rows (1 KB each) go straight into the second tile half, row h at
  // h kPitch, once for both tile groups; wave w moves rows w, w + 8, ...
  {
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(a.q) + (int64_t)row * a.H * (2 * kD);
#pragma unroll
    for (int i = 0; i < HPB / kAttWaves; ++i) {
      const int hl = wave + kAttWaves * i;
      const int hq = min(hg * HPB + hl, a.H - 1);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(qb + (int64_t)hq * (2 * kD) + 16 * lane),
                                       (lds_void*)(tbB + hl * kPitch), 16, 0, 0);
    }
  }
  const double fr = tid < a.rope_dim / 2 ? a.inv_freq[tid] : 0.0;

  const int64_t p = a.q_pos[row];

  // ---- the row set of this query: entries, then window rows
  const int kv_nv = min(max(a.kv_n_valid[b], 0), a.kv_cap);
  int n_ent;
  if (CSA) n_ent = a.topk;
  else n_ent = visible_rows_att(p, a.kv_pos0[b], a.kv_window, a.kv_stride, a.kv_n_valid[b], a.kv_cap);
  const int64_t wp0 = a.win_pos0[b];
  const int w_nv = min(max(a.win_n_valid[b], 0), a.win_cap);
  int64_t r_lo = p - a.W + 1 - wp0;
  int64_t r_hi = p - wp0;
  if (r_lo < 0) r_lo = 0;
  if (r_hi > w_nv - 1) r_hi = w_nv - 1;
  const int n_win = (a.W > 0 && r_hi >= r_lo) ? (int)(r_hi - r_lo + 1) : 0;
  const int n_slots = n_ent + n_win;
  const int s1 = min(n_slots, s0 + a.slots_per_split);
  const int ntile = s1 > s0 ? (s1 - s0 + T - 1) / T : 0;

  // ---- rows.  A step stages tiles NG pr .. NG pr + NG - 1 (64 rows); wave w moves rows
  // w + 8 i (i < RPT) of each.  Lane k < 8 of the wave prepares the row of tile
  // NG pr + k / RPT, tile row w + 8 (k % RPT), a step ahead: its number (a kv row >= 0,
  // -2 - a window row, or -1 for no row) and its byte offset from the kv base; the loads then
  // take both from that lane.
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(a.kv) + (int64_t)b * a.kv_cap * kRowB;
  const uint8_t* winb = reinterpret_cast<const uint8_t*>(a.win) + (int64_t)b * a.win_cap * (2 * kD);
  const int64_t win_off = winb - kvb;   // window rows are addressed from the kv base too
  struct PairRows {
    int r;          // row number (lanes 0..7)
    int64_t off;    // byte offset of the row from kvb (any valid row when there is none)
  };
  auto pair_rows = [&](int pr, int j) -> PairRows {
    const int k = lane & 7;
    const int t = NG * pr + k / RPT;
    const int slot = s0 + t * T + wave + 8 * (k % RPT);
    int r = -1;
    if (lane < 8 && t < ntile && slot < s1) {
      if (slot >= n_ent) r = -2 - (int)(r_lo + (slot - n_ent));
      else if (!CSA) r = slot;
      else r = (j >= 0 && j < kv_nv) ? j : -1;
    }
    const int64_t off = r >= 0 ? (int64_t)r * kRowB
                               : (r <= -2 ? win_off + (int64_t)(-2 - r) * (2 * kD) : 0);
    return PairRows{r, off};
  };
  // bf16 rows go straight into LDS (1 KB per instruction, 16 B per lane).  The valid flags
  // of a step are written first; the 8 loads may then be spread over the compute.
  auto mark_pair = [&](int pr, const PairRows& pr_rows, int bnxt) {
    if (lane < 8) {
      const int t = NG * pr + lane / RPT;
      if (t < ntile) tvalid[bnxt + lane / RPT][wave + 8 * (lane % RPT)] = pr_rows.r != -1;
    }
  };
  // LDS address of lane-k row of a step in a half
  auto row_dst = [&](uint16_t* half, int k) -> uint16_t* {
    return half + ((k / RPT) * T + wave + 8 * (k % RPT)) * kPitch;
  };
  auto issue_row = [&](int pr, const PairRows& pr_rows, int k, uint16_t* half) {
    const int t = NG * pr + k / RPT;
    if (t >= ntile) return;
    // fp8/fp4 caches: entry rows take the register path, and empty slots (-1) are zero-filled
    // there, since the bytes of a quantized row read as bf16 may be NaN (masked scores do not
    // cancel a NaN in P x V)
    if (QKV && __builtin_amdgcn_readlane(pr_rows.r, k) >= -1) return;
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(pr_rows.off >> 32), k);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)pr_rows.off, k);
    const int64_t off = (int64_t)((hi << 32) | lo);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kvb + off + 16 * lane),
                                     (lds_void*)row_dst(half, k), 16, 0, 0);
  };
  // fp8 / fp4 entry rows: codes and the channel block's scale go through registers and
  // are widened to bf16 (code * scale, rounded; exact for fp4) on the way into LDS.  Lane
  // l holds channels 8l .. 8l + 7 of the row: 8 fp8 codes, or 8 fp4 codes in one word.
  u32x2 pre8[8];
  float pres[8];
  auto fetch_q = [&](int pr, const PairRows& pr_rows) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = __builtin_amdgcn_readlane(pr_rows.r, k);
      pre8[k] = u32x2{0u, 0u};
      pres[k] = 0.f;
      if (NG * pr + k / RPT < ntile && r >= 0) {
        const int64_t rg = (int64_t)b * a.kv_cap + r;
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.kv) + rg * kRowB;
        if (KVF == CSA_FP4_E2M1) pre8[k][0] = *reinterpret_cast<const uint32_t*>(src + 4 * lane);
        else pre8[k] = *reinterpret_cast<const u32x2*>(src + 8 * lane);
        pres[k] = a.kv_scales[rg * (kD / a.kv_scale_block) + (8 * lane) / a.kv_scale_block];
      }
    }
  };
  auto store_q = [&](int pr, const PairRows& pr_rows, uint16_t* half) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = NG * pr + k / RPT;
      const int r = __builtin_amdgcn_readlane(pr_rows.r, k);
      if (t < ntile && r >= -1) {
        const float sc = pres[k];
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (r == -1) {
        } else if (KVF == CSA_FP4_E2M1) {
          // gfx950's scaled converter: byte i (channels 2i, 2i + 1 in its low and high nibbles)
          // times the block's power-of-two scale, to a bf16 pair; exact, as code x scale fits
          // bf16 (checked bit for bit against the E2M1 definition for every byte and every
          // power-of-two scale 2^-127 .. 2^127)
          const uint32_t w = pre8[k][0];
          v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
          v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
          v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
          v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
        } else {
          const f32x2 f0 = fp8x2_lo(pre8[k][0]), f1 = fp8x2_hi(pre8[k][0]);
          const f32x2 f2 = fp8x2_lo(pre8[k][1]), f3 = fp8x2_hi(pre8[k][1]);
          v[0] = pack_bf16x2(f0[0] * sc, f0[1] * sc);
          v[1] = pack_bf16x2(f1[0] * sc, f1[1] * sc);
          v[2] = pack_bf16x2(f2[0] * sc, f2[1] * sc);
          v[3] = pack_bf16x2(f3[0] * sc, f3[1] * sc);
        }
        *reinterpret_cast<u32x4*>(row_dst(half, k) + 8 * lane) = v;
      }
    }
  };

  // ---- prologue: the first step's rows go out as soon as their indices arrive (the query
  // loads behind them complete later, in order), and the rotation table is built while
  // everything is in flight
  const int npair = (ntile + NG - 1) / NG;
  const PairRows rows0 = pair_rows(0, idx0);
  if (ntile > 0) {
    mark_pair(0, rows0, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) issue_row(0, rows0, k, tbA);
    if (QKV) { fetch_q(0, rows0); store_q(0, rows0, tbA); }
  }
  if (tid < a.rope_dim / 2) {
    float cs, sn;
    rope_cs(p, fr, cs, sn);
    rtab[tid] = f32x2{cs, sn};
  }
  // the query rows have landed once only this wave's first-step tile loads, issued after them,
  // may still be in flight (quantized rows have completed all loads in store_q already)
  if (!QKV) {
    switch (ntile > 0 ? min(8, ntile * RPT) : 0) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<1>(); break;
      case 2: wait_vmcnt<2>(); break;
      case 3: wait_vmcnt<3>(); break;
      case 4: wait_vmcnt<4>(); break;
      case 5: wait_vmcnt<5>(); break;
      case 6: wait_vmcnt<6>(); break;
      case 7: wait_vmcnt<7>(); break;
      default: wait_vmcnt<8>(); break;
    }
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  // ---- query fragments (B operand of S^T = K Q^T): head = n, channels 32c + 8g + [0, 8).
  // The rotated query is not a bf16 value: its last two chunks (channels 448..511, which
  // hold the rotated pairs for rope_dim <= 64) are carried as bf16 hi + lo so the logits
  // keep fp32 accuracy; rotated channels below 448 (rope_dim > 64) are rounded to bf16.
  bf16x8 qf[16];
  bf16x8 qlo[2];
  {
    const int rot0 = kD - a.rope_dim;
    const uint16_t* qs = tbB + (hw * 16 + n) * kPitch + 8 * g;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      u32x4 v = head_ok ? *reinterpret_cast<const u32x4*>(qs + 32 * c) : u32x4{0u, 0u, 0u, 0u};
      u32x4 lo = {0u, 0u, 0u, 0u};
      if (32 * c + 32 > rot0 && a.rope_dim > 0) {
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          const int d = 32 * c + 8 * g + 2 * k2;
          if (d >= rot0) {
            const f32x2 t2 = rtab[(d - rot0) >> 1];
            const float cs = t2[0], sn = t2[1];
            const float x0 = bf16lo_to_f32(v[k2]), x1 = bf16hi_to_f32(v[k2]);
            const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
            v[k2] = pack_bf16x2(y0, y1);
            lo[k2] = pack_bf16x2(y0 - bf16lo_to_f32(v[k2]), y1 - bf16hi_to_f32(v[k2]));
          }
        }
      }
      qf[c] = __builtin_bit_cast(bf16x8, v);
      if (c >= 14) qlo[c - 14] = __builtin_bit_cast(bf16x8, lo);
    }
  }
  const bool q_split = a.rope_dim > 0;

  // ---- online softmax state (per lane: head n; the 4 lanes of a head hold equal m).  The
  // reference maximum starts at the first tile's maximum (so a dominant row there gets weight
  // exactly 1); the sink joins once, in the epilogue or in the split merge.  l_run is the
  // exact fp32 sum of the weights (for lse); n_run sums the weights as rounded to bf16 for
  // the PV product and normalises the output, so the rounding of a dominant weight cancels
  // between numerator and denominator.
  float m_run = kNegBig, l_run = 0.f, n_run = 0.f;
  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One step: half `cur` holds step pr (buffer ids bcur .. bcur + NG - 1), `nxt` receives
  // step pr + 1.
  auto pair_step = [&](int pr, const uint16_t* cur, uint16_t* nxt, int bcur) {
    // this wave's loads of step pr are the only tile loads outstanding; after the barrier the
    // step is visible to all and every wave is done with step pr - 1, whose buffers take step
    // pr + 1; the row numbers of step pr + 2 are fetched meanwhile
    wait_vmcnt<0>();
    __syncthreads();
    const PairRows rows_cur = pair_rows(pr + 1, idx_next);
    const bool more = pr + 1 < npair;   // false whenever this group has no tile in step pr
    if (more) {
      mark_pair(pr + 1, rows_cur, bcur ^ NG);
#pragma unroll
      for (int k = 0; k < 8; ++k) issue_row(pr + 1, rows_cur, k, nxt);
      if (QKV) fetch_q(pr + 1, rows_cur);
    }
    idx_next = pair_idx(pr + 2);
    const int t = NG * pr + grp;
    if (t < ntile) {
    const int buf = bcur + grp;
    const uint16_t* tl = cur + grp * T * kPitch;

    // S^T = K Q^T for rows 16kb + [0,16) of the tile
    constexpr int KB = T / 16;
    f32x4 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* rp = &tl[(16 * kb + n) * kPitch + 8 * g];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(rp + 32 * c);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], sacc[kb], 0, 0, 0);
        if (c >= 14 && q_split)
          sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qlo[c - 14], sacc[kb], 0, 0, 0);
      }
    }
    // online softmax over this tile's rows 16kb + 4g + i (lane's head n)
    float sv[4 * KB];
    int vmask = 0;
    float tmax = kNegBig;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      // valid flags of rows 16kb + 4g + [0, 4): one 32-bit LDS read
      const uint32_t vf = *reinterpret_cast<const uint32_t*>(&tvalid[buf][16 * kb + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * kb + i;
        const bool ok = (vf >> (8 * i)) & 0xffu;
        sv[e] = sacc[kb][i] * a.scale_log2;
        if (ok) { vmask |= 1 << e; tmax = fmaxf(tmax, sv[e]); }
      }
    }
    tmax = max_lane_groups(tmax);
    // Lazy rescaling: the reference maximum m_run only moves when a tile's maximum exceeds it
    // by more than kRescale (log2 units), so the 128 output accumulators are rescaled rarely;
    // in between, weights exp2(s - m_run) stay below 2^kRescale, well inside bf16 and fp32.
    const bool grow = tmax > m_run + kRescale;
    if (__any(grow)) {
      const float m_new = grow ? tmax : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
      n_run *= alpha;
      // nothing accumulated yet (first tile with rows): the accumulators are zero already
      if (__any(grow && m_run > kNegBig)) {
#pragma unroll
        for (int db = 0; db < 32; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;
      }
      m_run = m_new;
    }
    float pv[4 * KB];
#pragma unroll
    for (int e = 0; e < 4 * KB; ++e) {
      pv[e] = (vmask >> e & 1) ? fast_exp2(sv[e] - m_run) : 0.f;
      l_run += pv[e];
    }
    uint32_t pw[2 * KB];
#pragma unroll
    for (int k = 0; k < 2 * KB; ++k) {
      pw[k] = pack_bf16x2(pv[2 * k], pv[2 * k + 1]);
      n_run += bf16lo_to_f32(pw[k]) + bf16hi_to_f32(pw[k]);
    }

    // O^T += V^T P^T: A operand (channel 16db + n, rows 16r + 4g + j) via transposing loads
    const int L = lane & 15;
    if constexpr (KB == 2) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)&tl[(4 * g + (L >> 2)) * kPitch + 16 * db + 4 * (L & 3)]);
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)&tl[(16 + 4 * g + (L >> 2)) * kPitch + 16 * db + 4 * (L & 3)]);
        typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
        const i16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, acc[db], 0, 0, 0);
      }
    } else {
      // 16-row tiles: K = 16 rows, the 16x16x16 shape (4 rows per lane, as in S^T's output)
      const i16x4 pf = __builtin_bit_cast(i16x4, u32x2{pw[0], pw[1]});
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)&tl[(4 * g + (L >> 2)) * kPitch + 16 * db + 4 * (L & 3)]);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, pf, acc[db], 0, 0, 0);
      }
    }
    }
    if (QKV && more) store_q(pr + 1, rows_cur, nxt);
  };
  for (int pr = 0; pr < npair; pr += 2) {
    pair_step(pr, tbA, tbB, 0);
    if (pr + 1 < npair) pair_step(pr + 1, tbB, tbA, NG);
  }

  // ---- merge the groups' states into group 0 through LDS (the tile buffers are free now):
  // rounds halve the number of groups, groups [span, 2 span) handing theirs to group - span
  wait_vmcnt<0>();
  __syncthreads();
#pragma unroll
  for (int span = NG / 2; span >= 1; span >>= 1) {
    // writer slot: 32 KB per wave, slots 0-1 in half A, 2-3 in half B
    auto slot_buf = [&](int sl) -> f32x4* {
      return reinterpret_cast<f32x4*>((sl < 2 ? tbA : tbB) + (sl & 1) * (32 * kWave * 8));
    };
    if (grp >= span && grp < 2 * span) {
      const int sl = (grp - span) * GW + hw;
      f32x4* mbuf = slot_buf(sl);   // [db][lane]
#pragma unroll
      for (int db = 0; db < 32; ++db) mbuf[db * kWave + lane] = acc[db];
      mrg_ml[sl][lane] = f32x4{m_run, l_run, n_run, 0.f};
    }
    __syncthreads();
    if (grp < span) {
      const int sl = grp * GW + hw;
      const f32x4* mbuf = slot_buf(sl);
      const f32x4 ml = mrg_ml[sl][lane];
      const float M = fmaxf(m_run, ml[0]);
      const float sa = fast_exp2(m_run - M), sb = fast_exp2(ml[0] - M);
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const f32x4 o = mbuf[db * kWave + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[db][i] = acc[db][i] * sa + o[i] * sb;
      }
      l_run = l_run * sa + ml[1] * sb;
      n_run = n_run * sa + ml[2] * sb;
      m_run = M;
    }
    if (span > 1) __syncthreads();
  }
  if (grp != 0) return;

  // ---- epilogue
  float l_tot = sum_lane_groups(l_run);
  const float n_tot = sum_lane_groups(n_run);
  if (!head_ok) return;
  if (a.nsplit == 1) {
    // fold in the sink: Z = l 2^(m - M) + 2^(sink - M), M = max(m, sink)
    const float sink2 = a.sink[head] * kLog2e;
    const float M = fmaxf(m_run, sink2);
    const float sc = exp2f(m_run - M);
    const float es = exp2f(sink2 - M);
    l_tot = l_tot * sc + es;
    m_run = M;
    const float inv = sc / (n_tot * sc + es);
    const int rot0 = kD - a.rope_dim;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc[db][i] * inv;
      const int d0 = 16 * db + 4 * g;
      if (16 * db + 16 > rot0 && a.rope_dim > 0) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int d = d0 + 2 * k2;
          if (d >= rot0) {
            // rotation by -q_pos: same cosine, negated sine
            const f32x2 t2 = rtab[(d - rot0) >> 1];
            const float cs = t2[0], sn = -t2[1];
            const float x0 = o[2 * k2], x1 = o[2 * k2 + 1];
            o[2 * k2] = x0 * cs - x1 * sn;
            o[2 * k2 + 1] = x0 * sn + x1 * cs;
          }
        }
      }
      const int64_t off = ((int64_t)row * a.H + head) * kD + d0;
      if (a.out_dtype == CSA_FP32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + off) = f32x4{o[0], o[1], o[2], o[3]};
      } else {
        u32x2 w2;
        w2[0] = pack_bf16x2(o[0], o[1]);
        w2[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + off) = w2;
      }
    }
    if (a.lse && g == 0) a.lse[(int64_t)row * a.H + head] = (m_run + log2f(l_tot)) * kLn2;
  } else {
    // The split's normalised output o / n in fp16 (11-bit significand: rounding within 2^-11
    // relative, far below the error the bf16 inputs carry), scaled by 2^-e so that the head's
    // largest magnitude sits below 2^14 whatever the range of the cache values; (m, n, l, e)
    // stay fp32.  Half the bytes of fp32 partials, written here and read by the merge.
    float amax = 0.f;
#pragma unroll
    for (int db = 0; db < 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(acc[db][i]));
    amax = max_lane_groups(amax);
    const float inv_n = n_tot > 0.f ? 1.f / n_tot : 0.f;
    int e = 0;
    if (amax * inv_n > 0.f) {
      int ex;
      (void)frexpf(amax * inv_n, &ex);   // amax / n = f 2^ex, f in [0.5, 1)
      e = ex - 14;
    }
    const float sc = ldexpf(inv_n, -e);
    const int64_t pr = ((int64_t)row * a.nsplit + split) * a.H + head;
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      u32x2 h;
      h[0] = pack_f16x2(acc[db][0] * sc, acc[db][1] * sc);
      h[1] = pack_f16x2(acc[db][2] * sc, acc[db][3] * sc);
      *reinterpret_cast<u32x2*>(a.part_o + pr * kD + 16 * db + 4 * g) = h;
    }
    if (g == 0) {
      *reinterpret_cast<f32x4*>(a.part_ml + 4 * pr) = f32x4{m_run, n_tot, l_tot, (float)e};
    }
  }
}

// Merge split partials: M = max(sink, m_s), o = sum 2^(m_s - M) n_s u_s / Zo with u_s = o_s / n_s
// (stored in fp16 times 2^-e_s) and Zo = 2^(sink - M) + sum n_s 2^(m_s - M) (n_s: the sum of the
// weights as rounded for the split's PV product), lse = M + log2(2^(sink - M) + sum l_s
// 2^(m_s - M)) with the exact sums l_s; then rotate back and store.  A block of 256 lanes merges 4
// (row, head) pairs, 8 channels per lane; splits are merged online, four per round, so that a
// round's (max, sum) and output loads are all in flight together.
constexpr int kCombineHeads = 4;
__global__ void __launch_bounds__(64 * kCombineHeads) k_attend_combine(AttendArgs a) {
  const int rows = a.B * a.Tq;
  // blocks in the order of the attention grid's XCD ranges: a row's merge runs on the XCD that
  // wrote its partials
  const int rh = (int)xcd_remap(blockIdx.x, gridDim.x) * kCombineHeads + (threadIdx.x >> 6);   // row * H + head
  if (rh >= rows * a.H) return;
  const int row = rh / a.H, head = rh % a.H;
  const int d0 = (threadIdx.x & 63) * 8;
  const int64_t p = a.q_pos[row];
  const float sink2 = a.sink[head] * kLog2e;
  const int64_t base = (int64_t)row * a.nsplit * a.H + head;        // partial (row, s, head) = base + s * H
  // online merge, 4 splits per round: each round's (max, sum) and output loads go out together
  float M = sink2, Z = 1.f, Zo = 1.f;   // relative to 2^M
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < a.nsplit; s0 += 4) {
    u32x4 v[4];
    float ms[4], ns[4], ls[4], es[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t pr = base + (int64_t)min(s0 + u, a.nsplit - 1) * a.H;
      const f32x4 ml = *reinterpret_cast<const f32x4*>(a.part_ml + 4 * pr);
      ms[u] = s0 + u < a.nsplit ? ml[0] : kNegBig;
      ns[u] = ml[1];
      ls[u] = ml[2];
      es[u] = ml[3];
      // read once: nontemporal loads keep them from displacing other lines
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.part_o + pr * kD + d0));
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < 4; ++u) Mn = fmaxf(Mn, ms[u]);
    const float r = exp2f(M - Mn);
    Z *= r;
    Zo *= r;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= r;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = exp2f(ms[u] - Mn);   // 0 for the padding of a partial round
      Z += ls[u] * w;
      Zo += ns[u] * w;
      const float wo = ldexpf(ns[u] * w, (int)es[u]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x2 h = unpack_f16x2(v[u][k]);
        o[2 * k] += wo * h[0];
        o[2 * k + 1] += wo * h[1];
      }
    }
    M = Mn;
  }
  const float inv = Zo > 0.f ? 1.f / Zo : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] *= inv;
  const int rot0 = kD - a.rope_dim;
  if (a.rope_dim > 0 && d0 + 8 > rot0) {
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const int d = d0 + 2 * k2;
      if (d >= rot0) {
        float cs, sn;
        rope_cs(-p, a.inv_freq[(d - rot0) >> 1], cs, sn);
        const float x0 = o[2 * k2], x1 = o[2 * k2 + 1];
        o[2 * k2] = x0 * cs - x1 * sn;
        o[2 * k2 + 1] = x0 * sn + x1 * cs;
      }
    }
  }
  const int64_t off = (int64_t)rh * kD + d0;
  if (a.out_dtype == CSA_FP32) {
    float* op = reinterpret_cast<float*>(a.out) + off;
    *reinterpret_cast<f32x4*>(op) = f32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(op + 4) = f32x4{o[4], o[5], o[6], o[7]};
  } else {
    u32x4 w4;
#pragma unroll
    for (int k = 0; k < 4; ++k) w4[k] = pack_bf16x2(o[2 * k], o[2 * k + 1]);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + off) = w4;
  }
  if (a.lse && d0 == 0) a.lse[rh] = (M + log2f(Z)) * kLn2;
}

// Splits of the row set for a block shape: enough that the grid has about kTargetBlocks
// blocks, at most one per two tiles, with the per-split count rounded up to whole tiles.
static int nsplit_for(int hpb, int rows, int H, int slot_cap) {
  const int tile = hpb == 64 ? AttCfg<64>::T : AttCfg<32>::T;
  const int HG = (H + hpb - 1) / hpb;
  const long long base = (long long)rows * HG;
  int ns = (int)((kTargetBlocks + base - 1) / base);
  const int max_ns = (slot_cap + 2 * tile - 1) / (2 * tile);   // at least two tiles per split
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  int sps = (slot_cap + ns - 1) / ns;
  sps = (sps + tile - 1) / tile * tile;
  if (sps < tile) sps = tile;
  return (slot_cap + sps - 1) / sps;
}

#ifndef CSA_ATT_HPB
#define CSA_ATT_HPB 0   // 0: chosen per call; 32 or 64: that shape always
#endif

// Block shape and splits of a call: 64 heads per block whenever that grid reaches about
// kTargetBlocks blocks (it does the fewest MFMAs per row: 32-row tiles); 32 heads per block
// when it cannot (few query rows over short row sets, as in 1M-token decode with top-k),
// where twice the blocks beat the cost of 16-row tiles.
AttendPlan attend_plan(int rows, int H, int slot_cap) {
  AttendPlan pl;
  int hpb = CSA_ATT_HPB;
  if (hpb == 0) {
    const long long blocks64 = (long long)rows * ((H + 63) / 64) * nsplit_for(64, rows, H, slot_cap);
    hpb = blocks64 < kTargetBlocks ? 32 : 64;
  }
  pl.hpb = hpb;
  pl.nsplit = nsplit_for(hpb, rows, H, slot_cap);
  const int tile = hpb == 64 ? AttCfg<64>::T : AttCfg<32>::T;
  int sps = (slot_cap + pl.nsplit - 1) / pl.nsplit;
  sps = (sps + tile - 1) / tile * tile;
  pl.sps = sps < tile ? tile : sps;
  return pl;
}

size_t attend_workspace(int rows, int H, int slot_cap, bool csa) {
  (void)csa;
  const int ns = attend_plan(rows, H, slot_cap).nsplit;
  if (ns <= 1) return 0;
  // fp16 partial outputs, then fp32 (m, n, l, e): the latter start 16-byte aligned (kD even)
  return (size_t)rows * ns * H * (kD * sizeof(uint16_t) + 4 * sizeof(float)) + 256;
}

template <int HPB>
static void launch_attend_shape(const AttendArgs& a, dim3 grid, hipStream_t s) {
  const dim3 blk(kAttThreads);
  const bool csa = a.csa_mode != 0;
  switch (a.kv_dtype) {
    case CSA_FP8_E4M3:
      if (csa) hipLaunchKernelGGL((k_attend<true, CSA_FP8_E4M3, HPB>), grid, blk, 0, s, a);
      else hipLaunchKernelGGL((k_attend<false, CSA_FP8_E4M3, HPB>), grid, blk, 0, s, a);
      break;
    case CSA_FP4_E2M1:
      if (csa) hipLaunchKernelGGL((k_attend<true, CSA_FP4_E2M1, HPB>), grid, blk, 0, s, a);
      else hipLaunchKernelGGL((k_attend<false, CSA_FP4_E2M1, HPB>), grid, blk, 0, s, a);
      break;
    default:
      if (csa) hipLaunchKernelGGL((k_attend<true, CSA_BF16, HPB>), grid, blk, 0, s, a);
      else hipLaunchKernelGGL((k_attend<false, CSA_BF16, HPB>), grid, blk, 0, s, a);
      break;
  }
}

hipError_t launch_attend(const AttendArgs& a0, hipStream_t s) {
  AttendArgs a = a0;
  const int rows = a.B * a.Tq;
  const AttendPlan pl = attend_plan(rows, a.H, a.slot_cap);
  a.nsplit = pl.nsplit;
  a.slots_per_split = pl.sps;
  const int HG = (a.H + pl.hpb - 1) / pl.hpb;
  const long long blocks = (long long)rows * HG * a.nsplit;
  const dim3 grid((unsigned)blocks);
  if (pl.hpb == 64) launch_attend_shape<64>(a, grid, s);
  else launch_attend_shape<32>(a, grid, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nsplit > 1) {
    hipLaunchKernelGGL(k_attend_combine, dim3((rows * a.H + kCombineHeads - 1) / kCombineHeads),
                       dim3(64 * kCombineHeads), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace csa
