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
//  * a block = NP wave pairs for one query row and one split of its row set; pair p owns
//    16 heads.  Rows are staged in LDS in 32-row tiles through a ring of four tile
//    buffers, so three tiles are in flight while one is consumed, and every wave of the
//    block uses every staged row (the block's 16 NP heads share it as key and value);
//  * scores are computed transposed, S^T = K Q^T (M = rows, N = heads, K = channels):
//    wave h of a pair scores rows 16h .. 16h + 15 of a tile for its pair's heads, so every
//    accumulator lane belongs to one head;
//  * the two waves of a pair exchange their tiles' maxima and their softmax weights P (fp32)
//    through LDS; then each computes O^T = V^T P^T (M = channels, N = heads, K = rows) over
//    all 32 rows for half the channels (wave h: channels 256h .. 256h + 255), so each wave
//    holds 64 accumulator registers instead of 128 and a block of eight waves covers 64
//    heads with one copy of each row;
//  * the V^T operand is read from the same row-major LDS tile with the gfx950 transposing
//    LDS load (ds_read_b64_tr_b16), so no transposed copy is stored;
//  * the loop is software pipelined by one tile: the scores of tile t + 1 and the P V
//    product of tile t run back to back, then the maxima and weights of tile t + 1 are
//    exchanged (two barriers per tile);
//  * bf16 rows reach LDS by direct DMA; fp8 and fp4 entry rows go through registers.  fp4
//    codes times their power-of-two scale are exact in bf16.  fp8 rows are staged as their
//    exact codes and the per-64-channel scales are applied in fp32: to the scores per
//    channel block, and to the weights per channel block in P V;
//  * the weights enter P V as bf16 hi + lo parts (fp8 rows: weight x row scale), so they
//    keep about 16 bits;
//  * the sink joins the denominator once, in the epilogue (one split) or the split merge;
//  * lazy rescaling: the reference maximum moves only when a tile exceeds it by 2^8;
//  * several splits of the row set run in parallel when the query rows alone cannot
//    fill the GPU; their (max, sums, normalised fp16 output) partials are merged by
//    k_attend_combine.  With one split the kernel normalises, rotates and stores.
#include "attend_dev.hpp"

namespace csa {

// ---------------------------------------------------------------- grouped kernel (bf16 caches)
//
// A block = 8 waves in tile groups: two groups of 4 waves holding 64 heads (32-row tiles), or four
// groups of 2 waves holding 32 heads (16-row tiles), 16 heads and all 512 channels per wave, for one
// query row and one split of its row set.  A step stages 64 rows (one tile per group) in LDS by
// DMA; each group uses its tile for both contractions (K = V), the groups take alternate tiles and
// merge their softmax states through LDS at the end, so each SIMD runs two waves whose load,
// softmax and MFMA phases overlap.  Two steps fit in LDS: the next step's rows stream in while the
// current one is consumed.  Scores and outputs are transposed as in the pair kernel below; the
// rotated query dims are carried as bf16 hi + lo; the sink joins once (epilogue or merge); lazy
// rescaling; weights rounded to bf16 for P V and normalised by their own sum.
// W waves per block, each moving 8 rows of every step: a step stages 8 W rows
template <int HPB, int W>
struct AttCfg {
  static constexpr int SR = 8 * W;               // rows staged per step (one tile per group)
  static constexpr int GW = HPB / 16;            // waves per tile group
  static constexpr int NG = W / GW;              // tile groups
  static constexpr int T = SR / NG;              // rows per tile
  static constexpr int RPT = T / W;              // rows of each tile a wave moves per step
  static_assert(T == kAttGroupTile64 * HPB / 64, "tile rows must match the plan's");
};

// Grouped kernel (bf16 caches); HPB, W: the block shape (AttCfg).  W = 4: one group of four
// waves (64 heads), a block small enough in LDS that two run on a CU.
template <bool CSA, int HPB, int W>
__global__ void __launch_bounds__(64 * W, 2) k_attend_grp(AttendArgs a) {
  constexpr bool QKV = false;
  constexpr int kRowB = 2 * kD;
  using Cfg = AttCfg<HPB, W>;
  constexpr int kAttWaves = W, kStepRows = Cfg::SR;
  constexpr int GW = Cfg::GW, NG = Cfg::NG, T = Cfg::T, RPT = Cfg::RPT;
  // the block's query rows go through the second tile half when they fit there, else (W = 4)
  // straight into registers
  constexpr bool kQInLds = HPB <= kStepRows;
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
    const int slot = s0 + t * T + wave + W * (k % RPT);
    int j = -1;
    if (CSA && lane < 8 && slot < s0 + a.slots_per_split && slot < a.topk) j = idxrow[slot];
    return j;
  };
  const int idx0 = pair_idx(0);
  int idx_next = pair_idx(1);
  // the block's HPB query rows (1 KB each) go straight into the second tile half, row h at
  // h kPitch, once for all tile groups; wave w moves rows w, w + W, ...  (W = 4: each wave's own
  // 16 heads into registers instead, raw; rotated below)
  u32x4 qraw[kQInLds ? 1 : 16];
  if constexpr (!kQInLds) {
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)row * a.H + min(head, a.H - 1)) * kD + 8 * g;
#pragma unroll
    for (int c = 0; c < 16; ++c) qraw[c] = *reinterpret_cast<const u32x4*>(qh + 32 * c);
  } else {
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
    const int slot = s0 + t * T + wave + W * (k % RPT);
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
      if (t < ntile) tvalid[bnxt + lane / RPT][wave + W * (lane % RPT)] = pr_rows.r != -1;
    }
  };
  // LDS address of lane-k row of a step in a half
  auto row_dst = [&](uint16_t* half, int k) -> uint16_t* {
    return half + ((k / RPT) * T + wave + W * (k % RPT)) * kPitch;
  };
  auto issue_row = [&](int pr, const PairRows& pr_rows, int k, uint16_t* half) {
    const int t = NG * pr + k / RPT;
    if (t >= ntile) return;
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(pr_rows.off >> 32), k);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)pr_rows.off, k);
    const int64_t off = (int64_t)((hi << 32) | lo);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kvb + off + 16 * lane),
                                     (lds_void*)row_dst(half, k), 16, 0, 0);
  };
  auto fetch_q = [&](int, const PairRows&) {};
  auto store_q = [&](int, const PairRows&, uint16_t*) {};

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
    const uint16_t* qs = tbB + (kQInLds ? (hw * 16 + n) * kPitch + 8 * g : 0);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      u32x4 v = !head_ok ? u32x4{0u, 0u, 0u, 0u} : (kQInLds ? *reinterpret_cast<const u32x4*>(qs + 32 * c) : qraw[c]);
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

    // S^T = K Q^T for rows 16kb + [0,16) of the tile: chunk by chunk over the row blocks, so that
    // the KB accumulation chains interleave; the lo parts of the rotated chunks are zero without
    // rotation and add nothing
    constexpr int KB = T / 16;
    // the compiler's MFMA / LDS-read interleaving strategy for this region (65K attend 27.7 ->
    // 27.1 us, HCA 1M 63.3 -> 60.9 us; the same hint on the P V region loses)
    __builtin_amdgcn_iglp_opt(1);
    f32x4 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* rp0 = &tl[n * kPitch + 8 * g];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(rp0 + 16 * kb * kPitch + 32 * c);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], sacc[kb], 0, 0, 0);
        if (c >= 14) sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qlo[c - 14], sacc[kb], 0, 0, 0);
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


// ---------------------------------------------------------------- wave-pair kernel (quantized caches)

// KVF: the compressed cache's storage (CSA_BF16, CSA_FP8_E4M3 or CSA_FP4_E2M1); NP: wave pairs.
template <bool CSA, int KVF, int NP>
__global__ void __launch_bounds__(AttShape<NP>::NT) k_attend(AttendArgs a) {
  using Sh = AttShape<NP>;
  constexpr int HPB = Sh::HPB, NW = Sh::NW, RPW = Sh::RPW;
  constexpr bool QKV = KVF != CSA_BF16;       // quantized entry rows take the register path
  constexpr bool F8 = KVF == CSA_FP8_E4M3;    // exact codes in LDS; block scales applied in fp32
  constexpr int kRowB = F8 ? kD : (KVF == CSA_FP4_E2M1 ? kD / 2 : 2 * kD);
  static_assert(HPB <= 2 * kTR, "the block's query rows are staged in two tile buffers");

  // Four tile buffers as four objects: the compiler can then see that the DMA into one does not
  // alias the reads of another (and does not wait for it before those reads).
  __shared__ __attribute__((aligned(16))) uint16_t tb0[kTR * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t tb1[kTR * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t tb2[kTR * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t tb3[kTR * kPitch];
  __shared__ __attribute__((aligned(16))) int32_t idxl[CSA ? kAttIdxMax : 4];   // the split's top-k indices
  __shared__ __attribute__((aligned(16))) float pbuf[2][NP][2][kWave][4];   // weights P (fp32), by parity
  __shared__ float mref[2][NP][2][16];          // the producing wave's reference of those weights
  __shared__ __attribute__((aligned(4))) uint8_t tvalid[4][kTR];
  __shared__ f32x2 rtab[kD / 2];                // (cos, sin) of q_pos * inv_freq[i], fp64-evaluated
  __shared__ __attribute__((aligned(16))) float qsc[F8 ? 4 : 1][kD / 64][kTR];   // fp8 row scales
  __shared__ f32x4 xch[NP][2][16];              // end of the row set: (l, m_own, amax) per wave and head

  const int HG = (a.H + HPB - 1) / HPB;
  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = logical % HG;
  const int split = (logical / HG) % a.nsplit;
  const int row = logical / (HG * a.nsplit);
  const int b = row / a.Tq;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int p = wave >> 1, h = wave & 1;                        // pair (16 heads), half
  const int n = lane & 15, g = lane >> 4;
  const int head = hg * HPB + 16 * p + n;
  const bool head_ok = head < a.H;

  // ---- loads that need only the block's coordinates go out first: the split's top-k indices
  // (CSA) and the block's query rows, both by DMA into LDS
  const int s0 = split * a.slots_per_split;
  if (CSA) {
    const int nidx = max(0, min(a.slots_per_split, a.topk - s0));
    const int32_t* irow = a.idx + (int64_t)row * a.topk;
    for (int i = wave; i * kWave < nidx; i += NW) {
      const int j = min(s0 + i * kWave + lane, a.topk - 1);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(irow + j), (lds_void*)(idxl + i * kWave), 4,
                                       0, 0);
    }
  }
  {
    // query row r (head hg HPB + r) at row r % 32 of tile buffer 2 + r / 32; wave w moves rows
    // w, w + NW, ...
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(a.q) + (int64_t)row * a.H * (2 * kD);
#pragma unroll
    for (int i = 0; i < HPB / NW; ++i) {
      const int r = wave + NW * i;              // i < kTR / NW: rows 0..31 (buffer 2), else 32..63
      const int hq = min(hg * HPB + r, a.H - 1);
      const void* src = qb + (int64_t)hq * (2 * kD) + 16 * lane;
      if (i < kTR / NW) __builtin_amdgcn_global_load_lds(src, (lds_void*)(tb2 + r * kPitch), 16, 0, 0);
      else __builtin_amdgcn_global_load_lds(src, (lds_void*)(tb3 + (r - kTR) * kPitch), 16, 0, 0);
    }
  }
  const int64_t pq = a.q_pos[row];
  if (tid < a.rope_dim / 2) {
    float cs, sn;
    rope_cs(pq, a.inv_freq[tid], cs, sn);
    rtab[tid] = f32x2{cs, sn};
  }

  // ---- the row set of this query: entries, then window rows
  const int kv_nv = min(max(a.kv_n_valid[b], 0), a.kv_cap);
  const int n_ent = CSA ? a.topk
                        : visible_rows_att(pq, a.kv_pos0[b], a.kv_window, a.kv_stride, a.kv_n_valid[b], a.kv_cap);
  const int64_t wp0 = a.win_pos0[b];
  const int w_nv = min(max(a.win_n_valid[b], 0), a.win_cap);
  int64_t r_lo = pq - a.W + 1 - wp0;
  int64_t r_hi = pq - wp0;
  if (r_lo < 0) r_lo = 0;
  if (r_hi > w_nv - 1) r_hi = w_nv - 1;
  const int n_win = (a.W > 0 && r_hi >= r_lo) ? (int)(r_hi - r_lo + 1) : 0;
  const int n_slots = n_ent + n_win;
  const int s1 = min(n_slots, s0 + a.slots_per_split);
  const int ntile = s1 > s0 ? (s1 - s0 + kTR - 1) / kTR : 0;

  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(a.kv) + (int64_t)b * a.kv_cap * kRowB;
  const uint8_t* winb = reinterpret_cast<const uint8_t*>(a.win) + (int64_t)b * a.win_cap * (2 * kD);
  const int64_t win_off = winb - kvb;   // window rows are addressed from the kv base too
  // the row a missing slot loads before it is zeroed: the first window row of the query when
  // there is one, else kv row 0 (bf16 caches only; quantized caches load nothing for it)
  const int ph_row = n_win > 0 ? -2 - (int)r_lo : 0;

  wait_vmcnt<0>();
  __syncthreads();   // indices and query rows in LDS

  // ---- rows.  Wave w moves rows w + NW i (i < RPW) of every tile.  Lane i < RPW holds the
  // number of the row it names: a kv row (>= 0), -2 - a window row, or -1 for none.
  auto tile_rows = [&](int t) -> int {
    const int slot = s0 + t * kTR + wave + NW * lane;
    int r = -1;
    if (lane < RPW && slot < s1) {
      if (slot >= n_ent) r = -2 - (int)(r_lo + (slot - n_ent));
      else if (!CSA) r = slot;
      else {
        const int j = idxl[slot - s0];
        r = (j >= 0 && j < kv_nv) ? j : -1;
      }
    }
    return r;
  };
  auto row_off = [&](int r) -> int64_t {
    return r >= 0 ? (int64_t)r * kRowB : (r <= -2 ? win_off + (int64_t)(-2 - r) * (2 * kD) : 0);
  };
  // flags and (bf16) the DMA of every row into its own slot: exactly RPW loads per wave per tile,
  // so that the load counter tells which tile has landed.  A missing row (-1) loads a valid
  // placeholder row and is zeroed once it has landed (zero_tile): stale or unwritten bytes could
  // be NaN, which a zero weight does not cancel in P V.
  auto issue_tile = [&](int rr, uint16_t* buf, int st) {
    if (lane < RPW) tvalid[st][wave + NW * lane] = rr != -1;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = __builtin_amdgcn_readlane(rr, i);
      if (QKV && r >= -1) continue;           // quantized entry rows go through registers
      const int64_t off = row_off(r == -1 ? ph_row : r);
      dma_row(kvb + off + 16 * lane, buf + (wave + NW * i) * kPitch);
    }
  };
  auto zero_tile = [&](int rr, uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      if (__builtin_amdgcn_readlane(rr, i) == -1)
        *reinterpret_cast<u32x4*>(buf + (wave + NW * i) * kPitch + 8 * lane) = u32x4{0u, 0u, 0u, 0u};
  };
  // quantized entry rows: codes and the channel block's scale through registers.  Lane l holds
  // channels 8l .. 8l + 7 of the row: 8 fp8 codes, or 8 fp4 codes in one word.
  u32x2 pre8[QKV ? RPW : 1];
  float pres[QKV ? RPW : 1];
  auto fetch_q = [&](int rr) {
    if constexpr (QKV) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int r = __builtin_amdgcn_readlane(rr, i);
        pre8[i] = u32x2{0u, 0u};
        pres[i] = 0.f;
        if (r >= 0) {
          const int64_t rg = (int64_t)b * a.kv_cap + r;
          const uint8_t* src = reinterpret_cast<const uint8_t*>(a.kv) + rg * kRowB;
          if (KVF == CSA_FP4_E2M1) pre8[i][0] = *reinterpret_cast<const uint32_t*>(src + 4 * lane);
          else pre8[i] = *reinterpret_cast<const u32x2*>(src + 8 * lane);
          pres[i] = a.kv_scales[rg * (kD / a.kv_scale_block) + (8 * lane) / a.kv_scale_block];
        }
      }
    }
  };
  auto store_q = [&](int rr, uint16_t* buf, int st) {
    if constexpr (QKV) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int r = __builtin_amdgcn_readlane(rr, i);
        const int tr = wave + NW * i;
        if (F8 && (lane & 7) == 0) qsc[st][lane >> 3][tr] = r >= 0 ? pres[i] : (r == -1 ? 0.f : 1.f);
        if (r < -1) continue;                  // window rows came by DMA
        u32x4 v = u32x4{0u, 0u, 0u, 0u};       // a missing row stays zero
        if (r >= 0) {
        if constexpr (KVF == CSA_FP4_E2M1) {
          // gfx950's scaled converter: byte i (channels 2i, 2i + 1 in its low and high nibbles)
          // times the block's power-of-two scale, to a bf16 pair; exact, as code x scale fits bf16
          const uint32_t w = pre8[i][0];
          const float sc = pres[i];
          v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
          v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
          v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
          v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
        } else {
          // E4M3FN codes to bf16, exactly (every E4M3 value is a bf16 value): the scaled
          // converter with scale 1, two codes to a bf16 pair
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t w = pre8[i][k];
            v[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
            v[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
          }
        }
        }
        *reinterpret_cast<u32x4*>(buf + tr * kPitch + 8 * lane) = v;
      }
    }
  };

  // ---- prologue: tiles 0 and 1 go out while the query fragments are read; tiles 2 and 3 once
  // the query rows (in tile buffers 2 and 3) are no longer needed
  const int rows0 = tile_rows(0), rows1 = tile_rows(1), rows2 = tile_rows(2), rows3 = tile_rows(3);
  int rows_next = tile_rows(4);
  if constexpr (!QKV) {
    if (ntile > 0) issue_tile(rows0, tb0, 0);
    if (ntile > 1) issue_tile(rows1, tb1, 1);
  } else {
    if (ntile > 0) { issue_tile(rows0, tb0, 0); fetch_q(rows0); }
  }
  // query fragments (B operand of S^T = K Q^T): head = n, channels 32c + 8g + [0, 8).  The
  // rotated query is not a bf16 value: its last two chunks (channels 448..511, which hold the
  // rotated pairs for rope_dim <= 64) are carried as bf16 hi + lo so the logits keep fp32
  // accuracy; rotated channels below 448 (rope_dim > 64) are rounded to bf16.
  bf16x8 qf[16];
  bf16x8 qlo[2];
  {
    const int rot0 = kD - a.rope_dim;
    const int qr = 16 * p + n;
    const uint16_t* qs = (p < 2 ? tb2 : tb3) + (qr % kTR) * kPitch + 8 * g;
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
  __syncthreads();   // every wave has its query fragments: tile buffers 2 and 3 are free
  if constexpr (!QKV) {
    if (ntile > 2) issue_tile(rows2, tb2, 2);
    if (ntile > 3) issue_tile(rows3, tb3, 3);
    wait_tiles<RPW>(max(0, min(ntile, 4) - 1));    // tile 0 has landed
    if (ntile > 0) zero_tile(rows0, tb0);
  } else {
    // quantized rows: one tile in registers at a time; tiles 0..2 are stored here, tile 3 is
    // left in flight for the loop
    wait_vmcnt<0>();
    if (ntile > 0) store_q(rows0, tb0, 0);
    if (ntile > 1) { issue_tile(rows1, tb1, 1); fetch_q(rows1); wait_vmcnt<0>(); store_q(rows1, tb1, 1); }
    if (ntile > 2) { issue_tile(rows2, tb2, 2); fetch_q(rows2); wait_vmcnt<0>(); store_q(rows2, tb2, 2); }
    if (ntile > 3) { issue_tile(rows3, tb3, 3); fetch_q(rows3); }
  }
  ring_barrier();

  // ---- online softmax state.  Lane (n, g) of a wave works for head n.  Two references per
  // wave, both integers in log2 units, so that moving weights between them is an exact
  // power-of-two scaling:
  //  * m_own, for the weights of this wave's own rows (16h .. 16h + 15 of each tile): it starts
  //    at the first tile's maximum (rounded up) and moves only when a tile's maximum exceeds it
  //    by more than kRescale, so weights stay below 2^kRescale; l_own sums them in fp32 (for lse);
  //  * m_acc, for this wave's P V accumulators, which take the weights of both waves of the
  //    pair, each rescaled from its producer's reference by an exact power of two; it moves
  //    lazily the same way.  The weights pass between the waves in fp32 and enter the P V
  //    product as bf16 hi + lo (fp8 rows: weight x row scale), so they keep about 16 bits
  //    instead of 8: with 8, a flat softmax over a few hundred rows puts the largest output
  //    error near 1 % of the output's RMS.  n_acc sums the weights and normalises the output.
  //    Both waves of a pair see the same weights and references, so they hold the same m_acc
  //    and n_acc.
  // The sink joins once, in the epilogue or in the split merge.
  float m_own = kNegBig, l_own = 0.f;
  float m_acc = kNegBig, n_acc = 0.f;
  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Scores of this wave's rows of the tile in `buf` (stage st): S^T for rows 16h + [0, 16),
  // then the weights of rows 16h + 4g + i against this wave's reference, published with that
  // reference in parity slot par of pbuf / mref.
  auto score = [&](const uint16_t* buf, int st, int par) {
    const uint16_t* rp = buf + (16 * h + n) * kPitch + 8 * g;
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (!F8) {
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(rp + 32 * c);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], sacc, 0, 0, 0);
        if (c >= 14 && q_split) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qlo[c - 14], sacc, 0, 0, 0);
      }
    } else {
      // exact codes: one partial product per 64-channel block, times the rows' block scale
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 2 * blk; c < 2 * blk + 2; ++c) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(rp + 32 * c);
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], part, 0, 0, 0);
          if (c >= 14 && q_split) part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qlo[c - 14], part, 0, 0, 0);
        }
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(&qsc[st][blk][16 * h + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[i] = fmaf(s4[i], part[i], sacc[i]);
      }
    }
    const uint32_t vf = *reinterpret_cast<const uint32_t*>(&tvalid[st][16 * h + 4 * g]);
    float sv[4];
    float tmax = kNegBig;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ((vf >> (8 * i)) & 0xffu) ? sacc[i] * a.scale_log2 : kNegBig;
      tmax = fmaxf(tmax, sv[i]);
    }
    tmax = max_lane_groups(tmax);
    // lazy rescaling of the own reference (see above); weights stay below 2^kRescale
    const bool grow = tmax > m_own + kRescale;
    if (__any(grow)) {
      const float m_new = grow ? ceilf(tmax) : m_own;
      l_own *= fast_exp2(m_own - m_new);
      m_own = m_new;
    }
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = sv[i] > kNegBig ? fast_exp2(sv[i] - m_own) : 0.f;
      l_own += pv[i];
    }
    *reinterpret_cast<f32x4*>(&pbuf[par][p][h][lane][0]) = f32x4{pv[0], pv[1], pv[2], pv[3]};
    if (g == 0) mref[par][p][h][n] = m_own;
  };
  // 2^k for an integer k (exact); 0 far below the range
  auto pow2i = [](float k) -> float { return ldexpf(1.f, (int)fmaxf(k, -200.f)); };
  // O^T += V^T P^T over the 32 rows of the tile in `buf`, channels 256h + [0, 256), with the pair's
  // weights from parity slot par.  The K index of the contraction is permuted: k = 8g' + j names
  // row 4g' + j (j < 4, wave 0's rows) or 16 + 4g' + j - 4 (wave 1's rows), for P (as each wave's
  // lanes hold it) and V^T (two transposing reads of four rows each) alike.
  auto pv_product = [&](const uint16_t* buf, int st, int par) {
    const float r0 = mref[par][p][0][n], r1 = mref[par][p][1][n];
    const float rt = fmaxf(r0, r1);
    const bool grow = rt > m_acc + kRescale;
    if (__any(grow)) {
      const float m_new = grow ? rt : m_acc;
      const float alpha = pow2i(m_acc - m_new);
      n_acc *= alpha;
      if (__any(grow && m_acc > kNegBig)) {
#pragma unroll
        for (int db = 0; db < 16; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;
      }
      m_acc = m_new;
    }
    // the producers' weights on this wave's reference: exact power-of-two rescaling
    const float f0 = pow2i(r0 - m_acc), f1 = pow2i(r1 - m_acc);
    float w[8];
    {
      const f32x4 pa = *reinterpret_cast<const f32x4*>(&pbuf[par][p][0][lane][0]);
      const f32x4 pb = *reinterpret_cast<const f32x4*>(&pbuf[par][p][1][lane][0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) { w[i] = pa[i] * f0; w[4 + i] = pb[i] * f1; }
    }
    n_acc += ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
    const int L = lane & 15;
    const uint16_t* v0p = buf + (4 * g + (L >> 2)) * kPitch + 256 * h + 4 * (L & 3);
    const uint16_t* v1p = buf + (16 + 4 * g + (L >> 2)) * kPitch + 256 * h + 4 * (L & 3);
    if constexpr (!F8) {
      u32x4 pw, pl;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pw[k] = pack_bf16x2(w[2 * k], w[2 * k + 1]);
        pl[k] = pack_bf16x2(w[2 * k] - bf16lo_to_f32(pw[k]), w[2 * k + 1] - bf16hi_to_f32(pw[k]));
      }
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw), pfl = __builtin_bit_cast(bf16x8, pl);
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0p + 16 * db));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1p + 16 * db));
        const i16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, acc[db], 0, 0, 0);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pfl, acc[db], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int bl = 0; bl < 4; ++bl) {
        // the weights times the rows' scale of channel block 4h + bl, as bf16 hi + lo
        const int blk = 4 * h + bl;
        const f32x4 sa = *reinterpret_cast<const f32x4*>(&qsc[st][blk][4 * g]);
        const f32x4 sb = *reinterpret_cast<const f32x4*>(&qsc[st][blk][16 + 4 * g]);
        float ws[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) { ws[i] = w[i] * sa[i]; ws[4 + i] = w[4 + i] * sb[i]; }
        u32x4 hi, lo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hi[k] = pack_bf16x2(ws[2 * k], ws[2 * k + 1]);
          lo[k] = pack_bf16x2(ws[2 * k] - bf16lo_to_f32(hi[k]), ws[2 * k + 1] - bf16hi_to_f32(hi[k]));
        }
        const bf16x8 pfh = __builtin_bit_cast(bf16x8, hi), pfl = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
          const int db = 4 * bl + d4;
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v0p + 16 * db));
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v1p + 16 * db));
          const i16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          const bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfh, acc[db], 0, 0, 0);
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfl, acc[db], 0, 0, 0);
        }
      }
    }
  };

  // tile 0: scores and weights
  if (ntile > 0) {
    score(tb0, 0, 0);
    if constexpr (!QKV) {
      wait_tiles<RPW>(max(0, min(ntile, 4) - 2));   // tile 1 has landed
      if (ntile > 1) zero_tile(rows1, tb1);
    }
    ring_barrier();
  }

  // One step, one barrier: the scores and weights of tile t + 1 (buffer bs, stage ss) and the
  // P V product of tile t (buffer bp, stage sp); after the barrier bp receives tile t + 4, and
  // (quantized rows) tile t + 3's registers are stored into buffer b3 (stage s3).
  int rows_reg = rows3;   // quantized rows: the tile whose codes are in registers
  // bz (bf16 rows): tile t + 2's buffer, whose missing rows are zeroed once it has landed.
  auto step = [&](int t, const uint16_t* bs, int ss, uint16_t* bp, int sp, uint16_t* b3, int s3, uint16_t* bz) {
    if (t + 1 < ntile) score(bs, ss, (t + 1) & 1);
    pv_product(bp, sp, t & 1);
    if constexpr (!QKV) {
      wait_tiles<RPW>(max(0, min(ntile, t + 4) - (t + 3)));   // tile t + 2 has landed
      if (t + 2 < ntile) zero_tile(tile_rows(t + 2), bz);
    }
    ring_barrier();   // weights of tile t + 1 and tile t + 2 visible; tile t and its weights done
    const int rr = rows_next;
    rows_next = tile_rows(t + 5);
    if constexpr (!QKV) {
      if (t + 4 < ntile) issue_tile(rr, bp, sp);
    } else {
      if (t + 3 < ntile) { wait_vmcnt<0>(); store_q(rows_reg, b3, s3); }
      if (t + 4 < ntile) { issue_tile(rr, bp, sp); fetch_q(rr); }
      rows_reg = rr;
    }
  };
  for (int t = 0; t < ntile; t += 4) {
    step(t, tb1, 1, tb0, 0, tb3, 3, tb2);
    if (t + 1 >= ntile) break;
    step(t + 1, tb2, 2, tb1, 1, tb0, 0, tb3);
    if (t + 2 >= ntile) break;
    step(t + 2, tb3, 3, tb2, 2, tb1, 1, tb0);
    if (t + 3 >= ntile) break;
    step(t + 3, tb0, 0, tb3, 3, tb2, 2, tb1);
  }

  // ---- epilogue: the pair's sums on the accumulator reference and (for partials) the largest
  // output magnitude per head
  const float l_w = sum_lane_groups(l_own);
  const float n_tot = sum_lane_groups(n_acc);
  float amax = 0.f;
  if (a.nsplit > 1) {
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(acc[db][i]));
    amax = max_lane_groups(amax);
  }
  if (g == 0) xch[p][h][n] = f32x4{l_w, m_own, amax, 0.f};
  ring_barrier();
  const f32x4 x0 = xch[p][0][n], x1 = xch[p][1][n];
  const float m_run = m_acc;
  // the exact sums of both waves' weights, each on its own reference, moved to m_acc
  float l_tot = x0[0] * fast_exp2(fmaxf(x0[1] - m_run, -200.f)) + x1[0] * fast_exp2(fmaxf(x1[1] - m_run, -200.f));
  if (!head_ok) return;
  if (a.nsplit == 1) {
    // fold in the sink: Z = l 2^(m - M) + 2^(sink - M), M = max(m, sink)
    const float sink2 = a.sink[head] * kLog2e;
    const float M = fmaxf(m_run, sink2);
    const float sc = exp2f(m_run - M);
    const float es = exp2f(sink2 - M);
    l_tot = l_tot * sc + es;
    const float inv = sc / (n_tot * sc + es);
    const int rot0 = kD - a.rope_dim;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc[db][i] * inv;
      const int d0 = 256 * h + 16 * db + 4 * g;
      if (d0 + 4 > rot0 && a.rope_dim > 0) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int d = d0 + 2 * k2;
          if (d >= rot0) {
            // rotation by -q_pos: same cosine, negated sine
            const f32x2 t2 = rtab[(d - rot0) >> 1];
            const float cs = t2[0], sn = -t2[1];
            const float y0 = o[2 * k2], y1 = o[2 * k2 + 1];
            o[2 * k2] = y0 * cs - y1 * sn;
            o[2 * k2 + 1] = y0 * sn + y1 * cs;
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
    if (a.lse && g == 0 && h == 0) a.lse[(int64_t)row * a.H + head] = (M + log2f(l_tot)) * kLn2;
  } else {
    // The split's normalised output o / n in fp16 (11-bit significand: rounding within 2^-11
    // relative, far below the error the bf16 inputs carry), scaled by 2^-e so that the head's
    // largest magnitude sits below 2^14 whatever the range of the cache values; (m, n, l, e)
    // stay fp32.  Half the bytes of fp32 partials, written here and read by the merge.
    const float am = fmaxf(x0[2], x1[2]);
    const float inv_n = n_tot > 0.f ? 1.f / n_tot : 0.f;
    int e = 0;
    if (am * inv_n > 0.f) {
      int ex;
      (void)frexpf(am * inv_n, &ex);   // amax / n = f 2^ex, f in [0.5, 1)
      e = ex - 14;
    }
    const float sc = ldexpf(inv_n, -e);
    const int64_t pr = ((int64_t)row * a.nsplit + split) * a.H + head;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      u32x2 hh;
      hh[0] = pack_f16x2(acc[db][0] * sc, acc[db][1] * sc);
      hh[1] = pack_f16x2(acc[db][2] * sc, acc[db][3] * sc);
      *reinterpret_cast<u32x2*>(a.part_o + pr * kD + 256 * h + 16 * db + 4 * g) = hh;
    }
    if (g == 0 && h == 0) *reinterpret_cast<f32x4*>(a.part_ml + 4 * pr) = f32x4{m_run, n_tot, l_tot, (float)e};
  }
}

// Merge split partials: M = max(sink, m_s), o = sum 2^(m_s - M) n_s u_s / Zo with u_s = o_s / n_s
// (stored in fp16 times 2^-e_s) and Zo = 2^(sink - M) + sum n_s 2^(m_s - M) (n_s: the sum of the
// weights as they entered the split's P V product), lse = M + log2(2^(sink - M) + sum l_s
// 2^(m_s - M)) with the exact sums l_s; then rotate back and store.  A block of 256 lanes merges 4
// (row, head) pairs, 8 channels per lane; splits are merged online, four per round, so that a
// round's (max, sum) and output loads are all in flight together.  The (cos, sin) table of the
// row's position is built by the whole wave, one frequency per lane, while the loads are in
// flight.
constexpr int kCombineHeads = 4;
__global__ void __launch_bounds__(64 * kCombineHeads) k_attend_combine(AttendArgs a) {
  __shared__ f32x2 rtab[kCombineHeads][kD / 2];
  const int rows = a.B * a.Tq;
  // blocks in the order of the attention grid's XCD ranges: a row's merge runs on the XCD that
  // wrote its partials
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rh = (int)xcd_remap(blockIdx.x, gridDim.x) * kCombineHeads + wave;   // row * H + head
  if (rh >= rows * a.H) return;
  const int row = rh / a.H, head = rh % a.H;
  const int d0 = lane * 8;
  const int64_t base = (int64_t)row * a.nsplit * a.H + head;        // partial (row, s, head) = base + s * H
  const float sink2 = a.sink[head] * kLog2e;
  // online merge, 4 splits per round: each round's (max, sum) and output loads go out together
  float M = sink2, Z = 1.f, Zo = 1.f;   // relative to 2^M
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // one round: four splits' (max, sums, e) and output slices, issued together; a round's loads go
  // out before the previous round is merged (two rounds in flight)
  struct Round {
    u32x4 v[4];
    float ms[4], ns[4], ls[4], es[4];
  };
  auto load_round = [&](int s0, Round& R) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t pr = base + (int64_t)min(s0 + u, a.nsplit - 1) * a.H;
      const f32x4 ml = *reinterpret_cast<const f32x4*>(a.part_ml + 4 * pr);
      R.ms[u] = s0 + u < a.nsplit ? ml[0] : kNegBig;
      R.ns[u] = ml[1];
      R.ls[u] = ml[2];
      R.es[u] = ml[3];
      // read once: nontemporal loads keep them from displacing other lines
      R.v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.part_o + pr * kD + d0));
    }
  };
  auto merge_round = [&](const Round& R) {
    float Mn = M;
#pragma unroll
    for (int u = 0; u < 4; ++u) Mn = fmaxf(Mn, R.ms[u]);
    const float r = fast_exp2(M - Mn);
    Z *= r;
    Zo *= r;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= r;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = fast_exp2(R.ms[u] - Mn);   // 0 for the padding of a partial round
      Z += R.ls[u] * w;
      Zo += R.ns[u] * w;
      const float wo = ldexpf(R.ns[u] * w, (int)R.es[u]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x2 hh = unpack_f16x2(R.v[u][k]);
        o[2 * k] += wo * hh[0];
        o[2 * k + 1] += wo * hh[1];
      }
    }
    M = Mn;
  };
  Round R0, R1;
  load_round(0, R0);
  if (a.rope_dim > 0) {
    const int64_t p = a.q_pos[row];
    for (int i = lane; i < a.rope_dim / 2; i += kWave) {
      float cs, sn;
      rope_cs(p, a.inv_freq[i], cs, sn);
      rtab[wave][i] = f32x2{cs, -sn};   // rotation by -q_pos: same cosine, negated sine
    }
  }
  for (int s0 = 0; s0 < a.nsplit; s0 += 8) {
    if (s0 + 4 < a.nsplit) load_round(s0 + 4, R1);
    merge_round(R0);
    if (s0 + 4 >= a.nsplit) break;
    if (s0 + 8 < a.nsplit) load_round(s0 + 8, R0);
    merge_round(R1);
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
        const f32x2 t2 = rtab[wave][(d - rot0) >> 1];
        const float x0 = o[2 * k2], x1 = o[2 * k2 + 1];
        o[2 * k2] = x0 * t2[0] - x1 * t2[1];
        o[2 * k2 + 1] = x0 * t2[1] + x1 * t2[0];
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

template <int NP>
static void launch_attend_pairs(const AttendArgs& a, dim3 grid, hipStream_t s) {
  const dim3 blk(AttShape<NP>::NT);
  const bool csa = a.csa_mode != 0;
  switch (a.kv_dtype) {
    case CSA_FP8_E4M3:
      if constexpr (NP == 2) {   // fp8 caches take the 32-head shape only
        if (csa) hipLaunchKernelGGL((k_attend<true, CSA_FP8_E4M3, 2>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_attend<false, CSA_FP8_E4M3, 2>), grid, blk, 0, s, a);
      }
      break;
    default:   // fp4 (bf16 caches take the grouped kernel)
      if (csa) hipLaunchKernelGGL((k_attend<true, CSA_FP4_E2M1, NP>), grid, blk, 0, s, a);
      else hipLaunchKernelGGL((k_attend<false, CSA_FP4_E2M1, NP>), grid, blk, 0, s, a);
      break;
  }
}

template <int HPB, int W>
static void launch_attend_groups(const AttendArgs& a, dim3 grid, hipStream_t s) {
  if (a.csa_mode != 0) hipLaunchKernelGGL((k_attend_grp<true, HPB, W>), grid, dim3(64 * W), 0, s, a);
  else hipLaunchKernelGGL((k_attend_grp<false, HPB, W>), grid, dim3(64 * W), 0, s, a);
}

hipError_t launch_attend(const AttendArgs& a0, hipStream_t s) {
  AttendArgs a = a0;
  const int rows = a.B * a.Tq;
  const AttendPlan pl = attend_plan(rows, a.H, a.slot_cap, a.csa_mode != 0, att_kind(a.kv_dtype));
  a.nsplit = pl.nsplit;
  a.slots_per_split = pl.sps;
  const int HG = (a.H + pl.hpb - 1) / pl.hpb;
  const long long blocks = (long long)rows * HG * a.nsplit;
  const dim3 grid((unsigned)blocks);
  if (pl.kind == kAttGroups4) {
    launch_attend_groups<64, 4>(a, grid, s);
  } else if (pl.kind == kAttGroups) {
    if (pl.hpb == 64) launch_attend_groups<64, 8>(a, grid, s);
    else launch_attend_groups<32, 8>(a, grid, s);
  } else {
    if (pl.hpb == 64) launch_attend_pairs<4>(a, grid, s);
    else launch_attend_pairs<2>(a, grid, s);
  }
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
