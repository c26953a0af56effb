// Softmax-pooled KV compression with fused partial RoPE and bf16 / fp8 / fp4 storage.
//
// Each cache row pools `window` raw tokens at step `stride` with a softmax taken
// separately per channel over the window's pooling logits, then rotates the last
// rope_dim channels at the row's position (its last token's) and stores the row
// (DeepSeek-V4-Pro vs Inkling, Component-by-component table: CSA row, HCA row,
// partial-RoPE row; DeepSeek-V4.1-Flash vs Inkling: cache quantized after RoPE).
//
// Layout of the work: a group of C/8 lanes owns one sequence's run of consecutive
// rows, each lane 8 channels (16-byte loads of kv and logits).  When window ==
// 2*stride (CSA: 8 tokens at stride 4) consecutive rows share half their tokens, so
// the group walks the raw stream once, block of `stride` tokens by block, keeps the
// previous block's partial softmax state (running max, sum of weights, weighted sum)
// in registers and combines it with the current block: every raw token is read from
// HBM once.  Other geometries (HCA 128/128, the raw-window write 1/1) read each
// row's own tokens.
//
// This header holds the device code and the launch planning of the compressor; its kernels
// are in compress.hip, and the indexer's scores launch can carry a decode step's compress
// blocks (the two calls share no data).
#pragma once
#include "common.hpp"
#include "internal.hpp"

namespace csa {

struct PoolState {
  float m[8], s[8], sv[8];
};

// Hardware exp2 (v_exp_f32, about 1 ulp; results below 2^-126 flush to zero, which only
// drops weights that small relative to the running maximum).
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void pool_reset(PoolState& p) {
#pragma unroll
  for (int i = 0; i < 8; ++i) { p.m[i] = kNegBig; p.s[i] = 0.f; p.sv[i] = 0.f; }
}

__device__ __forceinline__ void pool_merge(PoolState& out, const PoolState& x, const PoolState& y) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float mn = fmaxf(x.m[i], y.m[i]);
    float a = fexp2(x.m[i] - mn), b = fexp2(y.m[i] - mn);
    out.m[i] = mn;
    out.s[i] = x.s[i] * a + y.s[i] * b;
    out.sv[i] = x.sv[i] * a + y.sv[i] * b;
  }
}

// Rotary inputs of a lane's 8 channels, loaded before the pooling so their latency overlaps
// it: the sequence's position origin and the frequencies of the lane's rotated pairs.
struct RopeIn {
  int64_t pos0;
  double fr[4];
};

__device__ __forceinline__ RopeIn rope_in(const CompressArgs& a, int b, int c0) {
  RopeIn r;
  r.pos0 = a.pos0[b];
  const int rot0 = a.C - a.rope_dim;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = c0 + 2 * k;
    r.fr[k] = (a.rope_dim > 0 && c >= rot0) ? a.inv_freq[(c - rot0) >> 1] : 0.0;
  }
  return r;
}

// A block of up to kB tokens of one lane's 8 channels (kv and logits), held in registers so
// that the next block's loads can be in flight while the current one is pooled.  Raw tokens are
// read once and entries written once: both go through nontemporal loads and stores, which keep
// the streams from displacing cached data (about 6-8 % faster over whole streams).
constexpr int kB = 4;
struct RawBlock {
  u32x4 v[kB], z[kB];
};
// tokens t0 + u * tstride, u < n
__device__ __forceinline__ void load_block(RawBlock& r, const uint16_t* kv, const uint16_t* lg, int64_t ld_tok,
                                           int64_t t0, int n, int c0, int tstride = 1) {
#pragma unroll
  for (int u = 0; u < kB; ++u) {
    if (u < n) {
      const int64_t t = t0 + (int64_t)u * tstride;
      r.v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kv + t * ld_tok + c0));
      r.z[u] = lg ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(lg + t * ld_tok + c0))
                  : u32x4{0u, 0u, 0u, 0u};
    }
  }
}
// Fold the n tokens of a register block into p: one maximum over the block, then one
// exponential per token and one rescale of the running state (1 + n exponentials per
// channel instead of 2n).
__device__ __forceinline__ void pool_regs(PoolState& p, const RawBlock& r, int n) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float z[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const uint32_t w = r.z[u][c >> 1];
      z[u] = u < n ? ((c & 1) ? bf16hi_to_f32(w) : bf16lo_to_f32(w)) * kLog2e : kNegBig;
    }
    float bm = z[0];
#pragma unroll
    for (int u = 1; u < kB; ++u) bm = fmaxf(bm, z[u]);
    const float mn = fmaxf(p.m[c], bm);
    const float al = fexp2(p.m[c] - mn);
    float s = p.s[c] * al, sv = p.sv[c] * al;
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (u < n) {
        const float v = (c & 1) ? bf16hi_to_f32(r.v[u][c >> 1]) : bf16lo_to_f32(r.v[u][c >> 1]);
        const float w = fexp2(z[u] - mn);
        s += w;
        sv += w * v;
      }
    }
    p.s[c] = s;
    p.sv[c] = sv;
    p.m[c] = mn;
  }
}

// Add the n raw tokens starting at token row t0 into p, kB at a time, the loads of the next
// block in flight while the current one is pooled.
__device__ __forceinline__ void pool_block(PoolState& p, const uint16_t* kv, const uint16_t* lg,
                                           int64_t ld_tok, int t0, int n, int c0) {
  RawBlock r0, r1;
  load_block(r0, kv, lg, ld_tok, t0, min(kB, n), c0);
  for (int t = 0; t < n; t += kB) {
    const int m = min(kB, n - t);
    if (t + kB < n) load_block(r1, kv, lg, ld_tok, t0 + t + kB, min(kB, n - t - kB), c0);
    pool_regs(p, r0, m);
    r0 = r1;
  }
}

// (cos, sin) of the row's position times the frequencies of the lane's rotated pairs (1, 0
// for pairs that are not rotated).  The row's position is that of its last token.
struct RopeTrig {
  float cs[4], sn[4];
};
__device__ __forceinline__ RopeTrig rope_trig(const CompressArgs& a, const RopeIn& ri, int row, int c0) {
  RopeTrig t;
  const int rot0 = a.C - a.rope_dim;
  const int64_t pos = ri.pos0 + (int64_t)row * a.stride + (a.window - 1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t.cs[k] = 1.f;
    t.sn[k] = 0.f;
    if (a.rope_dim > 0 && c0 + 2 * k >= rot0) rope_cs(pos, ri.fr[k], t.cs[k], t.sn[k]);
  }
  return t;
}

// Finish one row: normalise, rotate, store.
__device__ __forceinline__ void finish_row(const PoolState& p, const CompressArgs& a, const RopeTrig& tr, int b,
                                           int row, int c0) {
  float e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = p.sv[i] / p.s[i];
  const int rot0 = a.C - a.rope_dim;
  if (c0 + 8 > rot0 && a.rope_dim > 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (c0 + 2 * k >= rot0) {
        const float x0 = e[2 * k], x1 = e[2 * k + 1];
        e[2 * k] = x0 * tr.cs[k] - x1 * tr.sn[k];
        e[2 * k + 1] = x0 * tr.sn[k] + x1 * tr.cs[k];
      }
    }
  }
  const int64_t rowoff = ((int64_t)b * a.cap + row) * a.C;
  if (a.dtype == CSA_BF16) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(e[2 * i], e[2 * i + 1]);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + rowoff + c0));
  } else if (a.dtype == CSA_FP4_E2M1) {
    // MXFP4: a 32-channel block spans 4 consecutive lanes; its scale is the power of two
    // that puts the block's largest magnitude in [4, 8), 1 for a block of zeros.
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(e[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    int ex = 0;
    (void)frexpf(amax, &ex);                        // amax = f * 2^ex, f in [0.5, 1)
    const int es = amax > 0.f ? min(max(ex - 3, -127), 127) : 0;
    const float scale = ldexpf(1.0f, es);
    const float inv = ldexpf(1.0f, -es);            // exact: the scale is a power of two
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= f32_to_fp4_e2m1(e[i] * inv) << (4 * i);
    // channel c0 + i in nibble i: even channels in the low nibble of their byte
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.out) + rowoff / 2 + c0 / 2));
    if ((c0 % 32) == 0) __builtin_nontemporal_store(scale, &a.scales[((int64_t)b * a.cap + row) * (a.C / 32) + c0 / 32]);
  } else {
    // fp8: one scale per scale_block channels = scale_block/8 consecutive lanes.
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(e[i]));
    for (int m = 1; m < a.scale_block / 8; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    float scale = amax / 448.0f;
    uint32_t lo = 0, hi = 0;
    if (scale > 0.f) {
      // codes: round to nearest even of e / scale, by gfx950's converter (OCP E4M3FN), on e times
      // the fp32 reciprocal of the scale (within an fp32 ulp of the quotient; |e / scale| <= 448, so
      // nothing saturates)
      const float inv = 1.0f / scale;
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(e[0] * inv, e[1] * inv, 0u, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(e[2] * inv, e[3] * inv, lo, true);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(e[4] * inv, e[5] * inv, 0u, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(e[6] * inv, e[7] * inv, hi, true);
    }
    u32x2 w;
    w[0] = lo;
    w[1] = hi;
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(a.out) + rowoff + c0));
    if ((c0 % a.scale_block) == 0) {
      int nsb = a.C / a.scale_block;
      __builtin_nontemporal_store(scale, &a.scales[((int64_t)b * a.cap + row) * nsb + c0 / a.scale_block]);
    }
  }
}

// Long windows (HCA: 128 tokens per row) and decode-sized calls: one block per (row,
// 128-channel slice).  The window's tokens are dealt round-robin to 16 groups of 16 lanes
// (8 channels per lane), so all of a row's loads are in flight at once instead of walking
// the window serially; the 16 partial softmax states are merged through LDS.  Requires C % 128 == 0 and fp8 scale
// blocks of at most 128 channels (one block never spans two slices).
constexpr int kSplitGroups = 16;
constexpr int kSliceC = 128;

// One block of the split layout: row i of sequence b, channel slice z.
__device__ __forceinline__ void compress_split_block(const CompressArgs& a, int i, int b, int z) {
  __shared__ float sm_m[kSplitGroups][kSliceC], sm_s[kSplitGroups][kSliceC], sm_v[kSplitGroups][kSliceC];
  const int li = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int cs = li * 8;                                    // channel within the slice
  const int c0 = z * kSliceC + cs;
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv) + (int64_t)b * a.ld_seq;
  const uint16_t* lg = a.logits ? reinterpret_cast<const uint16_t*>(a.logits) + (int64_t)b * a.ld_seq
                                : nullptr;
  const RopeIn ri = rope_in(a, b, c0);
  PoolState p;
  pool_reset(p);
  const int t0 = i * a.stride;
  // group g takes tokens g, g + 16, g + 32, ... of the window, kB of them per load round,
  // the next round's loads in flight while the current one is pooled
  const int mine = g < a.window ? (a.window - 1 - g) / kSplitGroups + 1 : 0;
  RawBlock r0, r1;
  load_block(r0, kv, lg, a.ld_tok, (int64_t)t0 + g, min(kB, mine), c0, kSplitGroups);
  // the merging group's rotation, taken while the window's tokens are in flight
  RopeTrig tr{};
  if (g == 0) tr = rope_trig(a, ri, a.first_row + i, c0);
  for (int u0 = 0; u0 < mine; u0 += kB) {
    const int m = min(kB, mine - u0);
    if (u0 + kB < mine)
      load_block(r1, kv, lg, a.ld_tok, (int64_t)t0 + g + (int64_t)(u0 + kB) * kSplitGroups, min(kB, mine - u0 - kB),
                 c0, kSplitGroups);
    pool_regs(p, r0, m);
    r0 = r1;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sm_m[g][cs + k] = p.m[k];
    sm_s[g][cs + k] = p.s[k];
    sm_v[g][cs + k] = p.sv[k];
  }
  __syncthreads();
  // one thread per channel merges the states of the groups that hold tokens, into group 0's slot
  if (threadIdx.x < kSliceC) {
    const int ch = threadIdx.x;
    const int nh = min(a.window, kSplitGroups);
    float m = kNegBig;
    for (int h = 0; h < nh; ++h) m = fmaxf(m, sm_m[h][ch]);
    float ss = 0.f, sv = 0.f;
    for (int h = 0; h < nh; ++h) {
      const float f = fexp2(sm_m[h][ch] - m);
      ss += sm_s[h][ch] * f;
      sv += sm_v[h][ch] * f;
    }
    sm_m[0][ch] = m;
    sm_s[0][ch] = ss;
    sm_v[0][ch] = sv;
  }
  __syncthreads();
  if (g != 0) return;
  PoolState q;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    q.m[k] = sm_m[0][cs + k];
    q.s[k] = sm_s[0][cs + k];
    q.sv[k] = sm_v[0][cs + k];
  }
  finish_row(q, a, tr, b, a.first_row + i, c0);
}

// Short windows (CSA: 8 tokens; the raw-window write: 1) and decode-sized calls: one group of
// C/8 lanes per (row, sequence), each lane loading its 8 channels of every token of the row
// (all loads in flight together), with no cross-group merge.  Block-unit u covers the
// 256 / (C/8) consecutive (row, sequence) pairs from u * groups on, sequence fastest.
__device__ __forceinline__ void compress_rows_block(const CompressArgs& a, int u) {
  const int lanes = a.C / 8;
  const int groups = 256 / lanes;
  const int g = threadIdx.x / lanes, li = threadIdx.x % lanes;
  const long long unit = (long long)u * groups + g;
  if (unit >= (long long)a.n_new * a.B) return;
  const int i = (int)(unit / a.B), b = (int)(unit % a.B);
  const int c0 = li * 8;
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv) + (int64_t)b * a.ld_seq;
  const uint16_t* lg = a.logits ? reinterpret_cast<const uint16_t*>(a.logits) + (int64_t)b * a.ld_seq
                                : nullptr;
  const RopeIn ri = rope_in(a, b, c0);
  // every token of the row in flight (window <= 2 kB), then the rotation while they arrive
  RawBlock r0, r1;
  const int64_t t0 = (int64_t)i * a.stride;
  const int n0 = min(kB, a.window), n1 = a.window - n0;
  load_block(r0, kv, lg, a.ld_tok, t0, n0, c0);
  if (n1 > 0) load_block(r1, kv, lg, a.ld_tok, t0 + kB, n1, c0);
  const RopeTrig tr = rope_trig(a, ri, a.first_row + i, c0);
  PoolState p;
  pool_reset(p);
  pool_regs(p, r0, n0);
  if (n1 > 0) pool_regs(p, r1, n1);
  finish_row(p, a, tr, b, a.first_row + i, c0);
}

// Several calls in one launch (a step's new entries and its raw-window write): block L
// belongs to call c when start[c] <= L < start[c + 1].  In the split layout its blocks are
// (row, sequence, slice) in that order of significance; in the rows layout they are the
// block-units of compress_rows_block.  The call is selected by a uniform branch so that its
// arguments stay in scalar registers.
constexpr int kBatchMax = 4;
constexpr int kLaySplit = 0, kLayRows = 1;
struct CompressBatch {
  CompressArgs a[kBatchMax];
  int start[kBatchMax + 1];
  int lay[kBatchMax];
  int n;
};
// Block L of a batched launch: the call c with start[c] <= L < start[c + 1], selected by a
// uniform branch so that its arguments stay in scalar registers.
__device__ __forceinline__ void compress_batch_block(const CompressBatch& bt, int L) {
  int c = 0;
  while (c + 1 < bt.n && L >= bt.start[c + 1]) ++c;
  auto run = [&](const CompressArgs& a) {
    const int r = L - bt.start[c];
    if (bt.lay[c] == kLayRows) {
      compress_rows_block(a, r);
      return;
    }
    const int nz = a.C / kSliceC;
    const int z = r % nz, rb = r / nz;
    compress_split_block(a, rb / a.B, rb % a.B, z);
  };
  switch (c) {
    case 0: run(bt.a[0]); break;
    case 1: run(bt.a[1]); break;
    case 2: run(bt.a[2]); break;
    default: run(bt.a[3]); break;
  }
}

// Layout of a call in the one-launch kernel, or -1 for the run-mode kernel.  Long windows
// take the split layout (128-channel slices, the window's tokens spread over 16 lane groups);
// few rows (a decode step) take the rows layout when the window is short (every token of a
// row loads at once in one lane group) and the split layout otherwise.  Many rows of a short
// window (prefill) take the run-mode kernel, which reads shared tokens once.
static inline int batch_layout(const CompressArgs& a) {
  const long long rows = (long long)a.n_new * a.B;
  const bool split_ok = a.C % kSliceC == 0 && (a.dtype == CSA_BF16 || a.scale_block <= kSliceC);
  if (split_ok && a.window >= 2 * kSplitGroups) return kLaySplit;
  if (rows > 512) return -1;
  if (a.window <= 2 * kB) return kLayRows;
  return split_ok ? kLaySplit : -1;
}

static inline long long batch_blocks(const CompressArgs& a, int lay) {
  const long long rows = (long long)a.n_new * a.B;
  if (lay == kLayRows) {
    const int groups = 256 / (a.C / 8);
    return (rows + groups - 1) / groups;
  }
  return rows * (a.C / kSliceC);
}


// Packs up to kBatchMax calls, skipping empty ones, into one launch of `total` blocks.
// Returns false when some call needs the run-mode kernel (or there are too many calls).
static inline bool make_compress_batch(const CompressArgs* a, int n, CompressBatch& bt, long long& total) {
  bt = CompressBatch{};
  total = 0;
  if (n < 1 || n > kBatchMax) return false;
  for (int i = 0; i < n; ++i)
    if (batch_layout(a[i]) < 0) return false;
  for (int i = 0; i < n; ++i) {
    if (a[i].n_new <= 0 || a[i].B <= 0) continue;   // nothing to write
    const int m = bt.n++;
    bt.a[m] = a[i];
    bt.lay[m] = batch_layout(a[i]);
    bt.start[m] = (int)total;
    total += batch_blocks(a[i], bt.lay[m]);
  }
  bt.start[bt.n] = (int)total;
  return true;
}

}  // namespace csa
