// Grouped low-rank output projection after the attention ("DeepSeek-V4-Pro" model atlas, Raw config
// fields o_groups 16, o_lora_rank 1024, hidden_size 7168): the heads' outputs are cut into G groups
// of H / G consecutive heads, group g's (H / G) * D values go through its own down factor wa[g]
// (R x (H / G) D), and the G * R codes, concatenated in group order, through the up factor wb
// (hidden x G R).  Two launches of one kernel, C = A B^T with B's rows (the factors' output rows)
// contiguous over K:
//   1. z[t, g R + r] = sum_k o[t, g (H / G) D + k] wa[g, r, k]      (grid over groups)
//   2. y[t, j]       = sum_k z[t, k] wb[j, k]
// z stays fp32 in the workspace.  The second product runs over four K ranges (partial tiles in the
// workspace, then summed in range order by k_sum_splits).
//
// Kernel design (gfx950, wave64, bf16 MFMA 16x16x32, fp32 accumulation).  A block computes a
// 32-row x 16 NB-column tile of C over its K range; its 8 waves take interleaved 32-wide K steps
// (wave w: steps w, w + 8, ...), so neighbouring waves read neighbouring 64-byte pieces of the same
// factor rows.  A wave loads the A and B fragments of U steps at once (A rows are the few query
// tokens, read from cache; B rows stream from HBM) and then issues their MFMAs, so a wave keeps
// U steps of loads in flight and no load is carried across the loop's back edge.  fp32 A (the
// codes z, or an fp32 attention output) enters as bf16 hi + lo parts, two MFMAs, so the products
// keep about 16 bits of A.  The eight waves' partial tiles are summed through LDS in a fixed order
// (deterministic), then stored.  At decode (a few dozen tokens) the launches are bound by the
// factors' bytes (bf16: 2 B per factor element, read once).
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {
constexpr int kGW = 8;    // waves per block
constexpr int kGM = 32;   // rows of C per block
}  // namespace

// NB: 16-column blocks of C per block; a wave issues the loads of kGU K steps together (fewer for
// wide tiles, whose B fragments take more registers).  With a.ksplit > 1 the block covers one of
// ksplit equal K ranges and stores an fp32 partial tile, summed by k_sum_splits.
template <int NB, bool AF32, bool OUT_BF16>
__global__ void __launch_bounds__(64 * kGW, 2) k_gemm_nt(GemmArgs a) {
  constexpr int kGU = NB >= 8 ? 2 : 4;
  __shared__ f32x4 red[kGW][2][NB][kWave];   // the waves' partial tiles
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int grp = blockIdx.y;
  const int ks = blockIdx.z % a.ksplit;
  const int m0 = (blockIdx.z / a.ksplit) * kGM;
  const int c0 = blockIdx.x * 16 * NB;
  const int nsteps = a.K / a.ksplit / 32;          // K steps of this block's range
  const int kbase = ks * (a.K / a.ksplit);

  const uint8_t* A = static_cast<const uint8_t*>(a.A) + (int64_t)grp * a.a_gstride * (AF32 ? 4 : 2);
  const uint16_t* Bm = a.B + (int64_t)grp * a.b_gstride;
  // A rows of this lane (row blocks 0 and 1), clamped into [0, M); rows past M are not stored
  const int64_t ar0 = min(m0 + n16, a.M - 1), ar1 = min(m0 + 16 + n16, a.M - 1);
  const uint8_t* arow[2] = {A + ar0 * a.lda * (AF32 ? 4 : 2), A + ar1 * a.lda * (AF32 ? 4 : 2)};
  const uint16_t* brow[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) brow[cb] = Bm + (int64_t)(c0 + 16 * cb + n16) * a.ldb;

  f32x4 acc[2][NB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int j0 = wave; j0 < nsteps; j0 += kGW * kGU) {
    u32x4 av[kGU][2][AF32 ? 2 : 1];
    u32x4 bv[kGU][NB];
    bool live[kGU];
#pragma unroll
    for (int u = 0; u < kGU; ++u) {
      const int s = j0 + kGW * u;
      live[u] = s < nsteps;
      const int k = kbase + 32 * min(s, nsteps - 1) + 8 * g;   // a step past the end re-reads the last (masked)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if constexpr (AF32) {
          const float* p = reinterpret_cast<const float*>(arow[rb]) + k;
          av[u][rb][0] = *reinterpret_cast<const u32x4*>(p);
          av[u][rb][1] = *reinterpret_cast<const u32x4*>(p + 4);
        } else {
          av[u][rb][0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(arow[rb]) + k);
        }
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) bv[u][cb] = *reinterpret_cast<const u32x4*>(brow[cb] + k);
    }
#pragma unroll
    for (int u = 0; u < kGU; ++u) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        bf16x8 ah, al;
        if constexpr (AF32) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = live[u] ? __uint_as_float(av[u][rb][0][i]) : 0.f;
            x[4 + i] = live[u] ? __uint_as_float(av[u][rb][1][i]) : 0.f;
          }
          u32x4 h, l;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
            l[i] = pack_bf16x2(x[2 * i] - bf16lo_to_f32(h[i]), x[2 * i + 1] - bf16hi_to_f32(h[i]));
          }
          ah = __builtin_bit_cast(bf16x8, h);
          al = __builtin_bit_cast(bf16x8, l);
        } else {
          const u32x4 z4 = {0u, 0u, 0u, 0u};
          ah = __builtin_bit_cast(bf16x8, live[u] ? av[u][rb][0] : z4);
        }
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const bf16x8 bf = __builtin_bit_cast(bf16x8, bv[u][cb]);
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bf, acc[rb][cb], 0, 0, 0);
          if constexpr (AF32) acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bf, acc[rb][cb], 0, 0, 0);
        }
      }
    }
  }

  // the waves' partial tiles, summed in wave order; lane (n16, g) of tile (rb, cb) holds rows
  // 16 rb + 4 g + i, column 16 cb + n16
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) red[wave][rb][cb][lane] = acc[rb][cb];
  __syncthreads();
  for (int e = threadIdx.x; e < 2 * NB * kWave; e += 64 * kGW) {
    const int rb = e / (NB * kWave), cb = (e / kWave) % NB, l = e % kWave;
    f32x4 s = red[0][rb][cb][l];
#pragma unroll
    for (int w = 1; w < kGW; ++w) {
      const f32x4 v = red[w][rb][cb][l];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += v[i];
    }
    const int col = c0 + 16 * cb + (l & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * rb + 4 * (l >> 4) + i;
      if (m >= a.M) continue;
      const int64_t off = (int64_t)grp * a.c_gstride + (int64_t)m * a.ldc + col;
      if (a.ksplit > 1) reinterpret_cast<float*>(a.C)[(int64_t)ks * a.p_stride + off] = s[i];
      else if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(a.C)[off] = (uint16_t)(pack_bf16x2(s[i], 0.f) & 0xffffu);
      else reinterpret_cast<float*>(a.C)[off] = s[i];
    }
  }
}

// the K ranges' partial tiles summed in range order (fixed: deterministic), written as y
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) k_sum_splits(const float* part, int64_t p_stride, int ksplit, int64_t n,
                                                    void* y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + i);
  for (int k = 1; k < ksplit; ++k) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + (int64_t)k * p_stride + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += v[e];
  }
  if constexpr (OUT_BF16) {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(y) + i) = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + i) = s;
  }
}

template <int NB, bool AF32>
static void launch_gemm(const GemmArgs& g, int groups, bool out_bf16, hipStream_t s) {
  const dim3 grid(g.N / (16 * NB), groups, ((g.M + kGM - 1) / kGM) * g.ksplit);
  if (out_bf16) hipLaunchKernelGGL((k_gemm_nt<NB, AF32, true>), grid, dim3(64 * kGW), 0, s, g);
  else hipLaunchKernelGGL((k_gemm_nt<NB, AF32, false>), grid, dim3(64 * kGW), 0, s, g);
}

hipError_t launch_out_proj(const OutProjArgs& p, hipStream_t s) {
  const int Kg = (p.H / p.G) * p.D;
  // 1. codes: one grid column per group, 64-column tiles of each group's R codes
  GemmArgs g1{};
  g1.A = p.o;
  g1.lda = (int64_t)p.H * p.D;
  g1.a_gstride = Kg;
  g1.B = static_cast<const uint16_t*>(p.wa);
  g1.ldb = Kg;
  g1.b_gstride = (int64_t)p.R * Kg;
  g1.C = p.z;
  g1.ldc = (int64_t)p.G * p.R;
  g1.c_gstride = p.R;
  g1.M = p.T;
  g1.N = p.R;
  g1.K = Kg;
  g1.ksplit = 1;
  if (p.o_dtype == CSA_FP32) launch_gemm<4, true>(g1, p.G, false, s);
  else launch_gemm<4, false>(g1, p.G, false, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. hidden: 128-column tiles over kOutSplit K ranges, so that each block reads a quarter of the
  // codes (every block of a K range reads all its codes: wide tiles keep that traffic low) and the
  // grid still has about 224 blocks; the ranges' partials are then summed
  GemmArgs g2{};
  g2.A = p.z;
  g2.lda = (int64_t)p.G * p.R;
  g2.a_gstride = 0;
  g2.B = static_cast<const uint16_t*>(p.wb);
  g2.ldb = (int64_t)p.G * p.R;
  g2.b_gstride = 0;
  g2.C = p.y;
  g2.ldc = p.hidden;
  g2.c_gstride = 0;
  g2.M = p.T;
  g2.N = p.hidden;
  g2.K = p.G * p.R;
  const bool split = p.hidden % 128 == 0 && g2.K % (32 * kOutSplit) == 0;
  if (split) {
    g2.ksplit = kOutSplit;
    g2.C = p.part;
    g2.p_stride = (int64_t)p.T * p.hidden;
    launch_gemm<8, true>(g2, 1, false, s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)p.T * p.hidden;
    const dim3 grid((unsigned)((n / 4 + 255) / 256));
    if (p.y_dtype == CSA_BF16) hipLaunchKernelGGL(k_sum_splits<true>, grid, dim3(256), 0, s, p.part, g2.p_stride, kOutSplit, n, p.y);
    else hipLaunchKernelGGL(k_sum_splits<false>, grid, dim3(256), 0, s, p.part, g2.p_stride, kOutSplit, n, p.y);
  } else {
    g2.ksplit = 1;
    launch_gemm<2, true>(g2, 1, p.y_dtype == CSA_BF16, s);
  }
  return hipGetLastError();
}

}  // namespace csa
