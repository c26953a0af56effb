// Device helpers shared by the attention kernels: the LDS tile layout, lane-group reductions,
// load-counter waits, the tile-ring barrier and the direct global-to-LDS row load.
#pragma once
#include "common.hpp"
#include "internal.hpp"

namespace csa {

constexpr int kD = 512;             // channels (head dim)
// bf16 per LDS row: 1056 B, so consecutive rows start 8 banks apart (no bank conflicts for the
// scores' 16-byte row reads or the transposing reads of P V at this pitch).
constexpr int kPitch = 528;
constexpr int kTR = kAttTile;       // rows per tile
constexpr float kRescale = 8.f;     // lazy-rescale threshold (log2 units)

// Block shape: NP wave pairs, 16 heads each.
template <int NP>
struct AttShape {
  static constexpr int HPB = 16 * NP;     // heads per block
  static constexpr int NW = 2 * NP;       // waves
  static constexpr int NT = 64 * NW;      // threads
  static constexpr int RPW = kTR / NW;    // rows of a tile each wave moves
};

__device__ __forceinline__ int visible_rows_att(int64_t qp, int64_t pos0, int window, int stride,
                                                int n_valid, int cap) {
  int nv = min(max(n_valid, 0), cap);
  int64_t num = qp - pos0 - (window - 1);
  if (num < 0) return 0;
  return (int)min((int64_t)nv, num / stride + 1);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;

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

// Wait until at most N vector-memory loads of this wave are outstanding (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima = no wait).  Loads
// complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier for the tile ring.  __syncthreads() is a release fence plus the barrier, and
// the fence waits for every LDS write of the wave, the DMA loads into LDS included: no tile could
// stay in flight across it.  Here the waits are explicit instead: this wave's own LDS stores
// (lgkmcnt(0)) before the barrier, and (by the caller, with wait_tiles) the DMA of exactly the
// tiles the next step reads.  The "memory" clobber keeps the compiler from moving LDS accesses
// across the barrier; it still counts the DMA loads that are in flight for every later LDS read.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// One 1 KB row from global memory into LDS (16 bytes per lane, lane i at lds_row + 16 i) by the
// direct global-to-LDS load, issued through inline asm: the compiler's own tracking of these loads
// cannot tell the four tile buffers apart, and would wait for every load in flight before any read
// of any tile buffer.  The ring's waits are explicit instead (wait_tiles before ring_barrier), and
// the "memory" clobber keeps LDS accesses from moving across the issue.
// m0 (the LDS base of the load) is a reserved register, so it is saved and restored around the
// load (the load takes m0 when it issues), with a wait state after each write of it.
__device__ __forceinline__ void dma_row(const void* src_lane, uint16_t* lds_row) {
  const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)lds_row;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "s"(base), "v"(src_lane)
      : "memory");
}

// wait until at most k tiles of RPW loads each are outstanding, k in 0..3
template <int RPW>
__device__ __forceinline__ void wait_tiles(int k) {
  switch (k) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<RPW>(); break;
    case 2: wait_vmcnt<2 * RPW>(); break;
    default: wait_vmcnt<3 * RPW>(); break;
  }
}

}  // namespace csa
