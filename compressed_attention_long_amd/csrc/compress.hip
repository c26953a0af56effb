// Kernels and launchers of the KV compressor (softmax pooling per channel over each row's
// window, partial RoPE, bf16 / fp8 / fp4 storage); the device code is in compress_dev.hpp.
#include "compress_dev.hpp"

namespace csa {

// grid: (ceil(n_new / run), B); block: groups of C/8 lanes, one run of rows per group.
// MODE (a separate kernel each, so that each path gets its own register allocation):
// kOverlapRegs, kOverlap (window = 2 stride, runs of rows walking the raw stream once; the
// first keeps a block of tokens in registers ahead of the pooling), kPerRow (every row its own
// window).
enum { kOverlapRegs = 0, kOverlap = 1, kPerRow = 2 };
template <int MODE>
__global__ void __launch_bounds__(256) k_compress(CompressArgs a) {
  const int lanes = a.C / 8;
  const int groups = blockDim.x / lanes;
  const int g = threadIdx.x / lanes;
  const int li = threadIdx.x % lanes;
  if (g >= groups) return;
  const int b = blockIdx.y;
  const int first = (blockIdx.x * groups + g) * a.run;   // first new row (relative) of this run
  if (first >= a.n_new) return;
  const int last = min(first + a.run, a.n_new);           // exclusive
  const int c0 = li * 8;
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv) + (int64_t)b * a.ld_seq;
  const uint16_t* lg = a.logits ? reinterpret_cast<const uint16_t*>(a.logits) + (int64_t)b * a.ld_seq
                                : nullptr;
  const RopeIn ri = rope_in(a, b, c0);
  if constexpr (MODE == kOverlapRegs) {
    // Overlapping rows: entry i = block i + block i+1 (blocks of `stride` tokens).  The
    // loads of block i + 2 are issued before block i + 1 is pooled.
    const int st = a.stride;
    PoolState prev, cur;
    RawBlock r0, r1;
    load_block(r0, kv, lg, a.ld_tok, first * st, st, c0);
    load_block(r1, kv, lg, a.ld_tok, (first + 1) * st, st, c0);
    pool_reset(prev);
    pool_regs(prev, r0, st);
    for (int i = first; i < last; ++i) {
      if (i + 1 < last) load_block(r0, kv, lg, a.ld_tok, (i + 2) * st, st, c0);
      pool_reset(cur);
      pool_regs(cur, r1, st);
      pool_merge(prev, prev, cur);   // in place: element by element
      finish_row(prev, a, rope_trig(a, ri, a.first_row + i, c0), b, a.first_row + i, c0);
      prev = cur;
      r1 = r0;
    }
  } else if constexpr (MODE == kOverlap) {
    PoolState prev, cur, both;
    pool_reset(prev);
    pool_block(prev, kv, lg, a.ld_tok, first * a.stride, a.stride, c0);
    for (int i = first; i < last; ++i) {
      pool_reset(cur);
      pool_block(cur, kv, lg, a.ld_tok, (i + 1) * a.stride, a.stride, c0);
      pool_merge(both, prev, cur);
      finish_row(both, a, rope_trig(a, ri, a.first_row + i, c0), b, a.first_row + i, c0);
      prev = cur;
    }
  } else {
    for (int i = first; i < last; ++i) {
      PoolState p;
      pool_reset(p);
      pool_block(p, kv, lg, a.ld_tok, i * a.stride, a.window, c0);
      finish_row(p, a, rope_trig(a, ri, a.first_row + i, c0), b, a.first_row + i, c0);
    }
  }
}

__global__ void __launch_bounds__(256) k_compress_split_batch(CompressBatch bt) {
  compress_batch_block(bt, blockIdx.x);
}

hipError_t launch_compress_batch(const CompressArgs* a, int n, hipStream_t s) {
  CompressBatch bt;
  long long total;
  if (!make_compress_batch(a, n, bt, total)) {
    for (int i = 0; i < n; ++i) {
      const hipError_t e = launch_compress(a[i], s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (bt.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_compress_split_batch, dim3((unsigned)total), dim3(256), 0, s, bt);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a0, hipStream_t s) {
  CompressArgs a = a0;
  if (a.n_new == 0 || a.B == 0) return hipSuccess;
  // long windows, or few rows (a decode step): the one-launch kernel with a single call
  if (batch_layout(a) >= 0) return launch_compress_batch(&a, 1, s);
  const int lanes = a.C / 8;
  const int groups = max(128, lanes) / lanes;   // blocks of 128 lanes (measured faster than 256)
  // Long runs amortise the extra leading block of overlapping windows; short runs keep
  // enough blocks in flight for small calls.
  int run = 1;
  if (a.window == 2 * a.stride) {
    long long rows = (long long)a.n_new * a.B;
    run = rows >= 4096 ? 16 : (rows >= 1024 ? 4 : 1);
  }
  a.run = run;
  const int runs = (a.n_new + run - 1) / run;
  dim3 grid((runs + groups - 1) / groups, a.B);
  if (a.window == 2 * a.stride && a.run > 1 && a.stride <= kB)
    hipLaunchKernelGGL(k_compress<kOverlapRegs>, grid, dim3(groups * lanes), 0, s, a);
  else if (a.window == 2 * a.stride && a.run > 1)
    hipLaunchKernelGGL(k_compress<kOverlap>, grid, dim3(groups * lanes), 0, s, a);
  else
    hipLaunchKernelGGL(k_compress<kPerRow>, grid, dim3(groups * lanes), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa
