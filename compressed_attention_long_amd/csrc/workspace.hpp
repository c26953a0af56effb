// Launch plans and workspace carving of the top-k selection and of attention: which stages or
// splits run and where their intermediate results sit in the caller's workspace.  Plain host C++
// (no HIP), shared by the C ABI (sizes and checks), the launchers (pointers) and a host test that
// checks every carving against the size it fits in.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace csa {

// Rows of up to this many entries take one register-resident block per row.
#ifndef CSA_TOPK_SINGLE_MAX
#define CSA_TOPK_SINGLE_MAX 16384
#endif
// 16,384 entries per stage-1 block and candidates per merge block: a 262,143-entry row takes
// one chunk stage and one merge (23.5 us for 4 rows, against 25.6 in three stages with 8,192).
constexpr int kTopkChunk = 16384;       // stage-1 entries per block
constexpr int kTopkMergeCands = 16384;  // candidates per merge block
constexpr int kTopkMaxK = 4096;         // largest k the C ABI accepts
static_assert(kTopkMergeCands / kTopkMaxK >= 2, "a merge block must take at least two chunks of the largest k");

struct TopkPlan {
  int mode;               // 0: one block per row; 1: chunked stages
  int chunk, nchunk, group;
};

// Plan for rows of up to `cap` entries, k <= kTopkMaxK.  Short rows (and up to 65,536 entries
// when there are at least 128 rows to fill the GPU) take one block per row.  Longer rows go
// through stage 1 (chunks of kTopkChunk entries, `nchunk` per row) and merge stages that each
// reduce `group` chunks of k candidates to one, until one block per row finishes.
inline TopkPlan topk_plan(int rows, int cap, int k) {
  TopkPlan pl{};
  if (cap <= CSA_TOPK_SINGLE_MAX || (cap <= 65536 && rows >= 128)) {
    pl.mode = 0;
    return pl;
  }
  pl.mode = 1;
  pl.chunk = kTopkChunk;
  pl.nchunk = (cap + kTopkChunk - 1) / kTopkChunk;
  pl.group = kTopkMergeCands / k;
  return pl;
}

// Byte offsets, from the start of the candidate area (256-byte aligned), of the two candidate
// areas of the chunked plan: A holds the stage-1 chunks [rows, nchunk, k], B the first merge
// stage's [rows, ceil(nchunk / group), k]; later merge stages alternate between them (each
// stage's output has at most as many chunks as B).  Each area is [keys u32 | indices i32 |
// counts i32 per chunk]; A and B start 256-byte aligned.  `end` is the first byte past B.
struct TopkCarve {
  size_t keyA, idxA, cntA, keyB, idxB, cntB, end;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

inline TopkCarve topk_carve(int rows, const TopkPlan& pl, int k) {
  TopkCarve c{};
  if (pl.mode != 1) return c;
  const size_t nA = (size_t)rows * pl.nchunk * k;
  const size_t c2 = (size_t)(pl.nchunk + pl.group - 1) / pl.group;
  const size_t nB = (size_t)rows * c2 * k;
  c.keyA = 0;
  c.idxA = c.keyA + nA * sizeof(uint32_t);
  c.cntA = c.idxA + nA * sizeof(int32_t);
  c.keyB = align256(c.cntA + (size_t)rows * pl.nchunk * sizeof(int32_t));
  c.idxB = c.keyB + nB * sizeof(uint32_t);
  c.cntB = c.idxB + nB * sizeof(int32_t);
  c.end = c.cntB + (size_t)rows * c2 * sizeof(int32_t);
  return c;
}

// Candidate-area bytes of a call (0 for the one-block plan).
inline size_t topk_workspace(int rows, int cap, int k) {
  const TopkPlan pl = topk_plan(rows, cap, k);
  if (pl.mode != 1) return 0;
  return align256(topk_carve(rows, pl, k).end);
}

// ---------------------------------------------------------------- attention

// Two kernels: the grouped kernel for bf16 caches (tile groups of 16-head waves holding all 512
// output channels, 64 rows per step, 32- or 16-row tiles) and the wave-pair kernel for quantized
// caches (pairs of waves sharing 16 heads, 32-row tiles through a four-buffer ring, fp8 scales
// applied in fp32).
constexpr int kAttGroups = 0, kAttPairs = 1, kAttGroups4 = 2;   // kernels: grouped (8 or 4 waves), wave pairs
constexpr int kAttGroupTile64 = 32;    // grouped kernel: rows per tile with 64 heads per block
constexpr int kAttTile = 32;           // wave-pair kernel: rows per tile
constexpr int kAttIdxMax = 1280;       // top-k indices of one split held in LDS (a multiple of 64)
constexpr int kAttTargetBlocks = 256;  // split until the grid has about this many blocks

// Storage kinds of the compressed KV cache, as the plan sees them.
constexpr int kAttBf16 = 0, kAttFp8 = 1, kAttFp4 = 2;

struct AttendPlan {
  int kind;     // kAttGroups, kAttGroups4 or kAttPairs
  int hpb;      // heads per block (64 or 32)
  int nsplit;   // splits of each query row's row set
  int sps;      // rows per split (whole tiles)
};

// Splits for a block shape with `tile`-row tiles: enough that the grid has about kAttTargetBlocks
// blocks, at least two tiles per split, at most `idx_max` slots per split (0: no limit); the
// per-split count is rounded up to whole tiles.  slot_cap = the longest row set (top-k or visible
// entries, plus the window).
inline AttendPlan attend_plan_for(int kind, int hpb, int tile, int idx_max, int rows, int H, int slot_cap,
                                  int target = kAttTargetBlocks) {
  AttendPlan pl{};
  pl.kind = kind;
  pl.hpb = hpb;
  const long long HG = (H + hpb - 1) / hpb;
  const long long base = (long long)rows * HG;
  long long ns = (target + base - 1) / base;
  const long long max_ns = ((long long)slot_cap + 2 * tile - 1) / (2 * tile);
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  if (idx_max > 0) {
    const long long min_ns = ((long long)slot_cap + idx_max - 1) / idx_max;
    if (ns < min_ns) ns = min_ns;
  }
  long long sps = ((long long)slot_cap + ns - 1) / ns;
  sps = (sps + tile - 1) / tile * tile;
  if (sps < tile) sps = tile;
  pl.sps = (int)sps;
  const long long n = ((long long)slot_cap + sps - 1) / sps;
  pl.nsplit = (int)(n < 1 ? 1 : n);
  return pl;
}

// The call's plan.  Either kernel takes 64 heads per block when that grid reaches about
// kAttTargetBlocks blocks (each staged row then serves the most heads), else 32 (few query rows
// over short row sets, as in 1M-token decode with top-k), where twice the blocks shorten the
// critical path.  fp8 caches always take 32 heads per block (their per-block scaling needs the
// registers of the larger shape's second pair).
inline AttendPlan attend_plan(int rows, int H, int slot_cap, bool csa, int kv_kind) {
  if (kv_kind == kAttBf16) {
    // 64 heads in 4-wave blocks, two per CU (their phases drift apart: prefill 1.85 -> 1.61 ms),
    // where the query rows alone fill two blocks per CU, so that no split is added (with splits
    // the extra partials cost what the kernel gains: HCA 1M even, 65K decode +4 us)
    const AttendPlan p4 = attend_plan_for(kAttGroups4, 64, kAttGroupTile64, 0, rows, H, slot_cap, 2 * kAttTargetBlocks);
    if (p4.nsplit == 1 && (long long)rows * ((H + 63) / 64) >= 2 * kAttTargetBlocks) return p4;
    const AttendPlan p64 = attend_plan_for(kAttGroups, 64, kAttGroupTile64, 0, rows, H, slot_cap);
    const long long blocks64 = (long long)rows * ((H + 63) / 64) * p64.nsplit;
    return blocks64 < kAttTargetBlocks ? attend_plan_for(kAttGroups, 32, kAttGroupTile64 / 2, 0, rows, H, slot_cap)
                                       : p64;
  }
  const int idx_max = csa ? kAttIdxMax : 0;
  const AttendPlan p64 = attend_plan_for(kAttPairs, 64, kAttTile, idx_max, rows, H, slot_cap);
  const long long blocks64 = (long long)rows * ((H + 63) / 64) * p64.nsplit;
  return (kv_kind == kAttFp8 || blocks64 < kAttTargetBlocks)
             ? attend_plan_for(kAttPairs, 32, kAttTile, idx_max, rows, H, slot_cap)
             : p64;
}

// Split partials in the workspace: fp16 outputs [rows, nsplit, H, 512] from byte 0, then fp32
// (max, normaliser, sum, exponent) [rows, nsplit, H, 4]; nothing when there is one split.
struct AttendCarve {
  size_t part_o, part_ml, end;
};
inline AttendCarve attend_carve(int rows, int H, const AttendPlan& pl) {
  AttendCarve c{};
  if (pl.nsplit <= 1) return c;
  const size_t units = (size_t)rows * pl.nsplit * H;
  c.part_o = 0;
  c.part_ml = units * 512 * sizeof(uint16_t);
  c.end = c.part_ml + units * 4 * sizeof(float);
  return c;
}
// Bytes for any cache format (the size query does not take the format): the largest of the plans.
inline size_t attend_workspace(int rows, int H, int slot_cap, bool csa) {
  size_t end = 0;
  for (int kind = kAttBf16; kind <= kAttFp4; ++kind) {
    const AttendCarve c = attend_carve(rows, H, attend_plan(rows, H, slot_cap, csa, kind));
    if (c.end > end) end = c.end;
  }
  return end == 0 ? 0 : align256(end);
}

}  // namespace csa
