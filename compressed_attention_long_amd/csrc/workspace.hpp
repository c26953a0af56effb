// Workspace plans of the top-k selection: which stages run and where their candidate lists sit
// in the caller's workspace.  Plain host C++ (no HIP), shared by the C ABI (sizes and checks),
// the launcher (pointers) and a host test that checks every carving against the size it fits in.
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

}  // namespace csa
