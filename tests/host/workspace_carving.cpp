// Host check of the workspace carving (compressed_attention_long_amd/csrc/workspace.hpp): for
// every top-k plan in a sweep of (rows, cap, k), every area a kernel writes lies inside the
// candidate bytes the C ABI asks for, the areas do not overlap, each starts 256-byte aligned,
// and every merge stage's output fits the area it is written to; for every attention plan in a
// sweep of (rows, heads, row-set length), the splits cover the row set, fit the LDS index list,
// and their partials fit the workspace.  Prints one line per failure
// and "checked N plans" at the end; exit status 1 on any failure.
#include <cstdio>
#include "workspace.hpp"

using namespace csa;

static int failures = 0;
#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      ++failures;                                 \
      std::printf("FAIL %s: ", #cond);            \
      std::printf(__VA_ARGS__);                   \
      std::printf("\n");                          \
    }                                             \
  } while (0)

int main() {
  const int rows_list[] = {1, 2, 3, 4, 7, 32, 127, 128, 129, 4096};
  const int cap_list[] = {1, 100, 16383, 16384, 16385, 20000, 32768, 65535, 65536, 65537, 70000, 100000,
                          140000, 262143, 300000, 524288, 1048576, 4000000};
  const int k_list[] = {1, 2, 64, 256, 512, 777, 1024, 2048, 4095, 4096};
  long n = 0;
  for (int rows : rows_list)
    for (int cap : cap_list)
      for (int k : k_list) {
        if (k > cap) continue;
        ++n;
        const TopkPlan pl = topk_plan(rows, cap, k);
        const size_t ws = topk_workspace(rows, cap, k);
        if (pl.mode == 0) {
          CHECK(ws == 0, "rows %d cap %d k %d: one-block plan asks for %zu bytes", rows, cap, k, ws);
          continue;
        }
        CHECK(pl.mode == 1, "rows %d cap %d k %d: mode %d", rows, cap, k, pl.mode);
        CHECK(pl.group >= 2, "rows %d cap %d k %d: merge group %d", rows, cap, k, pl.group);
        CHECK((long long)pl.nchunk * pl.chunk >= cap, "rows %d cap %d k %d: chunks do not cover the row", rows,
              cap, k);
        const TopkCarve c = topk_carve(rows, pl, k);
        const size_t nA = (size_t)rows * pl.nchunk * k;
        const int c2 = (pl.nchunk + pl.group - 1) / pl.group;
        const size_t nB = (size_t)rows * c2 * k;
        // areas in order, no overlap, inside the workspace
        CHECK(c.idxA >= c.keyA + nA * 4 && c.cntA >= c.idxA + nA * 4, "rows %d cap %d k %d: area A overlaps",
              rows, cap, k);
        CHECK(c.keyB >= c.cntA + (size_t)rows * pl.nchunk * 4, "rows %d cap %d k %d: B starts inside A", rows,
              cap, k);
        CHECK(c.idxB >= c.keyB + nB * 4 && c.cntB >= c.idxB + nB * 4, "rows %d cap %d k %d: area B overlaps",
              rows, cap, k);
        CHECK(c.cntB + (size_t)rows * c2 * 4 <= ws, "rows %d cap %d k %d: B ends at %zu past %zu", rows, cap, k,
              c.cntB + (size_t)rows * c2 * 4, ws);
        CHECK(c.keyA % 256 == 0 && c.keyB % 256 == 0 && ws % 256 == 0, "rows %d cap %d k %d: alignment", rows,
              cap, k);
        CHECK(c.idxA % 4 == 0 && c.cntA % 4 == 0 && c.idxB % 4 == 0 && c.cntB % 4 == 0,
              "rows %d cap %d k %d: word alignment", rows, cap, k);
        // the launcher's stage loop: every intermediate stage's chunks fit the area written
        int chunks = pl.nchunk;
        bool in_A = true;
        int stages = 0;
        while (chunks > pl.group) {
          const int out_chunks = (chunks + pl.group - 1) / pl.group;
          const int capacity = in_A ? c2 : pl.nchunk;
          CHECK(out_chunks <= capacity, "rows %d cap %d k %d: stage %d writes %d chunks into room for %d", rows,
                cap, k, stages, out_chunks, capacity);
          chunks = out_chunks;
          in_A = !in_A;
          ++stages;
          if (stages > 64) break;
        }
        CHECK(stages <= 64, "rows %d cap %d k %d: merge stages do not converge", rows, cap, k);
        // the final merge block takes every remaining chunk: at most kTopkMergeCands candidates
        CHECK((long long)chunks * k <= kTopkMergeCands, "rows %d cap %d k %d: final merge of %d chunks", rows, cap,
              k, chunks);
      }
  // attention: every split's rows lie inside the row set's slots, (CSA) a split's top-k slots fit
  // the LDS index list, and the partials fit the workspace
  const int arows[] = {1, 2, 4, 6, 8, 16, 32, 64, 128, 256, 4096, 16384};
  const int aheads[] = {1, 8, 16, 24, 64, 100, 128};
  const int aslots[] = {0, 1, 31, 32, 33, 129, 300, 640, 1152, 1280, 1281, 2000, 4224, 8320, 33000, 262271};
  for (int rows : arows)
    for (int H : aheads)
      for (int slots : aslots)
        for (int csa = 0; csa < 2; ++csa)
          for (int kind = kAttBf16; kind <= kAttFp4; ++kind) {
          ++n;
          const AttendPlan pl = attend_plan(rows, H, slots, csa != 0, kind);
          CHECK(kind != kAttFp8 || pl.hpb == 32, "rows %d H %d slots %d: fp8 plan with %d heads per block", rows, H,
                slots, pl.hpb);
          CHECK((kind == kAttBf16) == (pl.kind == kAttGroups || pl.kind == kAttGroups4), "rows %d H %d slots %d: kernel kind",
                rows, H, slots);
          CHECK(pl.kind != kAttGroups4 || (pl.hpb == 64 && pl.nsplit == 1), "rows %d H %d slots %d: 4-wave plan", rows, H,
                slots);
          const int tile = pl.kind != kAttPairs ? (pl.hpb == 64 ? kAttGroupTile64 : kAttGroupTile64 / 2) : kAttTile;
          CHECK(pl.hpb == 32 || pl.hpb == 64, "rows %d H %d slots %d: %d heads per block", rows, H, slots, pl.hpb);
          CHECK(pl.nsplit >= 1 && pl.sps >= tile && pl.sps % tile == 0,
                "rows %d H %d slots %d: %d splits of %d", rows, H, slots, pl.nsplit, pl.sps);
          CHECK((long long)pl.nsplit * pl.sps >= slots, "rows %d H %d slots %d: splits do not cover the rows", rows,
                H, slots);
          CHECK(slots == 0 || (long long)(pl.nsplit - 1) * pl.sps < slots, "rows %d H %d slots %d: an empty split",
                rows, H, slots);
          if (csa && pl.kind == kAttPairs)
            CHECK(pl.sps <= kAttIdxMax, "rows %d H %d slots %d: %d slots per split", rows, H, slots, pl.sps);
          const size_t ws = attend_workspace(rows, H, slots, csa != 0);
          const AttendCarve c = attend_carve(rows, H, pl);
          const size_t units = (size_t)rows * pl.nsplit * H;
          if (pl.nsplit == 1) {
            CHECK(c.end == 0, "rows %d H %d slots %d: one split carves %zu bytes", rows, H, slots, c.end);
          } else {
            CHECK(c.part_ml >= c.part_o + units * 512 * 2, "rows %d H %d slots %d: partials overlap", rows, H, slots);
            CHECK(c.part_ml % 16 == 0, "rows %d H %d slots %d: (m, n, l, e) not 16-byte aligned", rows, H, slots);
            CHECK(c.part_ml + units * 16 <= ws, "rows %d H %d slots %d: partials end past %zu", rows, H, slots, ws);
          }
        }
  std::printf("checked %ld plans, %d failures\n", n, failures);
  return failures ? 1 : 0;
}
