// Internal launch interfaces between the C ABI (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "csa.h"
#include "workspace.hpp"

namespace csa {

struct CompressArgs {
  const void* kv;
  const void* logits;
  int64_t ld_tok, ld_seq;
  int B, T_raw, first_row, n_new;
  void* out;
  float* scales;
  const int64_t* pos0;
  int dtype, cap, C, scale_block, window, stride;
  const double* inv_freq;
  int rope_dim;
  int run;   // rows per lane group (set by the launcher)
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);
// several compress calls: one launch when all are small, else one launch each
hipError_t launch_compress_batch(const CompressArgs* a, int n, hipStream_t s);

struct IndexArgs {
  const void* q_idx;      // bf16 [rows, Hi, Di]
  const float* w;         // [rows, Hi]
  const int64_t* q_pos;   // [rows]
  int B, Tq, Hi, Di;
  const void* keys;       // [B, cap, Di]
  const float* key_scales;  // [B, cap] (fp8) or null
  const int32_t* n_valid;
  const int64_t* pos0;
  int key_dtype, cap, window, stride;
  int topk;
  float* scores;          // [rows, cap]
  int32_t* idx_out;       // [rows, topk]
  // chunked top-k (long rows): stage-1 candidates [rows, nchunk, topk] and counts [rows, nchunk];
  // the launcher carves its candidate areas from cand_key (the workspace part it points to)
  uint32_t* cand_key;
  int32_t* cand_idx;
  int* cand_count;
  int chunk, nchunk;      // set by the launcher
};
hipError_t launch_index_scores(const IndexArgs& a, hipStream_t s);
// the scores launch carrying compress calls (the batch layouts of launch_compress_batch); falls
// back to separate launches when the calls need the run-mode kernel or the scores take the
// many-row kernel
hipError_t launch_index_scores_compress(const IndexArgs& a, const CompressArgs* calls, int n, hipStream_t s);
hipError_t launch_topk(const IndexArgs& a, hipStream_t s);

struct AttendArgs {
  const void* q;          // bf16 [rows, H, 512]
  const int64_t* q_pos;   // [rows]
  int B, Tq, H;
  // compressed KV cache
  const void* kv;
  const float* kv_scales;
  const int32_t* kv_n_valid;
  const int64_t* kv_pos0;
  int kv_dtype, kv_cap, kv_scale_block, kv_window, kv_stride;
  // selection (CSA) or dense (HCA)
  const int32_t* idx;     // [rows, topk] (CSA)
  int topk;
  int csa_mode;           // 1: rows from idx (CSA); 0: every visible entry (HCA)
  // window cache
  const void* win;
  const int32_t* win_n_valid;
  const int64_t* win_pos0;
  int win_cap, W;
  const float* sink;
  const double* inv_freq;
  int rope_dim;
  float scale_log2;       // softmax_scale * log2(e)
  void* out;
  int out_dtype;
  float* lse;
  // split-KV partials
  int nsplit, slot_cap, slots_per_split;
  uint16_t* part_o;       // [rows, nsplit, H, 512] fp16: o / n times 2^-e
  float* part_ml;         // [rows, nsplit, H, 4]: reference max, normaliser n, exact sum, e
};
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);
// C = A B^T for the output projection: A element (m, k) of group g at A + g a_gstride + m lda + k
// (fp32 or bf16 elements), B (bf16) rows of K contiguous elements, C fp32 or bf16
struct GemmArgs {
  const void* A;
  int64_t lda, a_gstride;
  const uint16_t* B;
  int64_t ldb, b_gstride;
  void* C;
  int64_t ldc, c_gstride;
  int M, N, K;
  int ksplit;           // K ranges of equal length; > 1: C holds fp32 partials, range r at C + r p_stride
  int64_t p_stride;
};
constexpr int kOutSplit = 4;   // K ranges of the output projection's second product
struct OutProjArgs {
  const void* o;      // [T, H, D], o_dtype CSA_FP32 or CSA_BF16
  int o_dtype, T, H, D, G, R, hidden;
  const void* wa;     // bf16 [G, R, (H / G) D]
  const void* wb;     // bf16 [hidden, G R]
  float* z;           // fp32 [T, G R] (workspace)
  float* part;        // fp32 [kOutSplit, T, hidden] (workspace): the second product's partials
  void* y;            // [T, hidden], y_dtype CSA_FP32 or CSA_BF16
  int y_dtype;
};
hipError_t launch_out_proj(const OutProjArgs& a, hipStream_t s);
// the plan's name for a cache storage code
inline int att_kind(int dtype) { return dtype == CSA_FP8_E4M3 ? kAttFp8 : (dtype == CSA_FP4_E2M1 ? kAttFp4 : kAttBf16); }

}  // namespace csa
