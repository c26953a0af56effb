// C ABI of the CSA/HCA hot path: host-side validation, workspace carving, launches.
// Validation never calls into HIP, so a failed call has no side effects and the
// checks run on machines without a GPU.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return CSA_OK;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

// Common checks of a cache descriptor.  `reads` = the call reads rows (needs n_valid).
int check_cache(const csa_cache_t* c, const char* name, bool reads) {
  REQUIRE(c != nullptr, CSA_EINVAL, "%s: cache descriptor is NULL", name);
  REQUIRE(c->data != nullptr, CSA_EINVAL, "%s: data is NULL", name);
  REQUIRE(c->pos0 != nullptr, CSA_EINVAL, "%s: pos0 is NULL", name);
  REQUIRE(!reads || c->n_valid != nullptr, CSA_EINVAL, "%s: n_valid is NULL", name);
  REQUIRE(c->cap >= 1, CSA_EINVAL, "%s: cap must be >= 1 (got %d)", name, c->cap);
  REQUIRE(c->C >= 1, CSA_EINVAL, "%s: C must be >= 1 (got %d)", name, c->C);
  REQUIRE(c->window >= 1 && c->stride >= 1, CSA_EINVAL, "%s: window and stride must be >= 1 (got %d, %d)",
          name, c->window, c->stride);
  REQUIRE(c->dtype == CSA_BF16 || c->dtype == CSA_FP8_E4M3 || c->dtype == CSA_FP4_E2M1, CSA_ENOTSUP,
          "%s: dtype %d not supported", name, c->dtype);
  REQUIRE(aligned(c->data, 16), CSA_EINVAL, "%s: data must be 16-byte aligned", name);
  if (c->dtype == CSA_FP4_E2M1) {
    REQUIRE(c->scales != nullptr, CSA_EINVAL, "%s: fp4 cache needs scales", name);
    REQUIRE(c->scale_block == 32 && c->C % 32 == 0, CSA_EINVAL,
            "%s: fp4 caches use 32-channel blocks (scale_block %d, C %d)", name, c->scale_block, c->C);
  }
  if (c->dtype == CSA_FP8_E4M3) {
    REQUIRE(c->scales != nullptr, CSA_EINVAL, "%s: fp8 cache needs scales", name);
    REQUIRE(c->scale_block >= 1 && c->C % c->scale_block == 0, CSA_EINVAL,
            "%s: scale_block %d must divide C %d", name, c->scale_block, c->C);
  }
  return CSA_OK;
}

int check_rope(const double* inv_freq, int rope_dim, int C) {
  REQUIRE(rope_dim >= 0 && rope_dim % 2 == 0 && rope_dim <= C, CSA_EINVAL,
          "rope_dim must be even and in [0, %d] (got %d)", C, rope_dim);
  REQUIRE(rope_dim == 0 || inv_freq != nullptr, CSA_EINVAL, "inv_freq is NULL");
  return CSA_OK;
}

}  // namespace

extern "C" {

const char* csa_last_error(void) { return g_err.c_str(); }

int csa_abi_version(void) { return 1; }

}  // extern "C"

namespace {

// Checks one csa_compress call and fills its launch arguments; `empty` when there is nothing
// to do (B == 0 or n_new == 0).
int compress_args(const void* kv, const void* logits, int64_t ld_tok, int64_t ld_seq, int B, int T_raw,
                  int first_row, int n_new, const csa_cache_t* out, const double* inv_freq, int rope_dim,
                  csa::CompressArgs& a, bool& empty) {
  empty = true;
  int rc = check_cache(out, "out", false);
  if (rc) return rc;
  REQUIRE(B >= 0 && n_new >= 0, CSA_EINVAL, "B and n_new must be >= 0 (got %d, %d)", B, n_new);
  if (B == 0 || n_new == 0) return CSA_OK;
  REQUIRE(kv != nullptr, CSA_EINVAL, "kv is NULL");
  REQUIRE(logits != nullptr || out->window == 1, CSA_EINVAL, "logits is NULL (allowed only when window == 1)");
  const int C = out->C;
  REQUIRE(C % 8 == 0 && C <= 2048 && (256 % (C / 8)) == 0, CSA_ENOTSUP,
          "C must be 8 times a divisor of 256 (got %d)", C);
  REQUIRE(first_row >= 0 && (int64_t)first_row + n_new <= out->cap, CSA_EINVAL,
          "rows [%d, %d) exceed cap %d", first_row, first_row + n_new, out->cap);
  REQUIRE((int64_t)T_raw >= (int64_t)(n_new - 1) * out->stride + out->window, CSA_EINVAL,
          "T_raw %d is too short for %d rows of window %d, stride %d", T_raw, n_new, out->window, out->stride);
  REQUIRE(ld_tok >= C && ld_tok % 8 == 0, CSA_EINVAL, "ld_tok must be >= C and a multiple of 8 (got %lld)",
          (long long)ld_tok);
  REQUIRE(B == 1 || (ld_seq >= (int64_t)T_raw * ld_tok && ld_seq % 8 == 0), CSA_EINVAL,
          "ld_seq must be >= T_raw * ld_tok and a multiple of 8 (got %lld)", (long long)ld_seq);
  REQUIRE(aligned(kv, 16) && (logits == nullptr || aligned(logits, 16)), CSA_EINVAL,
          "kv and logits must be 16-byte aligned");
  if (out->dtype == CSA_FP8_E4M3) {
    const int sb = out->scale_block;
    REQUIRE(sb % 8 == 0 && sb <= 512 && ((sb / 8) & (sb / 8 - 1)) == 0, CSA_ENOTSUP,
            "fp8 scale_block must be 8 times a power of two, at most 512 (got %d)", sb);
  }
  rc = check_rope(inv_freq, rope_dim, C);
  if (rc) return rc;
  a = csa::CompressArgs{};
  a.kv = kv;
  a.logits = out->window == 1 ? nullptr : logits;
  a.ld_tok = ld_tok;
  a.ld_seq = ld_seq;
  a.B = B;
  a.T_raw = T_raw;
  a.first_row = first_row;
  a.n_new = n_new;
  a.out = out->data;
  a.scales = out->scales;
  a.pos0 = out->pos0;
  a.dtype = out->dtype;
  a.cap = out->cap;
  a.C = C;
  a.scale_block = out->scale_block;
  a.window = out->window;
  a.stride = out->stride;
  a.inv_freq = inv_freq;
  a.rope_dim = rope_dim;
  empty = false;
  return CSA_OK;
}

}  // namespace

extern "C" {

int csa_compress(const void* kv, const void* logits, int64_t ld_tok, int64_t ld_seq, int B, int T_raw,
                 int first_row, int n_new, const csa_cache_t* out, const double* inv_freq, int rope_dim,
                 hipStream_t stream) {
  csa::CompressArgs a;
  bool empty;
  const int rc = compress_args(kv, logits, ld_tok, ld_seq, B, T_raw, first_row, n_new, out, inv_freq, rope_dim,
                               a, empty);
  if (rc) return rc;
  if (empty) return ok();
  hipError_t e = csa::launch_compress(a, stream);
  REQUIRE(e == hipSuccess, CSA_EHIP, "compress launch failed: %s", hipGetErrorString(e));
  return ok();
}

int csa_compress_batch(const csa_compress_call_t* calls, int n_calls, hipStream_t stream) {
  REQUIRE(n_calls >= 0, CSA_EINVAL, "n_calls must be >= 0 (got %d)", n_calls);
  REQUIRE(n_calls == 0 || calls != nullptr, CSA_EINVAL, "calls is NULL");
  std::vector<csa::CompressArgs> todo;
  for (int i = 0; i < n_calls; ++i) {
    const csa_compress_call_t& c = calls[i];
    csa::CompressArgs a;
    bool empty;
    const int rc = compress_args(c.kv, c.logits, c.ld_tok, c.ld_seq, c.B, c.T_raw, c.first_row, c.n_new, c.out,
                                 c.inv_freq, c.rope_dim, a, empty);
    if (rc) {
      g_err = "call " + std::to_string(i) + ": " + g_err;
      return rc;
    }
    if (!empty) todo.push_back(a);
  }
  if (todo.empty()) return ok();
  hipError_t e = csa::launch_compress_batch(todo.data(), (int)todo.size(), stream);
  REQUIRE(e == hipSuccess, CSA_EHIP, "compress launch failed: %s", hipGetErrorString(e));
  return ok();
}

static size_t index_scores_bytes(int B, int Tq, int cap) {
  return ((size_t)B * Tq * cap * sizeof(float) + 255) / 256 * 256;
}

size_t csa_index_topk_workspace_bytes(int B, int Tq, int Hi, int cap, int topk) {
  (void)Hi;
  if (B <= 0 || Tq <= 0 || cap <= 0 || topk <= 0) return 0;
  return index_scores_bytes(B, Tq, cap) + csa::topk_workspace(B * Tq, cap, topk);
}

// Validation and argument block of an index/top-k call; `empty` when there is nothing to do.
static int index_args(const void* q_idx, const float* w, const int64_t* q_pos, int B, int Tq, int Hi,
                      const csa_cache_t* keys, int topk, int32_t* idx_out, float* scores_out, void* workspace,
                      size_t workspace_bytes, csa::IndexArgs& a, bool& empty) {
  empty = false;
  int rc = check_cache(keys, "keys", true);
  if (rc) return rc;
  REQUIRE(B >= 0 && Tq >= 0, CSA_EINVAL, "B and Tq must be >= 0");
  REQUIRE(topk >= 1 && topk <= keys->cap && topk <= 4096, CSA_EINVAL, "topk must be in [1, min(cap=%d, 4096)] (got %d)",
          keys->cap, topk);
  if (B == 0 || Tq == 0) {
    empty = true;
    return CSA_OK;
  }
  REQUIRE(q_idx && w && q_pos && idx_out, CSA_EINVAL, "q_idx, w, q_pos and idx_out must be non-NULL");
  REQUIRE(Hi >= 1 && Hi <= 64, CSA_ENOTSUP, "Hi must be in [1, 64] (got %d)", Hi);
  REQUIRE(keys->C == 128, CSA_ENOTSUP, "indexer key dim must be 128 (got %d)", keys->C);
  REQUIRE(keys->dtype != CSA_FP4_E2M1, CSA_ENOTSUP, "fp4 indexer keys are not supported");
  REQUIRE(keys->dtype == CSA_BF16 || keys->scale_block == keys->C, CSA_ENOTSUP,
          "fp8 indexer keys need one scale per key (scale_block == C)");
  REQUIRE(aligned(q_idx, 16), CSA_EINVAL, "q_idx must be 16-byte aligned");
  const int64_t rows = (int64_t)B * Tq;
  REQUIRE(rows <= 0x7fffffff && (keys->cap + 1023) / 1024 <= 65535, CSA_ENOTSUP, "problem too large");
  // workspace: [scores unless scores_out is given][two-stage top-k candidates of long rows]
  const size_t sc_bytes = scores_out ? 0 : index_scores_bytes(B, Tq, keys->cap);
  const csa::TopkPlan plan = csa::topk_plan((int)rows, keys->cap, topk);
  const size_t cand_bytes = csa::topk_workspace((int)rows, keys->cap, topk);
  const size_t need = sc_bytes + cand_bytes;
  if (need > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, CSA_EWORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    REQUIRE(aligned(workspace, 256), CSA_EINVAL, "workspace must be 256-byte aligned");
  }
  if (scores_out) REQUIRE(aligned(scores_out, 16), CSA_EINVAL, "scores_out must be 16-byte aligned");
  float* scores = scores_out ? scores_out : static_cast<float*>(workspace);
  uint8_t* cand = static_cast<uint8_t*>(workspace) + sc_bytes;
  a = csa::IndexArgs{};
  a.q_idx = q_idx;
  a.w = w;
  a.q_pos = q_pos;
  a.B = B;
  a.Tq = Tq;
  a.Hi = Hi;
  a.Di = keys->C;
  a.keys = keys->data;
  a.key_scales = keys->dtype == CSA_FP8_E4M3 ? keys->scales : nullptr;
  a.n_valid = keys->n_valid;
  a.pos0 = keys->pos0;
  a.key_dtype = keys->dtype;
  a.cap = keys->cap;
  a.window = keys->window;
  a.stride = keys->stride;
  a.topk = topk;
  a.scores = scores;
  a.idx_out = idx_out;
  if (plan.mode == 1) a.cand_key = reinterpret_cast<uint32_t*>(cand);   // carved by the launcher
  return CSA_OK;
}

int csa_index_topk(const void* q_idx, const float* w, const int64_t* q_pos, int B, int Tq, int Hi,
                   const csa_cache_t* keys, int topk, int32_t* idx_out, float* scores_out, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  csa::IndexArgs a;
  bool empty;
  const int rc = index_args(q_idx, w, q_pos, B, Tq, Hi, keys, topk, idx_out, scores_out, workspace,
                            workspace_bytes, a, empty);
  if (rc) return rc;
  if (empty) return ok();
  hipError_t e = csa::launch_index_scores(a, stream);
  REQUIRE(e == hipSuccess, CSA_EHIP, "index score launch failed: %s", hipGetErrorString(e));
  e = csa::launch_topk(a, stream);
  REQUIRE(e == hipSuccess, CSA_EHIP, "top-k launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Byte range [lo, hi) of a device buffer, for the overlap checks of the combined call.
struct Span {
  uintptr_t lo, hi;
};
static Span span(const void* p, size_t bytes) {
  const uintptr_t u = reinterpret_cast<uintptr_t>(p);
  return Span{u, u + (p ? bytes : 0)};
}
static bool overlap(Span x, Span y) { return x.lo < y.hi && y.lo < x.hi; }

int csa_index_topk_compress(const csa_compress_call_t* calls, int n_calls, const void* q_idx, const float* w,
                            const int64_t* q_pos, int B, int Tq, int Hi, const csa_cache_t* keys, int topk,
                            int32_t* idx_out, float* scores_out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  REQUIRE(n_calls >= 0, CSA_EINVAL, "n_calls must be >= 0 (got %d)", n_calls);
  REQUIRE(n_calls == 0 || calls != nullptr, CSA_EINVAL, "calls is NULL");
  std::vector<csa::CompressArgs> todo;
  for (int i = 0; i < n_calls; ++i) {
    const csa_compress_call_t& c = calls[i];
    csa::CompressArgs ca;
    bool cempty;
    const int rc = compress_args(c.kv, c.logits, c.ld_tok, c.ld_seq, c.B, c.T_raw, c.first_row, c.n_new, c.out,
                                 c.inv_freq, c.rope_dim, ca, cempty);
    if (rc) {
      g_err = "call " + std::to_string(i) + ": " + g_err;
      return rc;
    }
    if (!cempty) todo.push_back(ca);
  }
  csa::IndexArgs a;
  bool empty;
  const int rc = index_args(q_idx, w, q_pos, B, Tq, Hi, keys, topk, idx_out, scores_out, workspace,
                            workspace_bytes, a, empty);
  if (rc) return rc;
  if (!empty) {
    // the compressor's outputs must not be anything the indexer reads or writes
    const int64_t rows = (int64_t)B * Tq;
    const size_t key_elt = keys->dtype == CSA_BF16 ? 2 : 1;
    const Span ins[] = {
        span(keys->data, (size_t)keys->cap * keys->C * key_elt * B),
        span(keys->scales, (size_t)keys->cap * 4 * B),
        span(q_idx, (size_t)rows * Hi * keys->C * 2),
        span(w, (size_t)rows * Hi * 4),
        span(a.scores, (size_t)rows * keys->cap * 4),
        span(idx_out, (size_t)rows * topk * 4),
        span(workspace, workspace ? workspace_bytes : 0),
    };
    for (size_t i = 0; i < todo.size(); ++i) {
      const csa::CompressArgs& ca = todo[i];
      const size_t row_b = ca.dtype == CSA_BF16 ? 2 * (size_t)ca.C : (ca.dtype == CSA_FP8_E4M3 ? ca.C : ca.C / 2);
      const Span outs[] = {span(ca.out, row_b * ca.cap * ca.B),
                           span(ca.scales, ca.scales ? (size_t)ca.cap * (ca.C / ca.scale_block) * 4 * ca.B : 0)};
      for (const Span& o : outs)
        for (const Span& x : ins)
          REQUIRE(!overlap(o, x), CSA_EINVAL, "compress output of call %d overlaps an indexer buffer", (int)i);
    }
  }
  hipError_t e = hipSuccess;
  if (empty) {
    if (!todo.empty()) e = csa::launch_compress_batch(todo.data(), (int)todo.size(), stream);
    REQUIRE(e == hipSuccess, CSA_EHIP, "compress launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  e = csa::launch_index_scores_compress(a, todo.data(), (int)todo.size(), stream);
  REQUIRE(e == hipSuccess, CSA_EHIP, "index score / compress launch failed: %s", hipGetErrorString(e));
  e = csa::launch_topk(a, stream);
  REQUIRE(e == hipSuccess, CSA_EHIP, "top-k launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t csa_attend_workspace_bytes(int B, int Tq, int H, int topk, int W) {
  if (B <= 0 || Tq <= 0 || H <= 0) return 0;
  return csa::attend_workspace(B * Tq, H, topk + (W > 0 ? W : 0), true);
}

size_t hca_attend_workspace_bytes(int B, int Tq, int H, int cap, int W) {
  if (B <= 0 || Tq <= 0 || H <= 0) return 0;
  return csa::attend_workspace(B * Tq, H, cap + (W > 0 ? W : 0), false);
}

static int attend_common(const void* q, const int64_t* q_pos, int B, int Tq, int H, const csa_cache_t* kv,
                         const int32_t* idx, int topk, bool csa_mode, const csa_cache_t* win, int W,
                         const float* sink, const double* inv_freq, int rope_dim, float softmax_scale, void* out,
                         int out_dtype, float* lse_out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  int rc = check_cache(kv, "kv", true);
  if (rc) return rc;
  rc = check_cache(win, "win", true);
  if (rc) return rc;
  REQUIRE(B >= 0 && Tq >= 0, CSA_EINVAL, "B and Tq must be >= 0");
  if (B == 0 || Tq == 0) return ok();
  REQUIRE(q && q_pos && sink && out, CSA_EINVAL, "q, q_pos, sink and out must be non-NULL");
  REQUIRE(H >= 1 && H <= 1024, CSA_EINVAL, "H must be in [1, 1024] (got %d)", H);
  REQUIRE(kv->C == 512 && win->C == 512, CSA_ENOTSUP, "head dim must be 512 (kv %d, win %d)", kv->C, win->C);
  REQUIRE(win->dtype == CSA_BF16, CSA_ENOTSUP, "window cache must be bf16");
  REQUIRE(win->window == 1 && win->stride == 1, CSA_EINVAL, "window cache must have window = stride = 1");
  REQUIRE(kv->dtype != CSA_FP8_E4M3 || kv->scale_block % 64 == 0, CSA_ENOTSUP,
          "fp8 KV scale_block must be a multiple of 64 (got %d)", kv->scale_block);
  REQUIRE(W >= 0, CSA_EINVAL, "W must be >= 0 (got %d)", W);
  REQUIRE(out_dtype == CSA_FP32 || out_dtype == CSA_BF16, CSA_ENOTSUP, "out_dtype must be FP32 or BF16");
  REQUIRE(aligned(q, 16) && aligned(out, 16), CSA_EINVAL, "q and out must be 16-byte aligned");
  if (csa_mode) {
    REQUIRE(topk >= 0 && topk <= kv->cap, CSA_EINVAL, "topk must be in [0, cap=%d] (got %d)", kv->cap, topk);
    REQUIRE(topk == 0 || idx != nullptr, CSA_EINVAL, "idx is NULL");
  }
  rc = check_rope(inv_freq, rope_dim, 512);
  if (rc) return rc;
  const int rows = B * Tq;
  const int slot_cap = (csa_mode ? topk : kv->cap) + W;
  const size_t need = csa::attend_workspace(rows, H, slot_cap, csa_mode);
  if (need > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, CSA_EWORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    REQUIRE(aligned(workspace, 256), CSA_EINVAL, "workspace must be 256-byte aligned");
  }
  csa::AttendArgs a{};
  a.q = q;
  a.q_pos = q_pos;
  a.B = B;
  a.Tq = Tq;
  a.H = H;
  a.kv = kv->data;
  a.kv_scales = kv->dtype != CSA_BF16 ? kv->scales : nullptr;
  a.kv_n_valid = kv->n_valid;
  a.kv_pos0 = kv->pos0;
  a.kv_dtype = kv->dtype;
  a.kv_cap = kv->cap;
  a.kv_scale_block = kv->scale_block;
  a.kv_window = kv->window;
  a.kv_stride = kv->stride;
  a.idx = csa_mode ? (topk > 0 ? idx : nullptr) : nullptr;
  a.topk = csa_mode ? topk : 0;
  a.win = win->data;
  a.win_n_valid = win->n_valid;
  a.win_pos0 = win->pos0;
  a.win_cap = win->cap;
  a.W = W;
  a.sink = sink;
  a.inv_freq = inv_freq;
  a.rope_dim = rope_dim;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = out;
  a.out_dtype = out_dtype;
  a.lse = lse_out;
  a.slot_cap = slot_cap;
  if (need > 0) {
    const csa::AttendCarve cv =
        csa::attend_carve(rows, H, csa::attend_plan(rows, H, slot_cap, csa_mode, csa::att_kind(kv->dtype)));
    a.part_o = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + cv.part_o);
    a.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + cv.part_ml);
  }
  a.csa_mode = csa_mode ? 1 : 0;
  hipError_t e;
  e = csa::launch_attend(a, stream);
  REQUIRE(e == hipSuccess, CSA_EHIP, "attend launch failed: %s", hipGetErrorString(e));
  return ok();
}

int csa_attend(const void* q, const int64_t* q_pos, int B, int Tq, int H, const csa_cache_t* kv,
               const int32_t* idx, int topk, const csa_cache_t* win, int W, const float* sink,
               const double* inv_freq, int rope_dim, float softmax_scale, void* out, int out_dtype,
               float* lse_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return attend_common(q, q_pos, B, Tq, H, kv, idx, topk, true, win, W, sink, inv_freq, rope_dim, softmax_scale,
                       out, out_dtype, lse_out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- output projection

extern "C" {

static size_t out_proj_z_bytes(int T, int G, int R) { return ((size_t)T * G * R * sizeof(float) + 255) / 256 * 256; }

size_t csa_out_proj_workspace_bytes(int T, int G, int R, int hidden) {
  if (T <= 0 || G <= 0 || R <= 0 || hidden <= 0) return 0;
  return out_proj_z_bytes(T, G, R) + (size_t)csa::kOutSplit * T * hidden * sizeof(float);
}

int csa_out_proj(const void* o, int o_dtype, int T, int H, int D, int G, const void* wa, int R, const void* wb,
                 int hidden, void* y, int y_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  REQUIRE(T >= 0, CSA_EINVAL, "T must be >= 0 (got %d)", T);
  if (T == 0) return ok();
  REQUIRE(o && wa && wb && y, CSA_EINVAL, "o, wa, wb and y must be non-NULL");
  REQUIRE(H >= 1 && D >= 1 && G >= 1 && R >= 1 && hidden >= 1, CSA_EINVAL,
          "H, D, G, R and hidden must be >= 1 (got %d, %d, %d, %d, %d)", H, D, G, R, hidden);
  REQUIRE(H % G == 0, CSA_EINVAL, "H (%d) must be a multiple of G (%d)", H, G);
  const long long Kg = (long long)(H / G) * D;
  REQUIRE(Kg % 32 == 0, CSA_ENOTSUP, "(H / G) * D must be a multiple of 32 (got %lld)", Kg);
  REQUIRE(R % 64 == 0, CSA_ENOTSUP, "R must be a multiple of 64 (got %d)", R);
  REQUIRE(hidden % 32 == 0, CSA_ENOTSUP, "hidden must be a multiple of 32 (got %d)", hidden);
  REQUIRE((long long)G * R <= (1LL << 30) && Kg <= (1LL << 30), CSA_EINVAL, "factor shapes too large");
  REQUIRE(o_dtype == CSA_FP32 || o_dtype == CSA_BF16, CSA_ENOTSUP, "o_dtype must be FP32 or BF16");
  REQUIRE(y_dtype == CSA_FP32 || y_dtype == CSA_BF16, CSA_ENOTSUP, "y_dtype must be FP32 or BF16");
  REQUIRE(aligned(o, 16) && aligned(wa, 16) && aligned(wb, 16) && aligned(y, 16), CSA_EINVAL,
          "o, wa, wb and y must be 16-byte aligned");
  const size_t need = csa_out_proj_workspace_bytes(T, G, R, hidden);
  REQUIRE(workspace != nullptr && workspace_bytes >= need, CSA_EWORKSPACE, "workspace of %zu bytes needed (got %zu)",
          need, workspace_bytes);
  REQUIRE(aligned(workspace, 256), CSA_EINVAL, "workspace must be 256-byte aligned");
  csa::OutProjArgs a{};
  a.o = o;
  a.o_dtype = o_dtype;
  a.T = T;
  a.H = H;
  a.D = D;
  a.G = G;
  a.R = R;
  a.hidden = hidden;
  a.wa = wa;
  a.wb = wb;
  a.z = static_cast<float*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + out_proj_z_bytes(T, G, R));
  a.y = y;
  a.y_dtype = y_dtype;
  const hipError_t e = csa::launch_out_proj(a, stream);
  REQUIRE(e == hipSuccess, CSA_EHIP, "output projection launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------- csa_attend without a workspace
//
// The split partials of csa_attend_noalloc live in this array: one copy per GPU the library runs
// on, kept until the process ends.  Host code never uses its name as an address (on the host it
// is only a stand-in): each device's address is looked up once, with that device current, and
// kept in g_scratch.
static __device__ __attribute__((aligned(256))) uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

extern "C" {

int csa_attend_noalloc(const void* q, const int64_t* q_pos, int B, int Tq, int H, const csa_cache_t* kv,
                       const int32_t* idx, int topk, const csa_cache_t* win, int W, const float* sink,
                       const double* inv_freq, int rope_dim, float softmax_scale, void* out, int out_dtype,
                       float* lse_out, hipStream_t stream) {
  // the scratch this call needs, from its sizes alone (bad sizes are reported by attend_common)
  size_t need = 0;
  if (B > 0 && Tq > 0 && H >= 1 && H <= 1024 && topk >= 0 && W >= 0 && (int64_t)B * Tq <= 0x7fffffff)
    need = csa::attend_workspace(B * Tq, H, topk + W, true);
  REQUIRE(need <= CSA_NOALLOC_SCRATCH_BYTES, CSA_EWORKSPACE,
          "this call needs %zu bytes of scratch; the no-allocation entry point holds %u (use csa_attend with a "
          "workspace)", need, (unsigned)CSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    REQUIRE(e == hipSuccess, CSA_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    REQUIRE(dev >= 0 && dev < kMaxDevices, CSA_ENOTSUP, "device %d: at most %d devices", dev, kMaxDevices);
    std::call_once(g_scratch_once[dev], [dev] {
      g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
    });
    REQUIRE(g_scratch_err[dev] == hipSuccess && g_scratch[dev] != nullptr, CSA_EHIP,
            "locating the scratch array on device %d failed: %s", dev, hipGetErrorString(g_scratch_err[dev]));
    ws = g_scratch[dev];
  }
  return attend_common(q, q_pos, B, Tq, H, kv, idx, topk, true, win, W, sink, inv_freq, rope_dim, softmax_scale,
                       out, out_dtype, lse_out, ws, ws ? (size_t)CSA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int hca_attend(const void* q, const int64_t* q_pos, int B, int Tq, int H, const csa_cache_t* kv,
               const csa_cache_t* win, int W, const float* sink, const double* inv_freq, int rope_dim,
               float softmax_scale, void* out, int out_dtype, float* lse_out, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  return attend_common(q, q_pos, B, Tq, H, kv, nullptr, 0, false, win, W, sink, inv_freq, rope_dim,
                       softmax_scale, out, out_dtype, lse_out, workspace, workspace_bytes, stream);
}

}  // extern "C"
