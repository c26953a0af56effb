/*
 * csa.h — C ABI of the compressed-attention hot path on AMD Instinct MI355X (gfx950).
 *
 * The path computes one attention layer of the two compressed variants the
 * DeepSeek-V4-Pro pages describe:
 *   - Compressed Sparse Attention (CSA): entries pool 8 raw tokens at stride 4,
 *     a lightning indexer scores them and keeps the top-k, and the query heads
 *     attend to those entries plus a sliding window of raw tokens;
 *   - Heavily Compressed Attention (HCA): entries pool 128 raw tokens, and the
 *     heads attend densely to every visible entry plus the window.
 * ("DeepSeek-V4-Pro vs Inkling", Component-by-component table, CSA and HCA
 * rows; the sink and partial-RoPE rows; "DeepSeek-V4-Pro" model atlas, Raw
 * config fields.)
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers owned by the caller, dense and
 *     row-major with the shapes given below.  The library never allocates
 *     device memory; scratch space is a caller-provided workspace whose size
 *     the matching *_workspace_bytes() query returns.
 *   - Every call is asynchronous on the given stream and never synchronises
 *     the host.  A call returns CSA_OK once its kernels are enqueued.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed call has no side effects.  Validation never touches the GPU, so
 *     it can be exercised on a machine without one.  Device-resident values
 *     (counts, positions, indices) cannot be checked on the host: kernels
 *     clamp them to the buffers they index, so bad values give wrong numbers
 *     but never an out-of-bounds access.
 *   - Results are deterministic: the same inputs and arguments give the same
 *     bits (no floating-point atomics; fixed split counts).
 *   - Nothing is thrown across the ABI.  On failure, csa_last_error() returns
 *     a thread-local message describing the first failed check.
 *   - Positions are int64.  Rotary inverse frequencies are a device array of
 *     rope_dim/2 doubles (base 160,000 on the pages; the caller may pass a
 *     YaRN-adjusted table).  Rotation angles and their sines and cosines are
 *     evaluated in fp64 on the device, the rotation itself in fp32.
 *   - Rotated dims are the last rope_dim of the C = 512 channels, in adjacent
 *     pairs (C-rope_dim+2i, C-rope_dim+2i+1) turned by angle pos * inv_freq[i].
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define CSA_OK          0
#define CSA_EINVAL     -1   /* null pointer, bad size, misaligned pointer, topk > capacity ... */
#define CSA_ENOTSUP    -2   /* a dtype or shape combination the library does not implement */
#define CSA_EWORKSPACE -3   /* workspace missing or smaller than *_workspace_bytes() */
#define CSA_EHIP       -4   /* a kernel launch reported a HIP error */

/* Element types of stored caches and outputs. */
#define CSA_BF16      0     /* bfloat16 */
#define CSA_FP8_E4M3  1     /* OCP FP8 E4M3FN codes (max 448, no infinities) with fp32 block scales */
#define CSA_FP32      2     /* output only */
#define CSA_FP4_E2M1  3     /* OCP MXFP4: E2M1 codes, two per byte, with power-of-two fp32 scales per
                               32 channels (compressed KV caches only) */

/*
 * A per-layer cache of rows, one set per sequence.  Used for the compressed
 * KV cache (window 8 / stride 4 for CSA, 128 / 128 for HCA), the indexer key
 * cache (one key per compressed entry) and the raw sliding-window cache
 * (window = stride = 1).
 *
 * Row j of sequence b covers raw positions
 *     [pos0[b] + j*stride, pos0[b] + j*stride + window)
 * and carries the position of its LAST raw token, pos0[b] + j*stride + window - 1:
 * it is rotated at that position and is visible to a query at position p only
 * if that position is <= p (an entry becomes visible when all its tokens are).
 *
 *   data       device [B, cap, C]: bf16 values, or fp8 codes (one byte each), or for
 *              fp4 [B, cap, C/2] bytes holding E2M1 codes, channel 2k in the low
 *              nibble of byte k and 2k+1 in the high nibble.
 *              Stored rows are already rotated (the cache is written after RoPE;
 *              "DeepSeek-V4.1-Flash vs Inkling", partial-RoPE row: the FP4 KV cache
 *              is quantized after RoPE).
 *   scales     device [B, cap, C / scale_block] fp32, fp8 and fp4 caches only (else
 *              NULL).  Value of element c of row j = code * scales[.., j, c / scale_block].
 *              Scales must be >= 0; fp4 caches use scale_block 32 and powers of two
 *              (the MX block scale: 2^(floor(log2 amax) - 2), scale 1 for a zero block).
 *   n_valid    device [B] int32: rows 0 .. n_valid[b]-1 hold data (read side).
 *              Values above cap are treated as cap, negative values as 0.
 *   pos0       device [B] int64.
 */
typedef struct csa_cache {
    void*          data;
    float*         scales;
    const int32_t* n_valid;
    const int64_t* pos0;
    int32_t        dtype;        /* CSA_BF16, CSA_FP8_E4M3 or CSA_FP4_E2M1 */
    int32_t        cap;          /* rows per sequence */
    int32_t        C;            /* channels per row */
    int32_t        scale_block;  /* channels per scale (fp8: any divisor of C; fp4: 32) */
    int32_t        window;       /* raw tokens per row */
    int32_t        stride;       /* raw tokens between consecutive rows */
} csa_cache_t;

/*
 * csa_compress — softmax pooling of raw tokens into cache rows, with RoPE.
 *
 * Source: CSA row (each entry pools 8 overlapping tokens at stride 4 with a
 * softmax taken separately per channel) and HCA row (128 tokens per entry) of
 * "DeepSeek-V4-Pro vs Inkling"; the stored cache holds rotated values
 * ("DeepSeek-V4.1-Flash vs Inkling", partial-RoPE row: quantized after RoPE).
 *
 * For each sequence b, new row j = first_row + i (0 <= i < n_new) and channel c:
 *     a_t     = exp(logits[b, i*stride + t, c]),  t = 0 .. window-1
 *     e[c]    = sum_t a_t * kv[b, i*stride + t, c] / sum_t a_t
 *     row     = rope(e, pos0[b] + j*stride + window - 1)
 * then stored as bf16 (round to nearest even) or, for an fp8 cache, as E4M3FN
 * codes with one scale per scale_block channels: scale = amax / 448 over the
 * block (fp32), code = round-to-nearest-even(e / scale), saturating at 448; a
 * block of zeros stores scale 0 and codes 0.
 *
 *   kv, logits  device bf16; element (b, t, c) at b*ld_seq + t*ld_tok + c.
 *               Raw row 0 of sequence b is the first raw token of new row
 *               first_row.  logits may be NULL when window == 1 (the
 *               raw-window write: each token rotated at its own position).
 *   T_raw       raw rows available per sequence; must be >= (n_new-1)*stride + window.
 *   out         cache written at rows [first_row, first_row + n_new) (<= cap).
 *               out->n_valid is not read or written: the caller keeps counts.
 *   inv_freq    device double[rope_dim/2]; rope_dim even, 0 <= rope_dim <= C.
 * Requires C % 8 == 0, C <= 1024, 16-byte aligned kv/logits/out->data, ld_tok % 8 == 0.
 */
int csa_compress(const void* kv, const void* logits, int64_t ld_tok, int64_t ld_seq,
                 int B, int T_raw, int first_row, int n_new, const csa_cache_t* out,
                 const double* inv_freq, int rope_dim, hipStream_t stream);

/*
 * csa_compress_batch — several csa_compress calls in one go.
 *
 * Source: as csa_compress.  A step of one layer compresses twice from the same
 * raw tokens: the entries its tokens complete (CSA/HCA rows of "DeepSeek-V4-Pro
 * vs Inkling") and the new raw tokens of the sliding window (window == stride
 * == 1).  The result is that of calling csa_compress with the fields of
 * calls[0], calls[1], ... in order; calls must not write the same rows of one
 * cache.  Every call is checked before anything is launched (the first failing
 * call's error is reported, prefixed with its position).  When every call is
 * small (at most 512 rows of rows x sequences, or windows of at least 32
 * tokens) and there are at most 4 of them, they run as a single kernel launch;
 * otherwise each runs as csa_compress would.
 *
 *   calls    host array of n_calls descriptors (read before the call returns).
 */
typedef struct {
  const void* kv;
  const void* logits;
  int64_t ld_tok, ld_seq;
  int B, T_raw, first_row, n_new;
  const csa_cache_t* out;
  const double* inv_freq;
  int rope_dim;
} csa_compress_call_t;

int csa_compress_batch(const csa_compress_call_t* calls, int n_calls, hipStream_t stream);

/*
 * csa_index_topk — lightning-indexer scores and top-k selection.
 *
 * Source: CSA row of "DeepSeek-V4-Pro vs Inkling" (64 indexer heads of dim
 * 128, ReLU scores weighted per head, the top 1,024 entries are kept) and the
 * atlas Raw config fields (index_n_heads, index_head_dim, index_topk).
 *
 * For query (b, t) and entry j of `keys` that is visible to it
 * (j < n_valid[b] and its position <= q_pos[b, t]):
 *     s[j] = sum_h w[b, t, h] * max(0, q_idx[b, t, h, :] . key_j)
 * with key_j the stored bf16 row, or fp8 codes times the row's scale.  The k
 * visible entries with the largest score are written, in ascending index
 * order, to idx_out[b, t, 0 .. k-1]; an exact tie goes to the smaller index.
 * When fewer than k entries are visible, all of them are written and the rest
 * of the row is -1.
 *
 *   q_idx      device bf16 [B, Tq, Hi, Di]     (Di == keys->C == 128)
 *   w          device fp32 [B, Tq, Hi]
 *   q_pos      device int64 [B, Tq]
 *   keys       indexer key cache: bf16, or fp8 with scale_block == C (one scale per key)
 *   topk       1 .. keys->cap, at most 4096
 *   idx_out    device int32 [B, Tq, topk]
 *   scores_out device fp32 [B, Tq, keys->cap] or NULL; invisible entries hold -inf.
 *   workspace  at least csa_index_topk_workspace_bytes(...) bytes, 256-byte aligned:
 *              the scores when scores_out is NULL, and for rows longer than 16384
 *              entries the candidate lists of a two-stage selection (the top k of
 *              each chunk of the row, then the top k of those).
 * Requires 1 <= Hi <= 64, 16-byte aligned q_idx and key rows.
 */
int csa_index_topk(const void* q_idx, const float* w, const int64_t* q_pos,
                   int B, int Tq, int Hi, const csa_cache_t* keys, int topk,
                   int32_t* idx_out, float* scores_out,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t csa_index_topk_workspace_bytes(int B, int Tq, int Hi, int cap, int topk);

/*
 * csa_index_topk_compress — a decode step's compress calls and its indexer / top-k with
 * fewer launches.
 *
 * Same effect as csa_compress_batch(calls, n_calls, stream) followed by csa_index_topk(...)
 * with the remaining arguments (the steps of one CSA layer, "DeepSeek-V4-Pro vs Inkling",
 * Component-by-component table, CSA row).  The compressor writes only the caches named in
 * `calls`, which the indexer does not read, so small calls (a decode step's new entry and
 * raw-window write) run as extra blocks of the indexer's scores launch.  Calls that need
 * the compressor's many-row kernel, or scores taken by the many-query-row kernel (bf16 keys
 * with Tq >= 16), fall back to separate launches with the same result.  The workspace is
 * csa_index_topk's.
 * Errors: as for the two calls (a bad compress call's message starts "call i: "), and
 * CSA_EINVAL when a compress output (cache data or scales) overlaps the indexer's keys,
 * key scales, q_idx, w, scores_out, idx_out or workspace.
 */
int csa_index_topk_compress(const csa_compress_call_t* calls, int n_calls,
                            const void* q_idx, const float* w, const int64_t* q_pos,
                            int B, int Tq, int Hi, const csa_cache_t* keys, int topk,
                            int32_t* idx_out, float* scores_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * csa_attend — shared-KV multi-query attention over the selected entries and
 * the sliding window, with a per-head sink and the output's inverse rotation.
 *
 * Source: CSA row (the query heads attend to the kept entries together with
 * the window tokens), sink row (one logit per head whose exponential joins the
 * denominator only) and partial-RoPE row (an entry is key and value at once;
 * the rotated dims of each head's output are turned back by the query
 * position) of "DeepSeek-V4-Pro vs Inkling"; atlas Raw config fields
 * (head_dim 512, one KV head, sliding_window 128).
 *
 * For query (b, t) at position p = q_pos[b, t] and each head h:
 *     U   = { kv rows idx[b, t, u] : 0 <= u < topk, 0 <= idx < n_valid }
 *           plus the window rows of `win` whose position lies in (p - W, p]
 *           (a plain union; an entry and a window token are distinct members)
 *     l_x = softmax_scale * rope(q[b, t, h], p) . x
 *     Z   = exp(sink[h]) + sum_{x in U} exp(l_x)
 *     out = rope(sum_x exp(l_x) / Z * x, -p),   lse = log Z
 *
 *   q          device bf16 [B, Tq, H, 512], un-rotated
 *   kv         compressed KV cache (C == 512): bf16, fp8 with scale_block a multiple of 64
 *              (the codes enter both products exactly; the block scales are applied in fp32),
 *              or fp4 (scale_block 32)
 *   idx        device int32 [B, Tq, topk] (-1 = unused slot), e.g. from csa_index_topk
 *   win        raw-window cache (window = stride = 1, C == 512, bf16, rotated rows)
 *   W          window length in raw tokens (>= 0)
 *   sink       device fp32 [H]
 *   out        device [B, Tq, H, 512], out_dtype CSA_FP32 or CSA_BF16
 *   lse_out    device fp32 [B, Tq, H] or NULL
 *   workspace  at least csa_attend_workspace_bytes(...) bytes, 256-byte aligned
 * Requires 1 <= H <= 1024, 0 <= topk <= kv->cap, 16-byte aligned q/out/kv rows.
 */
int csa_attend(const void* q, const int64_t* q_pos, int B, int Tq, int H,
               const csa_cache_t* kv, const int32_t* idx, int topk,
               const csa_cache_t* win, int W, const float* sink,
               const double* inv_freq, int rope_dim, float softmax_scale,
               void* out, int out_dtype, float* lse_out,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t csa_attend_workspace_bytes(int B, int Tq, int H, int topk, int W);

/*
 * csa_attend_noalloc — csa_attend for callers that cannot allocate a workspace.
 *
 * For code that must not allocate device memory: work captured into a HIP graph, tight serving
 * loops, harnesses that forbid it.  Same arguments and result as csa_attend, without the
 * workspace: the split partials live in a scratch array inside the library, one per GPU, of
 * CSA_NOALLOC_SCRATCH_BYTES bytes, held from the first call on that GPU (with that GPU current)
 * until the process ends.  Nothing is allocated or freed by the call.
 *   - CSA_EWORKSPACE when the call needs more scratch than that (csa_attend_workspace_bytes of
 *     the same arguments is larger), checked on the host before anything is launched;
 *   - every call on one GPU shares that GPU's array, which keeps the last call's contents:
 *     calls that overlap on one GPU (other streams, or graph replays in flight together) race
 *     and must be serialised by the caller;
 *   - the array is located on the current device: the stream must belong to it.
 */
#define CSA_NOALLOC_SCRATCH_BYTES (32u << 20)

int csa_attend_noalloc(const void* q, const int64_t* q_pos, int B, int Tq, int H,
                       const csa_cache_t* kv, const int32_t* idx, int topk,
                       const csa_cache_t* win, int W, const float* sink,
                       const double* inv_freq, int rope_dim, float softmax_scale,
                       void* out, int out_dtype, float* lse_out, hipStream_t stream);

/*
 * hca_attend — as csa_attend, with U = every kv row visible to the query
 * (j < n_valid[b] and position <= p) plus the window rows.
 *
 * Source: HCA row of "DeepSeek-V4-Pro vs Inkling" (dense shared-KV attention
 * over all compressed entries plus a 128-token window) and the sink and
 * partial-RoPE rows.
 */
int hca_attend(const void* q, const int64_t* q_pos, int B, int Tq, int H,
               const csa_cache_t* kv, const csa_cache_t* win, int W, const float* sink,
               const double* inv_freq, int rope_dim, float softmax_scale,
               void* out, int out_dtype, float* lse_out,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t hca_attend_workspace_bytes(int B, int Tq, int H, int cap, int W);

/*
 * csa_out_proj — grouped low-rank output projection of the attention output.
 *
 * Source: "DeepSeek-V4-Pro" model atlas, Raw config fields o_groups (16), o_lora_rank (1024) and
 * hidden_size (7168); the fields alone are given, and the plainest reading they support is taken:
 * the H heads' outputs (after the inverse rotation, as csa_attend / hca_attend write them) form G
 * groups of H / G consecutive heads; group g's (H / G) * D values go through its own down factor,
 * the G * R codes, concatenated in group order, through one up factor:
 *     z[t, g, r] = sum_k o[t, g (H / G) D + k] * wa[g, r, k]        (k < (H / G) D)
 *     y[t, j]    = sum_{g, r} z[t, g, r] * wb[j, g R + r]
 *
 *   o          device [T, H, D], o_dtype CSA_FP32 or CSA_BF16 (16-byte aligned)
 *   wa         device bf16 [G, R, (H / G) D] (each code's weights contiguous; 16-byte aligned)
 *   wb         device bf16 [hidden, G R] (each output's weights contiguous; 16-byte aligned)
 *   y          device [T, hidden], y_dtype CSA_FP32 or CSA_BF16 (16-byte aligned)
 *   workspace  at least csa_out_proj_workspace_bytes(T, G, R, hidden) bytes (the fp32 codes z and
 *              the second product's partial sums), 256-byte aligned; its contents need not be kept
 *              between calls
 * Products of fp32 inputs (o, and the codes z) enter as bf16 hi + lo parts (about 16 bits);
 * sums are fp32 in a fixed order (results are deterministic).  Requires H a multiple of G,
 * (H / G) D a multiple of 32, R a multiple of 64, hidden a multiple of 32 (CSA_ENOTSUP otherwise).
 * T = 0 is a no-op.  Errors as for the other calls; nothing is launched on failure.
 */
int csa_out_proj(const void* o, int o_dtype, int T, int H, int D, int G,
                 const void* wa, int R, const void* wb, int hidden,
                 void* y, int y_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t csa_out_proj_workspace_bytes(int T, int G, int R, int hidden);

/* Thread-local description of the last failure (empty string after success). */
const char* csa_last_error(void);

/* ABI version of this library. */
int csa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
