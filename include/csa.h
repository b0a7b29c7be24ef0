/*
 * csa.h - C ABI of the CSA / HCA attention hot path (DeepSeek-V4 compressed sparse
 * attention) for AMD Instinct MI355X (gfx950).
 *
 * Five stages, each one asynchronous call on a caller-given HIP stream:
 *   csa_compress     overlapping (CSA) or single-stream (HCA) block compressor
 *   csa_index_score  lightning-indexer scores under causal block visibility
 *   csa_topk         per-query top-k selection of compressed entries
 *   csa_sparse_attn  shared-KV MQA over [SWA window || selected entries || sink]
 *   hca_dense_attn   shared-KV MQA over [SWA window || every visible entry || sink]
 *
 * Sources (web pages, cited by title and section):
 *   [HCA-CSA]  zdszero.github.io "hca_csa"
 *   [KV-COMP]  jerry609.github.io "DeepSeek-V4 的 KV 压缩：从删 token 误解到预算检索"
 *   [V4-CSA2]  yuyanqi.com "DeepSeek-V4 CSA/HCA 与 DeepSeek-V4.1 CSA2"
 *   [ATTN-CMP] blog.javazero.top "DeepSeek 注意力结构对比"
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller; tensors are dense
 *     row-major in the shape given.  Inputs and outputs must not alias.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     only enqueue work; they never synchronise and never allocate device memory.
 *     Scratch memory comes from the caller's `ws` buffer, sized by the matching
 *     *_workspace_size() query and 16-byte aligned (hipMalloc gives 256); ws may
 *     be NULL when that size is 0.
 *   - The library keeps no state between calls: calls on different streams with
 *     different buffers may run concurrently.  Two calls that share a workspace
 *     buffer must be ordered by the caller.
 *   - Return value: CSA_OK when the work was enqueued.  Argument errors are
 *     detected before anything is launched (CSA_ERR_INVALID_ARG for bad values,
 *     CSA_ERR_UNSUPPORTED for a valid shape the library has no kernel for,
 *     CSA_ERR_WORKSPACE when ws_bytes is too small); CSA_ERR_HIP reports a
 *     launch failure from the HIP runtime.  Errors that happen while kernels run
 *     surface at the caller's next synchronisation, as for any HIP kernel.
 *   - bf16 = bfloat16 bit patterns (uint16); fp8 = OCP e4m3fn codes (uint8) with an
 *     fp32 scale per row (real value = decode(code) * scale).
 */
#ifndef CSA_MI355X_H
#define CSA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1,
  CSA_ERR_UNSUPPORTED = 2,
  CSA_ERR_WORKSPACE = 3,
  CSA_ERR_HIP = 4,
  CSA_ERR_SCRATCH = 5
} csa_status;

/* Element types.  CSA_FP4_E2M1 as a compressor output means MXFP4 rows (E2M1 codes, two per
 * byte with the even channel in the low nibble, and one E8M0 scale byte per 32 channels);
 * CSA_PACKED_FP4_E4M3 and CSA_PACKED_FP8_ROPE are compressor outputs only: the packed
 * main-KV rows that the attention calls read with kv_format CSA_KV_FP4_E4M3 and
 * CSA_KV_FP8_ROPE_BF16 (csa_kv_format below). */
typedef enum {
  CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3 = 2, CSA_FP4_E2M1 = 3,
  CSA_PACKED_FP4_E4M3 = 4, CSA_PACKED_FP8_ROPE = 5
} csa_dtype;

/* Cache layouts of compressed entries: row-major [B, Nc, c], or (indexer keys, c = 128,
 * FP8 codes) the 16-entry blocks of csa_index_keys_b16. */
typedef enum { CSA_LAYOUT_ROWS = 0, CSA_LAYOUT_B16 = 1 } csa_layout;

/* Storage formats of the compressed main-KV cache read by the attention calls (c = 512,
 * one row per entry, rows of one batch element contiguous, [B, Nc, row bytes]):
 *   CSA_KV_BF16           the row as c bf16 values (1024 bytes).
 *   CSA_KV_FP4_E4M3       [V4-CSA2] section 16.1, [ATTN-CMP] section on CSA2: 512 E2M1
 *                         codes, two per byte with the even channel in the low nibble
 *                         (bytes 0..255), then one E4M3 scale per 16 channels (bytes
 *                         256..287); channel i = E2M1(code i) * E4M3(scale i/16).  288 bytes.
 *   CSA_KV_FP8_ROPE_BF16  [ATTN-CMP] section "CSA（DeepSeek-V4）": the 448 channels without
 *                         RoPE as e4m3 codes (bytes 0..447) times one power-of-two scale
 *                         2^(e - 127) per row, e = byte 576 (E8M0); the 64 RoPE channels as
 *                         bf16 (bytes 448..575); bytes 577..583 unused.  584 bytes.
 * Every value of these formats is a bf16 number, so the attention reads them exactly. */
typedef enum { CSA_KV_BF16 = 0, CSA_KV_FP4_E4M3 = 1, CSA_KV_FP8_ROPE_BF16 = 2 } csa_kv_format;

/* Human-readable name of a status code (static string, never NULL). */
const char* csa_status_string(int status);

/* ABI version: 10000 * major + 100 * minor + patch. */
int csa_version(void);

/* ------------------------------------------------------------------------------
 * Stage 1: block compressor.
 * [HCA-CSA] "CSA 的重叠窗口" (overlapping window) and "HCA：同一个算子，关掉重叠"
 * (single stream); [KV-COMP] section 9.2 (learned gated pooling).
 *
 * Every token h_t of the chunk is projected to contents C and gate logits Z.
 * Entry i of the chunk is, channel by channel, a softmax-weighted sum over its
 * slots: with overlap the m a-slots of block i (logit Z^a + B^a, value C^a) and the
 * m b-slots of block i-1 (logit Z^b + B^b, value C^b); without overlap the m slots
 * of block i.  The pooled vector u_i goes through RMSNorm (unit gain) and RoPE on
 * its last d_rope channels at position p0 + m*i (the block's first token):
 *     out_i = RoPE(u_i / sqrt(mean(u_i^2) + rms_eps)).
 *
 *   hidden      [B, T, d]  in_dtype (CSA_F32 or CSA_BF16): tokens at positions p0 .. p0+T-1
 *   hidden_prev [B, m, d]  in_dtype: the m tokens before p0 (only their b-stream is used,
 *               for entry 0); NULL means there is no previous block: entry 0's b-slots
 *               are padding (logit -inf, content 0).  overlap=1 with p0 > 0 requires it.
 *   w_proj      [S*c, d]   in_dtype, "out x in" layout (proj = hidden @ w_proj^T):
 *               overlap=1: S = 4 stream blocks (C^a | Z^a | C^b | Z^b);
 *               overlap=0: S = 2 (C | Z).
 *   bias        [S/2, m, c] fp32 position bias: (B^a, B^b) or (B).
 *   Requires T % m == 0, p0 % m == 0, p0 >= 0, 0 <= d_rope <= c, d_rope and c even,
 *   c <= 1024.
 *   out         [B, T/m, c]  out_dtype: CSA_F32 or CSA_BF16 (RNE), or CSA_FP8_E4M3 codes
 *               with out_scale [B, T/m] fp32 = amax/448 of the row (RNE, saturating;
 *               an all-zero row gets scale 0 and zero codes).  Low-precision caches:
 *               CSA_FP4_E2M1: MXFP4 codes [B, T/m, c/2] with out_scale taken as uint8
 *               E8M0 bytes [B, T/m, c/32] (block exponent floor(log2 amax) - 2, clamped to
 *               [-127, 127]; values to the nearest E2M1, ties to even, saturating; c % 32
 *               == 0);  CSA_PACKED_FP4_E4M3 / CSA_PACKED_FP8_ROPE (c = 512; the FP8 one
 *               with d_rope = 64): packed rows [B, T/m, 288] / [B, T/m, 584] as described
 *               under csa_kv_format (E4M3 scale = amax/6 per 16 channels, RNE; FP8 row
 *               exponent e = ceil(log2(amax/448)) over the 448 channels without RoPE, the
 *               RoPE channels in bf16, RNE).  out_scale is ignored for the types without
 *               a separate scale.
 *   out_layout  CSA_LAYOUT_ROWS: out as above (the chunk's entries only; Nc_max unused).
 *               CSA_LAYOUT_B16 (CSA_FP8_E4M3 with c = 128): out is the sequence caches of
 *               Nc_max entries in the 16-entry blocks of csa_index_keys_b16
 *               (csa_index_keys_b16_size(B, Nc_max) bytes) and out_scale [B, Nc_max]; entry i
 *               of the chunk is cache entry p0/m + i (p0/m + T/m <= Nc_max); other entries
 *               are left as they are.  The bytes equal csa_index_keys_b16 of the rows.
 *   ws          >= csa_compress_workspace_size(...) bytes (the projection, or for bf16
 *               inputs with overlap and m = 4 the pooled vectors, which need less).
 * The bf16 overlapping compressor with m = 4 and c % 64 == 0 runs the projection and the
 * pooling in one kernel; other shapes project first, then pool.  Results agree within
 * fp32 rounding order.
 * ------------------------------------------------------------------------------ */
size_t csa_compress_workspace_size(int B, int T, int m, int c, int overlap, int has_prev);

int csa_compress(const void* hidden, const void* hidden_prev, int in_dtype,
                 const void* w_proj, const float* bias, int overlap,
                 int B, int T, int d, int m, int c, int d_rope, float rope_theta,
                 float rms_eps, int64_t p0,
                 void* out, float* out_scale, int out_dtype, int out_layout, int Nc_max,
                 void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * Stage 1, CSA2 form (DeepSeek-V4.1): main KV entries and the indexer keys derived from
 * them.  [V4-CSA2] sections 6.1, 7.2 (one KV projection and one gate; each entry pools only
 * its own m-token block, per channel a softmax over the block's gate values, no position
 * bias), 7.5 and 15.1 (ratio 1: no gate, the entry is the normalised projection), 6.2 (the
 * indexer key is a projection of the main latent) and 7.4 (RoPE at the block's first
 * token); [ATTN-CMP] section on CSA2 (wk applied to the latent before RoPE, then k_norm and
 * RoPE with the indexer's own theta).
 *
 *   latent_i = RMSNorm(sum_r softmax_r(Z_r) * C_r)   (ratio 1: RMSNorm(C_i))
 *   kv_i     = RoPE(latent_i) at position p0 + m*i, theta_kv, last d_rope channels
 *   kI_i     = RoPE(RMSNorm(latent_i . W_k^T)) at the same position, theta_k, last d_rope
 * RMSNorm has unit gain and rms_eps.
 *
 *   hidden [B, T, d] in_dtype (CSA_F32 or CSA_BF16 with d % 64 == 0, c % 8 == 0), positions
 *          p0 .. p0+T-1;  T % m == 0, p0 % m == 0.
 *   w_proj [S*c, d] in_dtype ("out x in"): S = 2 (C | Z) for m > 1, S = 1 (C) for m = 1.
 *   w_k    [d_I, c] in_dtype ("out x in"), 16-byte aligned;  c <= 1024, d_I <= 256, even;
 *          d_rope even, <= c and <= d_I.
 *   kv_out [B, T/m, c] and k_out [B, T/m, d_I] in CSA_F32, CSA_BF16 or CSA_FP8_E4M3 (with
 *          kv_scale / k_scale [B, T/m] = amax/448 of the row), or in the low-precision
 *          types of csa_compress: CSA_FP4_E2M1 (MXFP4, scales as E8M0 bytes through
 *          kv_scale / k_scale) for either, CSA_PACKED_FP4_E4M3 or CSA_PACKED_FP8_ROPE
 *          (c = 512; d_rope = 64 for the FP8 one) for kv_out.
 *   ws     >= csa2_compress_workspace_size(B, T, m, c) bytes (the projection).
 * ------------------------------------------------------------------------------ */
size_t csa2_compress_workspace_size(int B, int T, int m, int c);

int csa2_compress(const void* hidden, int in_dtype, const void* w_proj, const void* w_k, int B, int T, int d,
                  int m, int c, int d_I, int d_rope, float theta_kv, float theta_k, float rms_eps,
                  int64_t p0, void* kv_out, float* kv_scale, int kv_dtype, void* k_out, float* k_scale,
                  int k_dtype, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * Stage 1, decode form: one new token per sequence.
 * [HCA-CSA] "KV cache：成品与原料" (an FP32 ring of the (C, Z) projections of the last 2m
 * tokens for CSA, m for HCA; an entry is produced only by the token that completes its
 * block; the HCA online state keeps one running (max, sum, weighted sum) per channel) and
 * "在 SGLang 里的落点" (the CSA emission reads the current and the previous block's slots);
 * [KV-COMP] section 9.3 (state until the block boundary, then one entry into the cache).
 *
 * For every sequence b, with t = pos[b] the position of its new token hidden[b]:
 *   1. the token's projection (C^a, Z^a, C^b, Z^b) (overlap = 1) or (C, Z) (overlap = 0)
 *      = w_proj . hidden[b] enters ring slot t mod 2m (overlap) or t mod m; with online = 1
 *      (requires overlap = 0) it updates the running triple instead;
 *   2. when emit != 0 and (t + 1) % m == 0, entry i = t / m is written to cache row i of
 *      sequence b, exactly as csa_compress computes it over the block's tokens (entry 0
 *      without a previous block: b-slots padded), i.e. RoPE(RMSNorm(pooled)) at position
 *      m*i.  Rows i >= Nc_max are not written.  emit = 0 only fills the state (to prime
 *      the ring with the last block of a prefill chunk before the first decode step).
 *   Sequences with pos[b] < 0 are skipped.
 * The state is valid for the entry of block i once the steps of block i (and, with
 * overlap, block i-1) have run on it; the online triple restarts at each block's first
 * token.  Nothing in it needs initialising.
 *
 *   hidden  [B, d] in_dtype (CSA_F32, or CSA_BF16 with d % 128 == 0)
 *   w_proj, bias, m, c, d_rope, rope_theta, rms_eps: as csa_compress
 *   pos     [B] int64 (device);  state: >= csa_compress_state_size(B, m, c, overlap, online)
 *           bytes, fp32, 16-byte aligned, one share per sequence, kept by the caller across
 *           calls.
 *   cache   CSA_LAYOUT_ROWS: [B, Nc_max, c] in out_dtype (CSA_F32, CSA_BF16, or
 *           CSA_FP8_E4M3 codes with cache_scale [B, Nc_max] = amax/448), or one of the
 *           low-precision types of csa_compress (CSA_FP4_E2M1 with E8M0 bytes
 *           [B, Nc_max, c/32] through cache_scale; packed rows [B, Nc_max, 288 / 584]);
 *           CSA_LAYOUT_B16: FP8 codes of c = 128 in 16-entry blocks
 *           (csa_index_keys_b16_size(B, Nc_max) bytes) + cache_scale [B, Nc_max].
 *   ws      >= csa_compress_decode_workspace_size(B, d, c, overlap, in_dtype) bytes (the projection
 *           of the B tokens, in partial sums over slices of the d inputs).
 * ------------------------------------------------------------------------------ */
size_t csa_compress_state_size(int B, int m, int c, int overlap, int online);
size_t csa_compress_decode_workspace_size(int B, int d, int c, int overlap, int in_dtype);

int csa_compress_decode(const void* hidden, int in_dtype, const void* w_proj, const float* bias,
                        int overlap, int online, int B, int d, int m, int c, int d_rope,
                        float rope_theta, float rms_eps, const int64_t* pos, int emit, float* state,
                        void* cache, float* cache_scale, int out_dtype, int out_layout, int Nc_max,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * The decode step of several compressors that read the same new tokens: a CSA layer's
 * main KV compressor and its indexer-key compressor, which both compress the layer's
 * hidden states ([HCA-CSA] "CSA：轻压缩 + 稀疏选择"; [KV-COMP] section 9.3).  The result
 * is exactly that of csa_compress_decode called once per compressor, in order, with the
 * same hidden, in_dtype, B, d, pos and emit; with bf16 inputs the compressors share one
 * projection launch and one step launch.
 *
 *   comps   n (1 or 2) compressors in host memory, read during the call.  Each holds the
 *           per-compressor arguments of csa_compress_decode, with the same meaning, layout
 *           and constraints.  The compressors' state, cache and cache_scale buffers must
 *           not overlap one another.
 *   ws      >= csa_compress_decode_many_workspace_size(B, d, in_dtype, n, comps) bytes,
 *           16-byte aligned (the projections of the B tokens for every compressor).
 * The arguments of every compressor are checked before anything is enqueued; the first
 * error found is returned.
 * ------------------------------------------------------------------------------ */
typedef struct csa_decode_compressor {
  const void* w_proj;
  const float* bias;
  int overlap, online, m, c, d_rope;
  float rope_theta, rms_eps;
  float* state;
  void* cache;
  float* cache_scale;
  int out_dtype, out_layout, Nc_max;
} csa_decode_compressor;

size_t csa_compress_decode_many_workspace_size(int B, int d, int in_dtype, int n,
                                               const csa_decode_compressor* comps);
int csa_compress_decode_many(const void* hidden, int in_dtype, int B, int d, const int64_t* pos,
                             int emit, int n, const csa_decode_compressor* comps, void* ws,
                             size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * Stage 2: lightning-indexer scores.
 * [HCA-CSA] "CSA：轻压缩 + 稀疏选择" (indexer equations); [KV-COMP] sections 9.4, 9.8.
 *
 *   scores[b,s,j] = sum_h w[b,s,h] * ReLU(qI[b,s,h,:] . KI[b,j,:])   for j < n_vis(b,s)
 *                 = -inf                                              otherwise,
 *   n_vis(b,s) = min(Nc, floor((q_pos[b,s] + 1) / m))  (entry j ends at token m*j+m-1).
 * No softmax and no 1/sqrt(d_I) factor.
 *
 * dtype CSA_FP8_E4M3: q [B,S,H_I,d_I] and k [B,Nc,d_I] are e4m3fn codes, q_scale
 *   [B,S,H_I] and k_scale [B,Nc] their per-row fp32 scales, which must be finite and
 *   >= 0 (amax/448 by construction).  Kernels for H_I = 64, d_I = 128.
 * dtype CSA_F32: q, k are fp32; q_scale and k_scale must be NULL.  Any H_I <= 64,
 *   d_I <= 256.
 *   w      [B,S,H_I] fp32 head weights;  q_pos [B,S] int64 absolute positions (>= 0).
 *   scores [B,S,Nc] fp32 output.
 * ------------------------------------------------------------------------------ */
int csa_index_score(const void* q, const float* q_scale, const float* w,
                    const void* k, const float* k_scale, int dtype,
                    const int64_t* q_pos, int B, int S, int H_I, int d_I, int Nc, int m,
                    float* scores, void* stream);

/* ------------------------------------------------------------------------------
 * Stages 2 and 3 in one call (FP8 inputs, H_I = 64, d_I = 128): the index scores of
 * csa_index_score and the selection of csa_topk, identical results.  For decode shapes
 * (S <= 4 and G = ceil(Nc / 4096) segments whose G*k candidates merge in one or two
 * levels, below) the scoring pass also selects the top-k of each 4096-entry segment while
 * the scores are in registers, and the merge passes finish the rows ([KV-COMP] section
 * 9.4: the union of segment top-k sets holds the row's top-k); other shapes run the two
 * stages back to back.
 *   Arguments as csa_index_score and csa_topk (k = top-k, 1 <= k <= 2048);
 *   scores [B,S,Nc] fp32 or NULL (then not written, except in the workspace);
 *   idx [B,S,k] int32 output;
 *   ws >= csa_index_topk_workspace_size(B, S, Nc, k) bytes (required, never NULL).
 * ------------------------------------------------------------------------------ */
size_t csa_index_topk_workspace_size(int B, int S, int Nc, int k);

int csa_index_topk(const void* q, const float* q_scale, const float* w,
                   const void* k_codes, const float* k_scale, const int64_t* q_pos,
                   int B, int S, int H_I, int d_I, int Nc, int m, int k,
                   float* scores, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * The fused path of csa_index_topk as two calls (decode shapes only: S <= 4, FP8,
 * H_I = 64, d_I = 128, and G = ceil(Nc / 4096) segment lists of k candidates that merge
 * in one level (G*k <= 36864) or in two (groups of M = clamp(round(sqrt(G)), 2,
 * floor(36864 / k)) lists first, then ceil(G / M) * k <= 36864 pairs); other shapes
 * return CSA_ERR_UNSUPPORTED).  [KV-COMP] section 9.4: the row's top-k lies in the union
 * of the top-k sets of its segments (and of groups of segments).
 *
 * csa_index_score_segments: the scores of csa_index_score (written when `scores` is not
 *   NULL) and, for every 4096-entry segment g of row r, the k best entries of the
 *   segment as pairs (key, entry) of two uint32: key = an order-preserving image of the
 *   score (0 = empty slot: fewer than k candidates), entries in ascending order.  cand:
 *   caller device memory of at least csa_index_segments_size(B, S, Nc, k) bytes,
 *   16-byte aligned, one equal share per row r = b*S + s; pair j of segment g is
 *   element g*k + j of row r's share (with one merge level the shares are exactly G*k
 *   pairs: cand[r][g][j]).
 * csa_topk_merge: idx [B,S,k] = the k best candidates of each row (key descending, then
 *   lower entry), ascending, padded with -1: exactly csa_topk of the same scores.  cand is
 *   read and, with two levels, also written: the first level's pairs go into the rest of
 *   each row's share (the segment pairs stay intact), so cand is not const and must not be
 *   shared with a concurrent call.  cand_bytes < csa_index_segments_size(B, S, Nc, k):
 *   CSA_ERR_WORKSPACE.
 * ------------------------------------------------------------------------------ */
size_t csa_index_segments_size(int B, int S, int Nc, int k);

int csa_index_score_segments(const void* q, const float* q_scale, const float* w,
                             const void* k_codes, const float* k_scale, const int64_t* q_pos,
                             int B, int S, int H_I, int d_I, int Nc, int m, int k,
                             float* scores, void* cand, size_t cand_bytes, void* stream);

int csa_topk_merge(void* cand, size_t cand_bytes, int B, int S, int Nc, int k, int32_t* idx, void* stream);

/* ------------------------------------------------------------------------------
 * The indexer keys in 16-entry blocks (decode scoring).  Same codes, another order:
 * block j of sequence b holds entries 16j .. 16j+15 as four 512-byte pieces, piece p
 * holding bytes 32p .. 32p+31 of each of the 16 entries in entry order (32 bytes per
 * entry), so that the 16 lanes of a quarter-wave that feed one matrix step read 512
 * contiguous bytes.  Entries past Nc in the last block are zero.
 *
 * csa_index_keys_b16_size: bytes of the blocked copy, B * ceil(Nc/16) * 2048 (0 on bad
 *   arguments).
 * csa_index_keys_b16: k_blocks = the blocked copy of k_codes [B,Nc,128] (e4m3 codes); both
 *   caller device memory, 16-byte aligned, not overlapping.  The copy is made once per key
 *   cache update, not per step.
 * csa_index_score_segments_b16: csa_index_score_segments with the keys in blocks
 *   (k_blocks as written by csa_index_keys_b16 for the same B and Nc; k_scale unchanged);
 *   the scores and candidate pairs are identical to csa_index_score_segments'.
 * ------------------------------------------------------------------------------ */
size_t csa_index_keys_b16_size(int B, int Nc);

int csa_index_keys_b16(const void* k_codes, void* k_blocks, int B, int Nc, void* stream);

int csa_index_score_segments_b16(const void* q, const float* q_scale, const float* w,
                                 const void* k_blocks, const float* k_scale, const int64_t* q_pos,
                                 int B, int S, int H_I, int d_I, int Nc, int m, int k,
                                 float* scores, void* cand, size_t cand_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * Index scores over microscaled caches ([V4-CSA2] sections 16.2 and 11.2: indexer keys of
 * 128 FP4 E2M1 values with one E8M0 scale per 32, 68 bytes; [ATTN-CMP] section on CSA2: the
 * indexer query in FP4 too; [KV-COMP] section 7: scores cast from FP32 to BF16 before the
 * top-k).  The score is csa_index_score's over the dequantised values,
 *   I[b,s,j] = sum_h w[b,s,h] * ReLU(q[b,s,h] . K[b,j])   (j < n_vis, else -inf),
 * each value being code * 2^(scale byte - 127) of its block of 32.
 *   elem_dtype CSA_FP4_E2M1: q [B,S,64,64] bytes (two codes per byte, the even value in the
 *     low nibble), k [B,Nc,64] bytes; CSA_FP8_E4M3: q [B,S,64,128], k [B,Nc,128] codes.
 *   q_scale [B,S,64,4], k_scale [B,Nc,4]: E8M0 bytes (block j = values 32j .. 32j+31).
 *   H_I = 64, d_I = 128.  FP4 block sums are exact in the matrix unit (products are
 *   multiples of 1/4); FP8 ones are not, so the FP8 form misses the 1e-5 bound of the
 *   e4m3 path of csa_index_score (kept for measuring that difference).
 *   score_bf16 != 0: every score is rounded to bf16 (RNE) before it is written or selected.
 *   cand NULL: scores [B,S,Nc] fp32 (required), any S.  cand not NULL: decode shapes as
 *   csa_index_score_segments (segment top-k pairs for csa_topk_merge /
 *   csa_topk_sparse_attn, >= csa_index_segments_size(B, S, Nc, k_top) bytes), scores
 *   optional.
 * ------------------------------------------------------------------------------ */
int csa_index_score_mx(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale,
                       int elem_dtype, const int64_t* q_pos, int B, int S, int H_I, int d_I, int Nc, int m,
                       int score_bf16, float* scores, int k_top, void* cand, size_t cand_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * The CSA2 hierarchical indexer ([V4-CSA2] section 11): the Full layer scores every entry,
 * keeps its own top-k, and scores blocks of 8 consecutive entries by their best entry; the
 * 2048 best blocks form a candidate pool of at most 16384 positions (11.1: a recall set
 * larger than top-k, so deeper layers can choose differently); each Reindex layer gathers
 * the pool's keys and scores them with its own query (gather, then score: sections 11 and
 * 15.2), and takes its own top-k.
 *
 * csa_index_score_segments_bmax: csa_index_score_segments (k_layout CSA_LAYOUT_ROWS, keys
 *   [B,Nc,128]) or csa_index_score_segments_b16 (CSA_LAYOUT_B16), the same scores and
 *   candidate pairs, and block_max [B,S,ceil(Nc/8)] fp32: the largest score of entries
 *   8j .. 8j+7 that the query sees, -inf for a block with none.  The pool's blocks are then
 *   csa_topk(block_max, k = n_blocks) (ascending block indices, -1 padded).
 * csa_index_score_pool: for the pool of blocks [B,S,n_blocks] int32 (block j = entries
 *   8j .. 8j+7; -1 = none) the pool's 8*n_blocks entries, pool entry e being position
 *   8*blocks[e/8] + e%8, scored as csa_index_score scores that position (-inf for no
 *   position or one the query does not see); scores [B,S,8*n_blocks] (pool order) or NULL;
 *   cand: the pairs of csa_index_score_segments for a row of 8*n_blocks entries, each pair
 *   carrying the POSITION (>= csa_index_pool_segments_size(B, S, n_blocks, k) bytes).
 *   csa_topk_merge(cand, ..., Nc = 8*n_blocks, k) then gives the Reindex layer's top-k as
 *   positions, ascending (ties to the lower position when the blocks are ascending).
 *   Keys row-major [B,Nc,128] FP8; decode shapes as csa_index_score_segments.
 * ------------------------------------------------------------------------------ */
int csa_index_score_segments_bmax(const void* q, const float* q_scale, const float* w, const void* k_keys,
                                  int k_layout, const float* k_scale, const int64_t* q_pos,
                                  int B, int S, int H_I, int d_I, int Nc, int m, int k,
                                  float* scores, void* cand, size_t cand_bytes, float* block_max,
                                  void* stream);

size_t csa_index_pool_segments_size(int B, int S, int n_blocks, int k);

int csa_index_score_pool(const void* q, const float* q_scale, const float* w, const void* k_codes,
                         const float* k_scale, const int64_t* q_pos, const int32_t* blocks,
                         int n_blocks, int B, int S, int H_I, int d_I, int Nc, int m, int k,
                         float* scores, void* cand, size_t cand_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * Stage 3: top-k selection.  [KV-COMP] sections 9.4 (S_t = TopK_k of the scores)
 * and 9.8 (invisible entries carry -inf and come out as -1).
 *
 *   scores [rows = B*S, Nc] fp32.  Candidates are the entries whose score is not
 *   -inf and not NaN (+0 and -0 compare equal).  Each row gets the indices of its
 *   min(k, n_cand) largest candidate scores, ties going to the lower index, written
 *   in ascending index order and padded with -1:  idx [rows, k] int32.
 *   1 <= k <= 2048.
 *   ws: NULL, or >= csa_topk_workspace_size(rows, Nc, k) bytes.  With ws, rows that
 *   are few or long are split over several workgroups; without it every row is
 *   handled by one workgroup, which holds at most 36864 scores (longer rows without
 *   ws: CSA_ERR_WORKSPACE).  The result is the same either way.  Rows longer than
 *   36864 * floor(36864 / k) entries: CSA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------------ */
size_t csa_topk_workspace_size(int rows, int Nc, int k);

int csa_topk(const float* scores, int B, int S, int Nc, int k, int32_t* idx,
             void* ws, size_t ws_bytes, void* stream);

/* csa_topk with the schedule forced: algo 0 = automatic, 1 = one workgroup per row,
 * 2 = several workgroups per row (needs ws).  For tuning and tests; same result. */
int csa_topk_algo(const float* scores, int B, int S, int Nc, int k, int32_t* idx,
                  void* ws, size_t ws_bytes, int algo, void* stream);

/* ------------------------------------------------------------------------------
 * Stage 4a: CSA core attention.  [HCA-CSA] "设计：近处看原文，远处看摘要" (one softmax
 * over [q K^swa || q K^comp || s_h], values [V^swa || V^comp || 0], K = V shared by
 * all heads); [KV-COMP] sections 9.5-9.6 (window indices concatenated with the
 * selected compressed indices).
 *
 * For query (b,s) and head h, with E = its window rows followed by the rows
 * kv_comp[b, j] for every j in idx[b,s,:] that is not -1:
 *     l_e = scale * (q[b,s,h,:] . kv_e)
 *     M   = max(sink[h], max_e l_e),  den = exp(sink[h] - M) + sum_e exp(l_e - M)
 *     out[b,s,h,:] = sum_e exp(l_e - M) * kv_e / den,   lse[b,s,h] = M + log(den).
 * The sink enters the denominator only (unscaled).
 *
 *   q      [B,S,H,c]   dtype (CSA_BF16: H = 64, c = 512;  CSA_F32: H <= 64, c <= 512)
 *   kv_comp[B,Nc,c]    dtype, when kv_format = CSA_KV_BF16; with dtype CSA_BF16 it may also
 *          be a cache of kv_format CSA_KV_FP4_E4M3 or CSA_KV_FP8_ROPE_BF16 (see csa_kv_format;
 *          16-byte aligned), read and decoded in the kernel: the result equals the call on
 *          the decoded bf16 rows.  Another format with CSA_F32: CSA_ERR_UNSUPPORTED.
 *   idx    [B,S,k] int32 in [-1, Nc), no duplicates.
 *   q_pos  [B,S] int64 positions (consecutive within a sequence), or NULL.  Only the
 *          window uses it: row r of swa holds position q_pos[b,S-1] - Ls + 1 + r, and
 *          rows of negative positions (a sequence shorter than Ls) are left out.  NULL:
 *          every row of swa is a real position.
 *   swa    [B,Ls,c]    dtype: raw KV of the Ls positions ending at the last query.
 *          Query s (of S consecutive queries) uses rows
 *          max(0, s+Ls-S-W+1) .. s+Ls-S  (positions t-W+1 .. t, t >= 0); requires Ls >= S.
 *   sink   [H] fp32;  scale > 0 (normally 1/sqrt(c)).
 *   inv_rope_d, rope_theta: 0 = no epilogue; else the output of query (b,s) at position
 *          t = q_pos[b,s] (q_pos required) has its last inv_rope_d channels rotated back by
 *          its own position before the cast, pair (2p, 2p+1) by the angle
 *          -t * rope_theta^(-2p/inv_rope_d) ([V4-CSA2] section 12.1 "Partial RoPE 与 inverse
 *          RoPE": rows rotated at their positions then contribute by relative distance;
 *          [ATTN-CMP] section "CSA（DeepSeek-V4）": the last 64 output dimensions rotated by
 *          RoPE(-t)).  inv_rope_d even, <= c.  lse is unaffected.
 *   out    [B,S,H,c]   dtype;  lse [B,S,H] fp32 natural log, or NULL.
 *   ws >= csa_attn_workspace_size(...) bytes (split partial results).
 * ------------------------------------------------------------------------------ */
size_t csa_attn_workspace_size(int B, int S, int H, int c, int max_rows, int dtype);

int csa_sparse_attn(const void* q, const void* kv_comp, const int32_t* idx,
                    const int64_t* q_pos, const void* swa, const float* sink, int dtype, int kv_format,
                    float scale, int B, int S, int H, int c, int Nc, int k, int Ls, int W,
                    int inv_rope_d, float rope_theta,
                    void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------
 * csa_sparse_attn for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * results as csa_sparse_attn (the same kernels, bit for bit), without a workspace: the
 * split partials go to one fixed scratch array of csa_sparse_attn_noalloc_max_bytes()
 * bytes (32 MiB) that the library holds on every GPU it runs on until the process ends.
 * The call itself allocates nothing (no hipMalloc, no hipFree); its first call on a
 * device looks up that device's scratch address.
 *   A call whose partials (csa_attn_workspace_size with max_rows = min(W, Ls) + k) exceed
 *   the scratch returns CSA_ERR_SCRATCH before anything is launched.
 *   All calls on one GPU share that GPU's scratch and leave their partials in it: two
 *   calls that may overlap on one GPU (different streams, not ordered) race and give
 *   wrong results; order them.  Nothing in the scratch needs clearing between calls
 *   (every partial a call reads, it has written).
 * ------------------------------------------------------------------------------ */
size_t csa_sparse_attn_noalloc_max_bytes(void);

int csa_sparse_attn_noalloc(const void* q, const void* kv_comp, const int32_t* idx, const int64_t* q_pos,
                            const void* swa, const float* sink, int dtype, int kv_format, float scale,
                            int B, int S, int H, int c, int Nc, int k, int Ls, int W,
                            int inv_rope_d, float rope_theta, void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------------
 * Stages 3 and 4a in one call (decode shapes): csa_topk_merge of the segment
 * candidates written by csa_index_score_segments, then csa_sparse_attn over the
 * selected entries.  [KV-COMP] section 9.4 (the row's top-k lies in the union of its
 * segments' top-k sets) and sections 9.5-9.6 (attention over window || selection).
 * Results identical to csa_topk_merge followed by csa_sparse_attn.
 *
 *   cand: the pairs of csa_index_score_segments for the same B, S, Nc and k, cand_bytes
 *   its size (>= csa_index_segments_size(B, S, Nc, k), else CSA_ERR_WORKSPACE).  When
 *   csa_topk_merge would take two levels, the first level runs here too and writes its
 *   pairs into the rest of each row's share of cand, as csa_topk_merge does (cand is not
 *   const); the attention workgroups then select from those.
 *   Supported: dtype CSA_BF16 (H = 64, c = 512), the shapes csa_index_score_segments
 *   accepts, and at most 8192 pairs per row to select from (the segment pairs, G*k, or
 *   with two levels the first level's); otherwise CSA_ERR_UNSUPPORTED.
 *   idx [B,S,k] int32: receives the selection (as csa_topk_merge writes it), or NULL.
 *   Other arguments and the workspace (max_rows = min(W, Ls) + k) as csa_sparse_attn.
 * ------------------------------------------------------------------------------ */
int csa_topk_sparse_attn(const void* q, const void* kv_comp, void* cand, size_t cand_bytes,
                         const int64_t* q_pos, const void* swa, const float* sink, int dtype,
                         int kv_format, float scale, int B, int S, int H, int c, int Nc, int k, int Ls, int W,
                         int inv_rope_d, float rope_theta,
                         void* out, float* lse, int32_t* idx, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------------
 * Stage 4b: HCA core attention.  [HCA-CSA] "HCA：重压缩 + 全量" (no indexer: every
 * completed, visible compressed entry plus the window and the sink); [KV-COMP]
 * section 9.8 (entry j visible iff t >= m*j + m - 1).
 *
 * Same as csa_sparse_attn with the remote set of query (b,s) being the entries
 * j < min(Nc, floor((q_pos[b,s] + 1) / m)).  q_pos [B,S] int64, consecutive
 * positions within a sequence (required; it also bounds the window as above).  The workspace query takes max_rows = W + Nc.
 * ------------------------------------------------------------------------------ */
int hca_dense_attn(const void* q, const void* kv_comp, const int64_t* q_pos, int m,
                   const void* swa, const float* sink, int dtype, int kv_format, float scale,
                   int B, int S, int H, int c, int Nc, int Ls, int W,
                   int inv_rope_d, float rope_theta,
                   void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_MI355X_H */
