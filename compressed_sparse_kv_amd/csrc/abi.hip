// C entry points: argument validation, then dispatch to the stage launchers.
// Every check runs on the host before anything is enqueued (see include/csa.h).
#include <algorithm>

#include "common.hpp"

namespace csa {
int launch_index_score(const void*, const float*, const float*, const void*, const float*, int, const int64_t*, int,
                       int, int, int, int, int, float*, hipStream_t);
int launch_topk(const float*, int, int, int, int32_t*, void*, size_t, int, hipStream_t);
size_t topk_workspace_bytes(int, int, int);
bool topk_supported(int, int, bool);
int launch_attention(bool, const void*, const void*, int, const int32_t*, const int64_t*, int, const void*, const float*,
                     int, float, int, int, int, int, int, int, int, int, int, float, void*, float*, void*, size_t,
                     hipStream_t);
size_t attn_workspace_bytes(int, int, int, int, int, int);
size_t attn_scratch_bytes();
int attn_scratch(void**);
int launch_compress(const void*, const void*, int, const void*, const float*, int, int, int, int, int, int, int,
                    float, float, int64_t, void*, float*, int, int, int, void*, hipStream_t);
size_t compress_workspace_bytes(int, int, int, int, int, int);
size_t compress_state_bytes(int, int, int, int, int);
size_t csa2_workspace_bytes(int, int, int, int);
int launch_csa2_compress(const void*, int, const void*, const void*, int, int, int, int, int, int, int, float, float,
                         float, int64_t, void*, float*, int, void*, float*, int, void*, hipStream_t);
size_t compress_decode_workspace_bytes(int, int, int, int, int);
size_t compress_decode_many_workspace_bytes(int, int, int, int, const csa_decode_compressor*);
int launch_compress_decode_many(const void*, int, int, int, const int64_t*, int, int, const csa_decode_compressor*,
                                void*, hipStream_t);
bool index_topk_fused_ok(int, int, int);
int index_topk_segments(int);
int launch_index_topk(const void*, const float*, const float*, const void*, const float*, const int64_t*, int, int,
                      int, int, int, float*, int32_t*, void*, hipStream_t);
int launch_index_segments(const void*, const float*, const float*, const void*, const float*, const int64_t*, int,
                          int, int, int, int, float*, uint2*, hipStream_t, bool, float*);
int launch_index_pool(const void*, const float*, const float*, const void*, const float*, const int64_t*,
                      const int32_t*, int, int, int, int, int, int, float*, uint2*, hipStream_t);
int launch_index_mx(const void*, const void*, const float*, const void*, const void*, int, const int64_t*, int, int,
                    int, int, int, float*, int, uint2*, hipStream_t);
size_t index_keys_b16_bytes(int, int);
int launch_index_keys_b16(const void*, void*, int, int, hipStream_t);
int launch_topk_merge(uint2*, int, int, int, int32_t*, hipStream_t);
size_t topk_merge_pairs_per_row(int, int);
int launch_topk_attention(const void*, const void*, int, const uint2*, int, size_t, const int64_t*, const void*,
                          const float*, float, int, int, int, int, int, int, int, float, void*, float*, int32_t*, void*,
                          size_t, hipStream_t);
int topk_attention_max_cand();
int topk_merge_group(int, int);
int launch_topk_merge_first(uint2*, int, int, int, size_t&, hipStream_t);
}  // namespace csa

using namespace csa;

#define CSA_REQUIRE(cond) \
  do {                    \
    if (!(cond)) return CSA_ERR_INVALID_ARG; \
  } while (0)

static hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" {

const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID_ARG: return "CSA_ERR_INVALID_ARG: an argument is out of range or a required pointer is NULL";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: no kernel for this dtype/shape combination";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace smaller than the size query returned";
    case CSA_ERR_HIP: return "CSA_ERR_HIP: the HIP runtime rejected a kernel launch";
    case CSA_ERR_SCRATCH:
      return "CSA_ERR_SCRATCH: the call needs more scratch than the library's fixed scratch array holds";
    default: return "unknown csa_status";
  }
}

int csa_version(void) { return 400; }

// ---- stage 1 ------------------------------------------------------------------------
size_t csa_compress_workspace_size(int B, int T, int m, int c, int overlap, int has_prev) {
  if (B <= 0 || T <= 0 || m <= 0 || c <= 0) return 0;
  return compress_workspace_bytes(B, T, m, c, overlap, has_prev);
}

// The entry types a compressor writes and what each needs (packed: the main-KV row formats).
static int check_entry_dtype(int dt, const void* out, const void* scale, int c, int d_rope, bool packed_ok) {
  if (dt == CSA_F32 || dt == CSA_BF16) return CSA_OK;
  if (dt == CSA_FP8_E4M3) return scale != nullptr ? CSA_OK : CSA_ERR_INVALID_ARG;
  if (dt == CSA_FP4_E2M1) {
    if (scale == nullptr) return CSA_ERR_INVALID_ARG;
    return c % 32 == 0 ? CSA_OK : CSA_ERR_UNSUPPORTED;
  }
  if (packed_ok && (dt == CSA_PACKED_FP4_E4M3 || dt == CSA_PACKED_FP8_ROPE)) {
    if (!aligned16(out)) return CSA_ERR_INVALID_ARG;
    return c == 512 && (dt == CSA_PACKED_FP4_E4M3 || d_rope == 64) ? CSA_OK : CSA_ERR_UNSUPPORTED;
  }
  return CSA_ERR_INVALID_ARG;
}

int csa_compress(const void* hidden, const void* hidden_prev, int in_dtype, const void* w_proj, const float* bias,
                 int overlap, int B, int T, int d, int m, int c, int d_rope, float rope_theta, float rms_eps,
                 int64_t p0, void* out, float* out_scale, int out_dtype, int out_layout, int Nc_max, void* ws,
                 size_t ws_bytes, void* stream) {
  CSA_REQUIRE(hidden && w_proj && bias && out);
  CSA_REQUIRE(out_layout == CSA_LAYOUT_ROWS || out_layout == CSA_LAYOUT_B16);
  CSA_REQUIRE(overlap == 0 || overlap == 1);
  CSA_REQUIRE(B > 0 && T > 0 && d > 0 && m > 0 && c > 0);
  CSA_REQUIRE(T % m == 0 && p0 >= 0 && p0 % m == 0);
  CSA_REQUIRE(c % 2 == 0 && c <= 1024 && d_rope >= 0 && d_rope <= c && d_rope % 2 == 0);
  CSA_REQUIRE(rms_eps >= 0.0f && rope_theta > 0.0f);
  CSA_REQUIRE(!(overlap && p0 > 0 && hidden_prev == nullptr));
  CSA_REQUIRE(in_dtype == CSA_F32 || in_dtype == CSA_BF16);
  const int ot = check_entry_dtype(out_dtype, out, out_scale, c, d_rope, true);
  if (ot != CSA_OK) return ot;
  if (in_dtype == CSA_BF16 && d % 64 != 0) return CSA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(B) * (T + m) * 4 * c > (int64_t{1} << 40)) return CSA_ERR_UNSUPPORTED;
  if (out_layout == CSA_LAYOUT_B16) {
    // the chunk's entries p0/m .. p0/m + T/m - 1 must lie inside the cache of Nc_max entries
    if (out_dtype != CSA_FP8_E4M3 || c != 128) return CSA_ERR_UNSUPPORTED;
    CSA_REQUIRE(Nc_max > 0 && p0 / m + T / m <= Nc_max && static_cast<int64_t>(B) * Nc_max * c < (int64_t{1} << 40));
  }
  const int has_prev = hidden_prev != nullptr;
  CSA_REQUIRE(aligned16(ws));
  if (ws == nullptr || ws_bytes < compress_workspace_bytes(B, T, m, c, overlap, has_prev)) return CSA_ERR_WORKSPACE;
  return launch_compress(hidden, hidden_prev, in_dtype, w_proj, bias, overlap, B, T, d, m, c, d_rope, rope_theta,
                         rms_eps, p0, out, out_scale, out_dtype, out_layout, Nc_max, ws, as_stream(stream));
}

size_t csa2_compress_workspace_size(int B, int T, int m, int c) {
  if (B <= 0 || T <= 0 || m <= 0 || c <= 0) return 0;
  return csa2_workspace_bytes(B, T, m, c);
}

int csa2_compress(const void* hidden, int in_dtype, const void* w_proj, const void* w_k, int B, int T, int d, int m,
                  int c, int d_I, int d_rope, float theta_kv, float theta_k, float rms_eps, int64_t p0, void* kv_out,
                  float* kv_scale, int kv_dtype, void* k_out, float* k_scale, int k_dtype, void* ws, size_t ws_bytes,
                  void* stream) {
  CSA_REQUIRE(hidden && w_proj && w_k && kv_out && k_out);
  CSA_REQUIRE(B > 0 && T > 0 && d > 0 && m > 0 && c > 0 && d_I > 0);
  CSA_REQUIRE(T % m == 0 && p0 >= 0 && p0 % m == 0);
  CSA_REQUIRE(c % 2 == 0 && c <= 1024 && d_I % 2 == 0 && d_I <= 256);
  CSA_REQUIRE(d_rope >= 0 && d_rope % 2 == 0 && d_rope <= c && d_rope <= d_I);
  CSA_REQUIRE(rms_eps >= 0.0f && theta_kv > 0.0f && theta_k > 0.0f);
  CSA_REQUIRE(in_dtype == CSA_F32 || in_dtype == CSA_BF16);
  const int kvt = check_entry_dtype(kv_dtype, kv_out, kv_scale, c, d_rope, true);
  if (kvt != CSA_OK) return kvt;
  const int kt = check_entry_dtype(k_dtype, k_out, k_scale, d_I, d_rope, false);
  if (kt != CSA_OK) return kt;
  if (in_dtype == CSA_BF16 && (d % 64 != 0 || c % 8 != 0)) return CSA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(B) * T * 2 * c > (int64_t{1} << 40)) return CSA_ERR_UNSUPPORTED;
  CSA_REQUIRE(aligned16(ws) && aligned16(w_k));
  if (ws == nullptr || ws_bytes < csa2_workspace_bytes(B, T, m, c)) return CSA_ERR_WORKSPACE;
  return launch_csa2_compress(hidden, in_dtype, w_proj, w_k, B, T, d, m, c, d_I, d_rope, theta_kv, theta_k, rms_eps,
                              p0, kv_out, kv_scale, kv_dtype, k_out, k_scale, k_dtype, ws, as_stream(stream));
}

size_t csa_compress_state_size(int B, int m, int c, int overlap, int online) {
  if (B <= 0 || m <= 0 || c <= 0) return 0;
  return compress_state_bytes(B, m, c, overlap, online);
}

size_t csa_compress_decode_workspace_size(int B, int d, int c, int overlap, int in_dtype) {
  if (B <= 0 || d <= 0 || c <= 0) return 0;
  return compress_decode_workspace_bytes(B, d, c, overlap, in_dtype);
}

// The checks of one decode compressor's arguments (every one before anything is enqueued).
static int check_decode_comp(int in_dtype, int B, int d, const csa_decode_compressor& k) {
  CSA_REQUIRE(k.w_proj && k.bias && k.state && k.cache);
  CSA_REQUIRE((k.overlap == 0 || k.overlap == 1) && (k.online == 0 || k.online == 1) && !(k.online && k.overlap));
  CSA_REQUIRE(B > 0 && d > 0 && k.m > 0 && k.c > 0 && k.Nc_max > 0);
  CSA_REQUIRE(k.c % 2 == 0 && k.c <= 1024 && k.d_rope >= 0 && k.d_rope <= k.c && k.d_rope % 2 == 0);
  CSA_REQUIRE(k.rms_eps >= 0.0f && k.rope_theta > 0.0f);
  CSA_REQUIRE(in_dtype == CSA_F32 || in_dtype == CSA_BF16);
  const int ot = check_entry_dtype(k.out_dtype, k.cache, k.cache_scale, k.c, k.d_rope, true);
  if (ot != CSA_OK) return ot;
  CSA_REQUIRE(k.out_layout == CSA_LAYOUT_ROWS || k.out_layout == CSA_LAYOUT_B16);
  CSA_REQUIRE(static_cast<int64_t>(B) * k.Nc_max * k.c < (int64_t{1} << 40));
  if (k.out_layout == CSA_LAYOUT_B16 && (k.out_dtype != CSA_FP8_E4M3 || k.c != 128)) return CSA_ERR_UNSUPPORTED;
  if (in_dtype == CSA_BF16 && d % 128 != 0) return CSA_ERR_UNSUPPORTED;
  CSA_REQUIRE(aligned16(k.state) && aligned16(k.w_proj));
  return CSA_OK;
}

int csa_compress_decode(const void* hidden, int in_dtype, const void* w_proj, const float* bias, int overlap,
                        int online, int B, int d, int m, int c, int d_rope, float rope_theta, float rms_eps,
                        const int64_t* pos, int emit, float* state, void* cache, float* cache_scale, int out_dtype,
                        int out_layout, int Nc_max, void* ws, size_t ws_bytes, void* stream) {
  const csa_decode_compressor k{w_proj, bias, overlap, online, m, c, d_rope, rope_theta, rms_eps, state, cache,
                                cache_scale, out_dtype, out_layout, Nc_max};
  return csa_compress_decode_many(hidden, in_dtype, B, d, pos, emit, 1, &k, ws, ws_bytes, stream);
}

size_t csa_compress_decode_many_workspace_size(int B, int d, int in_dtype, int n, const csa_decode_compressor* comps) {
  if (B <= 0 || d <= 0 || n < 1 || n > 2 || comps == nullptr) return 0;
  for (int i = 0; i < n; ++i)
    if (comps[i].c <= 0) return 0;
  return compress_decode_many_workspace_bytes(B, d, in_dtype, n, comps);
}

int csa_compress_decode_many(const void* hidden, int in_dtype, int B, int d, const int64_t* pos, int emit, int n,
                             const csa_decode_compressor* comps, void* ws, size_t ws_bytes, void* stream) {
  CSA_REQUIRE(hidden && pos && comps && n >= 1 && n <= 2);
  for (int i = 0; i < n; ++i) {
    const int rc = check_decode_comp(in_dtype, B, d, comps[i]);
    if (rc != CSA_OK) return rc;
  }
  CSA_REQUIRE(aligned16(ws) && aligned16(hidden));
  if (ws == nullptr || ws_bytes < compress_decode_many_workspace_bytes(B, d, in_dtype, n, comps))
    return CSA_ERR_WORKSPACE;
  return launch_compress_decode_many(hidden, in_dtype, B, d, pos, emit, n, comps, ws, as_stream(stream));
}

// ---- stage 2 ------------------------------------------------------------------------
int csa_index_score(const void* q, const float* q_scale, const float* w, const void* k, const float* k_scale,
                    int dtype, const int64_t* q_pos, int B, int S, int H_I, int d_I, int Nc, int m, float* scores,
                    void* stream) {
  CSA_REQUIRE(q && w && k && q_pos && scores);
  CSA_REQUIRE(B > 0 && S > 0 && H_I > 0 && d_I > 0 && Nc > 0 && m > 0);
  CSA_REQUIRE(static_cast<int64_t>(B) * S * Nc < (int64_t{1} << 40));
  if (dtype == CSA_FP8_E4M3) {
    CSA_REQUIRE(q_scale && k_scale);
    if (H_I != 64 || d_I != 128) return CSA_ERR_UNSUPPORTED;
  } else if (dtype == CSA_F32) {
    CSA_REQUIRE(q_scale == nullptr && k_scale == nullptr);
    if (H_I > 64 || d_I > 256) return CSA_ERR_UNSUPPORTED;
  } else {
    return CSA_ERR_INVALID_ARG;
  }
  return launch_index_score(q, q_scale, w, k, k_scale, dtype, q_pos, B, S, H_I, d_I, Nc, m, scores,
                            as_stream(stream));
}

// ---- stages 2 + 3 -------------------------------------------------------------------
static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

size_t csa_index_topk_workspace_size(int B, int S, int Nc, int k) {
  if (B <= 0 || S <= 0 || Nc <= 0 || k <= 0) return 0;
  const size_t rows = static_cast<size_t>(B) * S;
  if (index_topk_fused_ok(S, Nc, k)) return rows * topk_merge_pairs_per_row(index_topk_segments(Nc), k) * sizeof(uint2);
  return align256(rows * Nc * sizeof(float)) + topk_workspace_bytes(static_cast<int>(rows), Nc, k);
}

int csa_index_topk(const void* q, const float* q_scale, const float* w, const void* k_codes, const float* k_scale,
                   const int64_t* q_pos, int B, int S, int H_I, int d_I, int Nc, int m, int k, float* scores,
                   int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  CSA_REQUIRE(q && q_scale && w && k_codes && k_scale && q_pos && idx);
  CSA_REQUIRE(B > 0 && S > 0 && Nc > 0 && m > 0 && k >= 1 && k <= 2048);
  const int64_t rows = static_cast<int64_t>(B) * S;
  CSA_REQUIRE(rows < (int64_t{1} << 31) && rows * Nc < (int64_t{1} << 40));
  if (H_I != 64 || d_I != 128) return CSA_ERR_UNSUPPORTED;
  if (!topk_supported(Nc, k, true)) return CSA_ERR_UNSUPPORTED;
  CSA_REQUIRE(aligned16(ws));
  if (ws == nullptr || ws_bytes < csa_index_topk_workspace_size(B, S, Nc, k)) return CSA_ERR_WORKSPACE;
  if (index_topk_fused_ok(S, Nc, k))
    return launch_index_topk(q, q_scale, w, k_codes, k_scale, q_pos, B, S, Nc, m, k, scores, idx, ws,
                             as_stream(stream));
  // other shapes: the two stages one after the other, scores in the workspace when not given
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  float* sc = scores;
  if (sc == nullptr) sc = reinterpret_cast<float*>(wsb);
  wsb += align256(static_cast<size_t>(rows) * Nc * sizeof(float));
  const size_t tk_bytes = topk_workspace_bytes(static_cast<int>(rows), Nc, k);
  int st = launch_index_score(q, q_scale, w, k_codes, k_scale, CSA_FP8_E4M3, q_pos, B, S, H_I, d_I, Nc, m, sc,
                              as_stream(stream));
  if (st != CSA_OK) return st;
  return launch_topk(sc, static_cast<int>(rows), Nc, k, idx, tk_bytes ? wsb : nullptr, tk_bytes, 0,
                     as_stream(stream));
}

size_t csa_index_segments_size(int B, int S, int Nc, int k) {
  if (B <= 0 || S <= 0 || Nc <= 0 || k <= 0 || !index_topk_fused_ok(S, Nc, k)) return 0;
  return static_cast<size_t>(B) * S * topk_merge_pairs_per_row(index_topk_segments(Nc), k) * sizeof(uint2);
}

static int index_score_segments(const void* q, const float* q_scale, const float* w, const void* k_codes,
                                const float* k_scale, const int64_t* q_pos, int B, int S, int H_I, int d_I, int Nc,
                                int m, int k, float* scores, void* cand, size_t cand_bytes, void* stream, bool b16,
                                float* bmax = nullptr) {
  CSA_REQUIRE(q && q_scale && w && k_codes && k_scale && q_pos && cand);
  CSA_REQUIRE(B > 0 && S > 0 && Nc > 0 && m > 0 && k >= 1 && k <= 2048);
  const int64_t rows = static_cast<int64_t>(B) * S;
  CSA_REQUIRE(rows < (int64_t{1} << 31) && rows * Nc < (int64_t{1} << 40));
  CSA_REQUIRE(aligned16(cand) && (!b16 || aligned16(k_codes)));
  if (H_I != 64 || d_I != 128 || !index_topk_fused_ok(S, Nc, k)) return CSA_ERR_UNSUPPORTED;
  if (cand_bytes < csa_index_segments_size(B, S, Nc, k)) return CSA_ERR_WORKSPACE;
  return launch_index_segments(q, q_scale, w, k_codes, k_scale, q_pos, B, S, Nc, m, k, scores,
                               static_cast<uint2*>(cand), as_stream(stream), b16, bmax);
}

int csa_index_score_segments(const void* q, const float* q_scale, const float* w, const void* k_codes,
                             const float* k_scale, const int64_t* q_pos, int B, int S, int H_I, int d_I, int Nc,
                             int m, int k, float* scores, void* cand, size_t cand_bytes, void* stream) {
  return index_score_segments(q, q_scale, w, k_codes, k_scale, q_pos, B, S, H_I, d_I, Nc, m, k, scores, cand,
                              cand_bytes, stream, false);
}

int csa_index_score_segments_b16(const void* q, const float* q_scale, const float* w, const void* k_blocks,
                                 const float* k_scale, const int64_t* q_pos, int B, int S, int H_I, int d_I, int Nc,
                                 int m, int k, float* scores, void* cand, size_t cand_bytes, void* stream) {
  return index_score_segments(q, q_scale, w, k_blocks, k_scale, q_pos, B, S, H_I, d_I, Nc, m, k, scores, cand,
                              cand_bytes, stream, true);
}

int csa_index_score_segments_bmax(const void* q, const float* q_scale, const float* w, const void* k_keys,
                                  int k_layout, const float* k_scale, const int64_t* q_pos, int B, int S, int H_I,
                                  int d_I, int Nc, int m, int k, float* scores, void* cand, size_t cand_bytes,
                                  float* block_max, void* stream) {
  CSA_REQUIRE(block_max && (k_layout == CSA_LAYOUT_ROWS || k_layout == CSA_LAYOUT_B16));
  return index_score_segments(q, q_scale, w, k_keys, k_scale, q_pos, B, S, H_I, d_I, Nc, m, k, scores, cand,
                              cand_bytes, stream, k_layout == CSA_LAYOUT_B16, block_max);
}

int csa_index_score_mx(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale,
                       int elem_dtype, const int64_t* q_pos, int B, int S, int H_I, int d_I, int Nc, int m,
                       int score_bf16, float* scores, int k_top, void* cand, size_t cand_bytes, void* stream) {
  CSA_REQUIRE(q && q_scale && w && k && k_scale && q_pos);
  CSA_REQUIRE(elem_dtype == CSA_FP4_E2M1 || elem_dtype == CSA_FP8_E4M3);
  CSA_REQUIRE(B > 0 && S > 0 && Nc > 0 && m > 0);
  const int64_t rows = static_cast<int64_t>(B) * S;
  CSA_REQUIRE(rows < (int64_t{1} << 31) && rows * Nc < (int64_t{1} << 40));
  if (H_I != 64 || d_I != 128) return CSA_ERR_UNSUPPORTED;
  CSA_REQUIRE(aligned16(q) && aligned16(k));
  if (cand == nullptr) {
    CSA_REQUIRE(scores != nullptr);
  } else {
    CSA_REQUIRE(k_top >= 1 && k_top <= 2048 && aligned16(cand));
    if (!index_topk_fused_ok(S, Nc, k_top)) return CSA_ERR_UNSUPPORTED;
    if (cand_bytes < csa_index_segments_size(B, S, Nc, k_top)) return CSA_ERR_WORKSPACE;
  }
  return launch_index_mx(q, q_scale, w, k, k_scale, elem_dtype == CSA_FP4_E2M1, q_pos, B, S, Nc, m, score_bf16 != 0,
                         scores, k_top, static_cast<uint2*>(cand), as_stream(stream));
}

size_t csa_index_pool_segments_size(int B, int S, int n_blocks, int k) {
  if (n_blocks <= 0 || n_blocks > (1 << 26)) return 0;
  return csa_index_segments_size(B, S, 8 * n_blocks, k);
}

int csa_index_score_pool(const void* q, const float* q_scale, const float* w, const void* k_codes,
                         const float* k_scale, const int64_t* q_pos, const int32_t* blocks, int n_blocks, int B, int S,
                         int H_I, int d_I, int Nc, int m, int k, float* scores, void* cand, size_t cand_bytes,
                         void* stream) {
  CSA_REQUIRE(q && q_scale && w && k_codes && k_scale && q_pos && blocks && cand);
  CSA_REQUIRE(B > 0 && S > 0 && Nc > 0 && m > 0 && k >= 1 && k <= 2048 && n_blocks > 0 && n_blocks <= (1 << 26));
  const int64_t rows = static_cast<int64_t>(B) * S;
  CSA_REQUIRE(rows < (int64_t{1} << 31) && rows * 8 * n_blocks < (int64_t{1} << 40));
  CSA_REQUIRE(aligned16(cand));
  if (H_I != 64 || d_I != 128 || !index_topk_fused_ok(S, 8 * n_blocks, k)) return CSA_ERR_UNSUPPORTED;
  if (cand_bytes < csa_index_pool_segments_size(B, S, n_blocks, k)) return CSA_ERR_WORKSPACE;
  return launch_index_pool(q, q_scale, w, k_codes, k_scale, q_pos, blocks, n_blocks, B, S, Nc, m, k, scores,
                           static_cast<uint2*>(cand), as_stream(stream));
}

size_t csa_index_keys_b16_size(int B, int Nc) {
  if (B <= 0 || Nc <= 0) return 0;
  return index_keys_b16_bytes(B, Nc);
}

int csa_index_keys_b16(const void* k_codes, void* k_blocks, int B, int Nc, void* stream) {
  CSA_REQUIRE(k_codes && k_blocks && B > 0 && Nc > 0);
  CSA_REQUIRE(static_cast<int64_t>(B) * Nc < (int64_t{1} << 34));
  CSA_REQUIRE(aligned16(k_codes) && aligned16(k_blocks));
  return launch_index_keys_b16(k_codes, k_blocks, B, Nc, as_stream(stream));
}

int csa_topk_merge(void* cand, size_t cand_bytes, int B, int S, int Nc, int k, int32_t* idx, void* stream) {
  CSA_REQUIRE(cand && idx);
  CSA_REQUIRE(B > 0 && S > 0 && Nc > 0 && k >= 1 && k <= 2048);
  CSA_REQUIRE(static_cast<int64_t>(B) * S < (int64_t{1} << 31));
  CSA_REQUIRE(aligned16(cand));
  if (!index_topk_fused_ok(S, Nc, k)) return CSA_ERR_UNSUPPORTED;
  if (cand_bytes < csa_index_segments_size(B, S, Nc, k)) return CSA_ERR_WORKSPACE;
  return launch_topk_merge(static_cast<uint2*>(cand), B * S, index_topk_segments(Nc), k, idx, as_stream(stream));
}

// ---- stage 3 ------------------------------------------------------------------------
size_t csa_topk_workspace_size(int rows, int Nc, int k) {
  if (rows <= 0 || Nc <= 0 || k <= 0) return 0;
  return topk_workspace_bytes(rows, Nc, k);
}

int csa_topk_algo(const float* scores, int B, int S, int Nc, int k, int32_t* idx, void* ws, size_t ws_bytes,
                  int algo, void* stream) {
  CSA_REQUIRE(scores && idx);
  CSA_REQUIRE(B > 0 && S > 0 && Nc > 0 && k >= 1 && k <= 2048);
  CSA_REQUIRE(algo >= 0 && algo <= 2);
  const int64_t rows = static_cast<int64_t>(B) * S;
  CSA_REQUIRE(rows < (int64_t{1} << 31) && rows * Nc < (int64_t{1} << 40));
  if (!topk_supported(Nc, k, true)) return CSA_ERR_UNSUPPORTED;
  CSA_REQUIRE(aligned16(ws));
  if (ws != nullptr && ws_bytes < topk_workspace_bytes(static_cast<int>(rows), Nc, k)) return CSA_ERR_WORKSPACE;
  if (ws == nullptr && (algo == 2 || !topk_supported(Nc, k, false))) return CSA_ERR_WORKSPACE;
  return launch_topk(scores, static_cast<int>(rows), Nc, k, idx, ws, ws_bytes, algo, as_stream(stream));
}

int csa_topk(const float* scores, int B, int S, int Nc, int k, int32_t* idx, void* ws, size_t ws_bytes,
             void* stream) {
  return csa_topk_algo(scores, B, S, Nc, k, idx, ws, ws_bytes, 0, stream);
}

// ---- stage 4 ------------------------------------------------------------------------
size_t csa_attn_workspace_size(int B, int S, int H, int c, int max_rows, int dtype) {
  if (B <= 0 || S <= 0 || H <= 0 || c <= 0 || max_rows <= 0) return 0;
  return attn_workspace_bytes(B, S, H, c, max_rows, dtype);
}

static int check_attn(const void* q, const void* kv, const void* swa, const float* sink, int dtype, int kv_format,
                      float scale, int B, int S, int H, int c, int Nc, int Ls, int W, const void* out, int inv_rope_d,
                      float rope_theta, const int64_t* q_pos) {
  CSA_REQUIRE(q && kv && swa && sink && out);
  CSA_REQUIRE(kv_format == CSA_KV_BF16 || kv_format == CSA_KV_FP4_E4M3 || kv_format == CSA_KV_FP8_ROPE_BF16);
  if (kv_format != CSA_KV_BF16 && dtype != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  CSA_REQUIRE(kv_format == CSA_KV_BF16 || aligned16(kv));
  CSA_REQUIRE(inv_rope_d >= 0 && inv_rope_d % 2 == 0 && inv_rope_d <= c);
  CSA_REQUIRE(inv_rope_d == 0 || (q_pos != nullptr && rope_theta > 0.0f));
  CSA_REQUIRE(B > 0 && S > 0 && H > 0 && c > 0 && Nc > 0 && W > 0 && Ls >= S);
  CSA_REQUIRE(scale > 0.0f);
  CSA_REQUIRE(static_cast<int64_t>(B) * S < (int64_t{1} << 31));
  if (dtype == CSA_BF16) {
    if (H != 64 || c != 512) return CSA_ERR_UNSUPPORTED;
  } else if (dtype == CSA_F32) {
    if (H > 64 || c > 512) return CSA_ERR_UNSUPPORTED;
  } else {
    return CSA_ERR_INVALID_ARG;
  }
  return CSA_OK;
}

int csa_sparse_attn(const void* q, const void* kv_comp, const int32_t* idx, const int64_t* q_pos, const void* swa,
                    const float* sink, int dtype, int kv_format, float scale, int B, int S, int H, int c, int Nc, int k, int Ls, int W,
                    int inv_rope_d, float rope_theta, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  const int st = check_attn(q, kv_comp, swa, sink, dtype, kv_format, scale, B, S, H, c, Nc, Ls, W, out, inv_rope_d, rope_theta,
                            q_pos);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(idx && k >= 1 && k <= 65536);
  CSA_REQUIRE(aligned16(ws));
  return launch_attention(false, q, kv_comp, kv_format, idx, q_pos, 1, swa, sink, dtype, scale, B, S, H, c, Nc, k, Ls, W,
                          inv_rope_d, rope_theta, out, lse, ws, ws_bytes, as_stream(stream));
}

size_t csa_sparse_attn_noalloc_max_bytes(void) { return attn_scratch_bytes(); }

int csa_sparse_attn_noalloc(const void* q, const void* kv_comp, const int32_t* idx, const int64_t* q_pos,
                            const void* swa, const float* sink, int dtype, int kv_format, float scale, int B, int S, int H, int c,
                            int Nc, int k, int Ls, int W, int inv_rope_d, float rope_theta, void* out, float* lse,
                            void* stream) {
  const int st = check_attn(q, kv_comp, swa, sink, dtype, kv_format, scale, B, S, H, c, Nc, Ls, W, out, inv_rope_d, rope_theta,
                            q_pos);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(idx && k >= 1 && k <= 65536);
  const size_t need = attn_workspace_bytes(B, S, H, c, std::min(W, Ls) + k, dtype);
  if (need > attn_scratch_bytes()) return CSA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = attn_scratch(&ws);
    if (rc != CSA_OK) return rc;
  }
  return launch_attention(false, q, kv_comp, kv_format, idx, q_pos, 1, swa, sink, dtype, scale, B, S, H, c, Nc, k, Ls, W,
                          inv_rope_d, rope_theta, out, lse, ws, need, as_stream(stream));
}

int csa_topk_sparse_attn(const void* q, const void* kv_comp, void* cand, size_t cand_bytes, const int64_t* q_pos,
                         const void* swa, const float* sink, int dtype, int kv_format, float scale, int B, int S,
                         int H, int c, int Nc, int k, int Ls, int W, int inv_rope_d, float rope_theta, void* out,
                         float* lse, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  const int st = check_attn(q, kv_comp, swa, sink, dtype, kv_format, scale, B, S, H, c, Nc, Ls, W, out, inv_rope_d, rope_theta,
                            q_pos);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(cand && k >= 1 && k <= 2048);
  CSA_REQUIRE(aligned16(cand) && aligned16(ws));
  if (dtype != CSA_BF16 || !index_topk_fused_ok(S, Nc, k)) return CSA_ERR_UNSUPPORTED;
  // the set the attention selects from: the segment pairs, or the first merge level's
  // when the segments hold more pairs than one workgroup selects from at once
  const int G = index_topk_segments(Nc);
  const int M = topk_merge_group(G, k);
  if (M < 0) return CSA_ERR_UNSUPPORTED;
  const long long n_sel = M == 0 ? static_cast<long long>(G) * k : static_cast<long long>((G + M - 1) / M) * k;
  if (n_sel > topk_attention_max_cand()) return CSA_ERR_UNSUPPORTED;
  if (cand_bytes < csa_index_segments_size(B, S, Nc, k)) return CSA_ERR_WORKSPACE;
  // every check before the first level is enqueued
  if (ws_bytes < attn_workspace_bytes(B, S, H, c, std::min(W, Ls) + k, dtype)) return CSA_ERR_WORKSPACE;
  const int rows = B * S;
  uint2* pairs = static_cast<uint2*>(cand);
  size_t offset = 0;
  const int n_cand = launch_topk_merge_first(pairs, rows, G, k, offset, as_stream(stream));
  if (n_cand < 0) return CSA_ERR_HIP;
  return launch_topk_attention(q, kv_comp, kv_format, pairs + offset, n_cand, topk_merge_pairs_per_row(G, k), q_pos, swa, sink,
                               scale, B, S, Nc, k, Ls, W, inv_rope_d, rope_theta, out, lse, idx, ws, ws_bytes,
                               as_stream(stream));
}

int hca_dense_attn(const void* q, const void* kv_comp, const int64_t* q_pos, int m, const void* swa, const float* sink,
                   int dtype, int kv_format, float scale, int B, int S, int H, int c, int Nc, int Ls, int W, int inv_rope_d,
                   float rope_theta, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  const int st = check_attn(q, kv_comp, swa, sink, dtype, kv_format, scale, B, S, H, c, Nc, Ls, W, out, inv_rope_d, rope_theta,
                            q_pos);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(q_pos && m > 0);
  CSA_REQUIRE(aligned16(ws));
  return launch_attention(true, q, kv_comp, kv_format, nullptr, q_pos, m, swa, sink, dtype, scale, B, S, H, c, Nc, 0, Ls, W,
                          inv_rope_d, rope_theta, out, lse, ws, ws_bytes, as_stream(stream));
}

}  // extern "C"
