// extern "C" entry points of libtplayer: argument validation on the host
// (before any HIP call, so invalid requests never launch anything), then
// dispatch to the kernel launchers.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace tpl {
tp_status gemm_bf16_mfma(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                         bool out_f32, bool aligned, hipStream_t s, int force_tile);
tp_status gemm_bf16_dma(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                        bool out_f32, bool vec_out, hipStream_t s, int force_tile);
tp_status gemm_bf16_dma_act(const void* x, const void* w, void* h, int64_t M, int64_t I, int64_t K,
                            int act, bool vec_out, hipStream_t s);
tp_status gemm_bf16_stream_act(const void* x, const void* w, void* h, int64_t M, int64_t I,
                               int64_t K, int act, hipStream_t s);
tp_status reduce_rmsnorm(const float* const* partials, int R, const void* residual, bool res_f32,
                         void* y, bool y_f32, const void* gamma, void* yn, int64_t M, int64_t N,
                         float eps, hipStream_t s);
tp_status gemm_bf16_stream(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                           bool out_f32, hipStream_t s);
tp_status gemm_f32(const float* x, const float* w, float* y, int64_t M, int64_t N, int64_t K,
                   hipStream_t s);
tp_status act_local(const void* g, const void* u, void* h, int64_t M, int64_t I, int64_t ld,
                    int act, bool bf16, bool vec, hipStream_t s);
tp_status reduce_partials(const float* const* partials, int R, const void* residual, bool res_f32,
                          void* y, int64_t total, bool bf16, bool vec, hipStream_t s);
tp_status rmsnorm(const void* x, bool x_f32, const void* gamma, void* y, int64_t M, int64_t N,
                  float eps, bool bf16, bool vec, hipStream_t s);
tp_status kv_append(const void* kn, const void* vn, int64_t new_stride, void* kc, void* vc,
                    const int64_t cs[3], int64_t B, int64_t H, int64_t D, int64_t pos,
                    hipStream_t s);
tp_status attn_decode(const void* q, const int64_t qs[3], const void* k, const void* v,
                      const int64_t kvs[3], void* o, const int64_t os[3], int64_t B, int64_t Skv,
                      int64_t Hq, int64_t Hkv, float scale, void* ws, hipStream_t s,
                      const void* kn = nullptr, const void* vn = nullptr, int64_t nstride = 0);
tp_status attn_prefill_tr(const void* q, const int64_t qs[3], const void* k, const void* v,
                          const int64_t kvs[3], void* o, const int64_t os[3], int64_t B,
                          int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv, int causal, float scale,
                          hipStream_t s);
bool attn_prefill_tr_ok(const int64_t kvs[3], int64_t Skv, int64_t D);
size_t attn_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv);
tp_status attn_decode_scratch(hipStream_t s, void** ptr, size_t* bytes);
tp_status attn_prefill(const void* q, const int64_t qs[3], const void* k, const void* v,
                       const int64_t kvs[3], void* o, const int64_t os[3], int64_t B, int64_t Sq,
                       int64_t Skv, int64_t Hq, int64_t Hkv, int causal, float scale,
                       hipStream_t s);

static thread_local char g_last_error[512] = "";

void set_hip_error(const char* where, hipError_t e) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

tp_status vocab_argmax_local(const float* logits, int64_t M, int64_t V, int64_t offset, float* mv,
                             int64_t* mi, bool vec, hipStream_t s);
int attn_paged_nsplit(int64_t B, int64_t Hkv, int64_t max_len, int64_t bs);
size_t attn_paged_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_len, int64_t bs);
tp_status attn_decode_paged(const void* q, const int64_t qs[2], const void* kp, const void* vp,
                            const int64_t ps[3], int64_t nblocks, const int* table, int64_t tstride,
                            const int* lens, int64_t max_len, int64_t bs, void* o,
                            const int64_t os[2], int64_t B, int64_t Hq, int64_t Hkv, float scale,
                            void* ws, hipStream_t s, const void* kn = nullptr,
                            const void* vn = nullptr, int64_t nstride = 0);
tp_status paged_kv_append(const void* kn, const void* vn, int64_t new_stride, void* kp, void* vp,
                          const int64_t ps[3], int64_t nblocks, const int* table, int64_t tstride,
                          int64_t maxblk, const int* lens, int64_t B, int64_t H, int64_t D, int64_t bs,
                          hipStream_t s);
tp_status vocab_argmax_reduce(const float* const* vals, const int64_t* const* idxs, int R, int64_t M,
                              float* ov, int64_t* oi, hipStream_t s);
}  // namespace tpl

namespace {

constexpr int64_t kIntMax = 0x7fffffff;

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
// Do the byte ranges [a, a + na) and [b, b + nb) share a byte?
inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}
// A sum's output may be its residual buffer itself (the residual stream
// updated in place) only when both have one storage type; any other overlap
// would let one thread's store clobber another thread's residual load.
inline bool bad_alias(const void* res, tp_dtype res_dt, const void* y, tp_dtype y_dt, int64_t n) {
  if (!res) return false;
  if (res == y && res_dt == y_dt) return false;
  return overlap(res, (size_t)n * (res_dt == TP_BF16 ? 2 : 4), y, (size_t)n * (y_dt == TP_BF16 ? 2 : 4));
}
inline size_t esize(tp_dtype dt) { return dt == TP_BF16 ? 2 : 4; }
inline bool dtype_ok(tp_dtype dt) { return dt == TP_F32 || dt == TP_BF16; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

tp_status linear_common(const void* x, const void* w, void* y, int64_t M, int64_t K, int64_t N,
                        tp_dtype dt, void* stream, bool out_f32) {
  if (!x || !w || !y) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (M <= 0 || K <= 0 || N <= 0) return TP_ERR_SHAPE;
  if (M > kIntMax || K > kIntMax || N > kIntMax) return TP_ERR_UNSUPPORTED;
  const size_t es = esize(dt);
  if (!aligned(x, es) || !aligned(w, es) || !aligned(y, out_f32 ? 4 : es)) return TP_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  if (dt == TP_F32)
    return tpl::gemm_f32(static_cast<const float*>(x), static_cast<const float*>(w),
                         static_cast<float*>(y), M, N, K, s);
  const bool vec = (K % 8 == 0) && aligned(x, 16) && aligned(w, 16);
  if (M <= 64 && vec && K < (int64_t{1} << 24)) return tpl::gemm_bf16_stream(x, w, y, M, N, K, out_f32, s);
  // Direct-to-LDS tile path: 32-bit buffer offsets cover a 256-row tile.
  if (vec && K < (int64_t{1} << 21)) {
    const bool vec_out = (N % 4 == 0) && aligned(y, out_f32 ? 16 : 8);
    return tpl::gemm_bf16_dma(x, w, y, M, N, K, out_f32, vec_out, s, -1);
  }
  return tpl::gemm_bf16_mfma(x, w, y, M, N, K, out_f32, vec, s, -1);
}

}  // namespace

extern "C" {

tp_status tp_column_linear(const void* x, const void* w, void* y, int64_t M, int64_t K, int64_t N,
                           tp_dtype dt, void* stream) {
  return linear_common(x, w, y, M, K, N, dt, stream, /*out_f32=*/dt == TP_F32);
}

tp_status tp_row_linear_partial(const void* x, const void* w, float* partial, int64_t M, int64_t K,
                                int64_t N, tp_dtype dt, void* stream) {
  return linear_common(x, w, partial, M, K, N, dt, stream, /*out_f32=*/true);
}

tp_status tp_column_linear_act(const void* x, const void* w, void* h, int64_t M, int64_t K,
                               int64_t I, tp_act act, tp_dtype dt, void* stream) {
  if (act == TP_ACT_NONE) return tp_column_linear(x, w, h, M, K, I, dt, stream);
  if (!x || !w || !h) return TP_ERR_NULL;
  if (act != TP_ACT_SWIGLU && act != TP_ACT_GELU) return TP_ERR_DTYPE;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (M <= 0 || K <= 0 || I <= 0) return TP_ERR_SHAPE;
  if (M > kIntMax || K > kIntMax || I > kIntMax) return TP_ERR_UNSUPPORTED;
  if (dt != TP_BF16) return TP_ERR_UNSUPPORTED;
  if (!aligned(x, 2) || !aligned(w, 2) || !aligned(h, 2)) return TP_ERR_ALIGN;
  // The fused kernels stream 16-byte vectors of both operands.
  if (K % 8 != 0 || !aligned(x, 16) || !aligned(w, 16)) return TP_ERR_UNSUPPORTED;
  const int64_t wrows = act == TP_ACT_SWIGLU ? 2 * I : I;
  if (wrows * K * 2 >= (int64_t{1} << 32)) return TP_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  if (M <= 64 && K < (int64_t{1} << 24)) return tpl::gemm_bf16_stream_act(x, w, h, M, I, K, (int)act, s);
  if (K >= (int64_t{1} << 21)) return TP_ERR_UNSUPPORTED;
  const bool vec_out = (I % 4 == 0) && aligned(h, 8);
  return tpl::gemm_bf16_dma_act(x, w, h, M, I, K, (int)act, vec_out, s);
}

tp_status tp_swiglu_local(const void* gate, const void* up, void* h, int64_t M, int64_t I,
                          int64_t ld, tp_act act, tp_dtype dt, void* stream) {
  if (!gate || !h) return TP_ERR_NULL;
  if (act != TP_ACT_NONE && act != TP_ACT_SWIGLU && act != TP_ACT_GELU) return TP_ERR_DTYPE;
  if (act == TP_ACT_SWIGLU && !up) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (M <= 0 || I <= 0 || ld < I) return TP_ERR_SHAPE;
  const size_t es = esize(dt);
  if (!aligned(gate, es) || !aligned(h, es) || (up && !aligned(up, es))) return TP_ERR_ALIGN;
  bool vec = (I % 8 == 0) && (ld % 8 == 0) && aligned(gate, 16) && aligned(h, 16) &&
             (act != TP_ACT_SWIGLU || aligned(up, 16));
  return tpl::act_local(gate, up, h, M, I, ld, (int)act, dt == TP_BF16, vec, as_stream(stream));
}

size_t tp_local_attention_workspace(int64_t B, int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv,
                                    int64_t D) {
  if (B <= 0 || Sq <= 0 || Skv <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return 0;
  const int64_t G = Hq / Hkv;
  if (Sq == 1 && G <= 32) return tpl::attn_decode_workspace(B, Hq, Hkv, Skv);
  return 0;
}

tp_status tp_local_attention(const void* q, const int64_t qs[3], const void* k, const void* v,
                             const int64_t kvs[3], void* o, const int64_t os[3], int64_t B,
                             int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv, int64_t D,
                             int causal, float scale, tp_dtype dt, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !qs || !kvs || !os) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (B <= 0 || Sq <= 0 || Skv <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return TP_ERR_SHAPE;
  if (Hq % Hkv != 0) return TP_ERR_SHAPE;
  if (causal && Sq > Skv) return TP_ERR_SHAPE;
  if (!isfinite(scale)) return TP_ERR_SHAPE;
  if (dt != TP_BF16 || D != 128) return TP_ERR_UNSUPPORTED;
  if (B > 65535 || Hq > 65535 || Skv > kIntMax || Sq > kIntMax) return TP_ERR_UNSUPPORTED;
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || kvs[i] < 0 || os[i] < 0) return TP_ERR_SHAPE;
    if (qs[i] % 8 || kvs[i] % 8 || os[i] % 4) return TP_ERR_ALIGN;
  }
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 8)) return TP_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  const size_t need = tp_local_attention_workspace(B, Sq, Skv, Hq, Hkv, D);
  // The decode kernel addresses one sequence's key span with 32-bit offsets.
  if (Sq == 1 && ((Skv - 1) * kvs[1] + D) * 2 >= (int64_t{1} << 31)) return TP_ERR_UNSUPPORTED;
  if (Sq == 1 && need == 0 && Hq / Hkv <= 32)
    return tpl::attn_decode(q, qs, k, v, kvs, o, os, B, Skv, Hq, Hkv, scale, nullptr, s);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return TP_ERR_ALIGN;
    return tpl::attn_decode(q, qs, k, v, kvs, o, os, B, Skv, Hq, Hkv, scale, workspace, s);
  }
  if (tpl::attn_prefill_tr_ok(kvs, Skv, D) && B * Hq * ((Sq + 255) / 256) <= kIntMax)
    return tpl::attn_prefill_tr(q, qs, k, v, kvs, o, os, B, Sq, Skv, Hq, Hkv, causal, scale, s);
  return tpl::attn_prefill(q, qs, k, v, kvs, o, os, B, Sq, Skv, Hq, Hkv, causal, scale, s);
}

tp_status tp_kv_append(const void* k_new, const void* v_new, int64_t new_stride, void* k_cache,
                       void* v_cache, const int64_t cs[3], int64_t B, int64_t Hkv, int64_t D,
                       int64_t T, int64_t pos, tp_dtype dt, void* stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !cs) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (dt != TP_BF16) return TP_ERR_UNSUPPORTED;
  if (B <= 0 || Hkv <= 0 || D <= 0 || pos < 0 || pos >= T || new_stride < Hkv * D) return TP_ERR_SHAPE;
  if (cs[0] < 0 || cs[1] < 0 || cs[2] < 0) return TP_ERR_SHAPE;
  if (!aligned(k_new, 2) || !aligned(v_new, 2) || !aligned(k_cache, 2) || !aligned(v_cache, 2))
    return TP_ERR_ALIGN;
  return tpl::kv_append(k_new, v_new, new_stride, k_cache, v_cache, cs, B, Hkv, D, pos,
                        as_stream(stream));
}

// The decode step's append + attention; `own_scratch` takes the partials
// buffer from the library's static array instead of `workspace`.
static tp_status decode_append_common(const void* q, const int64_t qs[2], const void* k_new,
                                      const void* v_new, int64_t new_stride, void* k_cache,
                                      void* v_cache, const int64_t cs[3], int64_t T, int64_t pos,
                                      void* o, const int64_t os[2], int64_t B, int64_t Hq,
                                      int64_t Hkv, int64_t D, float scale, tp_dtype dt,
                                      void* workspace, size_t workspace_bytes, bool own_scratch,
                                      void* stream) {
  if (!q || !qs || !k_new || !v_new || !k_cache || !v_cache || !cs || !o || !os) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return TP_ERR_SHAPE;
  if (pos < 0 || pos >= T || new_stride < Hkv * D) return TP_ERR_SHAPE;
  if (!isfinite(scale)) return TP_ERR_SHAPE;
  if (dt != TP_BF16 || D != 128 || Hq / Hkv > 32) return TP_ERR_UNSUPPORTED;
  if (B > 65535 || Hkv > 65535 || pos >= kIntMax) return TP_ERR_UNSUPPORTED;
  for (int i = 0; i < 3; ++i) {
    if (cs[i] < 0) return TP_ERR_SHAPE;
    if (cs[i] % 8) return TP_ERR_ALIGN;
  }
  for (int i = 0; i < 2; ++i) {
    if (qs[i] < 0 || os[i] < 0) return TP_ERR_SHAPE;
    if (qs[i] % 8 || os[i] % 4) return TP_ERR_ALIGN;
  }
  if (new_stride % 8) return TP_ERR_ALIGN;
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(o, 8))
    return TP_ERR_ALIGN;
  const int64_t Skv = pos + 1;
  // the kernel addresses one sequence's key span with 32-bit offsets
  if ((pos * cs[1] + D) * 2 >= (int64_t{1} << 31)) return TP_ERR_UNSUPPORTED;
  const size_t need = tpl::attn_decode_workspace(B, Hq, Hkv, Skv);
  if (own_scratch && need > 0) {
    const tp_status st = tpl::attn_decode_scratch(as_stream(stream), &workspace, &workspace_bytes);
    if (st != TP_OK) return st;
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return TP_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return TP_ERR_ALIGN;
  const int64_t q3[3] = {qs[0], 0, qs[1]}, o3[3] = {os[0], 0, os[1]};
  return tpl::attn_decode(q, q3, k_cache, v_cache, cs, o, o3, B, Skv, Hq, Hkv, scale,
                          need > 0 ? workspace : nullptr, as_stream(stream), k_new, v_new,
                          new_stride);
}

tp_status tp_decode_attention_append(const void* q, const int64_t qs[2], const void* k_new,
                                     const void* v_new, int64_t new_stride, void* k_cache,
                                     void* v_cache, const int64_t cs[3], int64_t T, int64_t pos,
                                     void* o, const int64_t os[2], int64_t B, int64_t Hq,
                                     int64_t Hkv, int64_t D, float scale, tp_dtype dt,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_append_common(q, qs, k_new, v_new, new_stride, k_cache, v_cache, cs, T, pos, o, os,
                              B, Hq, Hkv, D, scale, dt, workspace, workspace_bytes, false, stream);
}

tp_status tp_decode_attention_append_noalloc(const void* q, const int64_t qs[2], const void* k_new,
                                             const void* v_new, int64_t new_stride, void* k_cache,
                                             void* v_cache, const int64_t cs[3], int64_t T,
                                             int64_t pos, void* o, const int64_t os[2], int64_t B,
                                             int64_t Hq, int64_t Hkv, int64_t D, float scale,
                                             tp_dtype dt, void* stream) {
  return decode_append_common(q, qs, k_new, v_new, new_stride, k_cache, v_cache, cs, T, pos, o, os,
                              B, Hq, Hkv, D, scale, dt, nullptr, 0, true, stream);
}

tp_status tp_reduce_partials(const float* const* partials, int64_t R, const void* residual,
                             tp_dtype res_dt, void* y, int64_t M, int64_t N, tp_dtype out_dt,
                             void* stream) {
  if (!partials || !y) return TP_ERR_NULL;
  if (R < 1 || R > 16) return TP_ERR_SHAPE;
  for (int64_t r = 0; r < R; ++r)
    if (!partials[r]) return TP_ERR_NULL;
  if (!dtype_ok(out_dt) || (residual && !dtype_ok(res_dt))) return TP_ERR_DTYPE;
  if (M <= 0 || N <= 0) return TP_ERR_SHAPE;
  if (bad_alias(residual, res_dt, y, out_dt, M * N)) return TP_ERR_SHAPE;
  const size_t es = esize(out_dt), rs = esize(res_dt);
  if (!aligned(y, es) || (residual && !aligned(residual, rs))) return TP_ERR_ALIGN;
  bool vec = ((M * N) % 4 == 0) && aligned(y, 4 * es) && (!residual || aligned(residual, 4 * rs));
  for (int64_t r = 0; r < R; ++r) {
    if (!aligned(partials[r], 4)) return TP_ERR_ALIGN;
    vec = vec && aligned(partials[r], 16);
  }
  return tpl::reduce_partials(partials, (int)R, residual, res_dt == TP_F32, y, M * N,
                              out_dt == TP_BF16, vec, as_stream(stream));
}

tp_status tp_reduce_partials_rmsnorm(const float* const* partials, int64_t R, const void* residual,
                                     tp_dtype res_dt, void* y, tp_dtype y_dt, const void* gamma,
                                     void* yn, int64_t M, int64_t N, float eps, tp_dtype dt,
                                     void* stream) {
  if (!partials || !y || !gamma || !yn) return TP_ERR_NULL;
  if (R < 1 || R > 16) return TP_ERR_SHAPE;
  for (int64_t r = 0; r < R; ++r)
    if (!partials[r]) return TP_ERR_NULL;
  if (!dtype_ok(dt) || !dtype_ok(y_dt) || (residual && !dtype_ok(res_dt))) return TP_ERR_DTYPE;
  if (M <= 0 || N <= 0 || !(eps >= 0.f) || !isfinite(eps)) return TP_ERR_SHAPE;
  if (M > kIntMax) return TP_ERR_UNSUPPORTED;
  if (bad_alias(residual, res_dt, y, y_dt, M * N)) return TP_ERR_SHAPE;
  const size_t es = esize(dt), ys = esize(y_dt), rs = esize(res_dt);
  if (!aligned(y, ys) || !aligned(yn, es) || !aligned(gamma, es) || (residual && !aligned(residual, rs)))
    return TP_ERR_ALIGN;
  bool fused = dt == TP_BF16 && N % 8 == 0 && aligned(y, 16) && aligned(yn, 16) && aligned(gamma, 16) &&
               (!residual || aligned(residual, 16));
  for (int64_t r = 0; r < R; ++r) {
    if (!aligned(partials[r], 4)) return TP_ERR_ALIGN;
    fused = fused && aligned(partials[r], 16);
  }
  if (fused)
    return tpl::reduce_rmsnorm(partials, (int)R, residual, res_dt == TP_F32, y, y_dt == TP_F32, gamma,
                               yn, M, N, eps, as_stream(stream));
  // other layouts: the two unfused calls (same results)
  const tp_status st = tp_reduce_partials(partials, R, residual, res_dt, y, M, N, y_dt, stream);
  if (st != TP_OK) return st;
  return tp_rmsnorm(y, y_dt, gamma, yn, M, N, eps, dt, stream);
}

size_t tp_paged_attention_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_context_len,
                                    int64_t block_size) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || max_context_len <= 0 || block_size < 16 ||
      block_size % 16)
    return 0;
  return tpl::attn_paged_workspace(B, Hq, Hkv, max_context_len, block_size);
}

static tp_status paged_decode_common(const void* q, const int64_t qs[2], const void* k_pool,
                                     const void* v_pool, const int64_t ps[3], int64_t num_blocks,
                                     const int32_t* block_table, int64_t table_stride,
                                     const int32_t* context_lens, int64_t max_context_len,
                                     int64_t block_size, void* o, const int64_t os[2], int64_t B,
                                     int64_t Hq, int64_t Hkv, int64_t D, float scale, tp_dtype dt,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     const void* k_new, const void* v_new, int64_t new_stride) {
  if (!q || !qs || !k_pool || !v_pool || !ps || !block_table || !context_lens || !o || !os)
    return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv || num_blocks <= 0 || max_context_len <= 0)
    return TP_ERR_SHAPE;
  if (!isfinite(scale)) return TP_ERR_SHAPE;
  if (block_size <= 0 || table_stride < (max_context_len + block_size - 1) / block_size) return TP_ERR_SHAPE;
  if (dt != TP_BF16 || D != 128 || block_size < 16 || block_size % 16) return TP_ERR_UNSUPPORTED;
  if (Hq / Hkv > 32 || B > 65535 || Hkv > 65535 || max_context_len > kIntMax) return TP_ERR_UNSUPPORTED;
  if (num_blocks > kIntMax) return TP_ERR_UNSUPPORTED;
  for (int i = 0; i < 3; ++i) {
    if (ps[i] < 0) return TP_ERR_SHAPE;
    if (ps[i] % 8) return TP_ERR_ALIGN;
  }
  for (int i = 0; i < 2; ++i) {
    if (qs[i] < 0 || os[i] < 0) return TP_ERR_SHAPE;
    if (qs[i] % 8 || os[i] % 4) return TP_ERR_ALIGN;
  }
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 8) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4))
    return TP_ERR_ALIGN;
  // one block's rows must be addressable with 31-bit byte offsets
  if (((block_size - 1) * ps[1] + D) * 2 >= (int64_t{1} << 31)) return TP_ERR_UNSUPPORTED;
  const size_t need = tpl::attn_paged_workspace(B, Hq, Hkv, max_context_len, block_size);
  if (need > 0 && (!workspace || workspace_bytes < need)) return TP_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 4)) return TP_ERR_ALIGN;
  return tpl::attn_decode_paged(q, qs, k_pool, v_pool, ps, num_blocks, block_table, table_stride,
                                context_lens, max_context_len, block_size, o, os, B, Hq, Hkv, scale,
                                workspace, as_stream(stream), k_new, v_new, new_stride);
}

tp_status tp_paged_attention_decode(const void* q, const int64_t qs[2], const void* k_pool,
                                    const void* v_pool, const int64_t ps[3], int64_t num_blocks,
                                    const int32_t* block_table, int64_t table_stride,
                                    const int32_t* context_lens, int64_t max_context_len,
                                    int64_t block_size, void* o, const int64_t os[2], int64_t B,
                                    int64_t Hq, int64_t Hkv, int64_t D, float scale, tp_dtype dt,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return paged_decode_common(q, qs, k_pool, v_pool, ps, num_blocks, block_table, table_stride,
                             context_lens, max_context_len, block_size, o, os, B, Hq, Hkv, D, scale,
                             dt, workspace, workspace_bytes, stream, nullptr, nullptr, 0);
}

tp_status tp_paged_decode_attention_append(
    const void* q, const int64_t qs[2], const void* k_new, const void* v_new, int64_t new_stride,
    void* k_pool, void* v_pool, const int64_t ps[3], int64_t num_blocks, const int32_t* block_table,
    int64_t table_stride, const int32_t* context_lens, int64_t max_context_len, int64_t block_size,
    void* o, const int64_t os[2], int64_t B, int64_t Hq, int64_t Hkv, int64_t D, float scale,
    tp_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new) return TP_ERR_NULL;
  if (new_stride < Hkv * D) return TP_ERR_SHAPE;
  if (new_stride % 8 || !aligned(k_new, 16) || !aligned(v_new, 16)) return TP_ERR_ALIGN;
  // every other argument as tp_paged_attention_decode, which validates them
  // and then runs the fused kernel when given the new rows
  return paged_decode_common(q, qs, k_pool, v_pool, ps, num_blocks, block_table, table_stride,
                             context_lens, max_context_len, block_size, o, os, B, Hq, Hkv, D, scale,
                             dt, workspace, workspace_bytes, stream, k_new, v_new, new_stride);
}

tp_status tp_paged_kv_append(const void* k_new, const void* v_new, int64_t new_stride, void* k_pool,
                             void* v_pool, const int64_t ps[3], int64_t num_blocks,
                             const int32_t* block_table, int64_t table_stride,
                             const int32_t* context_lens, int64_t B, int64_t Hkv, int64_t D,
                             int64_t block_size, tp_dtype dt, void* stream) {
  if (!k_new || !v_new || !k_pool || !v_pool || !ps || !block_table || !context_lens) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (B <= 0 || Hkv <= 0 || D <= 0 || num_blocks <= 0 || table_stride <= 0 || block_size <= 0)
    return TP_ERR_SHAPE;
  if (new_stride < Hkv * D) return TP_ERR_SHAPE;
  for (int i = 0; i < 3; ++i)
    if (ps[i] < 0) return TP_ERR_SHAPE;
  if (dt != TP_BF16) return TP_ERR_UNSUPPORTED;
  if (!aligned(k_new, 2) || !aligned(v_new, 2) || !aligned(k_pool, 2) || !aligned(v_pool, 2) ||
      !aligned(block_table, 4) || !aligned(context_lens, 4))
    return TP_ERR_ALIGN;
  return tpl::paged_kv_append(k_new, v_new, new_stride, k_pool, v_pool, ps, num_blocks, block_table,
                              table_stride, table_stride, context_lens, B, Hkv, D, block_size,
                              as_stream(stream));
}

tp_status tp_vocab_argmax_local(const float* logits, int64_t M, int64_t V_r, int64_t vocab_offset,
                                float* max_val, int64_t* max_idx, void* stream) {
  if (!logits || !max_val || !max_idx) return TP_ERR_NULL;
  if (M <= 0 || V_r <= 0 || vocab_offset < 0) return TP_ERR_SHAPE;
  if (M > kIntMax || V_r > kIntMax) return TP_ERR_UNSUPPORTED;
  if (!aligned(logits, 4) || !aligned(max_val, 4) || !aligned(max_idx, 8)) return TP_ERR_ALIGN;
  const bool vec = V_r % 4 == 0 && aligned(logits, 16);
  return tpl::vocab_argmax_local(logits, M, V_r, vocab_offset, max_val, max_idx, vec, as_stream(stream));
}

tp_status tp_vocab_argmax_reduce(const float* const* vals, const int64_t* const* idxs, int64_t R,
                                 int64_t M, float* out_val, int64_t* out_idx, void* stream) {
  if (!vals || !idxs || !out_val || !out_idx) return TP_ERR_NULL;
  if (R < 1 || R > tpl::kMaxArgmaxRanks || M <= 0) return TP_ERR_SHAPE;
  for (int64_t r = 0; r < R; ++r) {
    if (!vals[r] || !idxs[r]) return TP_ERR_NULL;
    if (!aligned(vals[r], 4) || !aligned(idxs[r], 8)) return TP_ERR_ALIGN;
  }
  if (!aligned(out_val, 4) || !aligned(out_idx, 8)) return TP_ERR_ALIGN;
  return tpl::vocab_argmax_reduce(vals, idxs, (int)R, M, out_val, out_idx, as_stream(stream));
}

tp_status tp_rmsnorm(const void* x, tp_dtype x_dt, const void* gamma, void* y, int64_t M, int64_t N,
                     float eps, tp_dtype dt, void* stream) {
  if (!x || !gamma || !y) return TP_ERR_NULL;
  if (!dtype_ok(dt) || !dtype_ok(x_dt)) return TP_ERR_DTYPE;
  if (M <= 0 || N <= 0 || !(eps >= 0.f) || !isfinite(eps)) return TP_ERR_SHAPE;
  if (M > kIntMax) return TP_ERR_UNSUPPORTED;
  const size_t es = esize(dt);
  if (!aligned(x, esize(x_dt)) || !aligned(gamma, es) || !aligned(y, es)) return TP_ERR_ALIGN;
  const bool vec = dt == TP_BF16 && (N % 8 == 0) && aligned(x, 16) && aligned(gamma, 16) &&
                   aligned(y, 16);
  return tpl::rmsnorm(x, x_dt == TP_F32, gamma, y, M, N, eps, dt == TP_BF16, vec, as_stream(stream));
}

const char* tp_status_string(tp_status s) {
  switch (s) {
    case TP_OK: return "ok";
    case TP_ERR_NULL: return "null pointer argument";
    case TP_ERR_SHAPE: return "invalid or inconsistent sizes";
    case TP_ERR_DTYPE: return "invalid dtype or activation";
    case TP_ERR_ALIGN: return "misaligned pointer or stride";
    case TP_ERR_WORKSPACE: return "workspace missing or too small";
    case TP_ERR_HIP: return "HIP runtime error";
    case TP_ERR_UNSUPPORTED: return "request outside the implemented kernels";
  }
  return "unknown status";
}

const char* tp_last_error(void) { return tpl::g_last_error; }

const char* tp_version(void) { return "tplayer 0.1 (gfx950)"; }

}  // extern "C"
