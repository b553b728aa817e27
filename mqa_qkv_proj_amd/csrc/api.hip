// C ABI of the library: host-side validation and dispatch to the gfx950 kernels.
// Every check runs before any HIP call, so a rejected call touches no device.
#include <algorithm>
#include <mutex>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "launch.h"
#include "mqa_qkv.h"

namespace {

thread_local char g_err[512] = "";

mqkv_status fail(mqkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

mqkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MQKV_OK;
  return fail(MQKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(mqkv_dtype t) { return t == MQKV_F32 || t == MQKV_BF16; }
int elem_align(mqkv_dtype t) { return t == MQKV_BF16 ? 8 : 4; }  // elements per 16 bytes
int elem_size(mqkv_dtype t) { return t == MQKV_BF16 ? 2 : 4; }

// Shared head-shape checks.
mqkv_status check_heads(int32_t H_q, int32_t H_kv, int32_t d) {
  if (H_q < 1 || H_kv < 1) return fail(MQKV_ERR_INVALID, "H_q=%d and H_kv=%d must be >= 1", H_q, H_kv);
  if (H_q % H_kv != 0) return fail(MQKV_ERR_INVALID, "H_q=%d is not a multiple of H_kv=%d", H_q, H_kv);
  if (d < 1) return fail(MQKV_ERR_INVALID, "d=%d must be >= 1", d);
  if (d != 64 && d != 128) return fail(MQKV_ERR_UNSUPPORTED, "head dim d=%d not supported (64 or 128)", d);
  return MQKV_OK;
}

bool split_ok(int32_t s) { return s >= 32 && s <= 65536 && s % 32 == 0; }

}  // namespace

extern "C" {

const char* mqkv_status_string(mqkv_status s) {
  switch (s) {
    case MQKV_OK: return "ok";
    case MQKV_ERR_INVALID: return "invalid argument";
    case MQKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case MQKV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* mqkv_last_error(void) { return g_err; }

int32_t mqkv_abi_version(void) { return 108; }

size_t qkv_proj_workspace_bytes(int64_t M, int64_t hidden, int32_t H_q, int32_t H_kv, int32_t d,
                                mqkv_dtype dtype) {
  if (M < 0 || hidden < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || (d != 64 && d != 128) ||
      dtype != MQKV_BF16)
    return 0;
  const int64_t N = (int64_t)(H_q + 2 * (int64_t)H_kv) * d;
  const mqkv::SkinnyPlan p = mqkv::plan_skinny(M, hidden, N);
  return p.ok ? p.ws_bytes : 0;
}

}  // extern "C"

namespace {

// Validation and dispatch shared by qkv_proj and qkv_proj_append.
mqkv_status proj_common(const void* x, const void* w_qkv, const void* bias, void* qkv, int64_t M,
                        int64_t hidden, int32_t H_q, int32_t H_kv, int32_t d, mqkv_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream, const mqkv::ProjEpilogue& app,
                        const char* what) {
  if (!dtype_ok(dtype)) return fail(MQKV_ERR_INVALID, "dtype %d unknown", (int)dtype);
  mqkv_status st = check_heads(H_q, H_kv, d);
  if (st != MQKV_OK) return st;
  if (M < 0) return fail(MQKV_ERR_INVALID, "M=%lld < 0", (long long)M);
  if (hidden < 1) return fail(MQKV_ERR_INVALID, "hidden=%lld < 1", (long long)hidden);
  if (hidden % elem_align(dtype) != 0)
    return fail(MQKV_ERR_INVALID, "hidden=%lld must be a multiple of %d", (long long)hidden, elem_align(dtype));
  if (!x || !w_qkv || !qkv) return fail(MQKV_ERR_INVALID, "x, w_qkv and qkv must be non-NULL");
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(qkv) || (bias && !aligned16(bias)) ||
      (workspace && !aligned16(workspace)))
    return fail(MQKV_ERR_INVALID, "data pointers must be 16-byte aligned");
  const int64_t N = (int64_t)(H_q + 2 * (int64_t)H_kv) * d;
  if (M > 0x7fffffff || hidden > 0x7fffffff || N > 0x7fffffff)
    return fail(MQKV_ERR_UNSUPPORTED, "sizes beyond 2^31-1 are not supported");
  if (M == 0) return MQKV_OK;
  return hip_status(mqkv::launch_qkv_gemm(x, w_qkv, bias, qkv, M, hidden, N, dtype == MQKV_BF16, workspace,
                                          workspace ? workspace_bytes : 0, (hipStream_t)stream, app),
                    what);
}

}  // namespace

extern "C" {

mqkv_status qkv_proj(const void* x, const void* w_qkv, const void* bias, void* qkv, int64_t M,
                     int64_t hidden, int32_t H_q, int32_t H_kv, int32_t d, mqkv_dtype dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const mqkv::ProjEpilogue none{};
  return proj_common(x, w_qkv, bias, qkv, M, hidden, H_q, H_kv, d, dtype, workspace, workspace_bytes, stream,
                     none, "qkv_proj launch");
}

mqkv_status qkv_proj_rope(const void* x, const void* w_qkv, const void* bias, void* qkv,
                          const int32_t* positions, const float* inv_freq, int64_t M, int64_t hidden,
                          int32_t H_q, int32_t H_kv, int32_t d, mqkv_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (!positions || !inv_freq) return fail(MQKV_ERR_INVALID, "positions and inv_freq must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(positions) & 3u) != 0 || (reinterpret_cast<uintptr_t>(inv_freq) & 3u) != 0)
    return fail(MQKV_ERR_INVALID, "positions and inv_freq must be 4-byte aligned");
  const mqkv_status st = check_heads(H_q, H_kv, d);
  if (st != MQKV_OK) return st;
  if ((int64_t)(H_q + 2 * (int64_t)H_kv) * d > 0x7fffffff)
    return fail(MQKV_ERR_UNSUPPORTED, "sizes beyond 2^31-1 are not supported");
  mqkv::ProjEpilogue ep{};
  ep.kcol = H_q * d;
  ep.vcol = (H_q + H_kv) * d;
  ep.inv_freq = inv_freq;
  ep.pos = positions;
  ep.rope_d = d;
  return proj_common(x, w_qkv, bias, qkv, M, hidden, H_q, H_kv, d, dtype, workspace, workspace_bytes, stream,
                     ep, "qkv_proj_rope launch");
}

}  // extern "C"

namespace {

// Validation and dispatch shared by qkv_proj_append and qkv_proj_append_rope.
mqkv_status append_common(const void* x, const void* w_qkv, const void* bias, void* qkv, void* k_cache,
                          void* v_cache, const int32_t* seq_lens, const float* inv_freq, int32_t B,
                          int64_t hidden, int32_t H_q, int32_t H_kv, int32_t d, int32_t L_max,
                          mqkv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream,
                          const char* what) {
  if (!k_cache || !v_cache || !seq_lens)
    return fail(MQKV_ERR_INVALID, "k_cache, v_cache and seq_lens must be non-NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0)
    return fail(MQKV_ERR_INVALID, "caches must be 16-byte aligned and seq_lens 4-byte aligned");
  if (B < 0) return fail(MQKV_ERR_INVALID, "B=%d < 0", B);
  if (L_max < 1) return fail(MQKV_ERR_INVALID, "L_max=%d must be >= 1", L_max);
  const mqkv_status st = check_heads(H_q, H_kv, d);
  if (st != MQKV_OK) return st;
  if ((int64_t)(H_q + 2 * (int64_t)H_kv) * d > 0x7fffffff)
    return fail(MQKV_ERR_UNSUPPORTED, "sizes beyond 2^31-1 are not supported");
  mqkv::ProjEpilogue ep{};
  ep.k_cache = k_cache;
  ep.v_cache = v_cache;
  ep.seq_lens = seq_lens;
  ep.kcol = H_q * d;
  ep.vcol = (H_q + H_kv) * d;
  ep.L_max = L_max;
  ep.inv_freq = inv_freq;  // nullptr: no rotation
  ep.pos = nullptr;        // rotation at seq_lens[b] - 1
  ep.rope_d = d;
  return proj_common(x, w_qkv, bias, qkv, B, hidden, H_q, H_kv, d, dtype, workspace, workspace_bytes, stream,
                     ep, what);
}

}  // namespace

extern "C" {

mqkv_status qkv_proj_append(const void* x, const void* w_qkv, const void* bias, void* qkv, void* k_cache,
                            void* v_cache, const int32_t* seq_lens, int32_t B, int64_t hidden, int32_t H_q,
                            int32_t H_kv, int32_t d, int32_t L_max, mqkv_dtype dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  return append_common(x, w_qkv, bias, qkv, k_cache, v_cache, seq_lens, nullptr, B, hidden, H_q, H_kv, d, L_max,
                       dtype, workspace, workspace_bytes, stream, "qkv_proj_append launch");
}

mqkv_status qkv_proj_append_rope(const void* x, const void* w_qkv, const void* bias, void* qkv, void* k_cache,
                                 void* v_cache, const int32_t* seq_lens, const float* inv_freq, int32_t B,
                                 int64_t hidden, int32_t H_q, int32_t H_kv, int32_t d, int32_t L_max,
                                 mqkv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (!inv_freq) return fail(MQKV_ERR_INVALID, "inv_freq must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(inv_freq) & 3u) != 0)
    return fail(MQKV_ERR_INVALID, "inv_freq must be 4-byte aligned");
  return append_common(x, w_qkv, bias, qkv, k_cache, v_cache, seq_lens, inv_freq, B, hidden, H_q, H_kv, d, L_max,
                       dtype, workspace, workspace_bytes, stream, "qkv_proj_append_rope launch");
}

size_t gqa_attn_prefill_workspace_bytes(int32_t B, int32_t L_kv, int32_t H_kv, int32_t d,
                                        mqkv_dtype in_dtype) {
  if (!dtype_ok(in_dtype) || B < 0 || L_kv < 1 || H_kv < 1 || (d != 64 && d != 128)) return 0;
  return mqkv::prefill_workspace_bytes(B, L_kv, H_kv, d, in_dtype == MQKV_BF16);
}

mqkv_status gqa_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t B, int32_t L_q, int32_t L_kv, int32_t H_q, int32_t H_kv,
                             int32_t d, int64_t q_tok_stride, int64_t kv_tok_stride, int32_t causal,
                             float scale, mqkv_dtype in_dtype, mqkv_dtype o_dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype))
    return fail(MQKV_ERR_INVALID, "dtype %d/%d unknown", (int)in_dtype, (int)o_dtype);
  mqkv_status st = check_heads(H_q, H_kv, d);
  if (st != MQKV_OK) return st;
  if (B < 0 || L_q < 0) return fail(MQKV_ERR_INVALID, "B=%d and L_q=%d must be >= 0", B, L_q);
  if (L_kv < 1) return fail(MQKV_ERR_INVALID, "L_kv=%d must be >= 1", L_kv);
  if (causal != 0 && causal != 1) return fail(MQKV_ERR_INVALID, "causal must be 0 or 1");
  if (causal && L_q > L_kv)
    return fail(MQKV_ERR_INVALID, "causal attention needs L_q (%d) <= L_kv (%d)", L_q, L_kv);
  if (!isfinite(scale) || scale < 0.0f) return fail(MQKV_ERR_INVALID, "scale must be finite and >= 0");
  if (!q || !k || !v || !o) return fail(MQKV_ERR_INVALID, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(MQKV_ERR_INVALID, "data pointers must be 16-byte aligned");
  const int ea = elem_align(in_dtype);
  if (q_tok_stride < (int64_t)H_q * d || kv_tok_stride < (int64_t)H_kv * d)
    return fail(MQKV_ERR_INVALID, "token strides must cover all heads (q >= %d, kv >= %d)", H_q * d,
                H_kv * d);
  if (q_tok_stride % ea != 0 || kv_tok_stride % ea != 0)
    return fail(MQKV_ERR_INVALID, "token strides must be multiples of %d elements", ea);
  if (in_dtype == MQKV_F32 && o_dtype != MQKV_F32)
    return fail(MQKV_ERR_UNSUPPORTED, "fp32 inputs need an fp32 output");
  if ((int64_t)L_kv * kv_tok_stride * elem_size(in_dtype) >= ((int64_t)1 << 31) ||
      (int64_t)L_q * q_tok_stride * elem_size(in_dtype) >= ((int64_t)1 << 31))
    return fail(MQKV_ERR_UNSUPPORTED, "one sequence's rows must span less than 2 GiB");
  if (B == 0 || L_q == 0) return MQKV_OK;
  const size_t need = mqkv::prefill_workspace_bytes(B, L_kv, H_kv, d, in_dtype == MQKV_BF16);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(MQKV_ERR_INVALID, "workspace must be 16-byte aligned and >= %zu bytes (got %zu)", need,
                workspace_bytes);
  mqkv::PrefillArgs a{q,      k,     v,         o,         lse,       B,         L_q,
                      L_kv,   H_q,   H_kv,      d,         q_tok_stride, kv_tok_stride,
                      causal != 0, scale, in_dtype == MQKV_BF16, o_dtype == MQKV_BF16,
                      workspace, workspace_bytes};
  return hip_status(mqkv::launch_prefill(a, (hipStream_t)stream), "gqa_attn_prefill launch");
}

size_t gqa_attn_prefill_varlen_workspace_bytes(int32_t B, int32_t max_L_kv, int32_t total_q, int32_t H_q,
                                               int32_t H_kv, int32_t d) {
  if (B < 1 || max_L_kv < 1 || total_q < 0 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || (d != 64 && d != 128))
    return 0;
  return mqkv::prefill_varlen_workspace_bytes(B, max_L_kv, total_q, H_q, H_kv, d);
}

mqkv_status gqa_attn_prefill_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t B,
                                    int32_t max_L_q, int32_t max_L_kv, int32_t total_q, int32_t total_kv,
                                    int32_t H_q, int32_t H_kv, int32_t d, int64_t q_tok_stride,
                                    int64_t kv_tok_stride, int32_t causal, float scale, mqkv_dtype in_dtype,
                                    mqkv_dtype o_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype))
    return fail(MQKV_ERR_INVALID, "dtype %d/%d unknown", (int)in_dtype, (int)o_dtype);
  mqkv_status st = check_heads(H_q, H_kv, d);
  if (st != MQKV_OK) return st;
  if (B < 0 || max_L_q < 0 || total_q < 0)
    return fail(MQKV_ERR_INVALID, "B=%d, max_L_q=%d and total_q=%d must be >= 0", B, max_L_q, total_q);
  if (max_L_kv < 1 || total_kv < 1)
    return fail(MQKV_ERR_INVALID, "max_L_kv=%d and total_kv=%d must be >= 1", max_L_kv, total_kv);
  if (causal != 0 && causal != 1) return fail(MQKV_ERR_INVALID, "causal must be 0 or 1");
  if (!isfinite(scale) || scale < 0.0f) return fail(MQKV_ERR_INVALID, "scale must be finite and >= 0");
  if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_kv)
    return fail(MQKV_ERR_INVALID, "q, k, v, o and the cu_seqlens arrays must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_kv) & 3u))
    return fail(MQKV_ERR_INVALID, "data pointers must be 16-byte aligned (cu_seqlens 4-byte)");
  const int ea = elem_align(in_dtype);
  if (q_tok_stride < (int64_t)H_q * d || kv_tok_stride < (int64_t)H_kv * d)
    return fail(MQKV_ERR_INVALID, "token strides must cover all heads (q >= %d, kv >= %d)", H_q * d,
                H_kv * d);
  if (q_tok_stride % ea != 0 || kv_tok_stride % ea != 0)
    return fail(MQKV_ERR_INVALID, "token strides must be multiples of %d elements", ea);
  if (in_dtype != MQKV_BF16) return fail(MQKV_ERR_UNSUPPORTED, "packed variable-length batches need bf16 inputs");
  if ((int64_t)max_L_kv * kv_tok_stride * 2 >= ((int64_t)1 << 31))
    return fail(MQKV_ERR_UNSUPPORTED, "one sequence's rows must span less than 2 GiB");
  if (B == 0 || max_L_q == 0 || total_q == 0) return MQKV_OK;
  const size_t need = mqkv::prefill_workspace_bytes(B, max_L_kv, H_kv, d, true);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(MQKV_ERR_INVALID, "workspace must be 16-byte aligned and >= %zu bytes (got %zu)", need,
                workspace_bytes);
  mqkv::PrefillArgs a{q,       k,     v,         o,         lse,       B,         max_L_q,
                      max_L_kv, H_q,  H_kv,      d,         q_tok_stride, kv_tok_stride,
                      causal != 0, scale, true, o_dtype == MQKV_BF16,
                      workspace, workspace_bytes};
  a.cu_q = cu_seqlens_q;
  a.cu_kv = cu_seqlens_kv;
  a.total_q = total_q;
  a.total_kv = total_kv;
  return hip_status(mqkv::launch_prefill(a, (hipStream_t)stream), "gqa_attn_prefill_varlen launch");
}

size_t gqa_attn_prefill_fp8_workspace_bytes(int32_t B, int32_t L_q, int32_t L_kv, int32_t H_q, int32_t H_kv,
                                            int32_t d) {
  if (B < 1 || L_q < 1 || L_kv < 1 || H_q < 1 || H_kv < 1 || d != 128) return 0;
  return mqkv::prefill_fp8_workspace_bytes(B, L_q, L_kv, H_q, H_kv, d);
}

mqkv_status gqa_attn_prefill_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const float* signs, int32_t B, int32_t L_q, int32_t L_kv, int32_t H_q,
                                 int32_t H_kv, int32_t d, int64_t q_tok_stride, int64_t kv_tok_stride,
                                 int32_t causal, float scale, mqkv_dtype o_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (!dtype_ok(o_dtype)) return fail(MQKV_ERR_INVALID, "dtype %d unknown", (int)o_dtype);
  mqkv_status st = check_heads(H_q, H_kv, d);
  if (st != MQKV_OK) return st;
  if (d != 128) return fail(MQKV_ERR_UNSUPPORTED, "FP8 prefill supports d=128 only (got %d)", d);
  if (B < 0 || L_q < 0) return fail(MQKV_ERR_INVALID, "B=%d and L_q=%d must be >= 0", B, L_q);
  if (L_kv < 1) return fail(MQKV_ERR_INVALID, "L_kv=%d must be >= 1", L_kv);
  if (causal != 0 && causal != 1) return fail(MQKV_ERR_INVALID, "causal must be 0 or 1");
  if (causal && L_q > L_kv)
    return fail(MQKV_ERR_INVALID, "causal attention needs L_q (%d) <= L_kv (%d)", L_q, L_kv);
  if (!isfinite(scale) || scale < 0.0f) return fail(MQKV_ERR_INVALID, "scale must be finite and >= 0");
  if (!q || !k || !v || !o) return fail(MQKV_ERR_INVALID, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)) ||
      (signs && !aligned16(signs)))
    return fail(MQKV_ERR_INVALID, "data pointers must be 16-byte aligned");
  if (q_tok_stride < (int64_t)H_q * d || kv_tok_stride < (int64_t)H_kv * d)
    return fail(MQKV_ERR_INVALID, "token strides must cover all heads (q >= %d, kv >= %d)", H_q * d,
                H_kv * d);
  if (q_tok_stride % 8 != 0 || kv_tok_stride % 8 != 0)
    return fail(MQKV_ERR_INVALID, "token strides must be multiples of 8 elements");
  if ((int64_t)L_kv * kv_tok_stride * 2 >= ((int64_t)1 << 31) || (int64_t)L_q * q_tok_stride * 2 >= ((int64_t)1 << 31))
    return fail(MQKV_ERR_UNSUPPORTED, "one sequence's rows must span less than 2 GiB");
  if (B == 0 || L_q == 0) return MQKV_OK;
  const size_t need = mqkv::prefill_fp8_workspace_bytes(B, L_q, L_kv, H_q, H_kv, d);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(MQKV_ERR_INVALID, "workspace must be 16-byte aligned and >= %zu bytes (got %zu)", need,
                workspace_bytes);
  mqkv::PrefillArgs a{q,      k,     v,         o,         lse,       B,         L_q,
                      L_kv,   H_q,   H_kv,      d,         q_tok_stride, kv_tok_stride,
                      causal != 0, scale, true, o_dtype == MQKV_BF16,
                      workspace, workspace_bytes};
  a.fp8 = true;
  a.signs = signs;
  return hip_status(mqkv::launch_prefill(a, (hipStream_t)stream), "gqa_attn_prefill_fp8 launch");
}

}  // extern "C"

namespace {

// Host validation of a decode call (gqa_attn_decode, gqa_attn_decode_noalloc).
mqkv_status decode_check(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                         void* o, float* lse, int32_t B, int32_t H_q, int32_t H_kv, int32_t d, int32_t L_max,
                         int64_t q_tok_stride, float scale, int32_t kv_split, mqkv_dtype in_dtype,
                         mqkv_dtype o_dtype) {
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype))
    return fail(MQKV_ERR_INVALID, "dtype %d/%d unknown", (int)in_dtype, (int)o_dtype);
  mqkv_status st = check_heads(H_q, H_kv, d);
  if (st != MQKV_OK) return st;
  if (B < 0) return fail(MQKV_ERR_INVALID, "B=%d must be >= 0", B);
  if (L_max < 1) return fail(MQKV_ERR_INVALID, "L_max=%d must be >= 1", L_max);
  if (kv_split != 0 && !split_ok(kv_split))
    return fail(MQKV_ERR_INVALID, "kv_split=%d must be 0 or a multiple of 32 in [32, 65536]", kv_split);
  if (!isfinite(scale) || scale < 0.0f) return fail(MQKV_ERR_INVALID, "scale must be finite and >= 0");
  if (!q || !k_cache || !v_cache || !seq_lens || !o)
    return fail(MQKV_ERR_INVALID, "q, k_cache, v_cache, seq_lens and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      (lse && !aligned16(lse)) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(MQKV_ERR_INVALID, "data pointers must be 16-byte aligned (seq_lens 4-byte)");
  const int ea = elem_align(in_dtype);
  if (q_tok_stride < (int64_t)H_q * d || q_tok_stride % ea != 0)
    return fail(MQKV_ERR_INVALID, "q_tok_stride must be >= H_q*d and a multiple of %d", ea);
  if (in_dtype == MQKV_F32 && o_dtype != MQKV_F32)
    return fail(MQKV_ERR_UNSUPPORTED, "fp32 inputs need an fp32 output");
  if ((int64_t)B * L_max * H_kv * d > ((int64_t)1 << 40))
    return fail(MQKV_ERR_UNSUPPORTED, "cache too large");
  return MQKV_OK;
}

// Workspace bytes one call of this dtype uses: partial outputs, then the
// (max, sum, V exponent, -) quads of every slot.
size_t decode_need(int32_t B, int32_t H_q, int32_t H_kv, int32_t d, int32_t L_max, int32_t kv_split, bool bf16) {
  const int slots = mqkv::decode_slots(B, H_q, H_kv, L_max, kv_split, bf16);
  const int64_t per = (int64_t)B * H_q * slots;
  return (size_t)(per * d * 4 + per * 4 * 4 + 256);
}

// Launch of a validated decode call on a workspace of at least decode_need bytes.
mqkv_status decode_launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                          void* o, float* lse, int32_t B, int32_t H_q, int32_t H_kv, int32_t d, int32_t L_max,
                          int64_t q_tok_stride, float scale, int32_t kv_split, void* workspace,
                          mqkv_dtype in_dtype, mqkv_dtype o_dtype, void* stream) {
  const bool bf16 = in_dtype == MQKV_BF16;
  const int32_t n_slot = mqkv::decode_slots(B, H_q, H_kv, L_max, kv_split, bf16);
  const int32_t split = kv_split > 0 ? kv_split : mqkv::decode_auto_split(B, H_q, H_kv, L_max, bf16);
  const int64_t per = (int64_t)B * H_q * n_slot;
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = part_o + per * d;
  mqkv::DecodeArgs a{q,     k_cache, v_cache, seq_lens, o,       lse,     B,
                     H_q,   H_kv,    d,       L_max,    q_tok_stride,     scale,
                     split, n_slot,  part_o,  part_ml,  bf16,    o_dtype == MQKV_BF16};
  a.auto_split = kv_split == 0;
  return hip_status(mqkv::launch_decode(a, (hipStream_t)stream), "gqa_attn_decode launch");
}

// Scratch of gqa_attn_decode_noalloc: a static device array (each GPU the
// library runs on holds its own copy until the process ends).  In host code
// `scratch` names a host-side stand-in, not device memory: host code uses only
// the device address hipGetSymbolAddress returns for it, looked up once per
// device with that device current and kept per device.
static __device__ __align__(256) unsigned char scratch[MQKV_DECODE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

mqkv_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "gqa_attn_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MQKV_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "gqa_attn_decode_noalloc: hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MQKV_ERR_HIP, "gqa_attn_decode_noalloc: no device address for the scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MQKV_OK;
}

}  // namespace

extern "C" {

size_t gqa_attn_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv, int32_t d,
                                       int32_t L_max, int32_t kv_split) {
  if (B < 0 || L_max < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || (d != 64 && d != 128))
    return 0;
  if (kv_split != 0 && !split_ok(kv_split)) return 0;
  // the query has no dtype: size for the larger of the two
  return std::max(decode_need(B, H_q, H_kv, d, L_max, kv_split, true),
                  decode_need(B, H_q, H_kv, d, L_max, kv_split, false));
}

mqkv_status gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, void* o, float* lse, int32_t B, int32_t H_q,
                            int32_t H_kv, int32_t d, int32_t L_max, int64_t q_tok_stride,
                            float scale, int32_t kv_split, void* workspace, size_t workspace_bytes,
                            mqkv_dtype in_dtype, mqkv_dtype o_dtype, void* stream) {
  g_err[0] = 0;
  mqkv_status st = decode_check(q, k_cache, v_cache, seq_lens, o, lse, B, H_q, H_kv, d, L_max, q_tok_stride,
                                scale, kv_split, in_dtype, o_dtype);
  if (st != MQKV_OK || B == 0) return st;
  const size_t need = gqa_attn_decode_workspace_bytes(B, H_q, H_kv, d, L_max, kv_split);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(MQKV_ERR_INVALID, "workspace must be 16-byte aligned and >= %zu bytes (got %zu)", need,
                workspace_bytes);
  return decode_launch(q, k_cache, v_cache, seq_lens, o, lse, B, H_q, H_kv, d, L_max, q_tok_stride, scale,
                       kv_split, workspace, in_dtype, o_dtype, stream);
}

mqkv_status gqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* seq_lens, void* o, float* lse, int32_t B, int32_t H_q,
                                    int32_t H_kv, int32_t d, int32_t L_max, int64_t q_tok_stride, float scale,
                                    int32_t kv_split, mqkv_dtype in_dtype, mqkv_dtype o_dtype, void* stream) {
  g_err[0] = 0;
  mqkv_status st = decode_check(q, k_cache, v_cache, seq_lens, o, lse, B, H_q, H_kv, d, L_max, q_tok_stride,
                                scale, kv_split, in_dtype, o_dtype);
  if (st != MQKV_OK || B == 0) return st;
  const size_t need = decode_need(B, H_q, H_kv, d, L_max, kv_split, in_dtype == MQKV_BF16);
  if (need > (size_t)MQKV_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(MQKV_ERR_UNSUPPORTED,
                "gqa_attn_decode_noalloc: these sizes need %zu bytes of scratch, beyond its %u-byte static buffer "
                "(use gqa_attn_decode with a workspace)", need, (unsigned)MQKV_DECODE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != MQKV_OK) return st;
  return decode_launch(q, k_cache, v_cache, seq_lens, o, lse, B, H_q, H_kv, d, L_max, q_tok_stride, scale,
                       kv_split, ws, in_dtype, o_dtype, stream);
}

mqkv_status gqa_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                                  int32_t B, int32_t H_q, int32_t H_kv, int32_t d, int32_t page_size,
                                  int32_t pages_per_seq, int32_t num_pages, int64_t q_tok_stride, float scale,
                                  int32_t kv_split, void* workspace, size_t workspace_bytes,
                                  mqkv_dtype in_dtype, mqkv_dtype o_dtype, void* stream) {
  g_err[0] = 0;
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype))
    return fail(MQKV_ERR_INVALID, "dtype %d/%d unknown", (int)in_dtype, (int)o_dtype);
  mqkv_status st = check_heads(H_q, H_kv, d);
  if (st != MQKV_OK) return st;
  if (B < 0) return fail(MQKV_ERR_INVALID, "B=%d must be >= 0", B);
  if (page_size < 16 || page_size % 16 != 0)
    return fail(MQKV_ERR_INVALID, "page_size=%d must be a positive multiple of 16", page_size);
  if (pages_per_seq < 1 || num_pages < 1)
    return fail(MQKV_ERR_INVALID, "pages_per_seq=%d and num_pages=%d must be >= 1", pages_per_seq, num_pages);
  if ((int64_t)pages_per_seq * page_size > 0x7fffffff)
    return fail(MQKV_ERR_UNSUPPORTED, "pages_per_seq * page_size beyond 2^31-1");
  const int32_t L_max = pages_per_seq * page_size;
  if (kv_split != 0 && !split_ok(kv_split))
    return fail(MQKV_ERR_INVALID, "kv_split=%d must be 0 or a multiple of 32 in [32, 65536]", kv_split);
  if (!isfinite(scale) || scale < 0.0f) return fail(MQKV_ERR_INVALID, "scale must be finite and >= 0");
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !o)
    return fail(MQKV_ERR_INVALID, "q, k_pages, v_pages, block_table, seq_lens and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) ||
      (lse && !aligned16(lse)) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return fail(MQKV_ERR_INVALID, "data pointers must be 16-byte aligned (seq_lens, block_table 4-byte)");
  const int ea = elem_align(in_dtype);
  if (q_tok_stride < (int64_t)H_q * d || q_tok_stride % ea != 0)
    return fail(MQKV_ERR_INVALID, "q_tok_stride must be >= H_q*d and a multiple of %d", ea);
  if (in_dtype != MQKV_BF16) return fail(MQKV_ERR_UNSUPPORTED, "paged caches need bf16 inputs");
  if ((int64_t)num_pages * page_size * H_kv * d > ((int64_t)1 << 40))
    return fail(MQKV_ERR_UNSUPPORTED, "page pool too large");
  if (B == 0) return MQKV_OK;
  const size_t need = gqa_attn_decode_workspace_bytes(B, H_q, H_kv, d, L_max, kv_split);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(MQKV_ERR_INVALID, "workspace must be 16-byte aligned and >= %zu bytes (got %zu)", need,
                workspace_bytes);
  const int32_t n_slot = mqkv::decode_slots(B, H_q, H_kv, L_max, kv_split, true);
  const int32_t split = kv_split > 0 ? kv_split : mqkv::decode_auto_split(B, H_q, H_kv, L_max, true);
  const int64_t per = (int64_t)B * H_q * n_slot;
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = part_o + per * d;
  mqkv::DecodeArgs a{q,     k_pages, v_pages, seq_lens, o,       lse,     B,
                     H_q,   H_kv,    d,       L_max,    q_tok_stride,     scale,
                     split, n_slot,  part_o,  part_ml,  true,
                     o_dtype == MQKV_BF16};
  a.block_table = block_table;
  a.page_size = page_size;
  a.pages_per_seq = pages_per_seq;
  a.num_pages = num_pages;
  a.auto_split = kv_split == 0;
  return hip_status(mqkv::launch_decode(a, (hipStream_t)stream), "gqa_attn_decode_paged launch");
}

}  // extern "C"
