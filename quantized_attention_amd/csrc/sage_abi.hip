// sage_abi.hip -- the C ABI declared in include/sage.h: host-side argument
// validation, buffer-size arithmetic and kernel launches.  No entry point
// makes a HIP call before every argument has been checked, so argument
// errors are reported identically on machines without a GPU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sage.h"

hipError_t sage_launch_quant_qk(const void* q, const void* k, int bf16, int B, int H, int H_kv,
                                int N, int d, int q_group, int smooth_k, int smooth_q,
                                int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                float* k_mean, float* q_mean, void* ws, hipStream_t st);
hipError_t sage_launch_quant(const void* q, const void* k, const void* v, int bf16, int B, int H,
                             int H_kv, int N, int d, int q_group, int smooth_k, int smooth_q,
                             int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                             float* k_mean, float* q_mean, uint8_t* v_f8, float* v_scale, void* ws,
                             hipStream_t st);
hipError_t sage_launch_mfma_peak(int kind, int iters, int nwg, long long* clocks, uint32_t* sink,
                                 hipStream_t st);
hipError_t sage_launch_delta_s(const void* k, int bf16, const float* k_mean, const float* q_mean,
                               int B, int H, int H_kv, int N, int d, float sm_scale, int bh0,
                               int nbh, int i0, int nrows, int causal, float* out,
                               hipStream_t st);
hipError_t sage_launch_quant_v(const void* v, int bf16, int B, int H_kv, int N, int d,
                               uint8_t* v_f8, float* v_scale, void* ws, hipStream_t st);
hipError_t sage_launch_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                const float* k_scale, const uint8_t* v_f8, const float* v_scale,
                                const uint8_t* v_e8, const float* delta_s, void* o, int bf16_out,
                                float* lse, const float* lse_corr, int B, int H, int H_kv, int N,
                                int d, int q_group, int causal, float sm_scale, int bk0, int nbk,
                                int qt0, int nqt, hipStream_t stream);
hipError_t sage_launch_quant_v_mxfp4(const void* v, int bf16, int B, int H_kv, int N, int d,
                                     uint8_t* v_f4, uint8_t* v_e8, hipStream_t st);
hipError_t sage_launch_lse_correction(const void* q, int bf16, const float* k_mean, int B, int H,
                                      int H_kv, int N, int d, float sm_scale, float* corr,
                                      hipStream_t st);
hipError_t sage_launch_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int H_kv,
                                int N, int d, int b, int h, int32_t* s_out, hipStream_t stream);
size_t sage_ws_quant_qk_bytes(int B, int H_kv, int N, int d);
size_t sage_ws_quant_v_bytes(int B, int H_kv, int N, int d);

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;   // sanity bound on any tensor

sage_status check_shape(int B, int H, int H_kv, int N, int d) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || N <= 0) return SAGE_ERR_SHAPE;
  if (d != 64 && d != 128) return SAGE_ERR_HEADDIM;
  if (H % H_kv != 0) return SAGE_ERR_GQA;
  // every tensor must be indexable: B*H*N*d (and the padded V) below 2^40;
  // B*H is a grid y-dimension (at most 65535); one head's K, V codes (and a
  // Delta S row, 4*N bytes) are read through 32-bit buffer-resource ranges,
  // so the padded N*d must stay below 2^32
  const int64_t npad = ((int64_t)N + SAGE_KV_TILE - 1) / SAGE_KV_TILE * SAGE_KV_TILE;
  if ((int64_t)B * H > 65535 || (int64_t)B * H * npad * d > kMaxElems) return SAGE_ERR_SHAPE;
  if (npad * d >= ((int64_t)1 << 32)) return SAGE_ERR_SHAPE;
  return SAGE_OK;
}

int64_t q_blocks(int N) { return ((int64_t)N + SAGE_BLKQ - 1) / SAGE_BLKQ; }

// One chunk of sage_attn_fwd_smooth_q: `groups` (b, kv head) groups with
// `rows` Q blocks of each of their query heads.
struct SqChunk {
  int64_t groups, rows;
};

// Rows an attention launch should have for its dispatch rounds to fill
// (about 2048 workgroups, 4 rounds at d = 128).
constexpr int64_t kSqTargetRows = 2048;

// `rows` spread evenly over the chunks it takes at most `rmax` at a time,
// rounded up to a multiple of 16 (the Delta S pass's row group) where that
// still fits.
int64_t even_rows(int64_t total, int64_t rmax) {
  const int64_t n = (total + rmax - 1) / rmax;
  const int64_t r = (total + n - 1) / n, r16 = (r + 15) / 16 * 16;
  return r16 <= rmax ? r16 : r;
}

// The chunk for a workspace of `cap` Delta S rows (N floats each), cap >= group:
//  1. whole groups with all their Q blocks, when a multiple of 8 groups (so
//     each (b, kv head) stays on one XCD's L2) fits and its attention launch
//     is no smaller than that of case 2: each Delta S pass then reads the K
//     of its groups once;
//  2. else every group with a range of Q blocks (one pass over K per range);
//  3. else (a workspace smaller than one row per head) one group at a time.
SqChunk smooth_q_chunk(int64_t nbk, int64_t group, int64_t nmb, int64_t cap) {
  const int64_t per = group * nmb;   // rows of one group
  int64_t g = cap / per;
  if (g >= nbk) return {nbk, nmb};
  if (cap < nbk * group) return {1, even_rows(nmb, cap / group)};
  const SqChunk by_rows = {nbk, even_rows(nmb, cap / (nbk * group))};
  g -= g % 8;
  if (g >= 8 && g * per >= by_rows.groups * group * by_rows.rows) {
    const int64_t n = (nbk + g - 1) / g;
    int64_t ge = ((nbk + n - 1) / n + 7) / 8 * 8;
    return {ge < g ? ge : g, nmb};
  }
  return by_rows;
}

// The default workspace: every head's rows for R Q blocks, R enough for
// kSqTargetRows rows in all, at least 32 (a Delta S pass over K per 32 Q
// blocks or fewer), a multiple of 16, at most the number of Q blocks.
int64_t smooth_q_default_rows(int B, int H, int N) {
  const int64_t bh = (int64_t)B * H;
  int64_t r = (kSqTargetRows + bh - 1) / bh;
  r = (r + 15) / 16 * 16;
  if (r < 32) r = 32;
  return r < q_blocks(N) ? r : q_blocks(N);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_q_group(int g) {
  return g == SAGE_QGROUP_BLOCK || g == SAGE_QGROUP_WAVE || g == SAGE_QGROUP_TOKEN;
}

sage_status from_hip(hipError_t e) { return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP; }

}  // namespace

extern "C" {

int sage_abi_version(void) { return SAGE_ABI_VERSION; }

const char* sage_status_str(sage_status s) {
  switch (s) {
    case SAGE_OK: return "ok";
    case SAGE_ERR_NULL: return "null pointer argument";
    case SAGE_ERR_SHAPE: return "invalid shape (B, H, H_kv, N must be positive and sizes bounded)";
    case SAGE_ERR_HEADDIM: return "head dim must be 64 or 128";
    case SAGE_ERR_GQA: return "H must be a multiple of H_kv";
    case SAGE_ERR_DTYPE: return "dtype must be SAGE_FP16 or SAGE_BF16";
    case SAGE_ERR_ARG: return "invalid argument (sm_scale, flag or index)";
    case SAGE_ERR_WORKSPACE: return "workspace missing or too small";
    case SAGE_ERR_HIP: return "HIP launch or runtime error";
    case SAGE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SAGE_ERR_SCRATCH: return "shapes need more than the library's fixed scratch array";
  }
  return "unknown status";
}

sage_status sage_buffer_sizes(int B, int H, int H_kv, int N, int d, int q_group,
                              sage_sizes* out) {
  if (!out) return SAGE_ERR_NULL;
  const sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (!valid_q_group(q_group)) return SAGE_ERR_ARG;
  const size_t b = B, h = H, hk = H_kv, n = N, dd = d, qg = q_group;
  const size_t nq = (n + qg - 1) / qg, nk = (n + SAGE_BLKK - 1) / SAGE_BLKK;
  const size_t npad = (n + SAGE_KV_TILE - 1) / SAGE_KV_TILE * SAGE_KV_TILE;
  out->q_i8 = b * h * n * dd;
  out->q_scale = b * h * nq * sizeof(float);
  out->k_i8 = b * hk * n * dd;
  out->k_scale = b * hk * nk * sizeof(float);
  out->k_mean = b * hk * dd * sizeof(float);
  out->v_f8 = b * hk * npad * dd;
  out->v_scale = b * hk * dd * sizeof(float);
  out->o = b * h * n * dd * 2;
  out->ws_quant_qk = sage_ws_quant_qk_bytes(B, H_kv, N, d);
  out->ws_quant_v = sage_ws_quant_v_bytes(B, H_kv, N, d);
  out->ws_quant_qkv = out->ws_quant_qk + out->ws_quant_v;
  const size_t nmb = (n + SAGE_BLKQ - 1) / SAGE_BLKQ;
  out->q_mean = b * h * nmb * dd * sizeof(float);
  out->ws_smooth_q = (size_t)((int64_t)B * H * smooth_q_default_rows(B, H, N) * N) * sizeof(float);
  out->v_f4 = b * hk * npad * dd / 2;
  out->v_e8 = b * hk * (npad / SAGE_KV_TILE) * 512;
  return SAGE_OK;
}

sage_status sage_quant_qk(const void* q, const void* k, sage_dtype dtype, int B, int H, int H_kv,
                          int N, int d, int q_group, int smooth_k, int smooth_q, int8_t* q_i8,
                          float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                          float* q_mean, void* workspace, size_t ws_bytes, void* stream) {
  if (!q || !k || !q_i8 || !q_scale || !k_i8 || !k_scale || !k_mean) return SAGE_ERR_NULL;
  if (smooth_q == 1 && !q_mean) return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!valid_q_group(q_group)) return SAGE_ERR_ARG;
  if (smooth_k != 0 && smooth_k != 1) return SAGE_ERR_ARG;
  if (smooth_q != 0 && smooth_q != 1) return SAGE_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_i8) || !aligned16(k_i8)) return SAGE_ERR_ALIGN;
  if (smooth_k) {
    if (!workspace) return SAGE_ERR_WORKSPACE;
    if (ws_bytes < sage_ws_quant_qk_bytes(B, H_kv, N, d)) return SAGE_ERR_WORKSPACE;
  }
  return from_hip(sage_launch_quant_qk(q, k, dtype == SAGE_BF16, B, H, H_kv, N, d, q_group,
                                       smooth_k, smooth_q, q_i8, q_scale, k_i8, k_scale, k_mean,
                                       q_mean, workspace, (hipStream_t)stream));
}

sage_status sage_quant_qkv(const void* q, const void* k, const void* v, sage_dtype dtype, int B,
                           int H, int H_kv, int N, int d, int q_group, int smooth_k, int smooth_q,
                           int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                           float* k_mean, float* q_mean, uint8_t* v_f8, float* v_scale,
                           void* workspace, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !q_i8 || !q_scale || !k_i8 || !k_scale || !k_mean || !v_f8 || !v_scale)
    return SAGE_ERR_NULL;
  if (smooth_q == 1 && !q_mean) return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!valid_q_group(q_group)) return SAGE_ERR_ARG;
  if (smooth_k != 0 && smooth_k != 1) return SAGE_ERR_ARG;
  if (smooth_q != 0 && smooth_q != 1) return SAGE_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_i8) || !aligned16(k_i8) ||
      !aligned16(v_f8))
    return SAGE_ERR_ALIGN;
  if (!workspace) return SAGE_ERR_WORKSPACE;
  if (ws_bytes < sage_ws_quant_qk_bytes(B, H_kv, N, d) + sage_ws_quant_v_bytes(B, H_kv, N, d))
    return SAGE_ERR_WORKSPACE;
  return from_hip(sage_launch_quant(q, k, v, dtype == SAGE_BF16, B, H, H_kv, N, d, q_group,
                                    smooth_k, smooth_q, q_i8, q_scale, k_i8, k_scale, k_mean,
                                    q_mean, v_f8, v_scale, workspace, (hipStream_t)stream));
}

sage_status sage_delta_s(const void* k, sage_dtype dtype, const float* k_mean,
                         const float* q_mean, int B, int H, int H_kv, int N, int d,
                         float sm_scale, int i0, int nrows, float* delta_s, void* stream) {
  if (!k || !k_mean || !q_mean || !delta_s) return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return SAGE_ERR_ARG;
  if (i0 < 0 || nrows < 1 || (int64_t)i0 + nrows > q_blocks(N)) return SAGE_ERR_ARG;
  if ((int64_t)B * H * nrows * N > kMaxElems) return SAGE_ERR_SHAPE;
  if (!aligned16(k) || !aligned16(q_mean) || !aligned16(delta_s)) return SAGE_ERR_ALIGN;
  return from_hip(sage_launch_delta_s(k, dtype == SAGE_BF16, k_mean, q_mean, B, H, H_kv, N, d,
                                      sm_scale, 0, B * H, i0, nrows, 0, delta_s,
                                      (hipStream_t)stream));
}

sage_status sage_quant_v(const void* v, sage_dtype dtype, int B, int H_kv, int N, int d,
                         uint8_t* v_f8, float* v_scale, void* workspace, size_t ws_bytes,
                         void* stream) {
  if (!v || !v_f8 || !v_scale) return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H_kv, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!aligned16(v) || !aligned16(v_f8)) return SAGE_ERR_ALIGN;
  if (!workspace) return SAGE_ERR_WORKSPACE;
  if (ws_bytes < sage_ws_quant_v_bytes(B, H_kv, N, d)) return SAGE_ERR_WORKSPACE;
  return from_hip(sage_launch_quant_v(v, dtype == SAGE_BF16, B, H_kv, N, d, v_f8, v_scale,
                                      workspace, (hipStream_t)stream));
}

sage_status sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                          const float* k_scale, const uint8_t* v_f8, const float* v_scale,
                          void* o, sage_dtype out_dtype, int B, int H, int H_kv, int N, int d,
                          int q_group, int causal, float sm_scale, void* stream) {
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v_f8 || !v_scale || !o) return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (out_dtype != SAGE_FP16 && out_dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!valid_q_group(q_group)) return SAGE_ERR_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_ARG;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return SAGE_ERR_ARG;
  if (!aligned16(q_i8) || !aligned16(k_i8) || !aligned16(v_f8) || !aligned16(o))
    return SAGE_ERR_ALIGN;
  return from_hip(sage_launch_attn_fwd(q_i8, q_scale, k_i8, k_scale, v_f8, v_scale, nullptr,
                                       nullptr, o, out_dtype == SAGE_BF16, nullptr, nullptr, B, H,
                                       H_kv, N, d, q_group, causal, sm_scale, 0, B * H_kv, 0,
                                       (int)q_blocks(N), (hipStream_t)stream));
}

sage_status sage_attn_fwd_lse(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                              const float* k_scale, const uint8_t* v_f8, const float* v_scale,
                              void* o, sage_dtype out_dtype, float* lse, const float* lse_corr,
                              int B, int H, int H_kv, int N, int d, int q_group, int causal,
                              float sm_scale, void* stream) {
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v_f8 || !v_scale || !o || !lse)
    return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (out_dtype != SAGE_FP16 && out_dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!valid_q_group(q_group)) return SAGE_ERR_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_ARG;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return SAGE_ERR_ARG;
  if (!aligned16(q_i8) || !aligned16(k_i8) || !aligned16(v_f8) || !aligned16(o))
    return SAGE_ERR_ALIGN;
  return from_hip(sage_launch_attn_fwd(q_i8, q_scale, k_i8, k_scale, v_f8, v_scale, nullptr,
                                       nullptr, o, out_dtype == SAGE_BF16, lse, lse_corr, B, H,
                                       H_kv, N, d, q_group, causal, sm_scale, 0, B * H_kv, 0,
                                       (int)q_blocks(N), (hipStream_t)stream));
}

sage_status sage_attn_fwd_smooth_q(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                   const float* k_scale, const uint8_t* v_f8,
                                   const float* v_scale, const void* k, sage_dtype k_dtype,
                                   const float* k_mean, const float* q_mean, void* o,
                                   sage_dtype out_dtype, float* lse, const float* lse_corr,
                                   int B, int H, int H_kv, int N, int d, int q_group, int causal,
                                   float sm_scale, void* workspace, size_t ws_bytes,
                                   void* stream) {
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v_f8 || !v_scale || !k || !k_mean || !q_mean ||
      !o)
    return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (k_dtype != SAGE_FP16 && k_dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (out_dtype != SAGE_FP16 && out_dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!valid_q_group(q_group)) return SAGE_ERR_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_ARG;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return SAGE_ERR_ARG;
  if (lse_corr && !lse) return SAGE_ERR_ARG;
  if (!aligned16(q_i8) || !aligned16(k_i8) || !aligned16(v_f8) || !aligned16(o) ||
      !aligned16(k) || !aligned16(q_mean))
    return SAGE_ERR_ALIGN;
  // the chunk: as many Delta S rows (N floats each) as the workspace holds
  const int64_t nmb = q_blocks(N), nbk = (int64_t)B * H_kv, group = H / H_kv;
  const int64_t cap = workspace ? (int64_t)(ws_bytes / ((size_t)N * sizeof(float))) : 0;
  if (cap < group) return SAGE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SAGE_ERR_ALIGN;
  const SqChunk ck = smooth_q_chunk(nbk, group, nmb, cap);
  float* ds = static_cast<float*>(workspace);
  const hipStream_t hs = (hipStream_t)stream;
  for (int64_t g0 = 0; g0 < nbk; g0 += ck.groups) {
    const int ng = (int)(nbk - g0 < ck.groups ? nbk - g0 : ck.groups);
    for (int64_t i0 = 0; i0 < nmb; i0 += ck.rows) {
      const int n = (int)(nmb - i0 < ck.rows ? nmb - i0 : ck.rows);
      hipError_t e = sage_launch_delta_s(k, k_dtype == SAGE_BF16, k_mean, q_mean, B, H, H_kv, N,
                                         d, sm_scale, (int)(g0 * group), (int)(ng * group),
                                         (int)i0, n, causal, ds, hs);
      if (e != hipSuccess) return SAGE_ERR_HIP;
      e = sage_launch_attn_fwd(q_i8, q_scale, k_i8, k_scale, v_f8, v_scale, nullptr, ds, o,
                               out_dtype == SAGE_BF16, lse, lse_corr, B, H, H_kv, N, d, q_group,
                               causal, sm_scale, (int)g0, ng, (int)i0, n, hs);
      if (e != hipSuccess) return SAGE_ERR_HIP;
    }
  }
  return SAGE_OK;
}

sage_status sage_quant_v_mxfp4(const void* v, sage_dtype dtype, int B, int H_kv, int N, int d,
                               uint8_t* v_f4, uint8_t* v_e8, void* stream) {
  if (!v || !v_f4 || !v_e8) return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H_kv, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!aligned16(v) || !aligned16(v_f4) || !aligned16(v_e8)) return SAGE_ERR_ALIGN;
  return from_hip(sage_launch_quant_v_mxfp4(v, dtype == SAGE_BF16, B, H_kv, N, d, v_f4, v_e8,
                                            (hipStream_t)stream));
}

sage_status sage_attn_fwd_mxfp4(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                const float* k_scale, const uint8_t* v_f4, const uint8_t* v_e8,
                                void* o, sage_dtype out_dtype, float* lse, const float* lse_corr,
                                int B, int H, int H_kv, int N, int d, int q_group, int causal,
                                float sm_scale, void* stream) {
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v_f4 || !v_e8 || !o) return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (out_dtype != SAGE_FP16 && out_dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!valid_q_group(q_group)) return SAGE_ERR_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_ARG;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return SAGE_ERR_ARG;
  if (!aligned16(q_i8) || !aligned16(k_i8) || !aligned16(v_f4) || !aligned16(v_e8) ||
      !aligned16(o))
    return SAGE_ERR_ALIGN;
  return from_hip(sage_launch_attn_fwd(q_i8, q_scale, k_i8, k_scale, v_f4, nullptr, v_e8, nullptr,
                                       o, out_dtype == SAGE_BF16, lse, lse_corr, B, H, H_kv, N, d,
                                       q_group, causal, sm_scale, 0, B * H_kv, 0, (int)q_blocks(N),
                                       (hipStream_t)stream));
}

sage_status sage_lse_correction(const void* q, sage_dtype dtype, const float* k_mean, int B, int H,
                                int H_kv, int N, int d, float sm_scale, float* corr,
                                void* stream) {
  if (!q || !k_mean || !corr) return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (dtype != SAGE_FP16 && dtype != SAGE_BF16) return SAGE_ERR_DTYPE;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return SAGE_ERR_ARG;
  if (!aligned16(q)) return SAGE_ERR_ALIGN;
  return from_hip(sage_launch_lse_correction(q, dtype == SAGE_BF16, k_mean, B, H, H_kv, N, d,
                                             sm_scale, corr, (hipStream_t)stream));
}

sage_status sage_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int H_kv, int N,
                          int d, int b, int h, int32_t* s_out, void* stream) {
  if (!q_i8 || !k_i8 || !s_out) return SAGE_ERR_NULL;
  sage_status st = check_shape(B, H, H_kv, N, d);
  if (st != SAGE_OK) return st;
  if (b < 0 || b >= B || h < 0 || h >= H) return SAGE_ERR_ARG;
  if ((int64_t)N * N > ((int64_t)1 << 34)) return SAGE_ERR_SHAPE;
  if (!aligned16(q_i8) || !aligned16(k_i8)) return SAGE_ERR_ALIGN;
  return from_hip(sage_launch_qk_int32(q_i8, k_i8, B, H, H_kv, N, d, b, h, s_out,
                                       (hipStream_t)stream));
}

sage_status sage_mfma_peak(int kind, int iters, int nwg, int64_t* clocks, uint32_t* sink,
                           int* wall_khz, void* stream) {
  if (!clocks || !sink || !wall_khz) return SAGE_ERR_NULL;
  if ((kind != 0 && kind != 1) || iters < 1 || iters > (1 << 18) || nwg < 1 || nwg > 65536)
    return SAGE_ERR_ARG;
  if (!aligned16(clocks) || !aligned16(sink)) return SAGE_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return SAGE_ERR_HIP;
  return from_hip(sage_launch_mfma_peak(kind, iters, nwg, reinterpret_cast<long long*>(clocks),
                                        sink, (hipStream_t)stream));
}

}  // extern "C"
