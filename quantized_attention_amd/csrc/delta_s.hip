// delta_s.hip -- the Delta S table of smooth Q for gfx950.
//
// Algorithm 1 of the SageAttention2 detail page subtracts each Q block's mean
// q_bar_i before quantizing Q and adds GEMV(q_bar_i, K_j^T) back to every
// score of the block; its pipeline figure computes that GEMV before
// quantization, on the smoothed K.  Here, for the flattened heads
// bh = bh0 + u (u < nbh, bh = b*H + h), the 128-token Q blocks i = i0 + r
// (r < nrows) and every key j:
//   out[u][r][j] = fp32(sum_c q_mean[b][h][i][c] * Ks[j][c] * sm_log2),
//   Ks[j][c] = float32(K[b][h_kv][j][c]) - k_mean[b][h_kv][c]
// (the values the K quantizer sees), already in the attention kernel's
// log2 score units.  The products of the float32 operands are exact in
// FP64 and the sums are taken in FP64 on the matrix cores
// (v_mfma_f64_16x16x4_f64), so the stored value is the float32 rounding of
// an almost exact sum: it does not depend on a summation order.  Each table
// entry decides scores that the FP8 rounding of P~ turns into codes, so its
// value must not move with the order of an FP32 sum.
//
// A range of heads and Q blocks at a time: the attention of smoothed Q
// consumes the rows in chunks, so its memory is heads x rows x N for a
// bounded number of heads x rows, never N^2/128 per head.
//
// Causal: Q block i attends keys below (i + 1) * 128 only, so a key past that
// bound never meets row i.  With `causal` set, a workgroup's 64 keys are
// computed for the rows from the first block whose range reaches them (in
// steps of 16 rows) and the entries above each block's diagonal are left
// unwritten: half the FP64 work of a causal table.
//
// Work split: a workgroup of 4 waves owns 64 keys of one (b, h).  Each wave
// keeps its 16 keys' smoothed K rows in registers as FP64 (the B operand,
// d/4 doubles per lane) and walks the range's mean rows 16 at a time (the
// A operand, read from L2).  Contraction index: MFMA s of a lane in
// group g = L/16 uses channel g*d/4 + s for both operands, so the d/4 MFMAs
// cover every channel, and each lane's channels are contiguous.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sage_device.hpp"

namespace sage {

typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int D, bool BF16>
__global__ __launch_bounds__(256) void delta_s_kernel(const void* __restrict__ k,
                                                      const float* __restrict__ k_mean,
                                                      const float* __restrict__ q_mean,
                                                      float* __restrict__ out, int H, int H_kv,
                                                      int N, int nmb, int bh0, int i0,
                                                      int nrows, int causal, float sm_log2) {
  constexpr int QD = D / 4;   // channels per lane group
  // first row of the range that reads this workgroup's keys (all of them
  // unless causal), rounded down to the 16-row MFMA group
  int rbeg = 0;
  if (causal) {
    rbeg = max(0, (int)(blockIdx.x * 64) / kBlkQ - i0) & ~15;
    if (rbeg >= nrows) return;
  }
  const int bh = bh0 + blockIdx.y, b = bh / H, h = bh % H, hk = h / (H / H_kv);
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int col = lane % 16, g = lane / 16;
  const int key = blockIdx.x * 64 + wave * 16 + col;
  // B operand: this lane's key, channels g*QD .. g*QD + QD - 1 (rows past N
  // read row N-1 and are not stored)
  double kb[QD];
  {
    const uint16_t* kr = reinterpret_cast<const uint16_t*>(k) +
                         ((size_t)(b * H_kv + hk) * N + min(key, N - 1)) * D + g * QD;
    const float* km = k_mean + (size_t)(b * H_kv + hk) * D + g * QD;
#pragma unroll
    for (int j = 0; j < QD / 8; ++j) {
      const uint4 u = *reinterpret_cast<const uint4*>(kr + j * 8);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float lo, hi;
        if (BF16) {
          lo = as_float((int)(w[i] << 16));
          hi = as_float((int)(w[i] & 0xFFFF0000u));
        } else {
          lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
          hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
        }
        kb[j * 8 + 2 * i] = (double)(lo - km[j * 8 + 2 * i]);
        kb[j * 8 + 2 * i + 1] = (double)(hi - km[j * 8 + 2 * i + 1]);
      }
    }
  }
  const float* qm = q_mean + ((size_t)bh * nmb + i0) * D;
  float* ob = out + (size_t)blockIdx.y * nrows * N;
  const double scale = (double)sm_log2;
  for (int r0 = rbeg; r0 < nrows; r0 += 16) {
    // A operand: mean row i0 + r0 + col (rows past the range read its last
    // row and are not stored)
    const float* qr = qm + (size_t)min(r0 + col, nrows - 1) * D + g * QD;
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < QD; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(qr + i);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.x, kb[i], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.y, kb[i + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.z, kb[i + 2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.w, kb[i + 3], acc, 0, 0, 0);
    }
    // lane L holds rows 4r + L/16 of the 16x16 result, column L%16 (its key)
    if (key < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = r0 + 4 * r + g;
        if (row < nrows) ob[(size_t)row * N + key] = (float)(acc[r] * scale);
      }
    }
  }
}

}  // namespace sage

hipError_t sage_launch_delta_s(const void* k, int bf16, const float* k_mean, const float* q_mean,
                               int B, int H, int H_kv, int N, int d, float sm_scale, int bh0,
                               int nbh, int i0, int nrows, int causal, float* out,
                               hipStream_t st) {
  using namespace sage;
  const int nmb = (N + kBlkQ - 1) / kBlkQ;
  if (i0 < 0 || nrows <= 0 || i0 + nrows > nmb) return hipErrorInvalidValue;
  if (bh0 < 0 || nbh <= 0 || bh0 + nbh > B * H || nbh > 65535) return hipErrorInvalidValue;
  // causal: keys from (i0 + nrows) * 128 on meet none of the range's rows
  const int nkeys = causal && (int64_t)(i0 + nrows) * kBlkQ < N ? (i0 + nrows) * kBlkQ : N;
  const dim3 grid((nkeys + 63) / 64, nbh), block(256);
  const float sm_log2 = sm_scale * kLog2e;
#define SAGE_DS(DD, BB)                                                                         \
  if (d == DD && (bf16 != 0) == BB) {                                                           \
    hipLaunchKernelGGL((delta_s_kernel<DD, BB>), grid, block, 0, st, k, k_mean, q_mean, out, H, \
                       H_kv, N, nmb, bh0, i0, nrows, causal, sm_log2);                          \
    return hipGetLastError();                                                                   \
  }
  SAGE_DS(64, false)
  SAGE_DS(64, true)
  SAGE_DS(128, false)
  SAGE_DS(128, true)
#undef SAGE_DS
  return hipErrorInvalidValue;
}
