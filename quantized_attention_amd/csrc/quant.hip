// quant.hip -- smoothing and quantization kernels for gfx950 (HBM-bound).
//
//   colstats_partial / colstats_final : per-channel token statistics of a
//       [N][d] slice: the exact FP64 sum of K (its mean smooths K: the
//       SageAttention synthesis page's Smooth K, Algorithm 1 preprocessing
//       on the SageAttention2 detail page) or the absolute max of V (the
//       per-channel FP8 scale of Algorithm 1's psi_V).
//   quant_int8        : per-block INT8 quantization of Q (128 or 32 tokens)
//       and of smoothed K (64 tokens): scale = amax/127, code = RNE(x/scale)
//       (deployment-guide page, quantization formula).
//   quant_int8_tok    : the same rules with one scale per Q token (the
//       per-thread granularity of the SageAttention2 detail page, Figure 4,
//       when each matrix-core lane holds one query).
//   q_block_mean      : per-channel mean of each 128-token Q block (Smooth Q,
//       Algorithm 1 of the SageAttention2 detail page: q_bar_i = mean(Q_i));
//       the quantizers then subtract the mean of the token's own block.
//   quant_v_fp8       : per-channel FP8 E4M3 quantization of V, written
//       transposed and key-permuted in the fragment layout of sage.h.
//   quant_v_mxfp4     : MXFP4 V (E2M1 codes, one E8M0 scale per 32
//       consecutive keys of a channel: the OCP microscaling format the
//       SageAttention3 synthesis page names), in the FP4 fragment layout.
//
// Every read of the fp16/bf16 inputs is a 16-byte vector load of 8 channels
// of one token; consecutive threads read consecutive 16-byte chunks.
// Results are deterministic: FP64 partial sums are combined in a fixed
// order (and are exact when every partial sum fits 53 bits), maxima are
// order-free, and every rounding is an explicit IEEE fp32 operation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sage_device.hpp"

namespace sage {

constexpr int kQuantThreads = 256;
constexpr int kStatChunk = 256;   // tokens per colstats_partial workgroup

template <bool BF16>
__device__ __forceinline__ void unpack8(const uint4 u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (BF16) {
      x[2 * i] = as_float((int)(w[i] << 16));
      x[2 * i + 1] = as_float((int)(w[i] & 0xFFFF0000u));
    } else {
      x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
      x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
  }
}

// The binary32 quotient v / s rounded to nearest, from y = RN(1/s): q0 = RN(v*y)
// is within one ulp of v/s, so the residual v - s*q0 is exact in one FMA and
// q0 + r*y (one more FMA) is the correctly rounded quotient (Markstein's
// theorem; s normal, quotient without overflow).  Three VALU operations
// instead of the full division sequence, bit-identical to x / s.
__device__ __forceinline__ float div_rn(float v, float s, float y) {
  const float q0 = v * y;
  const float r = fmaf(-s, q0, v);
  return fmaf(r, y, q0);
}
// Scales below this use true division (1/s would overflow or lose range).
constexpr float kDivRnMinScale = 1e-30f;

// ---------------------------------------------------------------------------
// Per-channel statistics over a chunk of kStatChunk tokens.
// MODE 0: FP64 sum (K).  MODE 1: abs max (V), stored as float.
// grid (nchunk, B*Hkv); ws layout [B*Hkv][nchunk][D] (double or float).
template <int D, bool BF16, int MODE>
__global__ __launch_bounds__(kQuantThreads) void colstats_partial(const void* __restrict__ x,
                                                                  void* __restrict__ ws, int N,
                                                                  int nchunk) {
  constexpr int TPR = D / 8;                    // threads per token row
  constexpr int RPP = kQuantThreads / TPR;      // rows per pass
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, cg = tid % TPR, rsub = tid / TPR;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x) + (size_t)bh * N * D;
  const int n0 = chunk * kStatChunk, n1 = min(N, n0 + kStatChunk);

  double acc[8];
  float mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { acc[i] = 0.0; mx[i] = 0.f; }
  for (int n = n0 + rsub; n < n1; n += RPP) {
    const uint4 u = *reinterpret_cast<const uint4*>(xs + (size_t)n * D + cg * 8);
    float v[8];
    unpack8<BF16>(u, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (MODE == 0) acc[i] += (double)v[i];
      else mx[i] = fmaxf(mx[i], fabsf(v[i]));
    }
  }
  // combine the RPP row groups in a fixed order
  __shared__ double red[RPP][D];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rsub][cg * 8 + i] = MODE == 0 ? acc[i] : (double)mx[i];
  __syncthreads();
  if (tid < D) {
    if (MODE == 0) {
      double s = 0.0;
      for (int r = 0; r < RPP; ++r) s += red[r][tid];
      reinterpret_cast<double*>(ws)[((size_t)bh * nchunk + chunk) * D + tid] = s;
    } else {
      float m = 0.f;
      for (int r = 0; r < RPP; ++r) m = fmaxf(m, (float)red[r][tid]);
      reinterpret_cast<float*>(ws)[((size_t)bh * nchunk + chunk) * D + tid] = m;
    }
  }
}

// MODE 0: out[bh][c] = float32(sum / N) (the K mean), or 0 when !enable.
// MODE 1: out[bh][c] = float32(amax / 448) (the V scale).
// kQuantThreads threads per (b, kv head): thread (r, c) combines chunks
// r, r + R, ... of channel c in order, then the R partials are combined in
// order (a fixed order, so the result is deterministic).
template <int D, int MODE>
__global__ __launch_bounds__(kQuantThreads) void colstats_final(const void* __restrict__ ws,
                                                                float* __restrict__ out, int N,
                                                                int nchunk, int enable) {
  constexpr int R = kQuantThreads / D;
  const int bh = blockIdx.x, c = threadIdx.x % D, r = threadIdx.x / D;
  __shared__ double red[R][D];
  if (MODE == 0) {
    const double* w = reinterpret_cast<const double*>(ws) + (size_t)bh * nchunk * D + c;
    double s = 0.0;
    if (enable) {
#pragma unroll 8
      for (int k = r; k < nchunk; k += R) s += w[(size_t)k * D];
    }
    red[r][c] = s;
  } else {
    const float* w = reinterpret_cast<const float*>(ws) + (size_t)bh * nchunk * D + c;
    float m = 0.f;
#pragma unroll 8
    for (int k = r; k < nchunk; k += R) m = fmaxf(m, w[(size_t)k * D]);
    red[r][c] = m;
  }
  __syncthreads();
  if (r == 0) {
    if (MODE == 0) {
      double s = red[0][c];
#pragma unroll
      for (int i = 1; i < R; ++i) s += red[i][c];
      out[(size_t)bh * D + c] = enable ? (float)(s / (double)N) : 0.f;
    } else {
      float m = (float)red[0][c];
#pragma unroll
      for (int i = 1; i < R; ++i) m = fmaxf(m, (float)red[i][c]);
      out[(size_t)bh * D + c] = m / 448.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// q_mean[bh][blk][c] = float32(sum / count) over the valid tokens of 128-token
// block blk: float64 partial sums per thread (exact for fp16/bf16 inputs under
// the K mean's condition), combined in a fixed order.  grid (nblk, B*H).
template <int D, bool BF16>
__global__ __launch_bounds__(kQuantThreads) void q_block_mean(const void* __restrict__ x,
                                                              float* __restrict__ q_mean, int N,
                                                              int nblk) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kQuantThreads / TPR;   // rows per pass
  const int blk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int rr = tid / TPR, cg = tid % TPR;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x) + (size_t)bh * N * D;
  double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int p = 0; p < kBlkQ / RPP; ++p) {
    const int row = blk * kBlkQ + p * RPP + rr;
    if (row < N) {
      float v[8];
      unpack8<BF16>(*reinterpret_cast<const uint4*>(xs + (size_t)row * D + cg * 8), v);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] += (double)v[i];
    }
  }
  __shared__ double red[RPP][D];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rr][cg * 8 + i] = s[i];
  __syncthreads();
  if (tid < D) {
    double t = red[0][tid];
    for (int r = 1; r < RPP; ++r) t += red[r][tid];
    const int cnt = min(kBlkQ, N - blk * kBlkQ);
    q_mean[((size_t)bh * nblk + blk) * D + tid] = (float)(t / (double)cnt);
  }
}

// ---------------------------------------------------------------------------
// Block max over the workgroup (all threads get the result).
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

// Mean subtracted before quantizing: none, the head's K mean mean[bh][c], or
// the Q mean of the token's 128-block mean[bh][row / 128][c].
enum { kNoMean = 0, kHeadMean = 1, kBlockMean = 2 };

// Per-block INT8 quantization of one block of BLK tokens x D channels
// (BLK <= 128, so a block lies in one 128-token mean block).
// SMOOTH: which mean (float32) is subtracted first.  grid (nblk, B*heads).
template <int D, int BLK, bool BF16, int SMOOTH>
__global__ __launch_bounds__(kQuantThreads) void quant_int8(const void* __restrict__ x,
                                                            const float* __restrict__ mean,
                                                            int8_t* __restrict__ codes,
                                                            float* __restrict__ scales, int N,
                                                            int nblk) {
  constexpr int TPR = D / 8;
  constexpr int PER = BLK * TPR / kQuantThreads;   // 16-byte chunks per thread
  const int blk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int cg = tid % TPR;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x) + (size_t)bh * N * D;
  int8_t* cs = codes + (size_t)bh * N * D;

  static_assert(BLK <= kBlkQ, "a block lies in one mean block");
  float mu[8];
  const size_t mrow = SMOOTH == kBlockMean
                          ? (size_t)bh * ((N + kBlkQ - 1) / kBlkQ) + (blk * BLK) / kBlkQ
                          : (size_t)bh;
#pragma unroll
  for (int i = 0; i < 8; ++i) mu[i] = SMOOTH ? mean[mrow * D + cg * 8 + i] : 0.f;

  float v[PER][8];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int row = blk * BLK + (p * kQuantThreads + tid) / TPR;
    if (row < N) {
      const uint4 u = *reinterpret_cast<const uint4*>(xs + (size_t)row * D + cg * 8);
      unpack8<BF16>(u, v[p]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (SMOOTH != kNoMean) v[p][i] = v[p][i] - mu[i];
        amax = fmaxf(amax, fabsf(v[p][i]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[p][i] = 0.f;
    }
  }
  __shared__ float red[kQuantThreads / 64];
  amax = block_max(amax, red);
  const float sc = amax / 127.0f;            // IEEE division
  if (tid == 0) scales[(size_t)bh * nblk + blk] = sc;
  auto emit = [&](auto fast_tag) __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const float rs = FAST ? 1.0f / sc : 0.f;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int row = blk * BLK + (p * kQuantThreads + tid) / TPR;
      if (row >= N) continue;
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float q = 0.f;
        if (FAST || sc > 0.f) {   // the fast path implies sc > 0
          const float x = FAST ? div_rn(v[p][i], sc, rs) : v[p][i] / sc;
          q = fminf(fmaxf(__builtin_rintf(x), -127.f), 127.f);
        }
        w[i / 4] |= ((uint32_t)(int)q & 0xFFu) << (8 * (i % 4));
      }
      *reinterpret_cast<uint2*>(cs + (size_t)row * D + cg * 8) = uint2{w[0], w[1]};
    }
  };
  // sc is the same for every thread of the block: branch on the scalar unit.
  if (__builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sc >= kDivRnMinScale ? 1.f : 0.f)))
    emit(std::true_type{});
  else
    emit(std::false_type{});
}

// Per-token INT8 quantization: one scale per token.  The D/8 consecutive
// threads of a token each load 8 channels; the token's amax is reduced by
// xor-shuffles among them.  SMOOTH: subtract the Q mean of the token's
// 128-block first.  grid (ceil(N / tokens per workgroup), B*heads).
template <int D, bool BF16, bool SMOOTH>
__global__ __launch_bounds__(kQuantThreads) void quant_int8_tok(const void* __restrict__ x,
                                                                const float* __restrict__ mean,
                                                                int8_t* __restrict__ codes,
                                                                float* __restrict__ scales, int N) {
  constexpr int TPR = D / 8;
  constexpr int TPB = kQuantThreads / TPR;   // tokens per workgroup
  static_assert(TPR <= 64 && (TPR & (TPR - 1)) == 0, "a token's threads share one wave");
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int row = blockIdx.x * TPB + tid / TPR, cg = tid % TPR;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x) + (size_t)bh * N * D;
  float v[8];
  float amax = 0.f;
  if (row < N) {
    unpack8<BF16>(*reinterpret_cast<const uint4*>(xs + (size_t)row * D + cg * 8), v);
    if (SMOOTH) {
      const float* mu =
          mean + ((size_t)bh * ((N + kBlkQ - 1) / kBlkQ) + row / kBlkQ) * D + cg * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] - mu[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float sc = amax / 127.0f;            // IEEE division
  auto emit = [&](auto fast_tag) __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_tag)::value;
    uint32_t w[2] = {0u, 0u};
    const float rs = FAST ? 1.0f / sc : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = 0.f;
      if (FAST || sc > 0.f) {
        const float y = FAST ? div_rn(v[i], sc, rs) : v[i] / sc;
        q = fminf(fmaxf(__builtin_rintf(y), -127.f), 127.f);
      }
      w[i / 4] |= ((uint32_t)(int)q & 0xFFu) << (8 * (i % 4));
    }
    *reinterpret_cast<uint2*>(codes + (size_t)bh * N * D + (size_t)row * D + cg * 8) =
        uint2{w[0], w[1]};
  };
  if (row < N) {
    if (cg == 0) scales[(size_t)bh * N + row] = sc;
    // the three-operation division when every token of the wave allows it
    if (__builtin_amdgcn_ballot_w64(!(sc >= kDivRnMinScale)) == 0) emit(std::true_type{});
    else emit(std::false_type{});
  }
}

// ---------------------------------------------------------------------------
// FP8 V.  Each 16-byte chunk of the v_f8 layout (sage.h) holds one channel
// and 16 keys, so one wave writes the 64 chunks (kb, cb, p, L = lane) of a
// (128-key tile, 32-channel block) pair for kb, p in {0, 1}: lane L gathers
// its channel cb*32 + L%32 for the 64 keys of its lane half straight from
// HBM (for each key, 32 lanes read 64 contiguous bytes) and stores whole
// 16-byte chunks, consecutive across the wave.  No LDS staging.
// grid (ceil(ntile * D/32 / 4), B*Hkv), 4 waves per workgroup.
template <int D, bool BF16>
__global__ __launch_bounds__(kQuantThreads) void quant_v_fp8(const void* __restrict__ x,
                                                             const float* __restrict__ vscale,
                                                             uint8_t* __restrict__ out, int N,
                                                             int ntile) {
  constexpr int NCB = D / 32;
  const int bh = blockIdx.y, lane = threadIdx.x % 64;
  const int pair = blockIdx.x * (kQuantThreads / 64) + threadIdx.x / 64;
  if (pair >= ntile * NCB) return;
  const int tile = pair / NCB, cb = pair % NCB;
  const int chan = cb * 32 + (lane % 32), g = lane / 32;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x) + (size_t)bh * N * D + chan;
  const float sv = vscale[(size_t)bh * D + chan];
  uint8_t* ot = out + ((size_t)bh * ntile + tile) * kKvTile * D;
  auto emit = [&](auto fast_tag, auto full_tag) __attribute__((always_inline)) {
  constexpr bool FAST = decltype(fast_tag)::value;
  constexpr bool FULL = decltype(full_tag)::value;   // every key of the tile is < N
  const float rv = FAST ? 1.0f / sv : 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      // byte i of the chunk: key = kb*64 + fp8_slot_key(g, p*16 + i)
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int n = tile * kKvTile + kb * 64 + fp8_slot_key(g, p * 16 + i);
        float v = 0.f;
        if (FULL || n < N) {
          const uint16_t h = xs[(size_t)n * D];
          v = BF16 ? as_float((int)((uint32_t)h << 16)) : (float)__builtin_bit_cast(_Float16, h);
        }
        const float x = FAST ? div_rn(v, sv, rv) : v / sv;
        y[i] = (sv > 0.f) ? fminf(fmaxf(x, -448.f), 448.f) : 0.f;
      }
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * q], y[4 * q + 1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * q + 2], y[4 * q + 3], pk, true);
        w[q] = (uint32_t)pk;
      }
      const int chunk = ((kb * NCB + cb) * 2 + p) * 64 + lane;
      *reinterpret_cast<uint4*>(ot + (size_t)chunk * 16) = uint4{w[0], w[1], w[2], w[3]};
    }
  };
  const bool fast = sv >= kDivRnMinScale || sv <= 0.f;   // sv <= 0: codes 0 either way
  if ((tile + 1) * kKvTile <= N) {
    if (fast) emit(std::true_type{}, std::true_type{});
    else emit(std::false_type{}, std::true_type{});
  } else {
    if (fast) emit(std::true_type{}, std::false_type{});
    else emit(std::false_type{}, std::false_type{});
  }
}

// ---------------------------------------------------------------------------
// MXFP4 V.  One wave per (128-key tile, 32-channel block): lane L holds
// channel cb*32 + L%32 and, for each 64-key half h of the tile, the 32 keys
// of block 2h + L/32.  The block's shared exponent is e = floor(log2 amax) - 2
// (clamped to E8M0's [-127, 127]; an all-zero block takes -127), its codes
// are RNE(v * 2^-e) saturated to +-6 (the scaling by a power of two is exact).
// The 16-byte chunk (tile, h, cb, L) holds nibble p = key mx_slot_key(p) of
// the block; the scale byte e + 127 sits at (tile, h, L, cb) of the scale
// array (4 bytes per (h, lane), one per channel block).  Keys >= N are 0.
// grid (ceil(ntile * D/32 / 4), B*Hkv), 4 waves per workgroup.
template <int D, bool BF16>
__global__ __launch_bounds__(kQuantThreads) void quant_v_mxfp4(const void* __restrict__ x,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               int N, int ntile) {
  constexpr int NCB = D / 32;
  const int bh = blockIdx.y, lane = threadIdx.x % 64;
  const int pair = blockIdx.x * (kQuantThreads / 64) + threadIdx.x / 64;
  if (pair >= ntile * NCB) return;
  const int tile = pair / NCB, cb = pair % NCB;
  const int chan = cb * 32 + (lane % 32), g = lane / 32;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(x) + (size_t)bh * N * D + chan;
  uint8_t* ct = codes + ((size_t)bh * ntile + tile) * (kKvTile / 2) * D;
  uint8_t* st = scales + ((size_t)bh * ntile + tile) * kMxScaleBytes;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float y[32];
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      const int n = tile * kKvTile + h * 64 + g * 32 + mx_slot_key(p);
      float v = 0.f;
      if (n < N) {
        const uint16_t u = xs[(size_t)n * D];
        v = BF16 ? as_float((int)((uint32_t)u << 16)) : (float)__builtin_bit_cast(_Float16, u);
      }
      y[p] = v;
      amax = fmaxf(amax, fabsf(v));
    }
    int e = -127;
    if (amax > 0.f) {
      int ex;
      frexpf(amax, &ex);                 // amax = f * 2^ex, f in [0.5, 1)
      e = min(max(ex - 3, -127), 127);   // floor(log2 amax) - 2
    }
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    static_for<16>([&](auto ji) {
      constexpr int j = decltype(ji)::value;
      w[j / 4] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[j / 4], ldexpf(y[2 * j], -e),
                                                         ldexpf(y[2 * j + 1], -e), 1.0f, j % 4);
    });
    *reinterpret_cast<uint4*>(ct + (size_t)((h * NCB + cb) * 64 + lane) * 16) =
        uint4{w[0], w[1], w[2], w[3]};
    st[(h * 64 + lane) * 4 + cb] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------------------
// corr[bh][n] = sm_scale * sum_c q[bh][n][c] * mean[bh_kv][c]: the part of
// every logit of row n that smoothing K removed (source-analysis page,
// smooth_k and LSE correction).  D/8 threads per row, 16-byte loads, fixed
// reduction order.  grid (ceil(N / rows per block), B*H).
template <int D, bool BF16>
__global__ __launch_bounds__(kQuantThreads) void lse_correction(const void* __restrict__ q,
                                                                const float* __restrict__ mean,
                                                                float* __restrict__ corr, int H,
                                                                int H_kv, int N, float sm_scale) {
  constexpr int TPR = D / 8;                     // threads per row
  constexpr int RPB = kQuantThreads / TPR;       // rows per block
  const int bh = blockIdx.y, tid = threadIdx.x, cg = tid % TPR;
  const int n = blockIdx.x * RPB + tid / TPR;
  const int b = bh / H, h = bh % H, hk = h / (H / H_kv);
  const float* mu = mean + (size_t)(b * H_kv + hk) * D + cg * 8;
  float acc = 0.f;
  if (n < N) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) +
                                                    ((size_t)bh * N + n) * D + cg * 8);
    float x[8];
    unpack8<BF16>(u, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(x[i], mu[i], acc);
  }
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (n < N && cg == 0) corr[(size_t)bh * N + n] = acc * sm_scale;
}

}  // namespace sage

// ---------------------------------------------------------------------------
// Host launchers.

namespace {
inline int nchunks(int N) { return (N + sage::kStatChunk - 1) / sage::kStatChunk; }
}  // namespace

size_t sage_ws_quant_qk_bytes(int B, int H_kv, int N, int d) {
  return (size_t)B * H_kv * nchunks(N) * d * sizeof(double);
}
size_t sage_ws_quant_v_bytes(int B, int H_kv, int N, int d) {
  return (size_t)B * H_kv * nchunks(N) * d * sizeof(float);
}

template <int D, bool BF16, bool SQ>
static void launch_quant_q(const void* q, const float* q_mean, int B, int H, int N, int q_group,
                           int8_t* q_i8, float* q_scale, hipStream_t st) {
  using namespace sage;
  constexpr int QM = SQ ? kBlockMean : kNoMean;
  if (q_group == kBlkQ) {
    const int nbq = (N + kBlkQ - 1) / kBlkQ;
    hipLaunchKernelGGL((quant_int8<D, kBlkQ, BF16, QM>), dim3(nbq, B * H), dim3(kQuantThreads), 0,
                       st, q, q_mean, q_i8, q_scale, N, nbq);
  } else if (q_group == kWaveQ) {
    const int nbq = (N + kWaveQ - 1) / kWaveQ;
    hipLaunchKernelGGL((quant_int8<D, kWaveQ, BF16, QM>), dim3(nbq, B * H), dim3(kQuantThreads), 0,
                       st, q, q_mean, q_i8, q_scale, N, nbq);
  } else {
    constexpr int tpb = kQuantThreads / (D / 8);
    hipLaunchKernelGGL((quant_int8_tok<D, BF16, SQ>), dim3((N + tpb - 1) / tpb, B * H),
                       dim3(kQuantThreads), 0, st, q, q_mean, q_i8, q_scale, N);
  }
}

template <int D, bool BF16>
static hipError_t quant_qk_impl(const void* q, const void* k, int B, int H, int H_kv, int N,
                                int q_group, int smooth_k, int smooth_q, int8_t* q_i8,
                                float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                                float* q_mean, void* ws, hipStream_t st) {
  using namespace sage;
  if (q_group != kBlkQ && q_group != kWaveQ && q_group != 1) return hipErrorInvalidValue;
  const int nc = nchunks(N);
  const int nbk = (N + kBlkK - 1) / kBlkK;
  if (smooth_k) {
    hipLaunchKernelGGL((colstats_partial<D, BF16, 0>), dim3(nc, B * H_kv), dim3(kQuantThreads), 0,
                       st, k, ws, N, nc);
  }
  hipLaunchKernelGGL((colstats_final<D, 0>), dim3(B * H_kv), dim3(kQuantThreads), 0, st, ws, k_mean,
                     N, nc, smooth_k);
  if (smooth_q) {
    const int nmb = (N + kBlkQ - 1) / kBlkQ;
    hipLaunchKernelGGL((q_block_mean<D, BF16>), dim3(nmb, B * H), dim3(kQuantThreads), 0, st, q,
                       q_mean, N, nmb);
    launch_quant_q<D, BF16, true>(q, q_mean, B, H, N, q_group, q_i8, q_scale, st);
  } else {
    launch_quant_q<D, BF16, false>(q, nullptr, B, H, N, q_group, q_i8, q_scale, st);
  }
  if (smooth_k)
    hipLaunchKernelGGL((quant_int8<D, kBlkK, BF16, kHeadMean>), dim3(nbk, B * H_kv),
                       dim3(kQuantThreads), 0, st, k, k_mean, k_i8, k_scale, N, nbk);
  else
    hipLaunchKernelGGL((quant_int8<D, kBlkK, BF16, kNoMean>), dim3(nbk, B * H_kv),
                       dim3(kQuantThreads), 0, st, k, nullptr, k_i8, k_scale, N, nbk);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t quant_v_impl(const void* v, int B, int H_kv, int N, uint8_t* v_f8,
                               float* v_scale, void* ws, hipStream_t st) {
  using namespace sage;
  const int nc = nchunks(N);
  const int nt = (N + kKvTile - 1) / kKvTile;
  hipLaunchKernelGGL((colstats_partial<D, BF16, 1>), dim3(nc, B * H_kv), dim3(kQuantThreads), 0, st,
                     v, ws, N, nc);
  hipLaunchKernelGGL((colstats_final<D, 1>), dim3(B * H_kv), dim3(kQuantThreads), 0, st, ws, v_scale,
                     N, nc, 1);
  const int pairs = nt * (D / 32), wpg = kQuantThreads / 64;
  hipLaunchKernelGGL((quant_v_fp8<D, BF16>), dim3((pairs + wpg - 1) / wpg, B * H_kv),
                     dim3(kQuantThreads), 0, st, v, v_scale, v_f8, N, nt);
  return hipGetLastError();
}

hipError_t sage_launch_quant_qk(const void* q, const void* k, int bf16, int B, int H, int H_kv,
                                int N, int d, int q_group, int smooth_k, int smooth_q,
                                int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                float* k_mean, float* q_mean, void* ws, hipStream_t st) {
#define SAGE_QQK(DD, BB)                                                                       \
  if (d == DD && (bf16 != 0) == BB)                                                            \
    return quant_qk_impl<DD, BB>(q, k, B, H, H_kv, N, q_group, smooth_k, smooth_q, q_i8,       \
                                 q_scale, k_i8, k_scale, k_mean, q_mean, ws, st);
  SAGE_QQK(64, false)
  SAGE_QQK(64, true)
  SAGE_QQK(128, false)
  SAGE_QQK(128, true)
#undef SAGE_QQK
  return hipErrorInvalidValue;
}

hipError_t sage_launch_quant_v(const void* v, int bf16, int B, int H_kv, int N, int d,
                               uint8_t* v_f8, float* v_scale, void* ws, hipStream_t st) {
  if (d == 64)
    return bf16 ? quant_v_impl<64, true>(v, B, H_kv, N, v_f8, v_scale, ws, st)
                : quant_v_impl<64, false>(v, B, H_kv, N, v_f8, v_scale, ws, st);
  if (d == 128)
    return bf16 ? quant_v_impl<128, true>(v, B, H_kv, N, v_f8, v_scale, ws, st)
                : quant_v_impl<128, false>(v, B, H_kv, N, v_f8, v_scale, ws, st);
  return hipErrorInvalidValue;
}

hipError_t sage_launch_quant_v_mxfp4(const void* v, int bf16, int B, int H_kv, int N, int d,
                                     uint8_t* v_f4, uint8_t* v_e8, hipStream_t st) {
  using namespace sage;
  const int nt = (N + kKvTile - 1) / kKvTile;
  const int wpg = kQuantThreads / 64;
#define SAGE_QV4(DD, BB)                                                                       \
  if (d == DD && (bf16 != 0) == BB) {                                                          \
    const int pairs = nt * (DD / 32);                                                          \
    hipLaunchKernelGGL((quant_v_mxfp4<DD, BB>), dim3((pairs + wpg - 1) / wpg, B * H_kv),       \
                       dim3(kQuantThreads), 0, st, v, v_f4, v_e8, N, nt);                      \
    return hipGetLastError();                                                                  \
  }
  SAGE_QV4(64, false)
  SAGE_QV4(64, true)
  SAGE_QV4(128, false)
  SAGE_QV4(128, true)
#undef SAGE_QV4
  return hipErrorInvalidValue;
}

hipError_t sage_launch_lse_correction(const void* q, int bf16, const float* k_mean, int B, int H,
                                      int H_kv, int N, int d, float sm_scale, float* corr,
                                      hipStream_t st) {
  using namespace sage;
  const int rpb = kQuantThreads / (d / 8);
  const dim3 grid((N + rpb - 1) / rpb, B * H), block(kQuantThreads);
#define SAGE_LSEC(DD, BB)                                                                      \
  if (d == DD && (bf16 != 0) == BB) {                                                          \
    hipLaunchKernelGGL((lse_correction<DD, BB>), grid, block, 0, st, q, k_mean, corr, H, H_kv, \
                       N, sm_scale);                                                           \
    return hipGetLastError();                                                                  \
  }
  SAGE_LSEC(64, false)
  SAGE_LSEC(64, true)
  SAGE_LSEC(128, false)
  SAGE_LSEC(128, true)
#undef SAGE_LSEC
  return hipErrorInvalidValue;
}
