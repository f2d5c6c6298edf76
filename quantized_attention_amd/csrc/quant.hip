// quant.hip -- smoothing and quantization kernels for gfx950 (HBM-bound).
//
//   kv_stats_partial / kv_stats_final : per-channel token statistics of K
//       and V in one pass over both: the exact FP64 sum of K (its mean
//       smooths K: the SageAttention synthesis page's Smooth K, Algorithm 1
//       preprocessing on the SageAttention2 detail page) and the absolute
//       max of V (the per-channel FP8 scale of Algorithm 1's psi_V).
//   quant_qkv_kernel  : one launch for every code, each workgroup in one role:
//       a 128-token Q block (Algorithm 1's smoothing block; optional smooth-Q
//       mean q_bar_i = mean(Q_i) subtracted; one scale per 128, 32 or 1
//       tokens, the per-block / per-warp / per-thread granularities of the
//       SageAttention2 detail page, Figure 4 and Table 6), a 64-token K block
//       (minus the K mean), or V tiles (per-channel FP8 E4M3, written
//       transposed and key-permuted in the fragment layout of sage.h).  INT8
//       rules: scale = amax/127, code = RNE(x/scale) (deployment-guide page,
//       quantization formula).
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
constexpr int kStatChunk = 256;   // tokens per kv_stats_partial workgroup

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
// One pass over a chunk of kStatChunk tokens of K and/or V of one (b, kv
// head): the FP64 column sums of K (for its mean) and the column amax of V
// (for its scales).  Each thread reads every RPP-th token row of its
// 8-channel group, kStatUnroll rows of each tensor in flight at a time; the
// RPP row groups are then combined in a fixed order.  The K sums are exact,
// so no order matters for them; amax is order-free.  grid (nchunk, B*Hkv);
// kws and vws are [B*Hkv][nchunk][D] (double, float).
constexpr int kStatUnroll = 4;
template <int D, bool BF16>
__global__ __launch_bounds__(kQuantThreads) void kv_stats_partial(const void* __restrict__ k,
                                                                  const void* __restrict__ v,
                                                                  double* __restrict__ kws,
                                                                  float* __restrict__ vws, int N,
                                                                  int nchunk, int do_k, int do_v) {
  constexpr int TPR = D / 8;                    // threads per token row
  constexpr int RPP = kQuantThreads / TPR;      // rows per pass
  constexpr int U = kStatUnroll;
  static_assert(2 * D <= kQuantThreads, "one thread per channel for each statistic");
  __shared__ double red_k[RPP][D];
  __shared__ float red_v[RPP][D];
  const int tid = threadIdx.x, cg = tid % TPR, rsub = tid / TPR;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const size_t base = (size_t)bh * N * D + cg * 8;
  const uint16_t* ks = reinterpret_cast<const uint16_t*>(k) + base;
  const uint16_t* vs = reinterpret_cast<const uint16_t*>(v) + base;
  const int n0 = chunk * kStatChunk, n1 = min(N, n0 + kStatChunk);
  double acc[8];
  float mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { acc[i] = 0.0; mx[i] = 0.f; }
  for (int n = n0 + rsub; n < n1; n += U * RPP) {
    uint4 uk[U], uv[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int r = n + j * RPP;
      if (r < n1) {
        if (do_k) uk[j] = *reinterpret_cast<const uint4*>(ks + (size_t)r * D);
        if (do_v) uv[j] = *reinterpret_cast<const uint4*>(vs + (size_t)r * D);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (n + j * RPP < n1) {
        float x[8];
        if (do_k) {
          unpack8<BF16>(uk[j], x);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += (double)x[i];
        }
        if (do_v) {
          unpack8<BF16>(uv[j], x);
#pragma unroll
          for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(x[i]));
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    red_k[rsub][cg * 8 + i] = acc[i];
    red_v[rsub][cg * 8 + i] = mx[i];
  }
  __syncthreads();
  // threads 0 .. D-1 combine the K sums, D .. 2D-1 the V maxima
  if (tid < D) {
    if (do_k) {
      double t = 0.0;
      for (int r = 0; r < RPP; ++r) t += red_k[r][tid];
      kws[((size_t)bh * nchunk + chunk) * D + tid] = t;
    }
  } else if (tid < 2 * D) {
    if (do_v) {
      const int c = tid - D;
      float m = 0.f;
      for (int r = 0; r < RPP; ++r) m = fmaxf(m, red_v[r][c]);
      vws[((size_t)bh * nchunk + chunk) * D + c] = m;
    }
  }
}

// The chunks combined: k_mean[bh][c] = float32(sum / N) (0 when !smooth_k)
// and v_scale[bh][c] = float32(amax / 448).  kQuantThreads threads per (b, kv
// head): thread (r, c) combines chunks r, r + R, ... of channel c in order,
// then the R partials are combined in order (a fixed order, so the result is
// deterministic; the K sums are exact, so order-free anyway).  grid (B*Hkv).
template <int D>
__global__ __launch_bounds__(kQuantThreads) void kv_stats_final(const double* __restrict__ kws,
                                                                const float* __restrict__ vws,
                                                                float* __restrict__ k_mean,
                                                                float* __restrict__ v_scale, int N,
                                                                int nchunk, int do_k, int smooth_k,
                                                                int do_v) {
  constexpr int R = kQuantThreads / D;
  const int bh = blockIdx.x, c = threadIdx.x % D, r = threadIdx.x / D;
  __shared__ double red[R][D];
  if (do_k) {
    const double* w = kws + (size_t)bh * nchunk * D + c;
    double s = 0.0;
    if (smooth_k) {
#pragma unroll 8
      for (int kk = r; kk < nchunk; kk += R) s += w[(size_t)kk * D];
    }
    red[r][c] = s;
    __syncthreads();
    if (r == 0) {
      double t = red[0][c];
#pragma unroll
      for (int i = 1; i < R; ++i) t += red[i][c];
      k_mean[(size_t)bh * D + c] = smooth_k ? (float)(t / (double)N) : 0.f;
    }
    __syncthreads();
  }
  if (do_v) {
    const float* w = vws + (size_t)bh * nchunk * D + c;
    float m = 0.f;
#pragma unroll 8
    for (int kk = r; kk < nchunk; kk += R) m = fmaxf(m, w[(size_t)kk * D]);
    red[r][c] = m;
    __syncthreads();
    if (r == 0) {
      float t = (float)red[0][c];
#pragma unroll
      for (int i = 1; i < R; ++i) t = fmaxf(t, (float)red[i][c]);
      v_scale[(size_t)bh * D + c] = t / 448.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// Max over the workgroup (all threads get the result); `red` holds one float
// per wave.
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int wave = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

// 8 values of one token row -> 8 INT8 codes: RNE(x / sc) clamped to +-127,
// 0 when sc == 0.  FAST: Markstein's three-operation quotient (sc normal and
// >= kDivRnMinScale), else the IEEE division.
template <bool FAST>
__device__ __forceinline__ uint2 codes8(const float* v, float sc) {
  const float rs = FAST ? 1.0f / sc : 0.f;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = 0.f;
    if (FAST || sc > 0.f) {
      const float x = FAST ? div_rn(v[i], sc, rs) : v[i] / sc;
      q = fminf(fmaxf(__builtin_rintf(x), -127.f), 127.f);
    }
    w[i / 4] |= ((uint32_t)(int)q & 0xFFu) << (8 * (i % 4));
  }
  return uint2{w[0], w[1]};
}

// Everything the quantization launch writes, and the shapes.
struct QuantArgs {
  const void* q;
  const void* k;
  const void* v;
  int8_t* q_i8;
  float* q_scale;
  float* q_mean;
  int8_t* k_i8;
  float* k_scale;
  const float* k_mean;
  uint8_t* v_f8;
  const float* v_scale;
  int N, nbq, nbk, ntile, nvw;   // per head: 128-token Q blocks, 64-token K blocks, V tiles, V workgroups
  int nQ, nK;                    // workgroups of the Q and K roles (the V role takes the rest)
  int smooth_k;
};

// Q role: one 128-token block (the smoothing block of Algorithm 1), with one
// scale per QG consecutive tokens (128, 32 or 1).  SQ: the block's
// per-channel mean q_bar = float32(exact sum / count) over its valid tokens
// is written to q_mean and subtracted (float32) before quantizing.
template <int D, bool BF16, int QG, bool SQ>
__device__ __forceinline__ void quant_q_block(const QuantArgs& a, int bh, int blk, double (*red)[D],
                                              float* fs) {
  constexpr int TPR = D / 8;                    // threads per token row
  constexpr int RPP = kQuantThreads / TPR;      // rows per pass
  constexpr int PER = kBlkQ / RPP;              // passes
  static_assert(RPP <= 32 && 32 % RPP == 0, "a 32-token group is whole passes");
  const int N = a.N;
  const int tid = threadIdx.x, cg = tid % TPR, rr = tid / TPR;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(a.q) + (size_t)bh * N * D;
  int8_t* cs = a.q_i8 + (size_t)bh * N * D;
  float v[PER][8];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int row = blk * kBlkQ + p * RPP + rr;
    if (row < N) {
      unpack8<BF16>(*reinterpret_cast<const uint4*>(xs + (size_t)row * D + cg * 8), v[p]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[p][i] = 0.f;
    }
  }
  if constexpr (SQ) {
    double sm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < PER; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) sm[i] += (double)v[p][i];
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rr][cg * 8 + i] = sm[i];
    __syncthreads();
    if (tid < D) {
      double t = red[0][tid];
      for (int r = 1; r < RPP; ++r) t += red[r][tid];
      const int cnt = min(kBlkQ, N - blk * kBlkQ);
      const float mu = (float)(t / (double)cnt);
      a.q_mean[((size_t)bh * a.nbq + blk) * D + tid] = mu;
      fs[tid] = mu;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PER; ++p)
      if (blk * kBlkQ + p * RPP + rr < N) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[p][i] = v[p][i] - fs[cg * 8 + i];
      }
  }
  float* wred = fs + D;   // per-wave partial maxima
  if constexpr (QG == kBlkQ) {
    float am = 0.f;
#pragma unroll
    for (int p = 0; p < PER; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[p][i]));
    const float sc = block_max(am, wred) / 127.0f;   // IEEE division
    if (tid == 0) a.q_scale[(size_t)bh * a.nbq + blk] = sc;
    const bool fast = __builtin_amdgcn_readfirstlane(sc >= kDivRnMinScale ? 1 : 0);
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int row = blk * kBlkQ + p * RPP + rr;
      if (row >= N) continue;
      const uint2 w = fast ? codes8<true>(v[p], sc) : codes8<false>(v[p], sc);
      *reinterpret_cast<uint2*>(cs + (size_t)row * D + cg * 8) = w;
    }
  } else if constexpr (QG == 32) {
    // pass p holds rows p*RPP .. +RPP of the block: group p*RPP/32
    float am[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < PER; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) am[p * RPP / 32] = fmaxf(am[p * RPP / 32], fabsf(v[p][i]));
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) am[g] = fmaxf(am[g], __shfl_xor(am[g], o));
    const int wave = tid / 64;
    __syncthreads();
    if ((tid & 63) == 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) wred[wave * 4 + g] = am[g];
    }
    __syncthreads();
    float sc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float m = wred[g];
#pragma unroll
      for (int w = 1; w < kQuantThreads / 64; ++w) m = fmaxf(m, wred[w * 4 + g]);
      sc[g] = m / 127.0f;                             // IEEE division
    }
    const int nq = (N + 31) / 32;
    if (tid < 4 && blk * 4 + tid < nq) a.q_scale[(size_t)bh * nq + blk * 4 + tid] = sc[tid];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int row = blk * kBlkQ + p * RPP + rr;
      if (row >= N) continue;
      const float s = sc[p * RPP / 32];
      const bool fast = __builtin_amdgcn_readfirstlane(s >= kDivRnMinScale ? 1 : 0);
      const uint2 w = fast ? codes8<true>(v[p], s) : codes8<false>(v[p], s);
      *reinterpret_cast<uint2*>(cs + (size_t)row * D + cg * 8) = w;
    }
  } else {
    static_assert(QG == 1, "Q groups of 128, 32 or 1 tokens");
    // one scale per token: its TPR threads are consecutive lanes of a wave
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int row = blk * kBlkQ + p * RPP + rr;
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[p][i]));
#pragma unroll
      for (int o = TPR / 2; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
      const float s = am / 127.0f;                    // IEEE division
      // the three-operation division when every token of the wave allows it
      const bool fast = __builtin_amdgcn_ballot_w64(!(s >= kDivRnMinScale)) == 0;
      if (row >= N) continue;
      if (cg == 0) a.q_scale[(size_t)bh * N + row] = s;
      const uint2 w = fast ? codes8<true>(v[p], s) : codes8<false>(v[p], s);
      *reinterpret_cast<uint2*>(cs + (size_t)row * D + cg * 8) = w;
    }
  }
}

// K role: one 64-token block of K (minus its mean when smoothing K).
template <int D, bool BF16>
__device__ __forceinline__ void quant_k_block(const QuantArgs& a, int bh, int blk, float* wred) {
  constexpr int TPR = D / 8;
  constexpr int PER = kBlkK * TPR / kQuantThreads;   // 16-byte chunks per thread
  const int N = a.N;
  const int tid = threadIdx.x, cg = tid % TPR;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(a.k) + (size_t)bh * N * D;
  int8_t* cs = a.k_i8 + (size_t)bh * N * D;
  float mu[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mu[i] = a.smooth_k ? a.k_mean[(size_t)bh * D + cg * 8 + i] : 0.f;
  float v[PER][8];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int row = blk * kBlkK + (p * kQuantThreads + tid) / TPR;
    if (row < N) {
      unpack8<BF16>(*reinterpret_cast<const uint4*>(xs + (size_t)row * D + cg * 8), v[p]);
      if (a.smooth_k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[p][i] = v[p][i] - mu[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[p][i]));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[p][i] = 0.f;
    }
  }
  const float sc = block_max(amax, wred) / 127.0f;   // IEEE division
  if (tid == 0) a.k_scale[(size_t)bh * a.nbk + blk] = sc;
  const bool fast = __builtin_amdgcn_readfirstlane(sc >= kDivRnMinScale ? 1 : 0);
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int row = blk * kBlkK + (p * kQuantThreads + tid) / TPR;
    if (row >= N) continue;
    const uint2 w = fast ? codes8<true>(v[p], sc) : codes8<false>(v[p], sc);
    *reinterpret_cast<uint2*>(cs + (size_t)row * D + cg * 8) = w;
  }
}

// V role.  Each 16-byte chunk of the v_f8 layout (sage.h) holds one channel
// and 16 keys, so one wave writes the 64 chunks (kb, cb, p, L = lane) of a
// (128-key tile, 32-channel block) pair for kb, p in {0, 1}: lane L gathers
// its channel cb*32 + L%32 for the 64 keys of its lane half straight from
// HBM (for each key, 32 lanes read 64 contiguous bytes) and stores whole
// 16-byte chunks, consecutive across the wave.  No LDS staging.  Workgroup
// w of a (b, kv head) takes pairs 4w .. 4w+3 (one per wave).
template <int D, bool BF16>
__device__ __forceinline__ void quant_v_wg(const QuantArgs& a, int bh, int w) {
  constexpr int NCB = D / 32;
  const int N = a.N, ntile = a.ntile;
  const int lane = threadIdx.x % 64;
  const int pair = w * (kQuantThreads / 64) + threadIdx.x / 64;
  if (pair >= ntile * NCB) return;
  const int tile = pair / NCB, cb = pair % NCB;
  const int chan = cb * 32 + (lane % 32), g = lane / 32;
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(a.v) + (size_t)bh * N * D + chan;
  const float sv = a.v_scale[(size_t)bh * D + chan];
  uint8_t* ot = a.v_f8 + ((size_t)bh * ntile + tile) * kKvTile * D;
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
        uint32_t wd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * q], y[4 * q + 1], 0, false);
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * q + 2], y[4 * q + 3], pk, true);
          wd[q] = (uint32_t)pk;
        }
        const int chunk = ((kb * NCB + cb) * 2 + p) * 64 + lane;
        *reinterpret_cast<uint4*>(ot + (size_t)chunk * 16) = uint4{wd[0], wd[1], wd[2], wd[3]};
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

// The quantization launch: workgroups [0, nQ) quantize 128-token Q blocks,
// [nQ, nQ + nK) 64-token K blocks, the rest V tiles (each role's work is
// independent; the K mean and V scales come from kv_stats_final).  One
// launch for what took one per tensor.  grid (nQ + nK + nV).
template <int D, bool BF16, int QG, bool SQ>
__global__ __launch_bounds__(kQuantThreads) void quant_qkv_kernel(QuantArgs a) {
  __shared__ double red[kQuantThreads / (D / 8)][D];
  __shared__ float fs[D + 16];
  int id = blockIdx.x;
  if (id < a.nQ) {
    quant_q_block<D, BF16, QG, SQ>(a, id / a.nbq, id % a.nbq, red, fs);
    return;
  }
  id -= a.nQ;
  if (id < a.nK) {
    quant_k_block<D, BF16>(a, id / a.nbk, id % a.nbk, fs);
    return;
  }
  id -= a.nK;
  quant_v_wg<D, BF16>(a, id / a.nvw, id % a.nvw);
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

// The three launches of a quantization call: column statistics of K (when
// smoothing it) and/or V, their combination into the K mean and V scales, and
// one launch quantizing Q and K (q != nullptr) and/or V (v != nullptr).
// ws: K sums [B*Hkv][nchunk][d] doubles, then V maxima as floats.
template <int D, bool BF16, int QG, bool SQ>
static hipError_t quant_impl(const void* q, const void* k, const void* v, int B, int H, int H_kv,
                             int N, int smooth_k, int8_t* q_i8, float* q_scale, int8_t* k_i8,
                             float* k_scale, float* k_mean, float* q_mean, uint8_t* v_f8,
                             float* v_scale, void* ws, hipStream_t st) {
  using namespace sage;
  const bool do_qk = q != nullptr, do_v = v != nullptr;
  const int nc = nchunks(N);
  double* kws = reinterpret_cast<double*>(ws);
  float* vws = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                        (do_qk && smooth_k ? sage_ws_quant_qk_bytes(B, H_kv, N, D) : 0));
  if ((do_qk && smooth_k) || do_v)
    hipLaunchKernelGGL((kv_stats_partial<D, BF16>), dim3(nc, B * H_kv), dim3(kQuantThreads), 0, st,
                       k, v, kws, vws, N, nc, (int)(do_qk && smooth_k), (int)do_v);
  hipLaunchKernelGGL((kv_stats_final<D>), dim3(B * H_kv), dim3(kQuantThreads), 0, st, kws, vws,
                     k_mean, v_scale, N, nc, (int)do_qk, smooth_k, (int)do_v);
  QuantArgs a;
  a.q = q; a.k = k; a.v = v;
  a.q_i8 = q_i8; a.q_scale = q_scale; a.q_mean = q_mean;
  a.k_i8 = k_i8; a.k_scale = k_scale; a.k_mean = k_mean;
  a.v_f8 = v_f8; a.v_scale = v_scale;
  a.N = N;
  a.nbq = (N + kBlkQ - 1) / kBlkQ;
  a.nbk = (N + kBlkK - 1) / kBlkK;
  a.ntile = (N + kKvTile - 1) / kKvTile;
  a.nvw = (a.ntile * (D / 32) + kQuantThreads / 64 - 1) / (kQuantThreads / 64);
  a.nQ = do_qk ? B * H * a.nbq : 0;
  a.nK = do_qk ? B * H_kv * a.nbk : 0;
  a.smooth_k = smooth_k;
  const long long nV = do_v ? (long long)B * H_kv * a.nvw : 0;
  const long long grid = (long long)a.nQ + a.nK + nV;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((quant_qkv_kernel<D, BF16, QG, SQ>), dim3((unsigned)grid), dim3(kQuantThreads),
                     0, st, a);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t quant_dispatch(const void* q, const void* k, const void* v, int B, int H,
                                 int H_kv, int N, int q_group, int smooth_k, int smooth_q,
                                 int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                 float* k_mean, float* q_mean, uint8_t* v_f8, float* v_scale,
                                 void* ws, hipStream_t st) {
#define SAGE_QI(QG, SQ)                                                                     \
  if (q_group == QG && (smooth_q != 0) == SQ)                                               \
    return quant_impl<D, BF16, QG, SQ>(q, k, v, B, H, H_kv, N, smooth_k, q_i8, q_scale, k_i8, \
                                       k_scale, k_mean, q_mean, v_f8, v_scale, ws, st);
  SAGE_QI(128, false)
  SAGE_QI(128, true)
  SAGE_QI(32, false)
  SAGE_QI(32, true)
  SAGE_QI(1, false)
  SAGE_QI(1, true)
#undef SAGE_QI
  return hipErrorInvalidValue;
}

hipError_t sage_launch_quant(const void* q, const void* k, const void* v, int bf16, int B, int H,
                             int H_kv, int N, int d, int q_group, int smooth_k, int smooth_q,
                             int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                             float* k_mean, float* q_mean, uint8_t* v_f8, float* v_scale, void* ws,
                             hipStream_t st) {
#define SAGE_QD(DD, BB)                                                                       \
  if (d == DD && (bf16 != 0) == BB)                                                           \
    return quant_dispatch<DD, BB>(q, k, v, B, H, H_kv, N, q_group, smooth_k, smooth_q, q_i8,   \
                                  q_scale, k_i8, k_scale, k_mean, q_mean, v_f8, v_scale, ws, st);
  SAGE_QD(64, false)
  SAGE_QD(64, true)
  SAGE_QD(128, false)
  SAGE_QD(128, true)
#undef SAGE_QD
  return hipErrorInvalidValue;
}

hipError_t sage_launch_quant_qk(const void* q, const void* k, int bf16, int B, int H, int H_kv,
                                int N, int d, int q_group, int smooth_k, int smooth_q,
                                int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                float* k_mean, float* q_mean, void* ws, hipStream_t st) {
  return sage_launch_quant(q, k, nullptr, bf16, B, H, H_kv, N, d, q_group, smooth_k, smooth_q, q_i8,
                           q_scale, k_i8, k_scale, k_mean, q_mean, nullptr, nullptr, ws, st);
}

hipError_t sage_launch_quant_v(const void* v, int bf16, int B, int H_kv, int N, int d,
                               uint8_t* v_f8, float* v_scale, void* ws, hipStream_t st) {
  return sage_launch_quant(nullptr, nullptr, v, bf16, B, H_kv, H_kv, N, d, 128, 0, 0, nullptr,
                           nullptr, nullptr, nullptr, nullptr, nullptr, v_f8, v_scale, ws, st);
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
