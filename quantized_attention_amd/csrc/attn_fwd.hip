// attn_fwd.hip -- INT8 QK^T / FP8 PV online-softmax attention for gfx950.
//
// Algorithm 1 of the SageAttention2 detail page (inner loop and final
// rescale), with INT8 Q/K codes and per-block FP32 scales, FP8 E4M3 V with
// per-channel scales, and P~ * 448 cast to FP8 before the P V product.
//
// Work decomposition: one workgroup = 4 waves = 128 queries of one head (one
// Q scale block); two (d = 128) or three (d = 64) workgroups share a CU.  Each wave owns 32 queries and computes S^T = K Q^T for a
// 128-key tile as four 32x32 INT8 MFMA blocks, so every lane holds the
// scores of ONE query (column L % 32) for 64 of the tile's keys; the other
// 64 keys sit in lane L ^ 32.  Row max and row sum are therefore in-lane
// plus one cross-half exchange.  P~ is converted to FP8 in registers and fed
// as the B operand of the 32x32x64 FP8 MFMA (O^T = V^T P^T); V^T arrives
// from HBM already permuted (sage.h, v_f8 layout) so that its keys line up
// with the register order of P.  K and V^T tiles are double-buffered in LDS.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <hip/hip_bf16.h>
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "sage_device.hpp"

namespace sage {

// The grid covers q tiles qt0 .. qt0 + nqt - 1 of the query heads of the
// (b, kv head) groups bk0 .. bk0 + total / (nqt * H/H_kv) - 1 (bk = b*H_kv + hk).
// SQ: Q was smoothed by its 128-block means; delta_s holds the Delta S rows
// of those heads and q tiles, [heads][nqt][N] (log2 units), added to every
// score.
// PV4: P V on the FP4 matrix cores in MXFP4 (v_f8 holds E2M1 codes, v_e8 the
// E8M0 scale bytes, see quant_v_mxfp4); P~ is quantized per 32 keys of a row.
template <int D, bool CAUSAL, bool BF16, bool SQ, bool PV4>
// d = 64 fits three workgroups per CU (168 registers), four with MXFP4 P V
// (128: no product by 448 and a smaller P, +3 % on a d = 64 video workload
// against three); d = 128 two.
__global__ __launch_bounds__(kWaves * 64, D == 64 ? (PV4 ? 4 : 3) : 2) void attn_fwd_kernel(
    const int8_t* __restrict__ q_i8, const float* __restrict__ q_scale,
    const int8_t* __restrict__ k_i8, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ v_f8, const float* __restrict__ v_scale,
    const uint8_t* __restrict__ v_e8, const float* __restrict__ delta_s,
    void* __restrict__ out, float* __restrict__ lse,
    const float* __restrict__ lse_corr, int H, int H_kv, int N, float lam, int qg_shift,
    int bk0, int qt0, int nqt, int total) {
  // Every float32 step of the softmax below is the one the oracle takes (each
  // named quantity rounded once); no multiply may be fused into a following add.
#pragma clang fp contract(off)
  constexpr int NKC = D / 32;                 // 32-wide channel chunks
  constexpr int KBYTES = kKvTile * D;         // K tile bytes
  constexpr int VBYTES = PV4 ? KBYTES / 2 : KBYTES;   // V tile bytes (FP8 or FP4 codes)
  constexpr int VSBYTES = PV4 ? kMxScaleBytes : 0;    // a tile's MXFP4 V scale bytes
  constexpr int DSBYTES = SQ ? kKvTile * 4 : 0;      // a tile's Delta S values
  static_assert(!(SQ && PV4), "Delta S and MXFP4 P V are separate variants");
  // K (with Delta S) and V tiles are double-buffered.
  __shared__ __attribute__((aligned(16))) char lds_k[2][KBYTES + DSBYTES];
  __shared__ __attribute__((aligned(16))) char lds_v[2][VBYTES + VSBYTES];
  // the kv head's V channel scales for the epilogue (FP8 P V), staged once at
  // the start so the epilogue does not wait on a global load
  __shared__ __attribute__((aligned(16))) float lds_vs[PV4 ? 4 : D];

  // ---- which (b, kv head, q tile, group member) this workgroup computes.
  // Non-causal (equal work per workgroup): each XCD takes a contiguous range
  // of logical ids, in which the `group` query heads that share a kv head are
  // adjacent and walk the q tiles together (they read the same K/V tiles).
  // Causal (q tile qt does qt+1 key tiles): the grid runs the q tiles
  // heaviest first, across all heads, with the (b, kv head) index varying
  // fastest.  The hardware deals consecutive ids round-robin to the 8 XCDs,
  // so every XCD gets the same mix of tile counts, each in heaviest-first
  // order, and when B*H_kv is a multiple of 8 each (b, kv head) stays on one
  // XCD (its K/V tiles stay in that XCD's L2).
  const int group = H / H_kv;
  int gm, qt, hk, b;
  if (CAUSAL) {
    const int nbk = total / (nqt * group);   // (b, kv head) groups in this launch
    int rest = blockIdx.x;
    const int bk = bk0 + rest % nbk; rest /= nbk;
    gm = rest % group;
    qt = qt0 + nqt - 1 - rest / group;
    b = bk / H_kv;
    hk = bk % H_kv;
  } else {
    int rest = xcd_remap(blockIdx.x, total);
    gm = rest % group; rest /= group;
    qt = qt0 + rest % nqt; rest /= nqt;
    const int bk = bk0 + rest;
    hk = bk % H_kv;
    b = bk / H_kv;
  }
  const int h = hk * group + gm;

  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int col = lane & 31, half = lane >> 5;
  // Matrix-core precedence (d = 128).  Each SIMD runs one wave of each of the
  // two workgroups on its CU.  At equal priority their MFMAs interleave one
  // by one, both waves reach their exponentials together, and the SIMD
  // alternates between MFMA-only and VALU-only stretches.  The workgroup in
  // an odd slot of its CU (HW_ID.TG_ID) takes priority 3 for its MFMA phase
  // (P V of tile t with the exponentials interleaved into it, the barrier,
  // QK^T of tile t+1), the other 2, and both drop to 0 after QK^T for the
  // row max and the first exponentials.  One wave then finishes its MFMA
  // phase first, and the other's follows while it computes exponentials:
  // +3 % at N = 32K, +7 % at N = 4K, +8 % on a causal 4K prefill.  d = 64
  // (three workgroups per CU) gains nothing.
  const bool mfma_first = (__builtin_amdgcn_s_getreg((3 << 11) | (16 << 6) | 4) & 1) != 0;
  auto prio_mfma = [&]() __attribute__((always_inline)) {
    if constexpr (D != 64) {
      __builtin_amdgcn_sched_barrier(0);
      if (mfma_first) __builtin_amdgcn_s_setprio(3);
      else __builtin_amdgcn_s_setprio(2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto prio_valu = [&]() __attribute__((always_inline)) {
    if constexpr (D != 64) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int q0 = qt * kBlockQ + wave * kWaveQ;
  const int qi = q0 + col;                    // this lane's query row

  const int8_t* qh = q_i8 + (size_t)(b * H + h) * N * D;
  const int8_t* kh = k_i8 + (size_t)(b * H_kv + hk) * N * D;
  const int ntk = (N + kKvTile - 1) / kKvTile;
  const uint8_t* vh = v_f8 + (size_t)(b * H_kv + hk) * ntk * VBYTES;
  const uint8_t* vsh = PV4 ? v_e8 + (size_t)(b * H_kv + hk) * ntk * VSBYTES : nullptr;
  // buffer resources of this head's K, V (and MXFP4 scales), Delta S row
  const rsrc_t rk = make_rsrc(kh, (uint32_t)N * D);
  const rsrc_t rv = make_rsrc(vh, (uint32_t)ntk * VBYTES);
  const int nkb = (N + kBlkK - 1) / kBlkK;
  const float* ksc = k_scale + (size_t)(b * H_kv + hk) * nkb;
  const int ntiles = CAUSAL ? qt + 1 : ntk;

  // Q fragments for the whole loop (B operand of S^T = K Q^T).
  i32x4 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    qf[kc] = (qi < N) ? *reinterpret_cast<const i32x4*>(qh + (size_t)qi * D + kc * 32 + half * 16)
                      : i32x4{0, 0, 0, 0};
  // this lane's Q scale: groups of 2^qg_shift consecutive queries (128, 32
  // or 1; rows past N read the last row's group)
  const int nqs = ((N - 1) >> qg_shift) + 1;
  const float dq = q_scale[(size_t)(b * H + h) * nqs + (min(qi, N - 1) >> qg_shift)];

  f32x16 acc_o[NKC];
#pragma unroll
  for (int c = 0; c < NKC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[c][r] = 0.f;
  float m_run = -INFINITY;   // running max of the log2-domain scores
  float l_part = 0.f;        // this lane's share of l = sum P~

  // this lane's byte offsets of its K blocks inside a tile
  constexpr int KNB = (kKvTile / 32) * NKC / kWaves;
  uint32_t koff[KNB];
#pragma unroll
  for (int i = 0; i < KNB; ++i) koff[i] = k_tile_offset<D>(i * kWaves + wave, lane);
  // Delta S row of this workgroup's Q block; waves 0 and 1 stage a tile's
  // 128 values (one float per lane; keys past N read zeros)
  // (the launch's heads are consecutive: local head b * H + h - bk0 * group)
  const rsrc_t rds = make_rsrc(SQ ? delta_s + ((size_t)(b * H + h - bk0 * group) * nqt + qt - qt0) * N
                                  : delta_s,
                               SQ ? (uint32_t)N * 4 : 0u);
  const rsrc_t rvs = make_rsrc(vsh, PV4 ? (uint32_t)ntk * VSBYTES : 0u);
  // K and V codes (and, for MXFP4, the tile's 512 scale bytes; with Delta S
  // the tile's 128 values: waves 0 and 1, one dword per lane) of tile t into
  // a stage
  auto load_k = [&](int t) __attribute__((always_inline)) {
    char* stage = lds_k[t & 1];
    load_k_tile<D>(rk, t * kKvTile, koff, stage, wave);
    if (SQ && wave < 2)
      buffer_to_lds<4>(rds, stage + KBYTES + wave * 256, (uint32_t)((wave * 64 + lane) * 4),
                       (uint32_t)t * kKvTile * 4);
  };
  auto load_v = [&](int t) __attribute__((always_inline)) {
    char* stage = lds_v[t & 1];
    load_v_tile<VBYTES>(rv, t, stage, wave, lane);
    if (PV4 && wave < 2)
      buffer_to_lds<4>(rvs, stage + VBYTES + wave * 256, (uint32_t)(wave * 256 + lane * 4),
                       (uint32_t)t * VSBYTES);
  };
  load_k(0);
  load_v(0);
  if constexpr (!PV4) {
    // waves 0 .. D/64-1: one scale per lane, straight into LDS (visible after
    // the first tile's wait and barrier)
    if (wave < D / 64) {
      const rsrc_t rvsc = make_rsrc(v_scale + (size_t)(b * H_kv + hk) * D, (uint32_t)D * 4);
      buffer_to_lds<4>(rvsc, reinterpret_cast<char*>(lds_vs) + wave * 256,
                       (uint32_t)((wave * 64 + lane) * 4), 0u);
    }
  }

  // One 128-key step of the online softmax.  MASK: the tile holds keys past
  // the diagonal (causal) or past N; only the last tile can.
  auto step = [&](int t, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // Tile t has landed in buffers t&1 for every wave; buffers (t+1)&1 were
    // last read in iteration t-1, which every wave has finished.
    wait_vmem();
    __syncthreads();
    if (t + 1 < ntiles) {
      load_k(t + 1);
      load_v(t + 1);
    }
    const char* kt = lds_k[t & 1];
    const char* vt = lds_v[t & 1];

    // ---- S^T = K Q^T on the INT8 matrix cores (exact int32 sums).
    // K fragments are read one 32-key block ahead of the MFMAs that use
    // them, so the LDS latency hides behind the previous block's MFMAs.
    i32x16 s[4];
    i32x4 kf[NKC];
    read_k_frags<NKC>(kt, lane, kf);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      i32x4 kn[NKC];
      if (kb + 1 < 4) read_k_frags<NKC>(kt + (kb + 1) * NKC * 1024, lane, kn);
      __builtin_amdgcn_sched_barrier(0);
      s[kb] = qk_frags<NKC>(kf, qf);
      __builtin_amdgcn_sched_barrier(0);
      if (kb + 1 < 4) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) kf[kc] = kn[kc];
      }
    }
    prio_valu();

    // Per 32-key block: the score factor c = (dQ * dK) * lam, each product
    // rounded once (the dequantization's scale product, then the softmax
    // constant sm_scale * log2 e).
    float ck[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int kidx = (t * kKvTile + kb * 32) / kBlkK;
      // in a tail tile a 32-key block may lie wholly past N: clamp the read
      // (its scores are masked anyway)
      const float dqk = dq * ksc[MASK ? min(kidx, nkb - 1) : kidx];
      ck[kb] = dqk * lam;
    }

    float xm = -INFINITY;
    float xk[4];   // MXFP4: each 32-key block's max over the whole row block
    if constexpr (SQ) {
      // ---- with Delta S: s becomes the float score x = S * ck + Delta S[key]
      // in log2 units, one rounding (masked: -inf), and the row max is taken
      // on those floats.
      const float* dt = reinterpret_cast<const float*>(lds_k[t & 1] + KBYTES);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // keys kb*32 + 8j + 4*half + (0..3) are registers 4j .. 4j+3
          const float4 d4 = *reinterpret_cast<const float4*>(dt + kb * 32 + 8 * j + 4 * half);
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            float x = fmaf((float)s[kb][r], ck[kb], dv[i]);
            if constexpr (MASK) {
              const int key = t * kKvTile + kb * 32 + 8 * j + 4 * half + i;
              if ((CAUSAL && key > qi) || key >= N) x = -INFINITY;
            }
            s[kb][r] = as_int(x);
          }
        }
        const i32x16& v = s[kb];
        float m = fmaxf(fmaxf(as_float(v[0]), as_float(v[1])), as_float(v[2]));
#pragma unroll
        for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, as_float(v[r])), as_float(v[r + 1]));
        xm = fmaxf(xm, fmaxf(m, as_float(v[15])));
      }
    } else {
      if constexpr (MASK) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = t * kKvTile + kb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
            if ((CAUSAL && key > qi) || key >= N) s[kb][r] = INT_MIN;
          }
      }

      // ---- tile row max (in-lane on the int bits, then across the lane halves).
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        // a depth-3 tree of max3 (short dependency chain)
        const i32x16& v = s[kb];
        const int m0 = max(max(v[0], v[1]), v[2]), m1 = max(max(v[3], v[4]), v[5]);
        const int m2 = max(max(v[6], v[7]), v[8]), m3 = max(max(v[9], v[10]), v[11]);
        const int m4 = max(max(v[12], v[13]), v[14]);
        const int fm = max(max(max(m0, m1), m2), max(max(m3, m4), v[15]));
        // the block's largest score x = S * c: rounding is monotonic, so
        // the max of the rounded products is the product of the max
        const float x = (float)fm * ck[kb];
        if constexpr (PV4) {
          xk[kb] = MASK ? (fm != INT_MIN ? x : -INFINITY) : x;
        } else {
          xm = MASK ? (fm != INT_MIN ? fmaxf(xm, x) : xm) : fmaxf(xm, x);
        }
      }
    }
    if constexpr (PV4) {
      // a block's 32 keys sit in both lane halves
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xk[kb] = max_xor32(xk[kb]);
      xm = fmaxf(fmaxf(xk[0], xk[1]), fmaxf(xk[2], xk[3]));
    } else {
      xm = max_xor32(xm);
    }
    const float m_new = fmaxf(m_run, xm);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_part *= alpha;
    // O is rescaled (when some row's max moved) just before the first P V
    // MFMA, so the max chain above, the conversions and the first
    // exponentials form one block the scheduler can interleave.
    // (Tile 0 skips it: O is still zero there.)
    auto rescale_o = [&]() __attribute__((always_inline)) {
      if (t > 0 && __builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int c = 0; c < NKC; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[c][r] *= alpha;
      }
    };

    // ---- P~ = 2^(x - m) with x = S * c (S the exact int32 sum, converted to
    // float exactly: |S| < 2^22), each step rounded once; l sums P~ unquantized;
    // (P~ * 448) is rounded to float32, then to FP8 E4M3 (nearest even,
    // saturating).  With Delta S, x is already in s.  Masked keys give 0.
    i32x8 pf[2];
    // The first two V fragments are read before the exponentials, the rest
    // two MFMAs ahead, so no FP8 MFMA waits on LDS.
    auto vfrag = [&](int idx) __attribute__((always_inline)) {
      const char* vp = vt + (idx * 2) * 1024 + lane * 16;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(vp);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(vp + 1024);
      return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    i32x8 va = vfrag(0), vb = vfrag(1);
    // P~ of elements r0 .. r0+NE-1 of 32-key block kb into its FP8 slots.
    auto exp_part = [&](int kb, int r0, auto ne_tag) __attribute__((always_inline)) {
      constexpr int NE = decltype(ne_tag)::value;
      float e[NE];
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        const int r = r0 + j;
        const float x = SQ ? as_float(s[kb][r]) : (float)s[kb][r] * ck[kb];
        e[j] = __builtin_amdgcn_exp2f(x - m_new);
        if constexpr (MASK && !SQ) e[j] = (s[kb][r] == INT_MIN) ? 0.f : e[j];
      }
      // this part's share of l as a tree (not a chain)
      float t[NE / 2];
#pragma unroll
      for (int j = 0; j < NE / 2; ++j) t[j] = e[2 * j] + e[2 * j + 1];
#pragma unroll
      for (int w = NE / 4; w >= 1; w /= 2)
#pragma unroll
        for (int j = 0; j < w; ++j) t[j] = t[2 * j] + t[2 * j + 1];
      l_part += t[0];
#pragma unroll
      for (int w = 0; w < NE / 4; ++w) {
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = e[4 * w + j] * 448.0f;
        // the high half is written by the second convert: any old value
        // does, and y's own register avoids zeroing one first
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], as_int(y[0]), false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
        pf[kb / 2][(kb % 2) * 4 + r0 / 4 + w] = pk;
      }
    };
    // ---- P, then O^T += V^T P^T on the FP8 matrix cores, overlapped: the
    // MFMAs of keys 0..63 go one at a time beside 1/NKC of the exponentials
    // of keys 64..127 (a wave's MFMAs overlap well with its own VALU work),
    // then those of keys 64..127.  With d = 128 the matrix-core precedence
    // starts with the first of them.
    auto exp_pv = [&]() __attribute__((always_inline)) {
      using E16 = std::integral_constant<int, 16>;
      using EC = std::integral_constant<int, 32 / NKC>;
      {
        exp_part(0, 0, E16{});
        exp_part(1, 0, E16{});
        pin(pf[0]);
        rescale_o();
        __builtin_amdgcn_sched_barrier(0);
        prio_mfma();

#pragma unroll
        for (int c = 0; c < NKC; ++c) {
          const i32x8 vn = vfrag(c + 2);
          acc_o[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pf[0], acc_o[c], 0, 0, 0,
                                                                       127, 0, 127);
          const int e0 = c * (32 / NKC);               // element over blocks 2, 3
          exp_part(2 + e0 / 16, e0 % 16, EC{});
          __builtin_amdgcn_sched_barrier(0);
          va = vb;
          vb = vn;
        }
#pragma unroll
        for (int c = 0; c < NKC; ++c) {
          const i32x8 vn = (NKC + c + 2 < 2 * NKC) ? vfrag(NKC + c + 2) : i32x8{};
          acc_o[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pf[1], acc_o[c], 0, 0, 0,
                                                                       127, 0, 127);
          __builtin_amdgcn_sched_barrier(0);
          va = vb;
          vb = vn;
        }
      }
    };
    if constexpr (PV4) {
      // ---- MXFP4: P~ = 2^(x - m) as above; block kb's shared exponent is
      // e = floor(log2 max P~) - 2 (clamped to [-127, 127], -127 for an
      // all-zero block), taken from the float32 P~ of the block's largest
      // score (the same value that element's own exponential gives); the
      // codes are E2M1(P~ / 2^e) (nearest, ties even, saturated to 6) by the
      // scaled convert; l sums P~ itself.
      int ex[4];
      uint32_t pk4[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float pm = __builtin_amdgcn_exp2f(xk[kb] - m_new);
        ex[kb] = pm > 0.f ? min(max(__builtin_amdgcn_frexp_expf(pm) - 3, -127), 127) : -127;
        const float sc = as_float((ex[kb] + 127) << 23);   // E8M0 code in the exponent field
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = (float)s[kb][r] * ck[kb];
          e[r] = __builtin_amdgcn_exp2f(x - m_new);
          if constexpr (MASK) e[r] = (s[kb][r] == INT_MIN) ? 0.f : e[r];
        }
        float u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = e[2 * j] + e[2 * j + 1];
#pragma unroll
        for (int w = 4; w >= 1; w /= 2)
#pragma unroll
          for (int j = 0; j < w; ++j) u[j] = u[2 * j] + u[2 * j + 1];
        l_part += u[0];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          uint32_t pk = 0u;
          static_for<4>([&](auto ji) {
            constexpr int j = decltype(ji)::value;
            pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk, e[8 * w + 2 * j],
                                                          e[8 * w + 2 * j + 1], sc, j);
          });
          pk4[kb][w] = pk;
        }
      }
      rescale_o();
      prio_mfma();
      // ---- O^T += V^T P^T on the FP4 matrix cores, 64 keys per MFMA: after
      // exchanging lane halves, half g holds all 32 keys of block 2h + g
      // (nibble p = key mx_slot_key(p)), as V's chunks do.
      const char* vsc = vt + VBYTES;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const auto r0 = __builtin_amdgcn_permlane32_swap(pk4[2 * hh][0], pk4[2 * hh + 1][0], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(pk4[2 * hh][1], pk4[2 * hh + 1][1], false, false);
        const i32x8 bop = {(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1], 0, 0, 0, 0};
        const int sb = (half ? ex[2 * hh + 1] : ex[2 * hh]) + 127;
        const int sa = *reinterpret_cast<const int*>(vsc + (hh * 64 + lane) * 4);
        static_for<NKC>([&](auto ci) {
          constexpr int c = decltype(ci)::value;
          const i32x4 a4 = *reinterpret_cast<const i32x4*>(vt + ((hh * NKC + c) * 64 + lane) * 16);
          const i32x8 aop = {a4[0], a4[1], a4[2], a4[3], 0, 0, 0, 0};
          // A and B are FP4 (format 4); A's scale is byte c of sa
          acc_o[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, acc_o[c], 4, 4, c,
                                                                       sa, 0, sb);
        });
      }
    } else {
      exp_pv();
    }
  };

  const bool last_masked = CAUSAL || (N % kKvTile) != 0;
  const int nfull = last_masked ? ntiles - 1 : ntiles;
  for (int t = 0; t < nfull; ++t) step(t, std::false_type{});
  if (last_masked) step(ntiles - 1, std::true_type{});

  // ---- O = O / (448 l) * dV (MXFP4: O / l, V's scales were applied by the
  // matrix cores).
#pragma unroll
  for (int c = 0; c < NKC; ++c) pin(acc_o[c]);
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  const float inv = 1.0f / (PV4 ? l_tot : l_tot * 448.0f);
  // Row log-sum-exp (natural log) of the scores the softmax used: the
  // running max m (log2 units) and l = sum 2^(x - m) give
  // ln sum exp(S) = ln 2 * (m + log2(l)); plus the caller's correction for
  // smoothed K (sm_scale * q . mean K) when given.
  if (lse != nullptr && half == 0 && qi < N) {
    const size_t row = (size_t)(b * H + h) * N + qi;
    float v = 0.69314718055994531f * (m_run + log2f(l_tot));
    if (lse_corr != nullptr) v += lse_corr[row];
    lse[row] = v;
  }
  if (qi < N) {
    char* orow = reinterpret_cast<char*>(out) + ((size_t)(b * H + h) * N + qi) * D * 2;
#pragma unroll
    for (int c = 0; c < NKC; ++c)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int ch = c * 32 + 8 * r4 + 4 * half;
        const float4 s4 = PV4 ? float4{1.f, 1.f, 1.f, 1.f}
                              : *reinterpret_cast<const float4*>(lds_vs + (PV4 ? 0 : ch));
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = acc_o[c][r4 * 4 + j] * inv * sv[j];
        uint2 pk;
        if (BF16) {
          __hip_bfloat16 x0 = __float2bfloat16(v[0]), x1 = __float2bfloat16(v[1]);
          __hip_bfloat16 x2 = __float2bfloat16(v[2]), x3 = __float2bfloat16(v[3]);
          pk.x = (uint32_t)__builtin_bit_cast(uint16_t, x0) | ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
          pk.y = (uint32_t)__builtin_bit_cast(uint16_t, x2) | ((uint32_t)__builtin_bit_cast(uint16_t, x3) << 16);
        } else {
          __half x0 = __float2half(v[0]), x1 = __float2half(v[1]);
          __half x2 = __float2half(v[2]), x3 = __float2half(v[3]);
          pk.x = (uint32_t)__builtin_bit_cast(uint16_t, x0) | ((uint32_t)__builtin_bit_cast(uint16_t, x1) << 16);
          pk.y = (uint32_t)__builtin_bit_cast(uint16_t, x2) | ((uint32_t)__builtin_bit_cast(uint16_t, x3) << 16);
        }
        *reinterpret_cast<uint2*>(orow + ch * 2) = pk;
      }
  }
}

// Diagnostic: exact int32 S = Q^ K^T of one head, through the same K tile
// loader (buffer loads, zeros past N), LDS fragment layout and qk_frags
// routine as attn_fwd_kernel.
template <int D>
__global__ __launch_bounds__(kWaves * 64) void qk_int32_kernel(
    const int8_t* __restrict__ q_i8, const int8_t* __restrict__ k_i8, int32_t* __restrict__ s_out,
    int N, size_t qoff, size_t kvoff) {
  constexpr int NKC = D / 32;
  __shared__ __attribute__((aligned(16))) char lds[kKvTile * D];
  const int qt = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int half = lane >> 5;
  const int qi = qt * kBlockQ + wave * kWaveQ + (lane & 31);
  const int8_t* qh = q_i8 + qoff;
  const int8_t* kh = k_i8 + kvoff;

  constexpr int KNB = (kKvTile / 32) * NKC / kWaves;
  uint32_t koff[KNB];
#pragma unroll
  for (int i = 0; i < KNB; ++i) koff[i] = k_tile_offset<D>(i * kWaves + wave, lane);
  load_k_tile<D>(make_rsrc(kh, (uint32_t)N * D), t * kKvTile, koff, lds, wave);
  wait_vmem();
  __syncthreads();
  i32x4 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    qf[kc] = (qi < N) ? *reinterpret_cast<const i32x4*>(qh + (size_t)qi * D + kc * 32 + half * 16)
                      : i32x4{0, 0, 0, 0};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    i32x4 kf[NKC];
    read_k_frags<NKC>(lds + kb * NKC * 1024, lane, kf);
    i32x16 s = qk_frags<NKC>(kf, qf);
    pin(s);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = t * kKvTile + kb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
      if (qi < N && key < N)
        s_out[(size_t)qi * N + key] = s[r];
    }
  }
}

}  // namespace sage

// ---------------------------------------------------------------------------
// Host launchers (called by the C ABI after validation).

hipError_t sage_launch_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                const float* k_scale, const uint8_t* v_f8, const float* v_scale,
                                const uint8_t* v_e8, const float* delta_s, void* o, int bf16_out,
                                float* lse, const float* lse_corr, int B, int H, int H_kv, int N,
                                int d, int q_group, int causal, float sm_scale, int bk0, int nbk,
                                int qt0, int nqt, hipStream_t stream) {
  using namespace sage;
  const int qg_shift = q_group == kBlkQ ? 7 : q_group == kWaveQ ? 5 : q_group == 1 ? 0 : -1;
  if (qg_shift < 0) return hipErrorInvalidValue;
  const int ntq = (N + kBlockQ - 1) / kBlockQ;
  if (qt0 < 0 || nqt <= 0 || qt0 + nqt > ntq) return hipErrorInvalidValue;
  if (bk0 < 0 || nbk <= 0 || bk0 + nbk > B * H_kv) return hipErrorInvalidValue;
  const long long total = (long long)nbk * (H / H_kv) * nqt;
  if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  const float lam = sm_scale * kLog2e;   // the softmax constant in log2 units
  dim3 grid((unsigned)total), block(kWaves * 64);
  const bool sq = delta_s != nullptr, pv4 = v_e8 != nullptr;
  if (sq && pv4) return hipErrorInvalidValue;
#define SAGE_ATTN_CASE(DD, CC, BB, SS, PP)                                                        \
  if (d == DD && (causal != 0) == CC && (bf16_out != 0) == BB && sq == SS && pv4 == PP) {          \
    hipLaunchKernelGGL((attn_fwd_kernel<DD, CC, BB, SS, PP>), grid, block, 0, stream, q_i8,       \
                       q_scale, k_i8, k_scale, v_f8, v_scale, v_e8, delta_s, o, lse, lse_corr, H, \
                       H_kv, N, lam, qg_shift, bk0, qt0, nqt, (int)total);                    \
    return hipGetLastError();                                                                     \
  }
#define SAGE_ATTN_CASES(SS, PP)              \
  SAGE_ATTN_CASE(64, false, false, SS, PP)  \
  SAGE_ATTN_CASE(64, false, true, SS, PP)   \
  SAGE_ATTN_CASE(64, true, false, SS, PP)   \
  SAGE_ATTN_CASE(64, true, true, SS, PP)    \
  SAGE_ATTN_CASE(128, false, false, SS, PP) \
  SAGE_ATTN_CASE(128, false, true, SS, PP)  \
  SAGE_ATTN_CASE(128, true, false, SS, PP)  \
  SAGE_ATTN_CASE(128, true, true, SS, PP)
  SAGE_ATTN_CASES(false, false)
  SAGE_ATTN_CASES(true, false)
  SAGE_ATTN_CASES(false, true)
#undef SAGE_ATTN_CASES
#undef SAGE_ATTN_CASE
  return hipErrorInvalidValue;
}

hipError_t sage_launch_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int H_kv,
                                int N, int d, int b, int h, int32_t* s_out, hipStream_t stream) {
  using namespace sage;
  const int nt = (N + kKvTile - 1) / kKvTile;
  const size_t qoff = (size_t)(b * H + h) * N * d;
  const size_t koff = (size_t)(b * H_kv + h / (H / H_kv)) * N * d;
  dim3 grid(nt, nt), block(kWaves * 64);
  if (d == 64)
    hipLaunchKernelGGL(qk_int32_kernel<64>, grid, block, 0, stream, q_i8, k_i8, s_out, N, qoff, koff);
  else if (d == 128)
    hipLaunchKernelGGL(qk_int32_kernel<128>, grid, block, 0, stream, q_i8, k_i8, s_out, N, qoff, koff);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
