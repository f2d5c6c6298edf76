// sage_device.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core conventions used throughout (CDNA 32x32 MFMA family):
//   A operand: lane L supplies row (L % 32) and the K-slice chosen by L / 32;
//   B operand: lane L supplies column (L % 32) and the same K-slice;
//   C/D (32x32, 16 values per lane): register r of lane L holds
//     row = 8*(r/4) + 4*(L/32) + (r%4), column = L % 32.
// A and B share the K-slice mapping, so a contraction over K is correct for
// any order of K inside the slices, as long as both operands use one order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sage {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlkQ = 128;     // Q tokens per INT8 scale (the default Q granularity)
constexpr int kBlkK = 64;      // K tokens per INT8 scale
constexpr int kKvTile = 128;   // keys per online-softmax step / V tile
constexpr int kMxScaleBytes = 512;   // MXFP4 V scale bytes per tile: 2 halves x 64 lanes x 4
constexpr int kWaveQ = 32;     // queries per wave (one 32-wide MFMA column block)
constexpr int kWaves = 4;      // waves per workgroup
constexpr int kBlockQ = kWaveQ * kWaves;   // queries per workgroup (== kBlkQ)
static_assert(kBlockQ == kBlkQ, "a 128-token Q scale block is one workgroup's queries");
static_assert(kBlkQ == 1 << 7 && kWaveQ == 1 << 5, "Q scale groups are shifts of the query index");

constexpr float kLog2e = 1.4426950408889634f;

// Bit casts through a by-value parameter.  (Applying __builtin_bit_cast
// directly to an ext_vector element, e.g. bit_cast<float>(v[r]), makes this
// compiler read element 0 for every r; going through a scalar is correct.)
__device__ __forceinline__ float as_float(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int as_int(float x) { return __builtin_bit_cast(int, x); }

// Force a matrix-core accumulator to be fully computed at this point.  The
// MFMA reads its operands from all 64 lanes regardless of the exec mask, so
// it must never be moved (with the loads feeding it) into a lane-divergent
// branch; an empty asm that "modifies" the value pins its computation here.
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

// Key (0..63 inside a 64-key half tile) held by byte s (0..31) of a lane in
// half g (0/1) of the 32x32x64 FP8 operand: bytes 0..15 come from the C/D
// registers r = 0..15 of the first 32-key S block, bytes 16..31 from the
// second block (see the C/D row formula above).
__host__ __device__ constexpr int fp8_slot_key(int g, int s) {
  return (s / 16) * 32 + ((s % 16) / 4) * 8 + g * 4 + (s % 4);
}

// max(x, x from lane L ^ 32) in every lane, on the VALU (v_permlane32_swap
// exchanges the lane halves of two registers) instead of an LDS permute.
// swap(x, y) returns {[x_lo, y_lo], [x_hi, y_hi]}; with y a copy of x the
// max of the two is the cross-half max.  The copy goes through an empty asm
// so the two operands are distinct values to the optimizer.
__device__ __forceinline__ float max_xor32(float x) {
  int a = __builtin_bit_cast(int, x), b = a;
  asm volatile("" : "+v"(b));
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}

// f(std::integral_constant<int, I>) for I = 0 .. N-1, each I a constant
// expression (for builtin arguments that must be immediates).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Key (0..31 inside a 32-key block) of nibble p (0..31) of a lane's 16-byte
// FP4 operand (32 keys of one block): nibbles 0..15 are the block's keys that
// lane half 0 holds in the C/D layout (8*(r/4) + r%4), nibbles 16..31 those of
// half 1 (8*(r/4) + 4 + r%4) -- the order of P after the lane-half exchange.
__host__ __device__ constexpr int mx_slot_key(int p) {
  return 8 * ((p % 16) / 4) + 4 * (p / 16) + (p % 4);
}

// Map a linear workgroup id to a logical work id so that each XCD (ids are
// dealt round-robin to the 8 XCDs) receives one contiguous range of logical
// ids.  A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int q = total / 8, rem = total % 8;
  const int x = id % 8, j = id / 8;
  return x * q + min(x, rem) + j;
}

// ---------------------------------------------------------------------------
// INT8 S^T tile: 32 keys x 32 queries from the lane's K fragments `kf` (A
// operand, one per 32-channel chunk) and Q fragments `qf` (B operand).
// Returns the 16 C/D values, the exact int32 sums (the accumulator starts
// from the inline constant 0: no register is seeded per tile).
template <int NKC>
__device__ __forceinline__ i32x16 qk_frags(const i32x4* kf, const i32x4* qf) {
  i32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0;
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kc], qf[kc], acc, 0, 0, 0);
  return acc;
}

// The lane's K fragments of one 32-key block: `kfrag` points at the block's
// LDS fragments (NKC x 1 KB, lane-major 16 bytes per lane).
template <int NKC>
__device__ __forceinline__ void read_k_frags(const char* kfrag, int lane, i32x4* kf) {
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) kf[kc] = *reinterpret_cast<const i32x4*>(kfrag + kc * 1024 + lane * 16);
}

typedef __attribute__((address_space(3))) void lds_void;

// Wait until this wave's outstanding vector-memory operations (including
// global->LDS loads) have completed: s_waitcnt vmcnt(0), other counters
// left alone.  Must precede the barrier that publishes LDS-load data.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Raw buffer resources (base, byte size; word 3 = the gfx9 raw-buffer format)
// for the tile loads: each lane passes a 32-bit offset computed once, the
// tile's offset is a scalar, and reads at or past the size return zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 (or 4) bytes per lane from the buffer into LDS: lane L of the
// instruction lands at byte 16*L (4*L) of `lds`.
template <int BYTES>
__device__ __forceinline__ void buffer_to_lds(rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword loads");
  if constexpr (BYTES == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, soff, 0, 0);
}

// K tile (kKvTile keys x D int8) -> LDS in fragment-major order, 16 bytes
// per lane per 1 KB block.  Block (kb32, kc) holds, for lane L, key
// kb32*32 + L%32 and channel bytes kc*32 + 16*(L/32) .. +16: exactly the
// A-operand fragment of the INT8 MFMA.  Wave w loads blocks w, w + 4, ...;
// `koff[i]` is the lane's byte offset of block i*4 + w relative to the
// tile's first key (tile-invariant).  Keys >= N read zeros (their scores are
// masked).
template <int D>
__device__ __forceinline__ uint32_t k_tile_offset(int blk, int lane) {
  constexpr int NKC = D / 32;
  const int kb32 = blk / NKC, kc = blk % NKC;
  return (uint32_t)((kb32 * 32 + lane % 32) * D + kc * 32 + 16 * (lane / 32));
}
template <int D>
__device__ __forceinline__ void load_k_tile(rsrc_t rk, int key0, const uint32_t* koff, char* lds_k,
                                            int wave) {
  constexpr int NKC = D / 32;
  constexpr int NB = (kKvTile / 32) * NKC;
  static_assert(NB % kWaves == 0, "whole blocks per wave");
  const uint32_t soff = (uint32_t)key0 * D;
#pragma unroll
  for (int i = 0; i < NB / kWaves; ++i)
    buffer_to_lds<16>(rk, lds_k + (i * kWaves + wave) * 1024, koff[i], soff);
}

// V tile (already fragment-ordered in HBM, BYTES bytes: kKvTile*D FP8 or
// half that of FP4 codes) -> LDS, a straight copy in 1 KB blocks.
template <int BYTES>
__device__ __forceinline__ void load_v_tile(rsrc_t rv, int t, char* lds_v, int wave, int lane) {
  constexpr int NB = BYTES / 1024;
  static_assert(NB % kWaves == 0, "whole blocks per wave");
  const uint32_t soff = (uint32_t)t * BYTES;
#pragma unroll
  for (int i = 0; i < NB / kWaves; ++i) {
    const int blk = i * kWaves + wave;
    buffer_to_lds<16>(rv, lds_v + blk * 1024, (uint32_t)(blk * 1024 + lane * 16), soff);
  }
}

}  // namespace sage
