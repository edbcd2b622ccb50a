// kd_device.hpp - device building blocks shared by the gfx950 kernels.
//
// The MFMA kernels compute tiles of C = A * B^T where A [rows, K] and B
// [rows, K] are both row-major with K contiguous (an "NT" contraction: logits
// z = W h^T, or dh = G W_s^T with the chunk of W_s transposed); the
// pipelined tile loop itself lives in kd_sweep.hpp.
//
// MFMA lane layouts (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32), as
// checked on the device:  A operand: lane l holds row (l & 31), k-slice
// 8*(l >> 5) .. +7 of a 16-wide k block (bf16) or k = (l >> 5) (fp32);
// B likewise with its row = output column; output register r of lane l holds
// row 8*(r/4) + 4*(l >> 5) + (r % 4), column (l & 31).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef float floatx16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float floatx4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round fp32 to bf16, nearest with ties to even (gfx950's v_cvt_pk_bf16_f32,
// which rounds finite values, ties and denormals alike the same way as the
// integer form u + 0x7FFF + ((u >> 16) & 1) taken over the top 16 bits).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Wave64 reductions (every lane receives the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// log(1 - e^x) for x < 0, in the two-branch form that stays accurate near 0
// (expm1) and far from it (log1p).
__device__ __forceinline__ float log1mexp_f32(float x) {
  return x > -0.69314718f ? logf(-expm1f(x)) : log1pf(-expf(x));
}

// h . W[v] for bf16 rows of d elements (d a multiple of 8, rows 16-byte
// aligned), computed by the whole wave: lane-strided fp32 partial sums, then a
// wave sum; the result is rounded to bf16 and returned as fp32.
__device__ __forceinline__ float wave_dot_bf16(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                               int64_t v, int32_t d, int lane) {
  const uint16_t* w = W + v * d;
  float acc = 0.f;
  for (int i = lane * 8; i < d; i += 64 * 8) {
    const u32x4 hv = *reinterpret_cast<const u32x4*>(h + i);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(w + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t hx = hv[e], wx = wv[e];
      acc = fmaf(__builtin_bit_cast(float, hx << 16), __builtin_bit_cast(float, wx << 16), acc);
      acc = fmaf(__builtin_bit_cast(float, hx & 0xFFFF0000u), __builtin_bit_cast(float, wx & 0xFFFF0000u), acc);
    }
  }
  return __builtin_bit_cast(float, f32_to_bf16_bits(wave_sum(acc)) << 16);
}

// Four such dot products at once (rows v[j] of W; v[j] < 0: no row, result
// unspecified), each accumulated and reduced exactly as wave_dot_bf16 does, so
// the same bits, with the loads of the four rows in flight together.
__device__ __forceinline__ void wave_dot4_bf16(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
                                               const int64_t (&v)[4], int32_t d, int lane, float (&out)[4]) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = lane * 8; i < d; i += 64 * 8) {
    const u32x4 hv = *reinterpret_cast<const u32x4*>(h + i);
    u32x4 wv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wv[j] = v[j] >= 0 ? *reinterpret_cast<const u32x4*>(W + v[j] * d + i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t hx = hv[e], wx = wv[j][e];
        acc[j] = fmaf(__builtin_bit_cast(float, hx << 16), __builtin_bit_cast(float, wx << 16), acc[j]);
        acc[j] = fmaf(__builtin_bit_cast(float, hx & 0xFFFF0000u), __builtin_bit_cast(float, wx & 0xFFFF0000u), acc[j]);
      }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = __builtin_bit_cast(float, f32_to_bf16_bits(wave_sum(acc[j])) << 16);
}

// --------------------------------------------------------------------------
// Raw buffer resource over [base, base + bytes): loads past the end return
// zero, which masks the vocabulary / token tails without branches.
// --------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (bytes < 0 ? 0 : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

template <int MB, int NB>
__device__ __forceinline__ void zero_acc(floatx16 (&acc)[MB][NB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
}

// Output row (within the wave's 32-row block) held by register r of this lane.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Block -> (token tile, vocabulary split): groups of G token tiles visit
// every split before the next group starts, so that the blocks of one XCD (a
// contiguous logical range after xcd_remap) share both W and h rows.
template <int G>
__device__ __forceinline__ void block_coords(int L, int n_tok_tiles, int n_splits, int& tt, int& sp) {
  constexpr int kTokGroup = G;
  const int per_group = kTokGroup * n_splits;
  const int group = L / per_group;
  const int within = L - group * per_group;
  const int rest = n_tok_tiles - group * kTokGroup;
  const int g_eff = rest < kTokGroup ? rest : kTokGroup;
  tt = group * kTokGroup + within % g_eff;
  sp = within / g_eff;
}

// XCD-aware block order: hardware block b runs on XCD b % 8; give each XCD a
// contiguous run of logical tiles so that blocks sharing operand rows meet in
// that XCD's L2. Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  if (nblocks & 7) return b;
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

// The XCD-ordered kernels launch their grid rounded up to a multiple of 8, so
// that the remap applies whatever the tile count (otherwise the token tiles of
// one vocabulary split would land on different XCDs and each fetch the same
// unembedding rows); the blocks past the tile count leave at once.
__host__ __device__ constexpr int xcd_grid(int n) { return (n + 7) & ~7; }

}  // namespace kd
