// kd_device.hpp - device building blocks shared by the gfx950 kernels.
//
// One workgroup = 256 threads = 4 wave64s arranged 2 x 2 over a TM x TN output
// tile of C = A * B^T, where A [rows, K] and B [rows, K] are both row-major
// with K contiguous (an "NT" contraction: logits z = W h^T, or dh = G W_s^T
// with W_s transposed per chunk). K is staged through LDS 128 bytes at a time
// (64 bf16 or 32 fp32 per row), double buffered: the global loads of stage
// i+1 are in flight while the MFMAs consume stage i.
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

// Round an fp32 value to bf16 (nearest, ties to even); finite inputs.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
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

}  // namespace kd
