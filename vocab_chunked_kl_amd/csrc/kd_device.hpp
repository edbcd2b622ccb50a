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

constexpr int kThreads = 256;
constexpr int kStageBytes = 128;                // K bytes per row per LDS stage
constexpr int kPitch = kStageBytes + 16;        // padded LDS row pitch (bank spread)
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

// --------------------------------------------------------------------------
// Global -> register staging of one K stage of a ROWS-row operand tile.
// Thread t moves 16-byte chunks c = t + 256 i: row c / 8, byte column (c % 8) * 16.
// The resource starts at the tile's first row and ends at the operand's last
// row, so rows past the end read as zero; `tail` zeroes the bytes at or past
// the row length in a partial last stage (only then is it evaluated).
// --------------------------------------------------------------------------
template <int ROWS>
struct Stage {
  static constexpr int kChunks = ROWS * 8 / kThreads;
  static_assert(kChunks >= 1 && ROWS * 8 % kThreads == 0, "tile rows must be a multiple of 32");
  u32x4 v[kChunks];

  // byte offset of this thread's chunk 0 inside the tile; chunk i sits
  // 32 * i rows further down
  __device__ __forceinline__ static int32_t lane_off(int tid, int64_t ld_bytes) {
    return (int32_t)((tid >> 3) * ld_bytes + (tid & 7) * 16);
  }

  // Branch-free: a lane whose 16 bytes lie at or past the row length (K
  // tail), or any lane when `valid` is false, reads from an offset past the
  // resource end, which returns zeros.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int32_t off0, int32_t row_step, int32_t kbyte0,
                                       int32_t kbytes, bool valid, int tid) {
    const bool in = valid && (kbyte0 + (tid & 7) * 16 < kbytes);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int32_t off = in ? off0 + i * row_step + kbyte0 : 0x7FFFFFF0;
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(lds + (c >> 3) * kPitch + (c & 7) * 16) = v[i];
    }
  }
};

// --------------------------------------------------------------------------
// MFMA on one LDS stage: acc[mb][nb] += A_rows(mb) . B_rows(nb) over the
// stage's 128 K bytes. a_row0 / b_row0: first LDS row of this wave's slice.
// Lane group g = lane >> 5 reads 16 bytes at offset 32 j + 16 g of sub-step j;
// bf16 issues one 32x32x16 MFMA per (mb, nb, j), fp32 four 32x32x2 MFMAs (the
// four floats of each lane pair up k = 8j + e and 8j + 4 + e, the same pairing
// on both operands, so every k is summed exactly once).
// --------------------------------------------------------------------------
template <bool kBf16, int MB, int NB>
__device__ __forceinline__ void mma_stage(floatx16 (&acc)[MB][NB], const char* ldsA, const char* ldsB, int a_row0,
                                          int b_row0, int lane) {
  const int r = lane & 31;
  const int g = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 a[MB], b[NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      a[mb] = *reinterpret_cast<const u32x4*>(ldsA + (a_row0 + mb * 32 + r) * kPitch + j * 32 + g * 16);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      b[nb] = *reinterpret_cast<const u32x4*>(ldsB + (b_row0 + nb * 32 + r) * kPitch + j * 32 + g * 16);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (kBf16) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[mb]),
                                                                __builtin_bit_cast(bf16x8, b[nb]), acc[mb][nb], 0, 0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // copy the element out first: a bit_cast of a vector-element lvalue
            // reads element 0 with this compiler
            const uint32_t ae = a[mb][e], be = b[nb][e];
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, ae),
                                                               __builtin_bit_cast(float, be), acc[mb][nb], 0, 0, 0);
          }
        }
      }
  }
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

// XCD-aware block order: hardware block b runs on XCD b % 8; give each XCD a
// contiguous run of logical tiles so that blocks sharing operand rows meet in
// that XCD's L2. Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
#ifdef KD_NO_XCD_REMAP
  return b;
#endif
  if (nblocks & 7) return b;
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

}  // namespace kd
