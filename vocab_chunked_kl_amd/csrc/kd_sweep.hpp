// kd_sweep.hpp - the pipelined MFMA tile loop shared by the logit-rebuilding
// kernels and the dh GEMM.
//
// A block owns a fixed B tile (TN rows: a token tile for the logit kernels, a
// d-tile of the transposed unembedding for dh) and walks a run of A tiles
// (TM rows each: vocabulary tiles, or one token tile for dh). For every A tile
// it contracts two operand pairs over their K extents into two fp32
// accumulators, acc1 = A1 . B1^T (K1 bytes) and acc2 = A2 . B2^T (K2 bytes;
// K2 may be 0), then hands both to the epilogue functor and zeroes them.
// For the logits: pair 1 = (W_s, h_s) -> z_s, pair 2 = (W_t, h_t) -> z_t,
// both for the same (vocabulary, token) tile, as the block logit rebuild of
// the Nitrobrew notes ("Nitrobrew 的两个动作") needs them side by side.
//
// Pipeline: a ring of three LDS stage buffers filled by direct-to-LDS buffer
// loads (no staging registers, no LDS store instructions). While stage i is
// multiplied, the loads of stages i+1 and i+2 are in flight; one barrier per
// stage recycles the buffer read in the previous step.
#pragma once

#include "kd_device.hpp"

#ifndef KD_SPAN2
#define KD_SPAN2 3
#endif

namespace kd {

struct PairDesc {
  const char* A;      // [a_rows, K] row-major
  const char* B;      // [b_rows, K] row-major
  int64_t lda, ldb;   // row pitch in bytes
  int64_t a_rows, b_rows;
  int32_t kbytes;     // contracted extent in bytes (multiple of 16)
};

// s_waitcnt immediate that waits until at most `n` vector-memory operations
// of this wave are outstanding (the LDS and export counters are not waited on).
__device__ __forceinline__ constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier with the wave's own LDS operations drained first. Written
// as one asm statement (a "memory" clobber keeps every memory access on its
// side) so that the compiler does not also drain the direct-to-LDS loads in
// flight: the stage ring below waits for those itself, one stage at a time.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// sched_group_barrier masks
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

// LDS stage layout: [A tile: TM rows][B tile: TN rows], 128 bytes per row,
// unpadded, with the 16-byte chunks of row R stored at slot (chunk ^ swz(R)),
// swz(R) = (R & 7) ^ ((R >> 3) & 3). Direct-to-LDS loads write 64 lanes x 16
// bytes contiguously (8 rows per instruction), and the XOR spreads the MFMA
// fragment reads of 16 consecutive rows over all banks.
__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 3); }

template <int TM, int TN>
struct Ring {
  static constexpr int kBytes = (TM + TN) * kStageBytes;
};

// Issue the direct-to-LDS loads of one stage (this wave's share of NW waves:
// (TM + TN) / (8 NW) instructions of 8 rows each). `a_base` / `b_base`:
// resources starting at the tile's first row; `lane_row` = (lane >> 3) * ld
// for each operand; a lane whose chunk lies at or past the row length, or
// every lane when `valid` is false, reads past the resource end and writes
// zeros.
template <int TM, int TN, int NW>
__device__ __forceinline__ void dma_stage(char* dst, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          int32_t a_lane_row, int32_t b_lane_row, int64_t lda, int64_t ldb,
                                          int32_t kbyte0, int32_t kbytes, bool valid, int wave, int lane) {
  constexpr int QA = TM / (8 * NW), QB = TN / (8 * NW);  // instructions per wave
  static_assert(QA * 8 * NW == TM && QB * 8 * NW == TN, "tile rows must split evenly over the waves");
  const int c_lo = lane & 7, c_hi = lane >> 3;
#pragma unroll
  for (int i = 0; i < QA; ++i) {
    const int q = wave * QA + i;                 // 8-row group index within the tile
    const int c = c_lo ^ c_hi ^ (q & 3);         // global chunk this lane moves
    const bool in = valid && (kbyte0 + c * 16 < kbytes);
    const int32_t off = in ? a_lane_row + (int32_t)(8 * q * lda) + c * 16 + kbyte0 : 0x7FFFFFF0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(dst + q * 1024), 16, off,
                                             0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < QB; ++i) {
    const int q = wave * QB + i;
    const int c = c_lo ^ c_hi ^ (q & 3);
    const bool in = valid && (kbyte0 + c * 16 < kbytes);
    const int32_t off = in ? b_lane_row + (int32_t)(8 * q * ldb) + c * 16 + kbyte0 : 0x7FFFFFF0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (__attribute__((address_space(3))) void*)(dst + TM * kStageBytes + q * 1024), 16, off, 0, 0, 0);
  }
}

// Pinned instruction order of one stage (sched_group_barrier takes literal
// counts, hence the compile-time recursion over MFMA index M): the LDS reads
// of sub-step 0 first; then each MFMA is followed by at most one LDS read of
// the next sub-step, and the `kLoads` direct-to-LDS loads are spread evenly
// over the first kSpan MFMAs.
template <int kMf, int kRd, int kLoads, int kSpan, int M = 0>
__device__ __forceinline__ void pin_stage_order() {
  if constexpr (M == 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kRd, 0);
  if constexpr (M < 4 * kMf) {
    constexpr int lo = M * kLoads / kSpan, hi = (M + 1) * kLoads / kSpan;
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (M < 3 * kMf && (M % kMf) < kRd) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    if constexpr (M < kSpan && hi > lo) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, hi - lo, 0);
    pin_stage_order<kMf, kRd, kLoads, kSpan, M + 1>();
  }
}

// MFMAs of one LDS stage for this wave: four k16 sub-steps, fragments double
// buffered in registers so the reads of sub-step j+1 overlap the MFMAs of j.
// a_off / b_off: this lane's row byte offset; colx[j]: its swizzled chunk
// byte offset for sub-step j. `issue` emits the direct-to-LDS loads of a later
// stage; they are spread between the MFMAs (a burst of loads right after the
// barrier would stall the wave's issue while the address unit drains them).
template <bool kBf16, int MB, int NB, int kLoads, int kSpanQ, class Issue>
__device__ __forceinline__ void mma_ring_stage(floatx16 (&acc)[MB][NB], const char* cur, int a_off, int b_off,
                                               const int (&colx)[4], Issue&& issue) {
  u32x4 fa[2][MB], fb[2][NB];
  auto rd = [&](int s, int j) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      fa[s][mb] = *reinterpret_cast<const u32x4*>(cur + a_off + colx[j] + mb * 32 * kStageBytes);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      fb[s][nb] = *reinterpret_cast<const u32x4*>(cur + b_off + colx[j] + nb * 32 * kStageBytes);
  };
  auto mm = [&](int s) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (kBf16) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[s][mb]),
                                                                __builtin_bit_cast(bf16x8, fb[s][nb]), acc[mb][nb], 0,
                                                                0, 0);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t ae = fa[s][mb][e], be = fb[s][nb][e];
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, ae),
                                                               __builtin_bit_cast(float, be), acc[mb][nb], 0, 0, 0);
          }
        }
      }
  };
  constexpr int kRd = MB + NB;
  constexpr int kMf = MB * NB * (kBf16 ? 1 : 4);
  constexpr int kTotMf = 4 * kMf;
  rd(0, 0);
  issue();
  rd(1, 1);
  mm(0);
  rd(0, 2);
  mm(1);
  rd(1, 3);
  mm(0);
  mm(1);
  pin_stage_order<kMf, kRd, kLoads, kSpanQ == 0 ? 1 : kSpanQ * kMf>();
}

// Shared LDS of the stage ring: three separate objects, so that the compiler
// sees that reads of one stage never alias the loads landing in another.
template <int TM, int TN>
struct RingLds {
  char* b0;
  char* b1;
  char* b2;
};

// WM x WN waves: wave w owns rows (w % WM) * TM / WM .. of the A tile and rows
// (w / WM) * TN / WN .. of the B tile; its accumulators are [MB][NB] 32 x 32
// MFMA blocks, MB = TM / (32 WM), NB = TN / (32 WN).
// kDual = false: one operand pair only (p2 is ignored, the epilogue gets acc1
// twice and no second accumulator is allocated).
template <bool kBf16, int TM, int TN, int WM, int WN, class Epi, int NBUF = 3, bool kDual = true>
__device__ __forceinline__ void sweep(const PairDesc& p1, const PairDesc& p2, int64_t b_row0, int a_tile_begin,
                                      int a_tile_end, const RingLds<TM, TN>& lds, Epi&& epi) {
  static_assert(NBUF == 2 || NBUF == 3, "ring of two or three stage buffers");
  constexpr int NW = WM * WN;
  constexpr int MB = TM / (32 * WM), NB = TN / (32 * WN);
  static_assert(MB * 32 * WM == TM && NB * 32 * WN == TN, "wave tiles must be multiples of 32");
  constexpr int kDma = (TM + TN) / (8 * NW);  // direct-to-LDS loads per wave per stage
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int a_off = ((wave % WM) * (TM / WM) + r32) * kStageBytes;
  const int b_off = (TM + (wave / WM) * (TN / WN) + r32) * kStageBytes;
  int colx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) colx[j] = ((2 * j + (lane >> 5)) ^ lds_swz(r32)) * 16;

  const int ks1 = (p1.kbytes + kStageBytes - 1) / kStageBytes;
  const int ks2 = kDual ? (p2.kbytes + kStageBytes - 1) / kStageBytes : 0;
  if (a_tile_end <= a_tile_begin || ks1 == 0) return;

  const int32_t la1 = (int32_t)((lane >> 3) * p1.lda), la2 = (int32_t)((lane >> 3) * p2.lda);
  const int32_t lb1 = (int32_t)((lane >> 3) * p1.ldb), lb2 = (int32_t)((lane >> 3) * p2.ldb);
  const __amdgpu_buffer_rsrc_t rb1 = make_rsrc(p1.B + b_row0 * p1.ldb, (p1.b_rows - b_row0) * p1.ldb);
  const __amdgpu_buffer_rsrc_t rb2 = make_rsrc(p2.B + b_row0 * p2.ldb, (p2.b_rows - b_row0) * p2.ldb);

  // Fetch cursor: the stage issued next (tile, pair, stage). The loads pick
  // their operand pair with selects, not branches, so that they stay in the
  // MFMA block and can be interleaved with it; the cursor advances after it.
  int ft = a_tile_begin, fp = 0, fs = 0;
  auto issue = [&](char* dst) {
    const bool valid = ft < a_tile_end;
    const bool second = kDual && fp != 0;
    const int64_t a_row0 = (int64_t)(valid ? ft : a_tile_begin) * TM;
    const char* A = second ? p2.A : p1.A;
    const int64_t lda = second ? p2.lda : p1.lda, ldb = second ? p2.ldb : p1.ldb;
    const int64_t a_rows = second ? p2.a_rows : p1.a_rows;
    dma_stage<TM, TN, NW>(dst, make_rsrc(A + a_row0 * lda, (a_rows - a_row0) * lda), second ? rb2 : rb1,
                      second ? la2 : la1, second ? lb2 : lb1, lda, ldb, fs * kStageBytes,
                      second ? p2.kbytes : p1.kbytes, valid, wave, lane);
  };
  auto advance = [&] {
    const bool wrap = fs + 1 == (fp == 0 ? ks1 : ks2);
    const int nfp = (fp == 0 && ks2 > 0) ? 1 : 0;
    ft += (wrap && nfp == 0) ? 1 : 0;
    fs = wrap ? 0 : fs + 1;
    fp = wrap ? nfp : fp;
  };

  // One ring step on buffer `cur`: wait for its loads (with three buffers the
  // next stage's loads stay in flight), barrier, refill the buffer read one
  // step earlier with the stage NBUF-1 ahead, multiply `cur`.
  auto step = [&](floatx16(&acc)[MB][NB], char* cur, char* refill) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NBUF == 3 ? kDma : 0));
    lds_barrier();
    mma_ring_stage<kBf16, MB, NB, kDma, NBUF == 3 ? 3 : KD_SPAN2>(acc, cur, a_off, b_off, colx, [&] { issue(refill); });
    advance();
  };
  // Run `ks` stages into `acc` starting with ring position `rot`.
  auto run = [&](floatx16(&acc)[MB][NB], int ks, int rot) {
    int s = 0;
    if constexpr (NBUF == 3) {
      switch (rot) {
        case 0:
          for (; s + 3 <= ks; s += 3) {
            step(acc, lds.b0, lds.b2);
            step(acc, lds.b1, lds.b0);
            step(acc, lds.b2, lds.b1);
          }
          if (s < ks) step(acc, lds.b0, lds.b2), ++s;
          if (s < ks) step(acc, lds.b1, lds.b0), ++s;
          break;
        case 1:
          for (; s + 3 <= ks; s += 3) {
            step(acc, lds.b1, lds.b0);
            step(acc, lds.b2, lds.b1);
            step(acc, lds.b0, lds.b2);
          }
          if (s < ks) step(acc, lds.b1, lds.b0), ++s;
          if (s < ks) step(acc, lds.b2, lds.b1), ++s;
          break;
        default:
          for (; s + 3 <= ks; s += 3) {
            step(acc, lds.b2, lds.b1);
            step(acc, lds.b0, lds.b2);
            step(acc, lds.b1, lds.b0);
          }
          if (s < ks) step(acc, lds.b2, lds.b1), ++s;
          if (s < ks) step(acc, lds.b0, lds.b2), ++s;
          break;
      }
    } else {
      if (rot == 0) {
        for (; s + 2 <= ks; s += 2) {
          step(acc, lds.b0, lds.b1);
          step(acc, lds.b1, lds.b0);
        }
        if (s < ks) step(acc, lds.b0, lds.b1);
      } else {
        for (; s + 2 <= ks; s += 2) {
          step(acc, lds.b1, lds.b0);
          step(acc, lds.b0, lds.b1);
        }
        if (s < ks) step(acc, lds.b1, lds.b0);
      }
    }
  };

  floatx16 acc1[MB][NB], acc2[kDual ? MB : 1][kDual ? NB : 1];
  zero_acc(acc1);
  if constexpr (kDual) zero_acc(acc2);
  issue(lds.b0);  // stage 0
  advance();
  if (NBUF == 3) {  // stage 1
    issue(lds.b1);
    advance();
  }
  int rot = 0;
  for (int tile = a_tile_begin; tile < a_tile_end; ++tile) {
    run(acc1, ks1, rot);
    rot = (rot + ks1) % NBUF;
    if constexpr (kDual) {
      if (ks2 > 0) {
        run(acc2, ks2, rot);
        rot = (rot + ks2) % NBUF;
      }
      epi(tile, acc1, acc2);
      zero_acc(acc2);
    } else {
      epi(tile, acc1, acc1);
    }
    zero_acc(acc1);
  }
  // drain the loads issued past the end before the LDS is reused
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
}

}  // namespace kd
