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
// Pipeline: the global->register prefetch of the next stage is in flight
// while the MFMAs run on the current LDS stage; registers are then written
// into the other LDS buffer and one barrier per stage publishes it. The
// epilogue runs between the MFMAs of a tile's last stage and the LDS store of
// the next tile's first stage, so its VALU/exp work overlaps those loads.
#pragma once

#include "kd_device.hpp"

namespace kd {

struct PairDesc {
  const char* A;      // [a_rows, K] row-major
  const char* B;      // [b_rows, K] row-major
  int64_t lda, ldb;   // row pitch in bytes
  int64_t a_rows, b_rows;
  int32_t kbytes;     // contracted extent in bytes (multiple of 16)
};

template <int TM, int TN>
struct SweepLds {
  char buf[2][(TM + TN) * kPitch];
};

template <bool kBf16, int TM, int TN, class Epi>
__device__ __forceinline__ void sweep(const PairDesc& p1, const PairDesc& p2, int64_t b_row0, int a_tile_begin,
                                      int a_tile_end, SweepLds<TM, TN>& lds, Epi&& epi) {
  constexpr int MB = TM / 64, NB = TN / 64;
  using SA = Stage<TM>;
  using SB = Stage<TN>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int a_row0w = (wave & 1) * (TM / 2);
  const int b_row0w = TM + (wave >> 1) * (TN / 2);  // B rows sit after A rows in an LDS stage

  const int ks1 = (p1.kbytes + kStageBytes - 1) / kStageBytes;
  const int ks2 = (p2.kbytes + kStageBytes - 1) / kStageBytes;
  if (a_tile_end <= a_tile_begin || ks1 == 0) return;

  // Per-lane chunk offsets inside a tile (stage 0); constant for the sweep.
  int32_t oa1[SA::kChunks], ob1[SB::kChunks], oa2[SA::kChunks], ob2[SB::kChunks];
#pragma unroll
  for (int i = 0; i < SA::kChunks; ++i) {
    oa1[i] = SA::lane_off(i, tid, p1.lda);
    oa2[i] = SA::lane_off(i, tid, p2.lda);
  }
#pragma unroll
  for (int i = 0; i < SB::kChunks; ++i) {
    ob1[i] = SB::lane_off(i, tid, p1.ldb);
    ob2[i] = SB::lane_off(i, tid, p2.ldb);
  }
  const __amdgpu_buffer_rsrc_t rb1 = make_rsrc(p1.B + b_row0 * p1.ldb, (p1.b_rows - b_row0) * p1.ldb);
  const __amdgpu_buffer_rsrc_t rb2 = make_rsrc(p2.B + b_row0 * p2.ldb, (p2.b_rows - b_row0) * p2.ldb);

  SA sa;
  SB sb;
  // Fetch stage `s` of pair `pr` of A tile `tile` into registers.
  auto load = [&](int tile, int pr, int s) {
    const int64_t a_row0 = (int64_t)tile * TM;
    if (pr == 0) {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(p1.A + a_row0 * p1.lda, (p1.a_rows - a_row0) * p1.lda);
      sa.load(ra, oa1, s * kStageBytes, p1.kbytes, tid);
      sb.load(rb1, ob1, s * kStageBytes, p1.kbytes, tid);
    } else {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(p2.A + a_row0 * p2.lda, (p2.a_rows - a_row0) * p2.lda);
      sa.load(ra, oa2, s * kStageBytes, p2.kbytes, tid);
      sb.load(rb2, ob2, s * kStageBytes, p2.kbytes, tid);
    }
  };
  auto store = [&](int b) {
    sa.store(lds.buf[b], tid);
    sb.store(lds.buf[b] + TM * kPitch, tid);
  };
  // The stage after (tile, pr, s); false past the end of the sweep.
  auto next = [&](int& tile, int& pr, int& s) -> bool {
    ++s;
    if (pr == 0 && s == ks1) {
      s = 0;
      if (ks2 > 0) pr = 1; else ++tile;
    } else if (pr == 1 && s == ks2) {
      s = 0;
      pr = 0;
      ++tile;
    }
    return tile < a_tile_end;
  };

  floatx16 acc1[MB][NB], acc2[MB][NB];
  zero_acc(acc1);
  zero_acc(acc2);

  int lt = a_tile_begin, lp = 0, ls = 0;  // stage in flight
  load(lt, lp, ls);
  store(0);
  __syncthreads();
  int buf = 0;

  for (int tile = a_tile_begin; tile < a_tile_end; ++tile) {
    for (int s = 0; s < ks1; ++s) {
      const bool more = next(lt, lp, ls);
      if (more) load(lt, lp, ls);
      mma_stage<kBf16>(acc1, lds.buf[buf], lds.buf[buf], a_row0w, b_row0w, lane);
      if (more) store(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    for (int s = 0; s < ks2; ++s) {
      const bool more = next(lt, lp, ls);
      if (more) load(lt, lp, ls);
      mma_stage<kBf16>(acc2, lds.buf[buf], lds.buf[buf], a_row0w, b_row0w, lane);
      if (s + 1 == ks2) {
        epi(tile, acc1, acc2);
        zero_acc(acc1);
        zero_acc(acc2);
      }
      if (more) store(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    if (ks2 == 0) {
      epi(tile, acc1, acc2);
      zero_acc(acc1);
    }
  }
}

}  // namespace kd
