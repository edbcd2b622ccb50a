// kd_kernels.hip - forward (divergence) and backward (dL/dh_s) kernels.
//
// Forward: one sweep over every (vocabulary tile, token tile): rebuild z_s and
// z_t for the tile with bf16 MFMA (fp32 accumulation), then fold the tile into
// per-token online statistics (running max and sum of exp for both models and
// a KL numerator), exactly the two actions of the Nitrobrew notes ("Nitrobrew
// 的两个动作": rebuild the logits of a vocabulary block, update the online
// softmax / log-sum-exp accumulators and the KL terms, discard the block).
// The vocabulary is split across workgroups; each writes one partial record
// per token and a merge kernel combines them (a log-sum-exp merge).
//
// The beta family follows the beta table of ars-opd-rebuild "03 · 层 2：
// White-box OPD 基线" (section 2.3): beta = 0 forward KL, beta = 1 reverse KL,
// both done in one sweep through the identity
//   KL(q||p) = sum_v q_v (s_v - t_v) - LSE(s) + LSE(t)     (and its mirror),
// and 0 < beta < 1, whose log-mixture needs the final log-sum-exps, in two
// sweeps (LSEs, then the mixture sums).
//
// Backward (Nitrobrew notes, "仓库实现": recompute per vocabulary block
// instead of storing logits): per vocabulary chunk, recompute the tile logits,
// form g = dloss/ds scaled by grad/tau and store it as bf16 [N, chunk]; then
// dh_s += G . W_s[chunk] with W_s[chunk] transposed once per chunk, and, when
// asked, dW_s[chunk] = G^T . h_s from a transposed copy of the same tile.
//
// Also here: the backward of the top-k style losses (a per-token coefficient
// kernel, a student-only recompute sweep and a fix-up of the listed entries
// before the same dh GEMM) and the row gather / scatter of token masking.
//
// All exponentials and logarithms are base 2 (v_exp_f32 / v_log_f32) on
// logits prescaled by log2(e)/tau; the per-token results are converted back
// to natural logarithms in the merge.
#include <math.h>

#include "kd_internal.h"
#include "kd_sweep.hpp"

namespace kd {

namespace {

constexpr float kNegInf = -INFINITY;

// The NBUF (2 to 4) LDS stage buffers of a sweep ring, as separate objects.
#define KD_RING_LDS_N(TM, TN, RB, NBUF)                                                             \
  __shared__ __attribute__((aligned(16))) char ring0_[Ring<TM, TN, RB>::kBytes];                    \
  __shared__ __attribute__((aligned(16))) char ring1_[Ring<TM, TN, RB>::kBytes];                    \
  __shared__ __attribute__((aligned(16))) char ring2_[(NBUF) > 2 ? Ring<TM, TN, RB>::kBytes : 16]; \
  __shared__ __attribute__((aligned(16))) char ring3_[(NBUF) > 3 ? Ring<TM, TN, RB>::kBytes : 16]; \
  const RingLds<NBUF> lds = ring_of<NBUF>(ring0_, ring1_, ring2_, ring3_)

template <int NBUF>
__device__ __forceinline__ RingLds<NBUF> ring_of(char* r0, char* r1, char* r2, char* r3) {
  char* all[4] = {r0, r1, r2, r3};
  RingLds<NBUF> r;
#pragma unroll
  for (int i = 0; i < NBUF; ++i) r.b[i] = all[i];
  return r;
}

struct LogitArgs {
  PairDesc ps, pt;   // (W_s, h_s) and (W_t, h_t)
  int64_t N, V;
  float c2;          // log2(e) / tau
  float inv_tau;
  float beta;
  int n_tok_tiles, n_splits, tiles_per_split, n_vtiles;
  int vt_offset;     // first vocabulary tile of the grid (backward chunks)
  float* part;       // forward partial statistics
  const float *lse_s, *lse_t, *aux, *grad;
  char* G;           // backward gradient chunk [N][chunk] (null: not written)
  int64_t ldg;       // G row pitch in bytes
  int64_t g_col0;    // vocabulary index of G's column 0
  char* GT;          // the same chunk transposed, [chunk][Np] (null: not written)
  int64_t ldgt;      // GT row pitch in bytes
  int64_t Np;        // tokens rounded up to the token tile (GT columns written)
  // Dominant-entry correction of dL/dh_s (null: off): per (split, token) the
  // sum of the G entries as stored, [n_splits][N]; per token the vocabulary
  // index of the entry whose student probability exceeds kBigQ (-1: none).
  float* esum;
  int32_t* big;
};

// A student probability above this belongs to at most one entry per token:
// the dominant entry, whose gradient the backward takes from the zero-sum
// identity instead of its own (cancelling) formula. kBigLq2Lo is the wider
// log2 threshold of the cheap per-tile check that guards the exact test.
constexpr float kBigLq2 = -0.73696559f;    // log2(0.6)
constexpr float kBigLq2Lo = -0.86249648f;  // log2(0.55)

__device__ __forceinline__ void merge_online(float& m, float& l, float m2, float l2) {
  const float mm = fmaxf(m, m2);
  const float f1 = (m == kNegInf) ? 0.f : fast_exp2(m - mm);
  const float f2 = (m2 == kNegInf) ? 0.f : fast_exp2(m2 - mm);
  l = l * f1 + l2 * f2;
  m = mm;
}

// Merge (ms, ls, mt, lt, acc) with a second record; `acc` is scaled like the
// student sums for reverse KL and like the teacher sums for forward KL.
template <int MODE>
__device__ __forceinline__ void merge_record(float& ms, float& ls, float& mt, float& lt, float& ac, float ms2,
                                             float ls2, float mt2, float lt2, float ac2) {
  const float mms = fmaxf(ms, ms2), mmt = fmaxf(mt, mt2);
  const float fs1 = (ms == kNegInf) ? 0.f : fast_exp2(ms - mms);
  const float fs2 = (ms2 == kNegInf) ? 0.f : fast_exp2(ms2 - mms);
  const float ft1 = (mt == kNegInf) ? 0.f : fast_exp2(mt - mmt);
  const float ft2 = (mt2 == kNegInf) ? 0.f : fast_exp2(mt2 - mmt);
  ls = ls * fs1 + ls2 * fs2;
  lt = lt * ft1 + lt2 * ft2;
  if (MODE == kModeRKL) ac = ac * fs1 + ac2 * fs2;
  if (MODE == kModeFKL) ac = ac * ft1 + ac2 * ft2;
  ms = mms;
  mt = mmt;
}

// ---------------------------------------------------------------------------
// Forward sweep. MODE: kModeFKL / kModeRKL (loss in one sweep), kModeLSE (only
// the log-sum-exps, first JSD sweep), kModeJSD (mixture sums given the LSEs).
// ---------------------------------------------------------------------------
template <bool kBf16, int MODE, bool kSmall, int kR2>
__global__ __launch_bounds__(kLogitThreads, 1) void fwd_kernel(LogitArgs a) {
  constexpr int TM = kTileV, TN = kSmall ? kSmallT : kTileT, WM = kLogitWM, WN = kLogitWN;
  constexpr int NBUF = kSmall ? kSmallBuf : kLogitBuf;
  constexpr int MB = TM / (32 * WM), NB = TN / (32 * WN);
  KD_RING_LDS_N(TM, TN, kLogitRB, NBUF);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  if (L >= a.n_tok_tiles * a.n_splits) return;  // grid padding
  int tt, sp;
  block_coords<kTokGroup>(L, a.n_tok_tiles, a.n_splits, tt, sp);
  const int vt0 = sp * a.tiles_per_split;
  const int vt1 = min(vt0 + a.tiles_per_split, a.n_vtiles);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave % WM, wn = wave / WM;
  const int64_t tok0 = (int64_t)tt * TN + wn * (TN / WN);
  const float c2 = a.c2;

  float ms[NB], ls[NB], mt[NB], lt[NB], ac[NB];
  float Ls2[NB], Lt2[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    ms[nb] = kNegInf;
    mt[nb] = kNegInf;
    ls[nb] = lt[nb] = ac[nb] = 0.f;
    Ls2[nb] = Lt2[nb] = 0.f;
    if (MODE == kModeJSD) {
      const int64_t n = tok0 + nb * 32 + (lane & 31);
      if (n < a.N) {
        Ls2[nb] = a.lse_s[n] * kLog2e;
        Lt2[nb] = a.lse_t[n] * kLog2e;
      }
    }
  }
  const float beta = a.beta, omb = 1.f - a.beta;

  // Epilogue of one vocabulary tile. Every tile but the vocabulary's last is
  // whole, and its copy of the epilogue (kFull) carries no row test: a test
  // per element (index, 64-bit compare, select) cost more instructions than
  // the arithmetic it guards.
  auto epi_tile = [&](auto kFull, int64_t vrow0, auto& zs, auto& zt) __attribute__((always_inline)) {
    constexpr bool full = decltype(kFull)::value;
    // rows of this wave's slice below V, relative to its first row (kFull: all)
    const int vlim = full ? TM : (int)max<int64_t>(0, min<int64_t>(a.V - vrow0, TM));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (MODE == kModeJSD) {
        float sl = 0.f, sx = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = full || (mb * 32 + acc_row(r, lane) < vlim);
            const float lq2 = fmaf(zs[mb][nb][r], c2, -Ls2[nb]);
            const float lp2 = fmaf(zt[mb][nb][r], c2, -Lt2[nb]);
            const float q = fast_exp2(lq2), p = fast_exp2(lp2);
            const float m = beta * p + omb * q;
            if (ok && m > 1e-37f) {
              const float lm2 = fast_log2(m);
              const float tqm = q * (lq2 - lm2);
              sl += beta * (p * (lp2 - lm2)) + omb * tqm;
              sx += tqm;
            }
          }
        ls[nb] += sl;
        lt[nb] += sx;
      } else {
        float mxs = kNegInf, mxt = kNegInf;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (full || (mb * 32 + acc_row(r, lane) < vlim)) {
              mxs = fmaxf(mxs, zs[mb][nb][r]);
              mxt = fmaxf(mxt, zt[mb][nb][r]);
            }
          }
        const float ms_new = fmaxf(ms[nb], mxs * c2);
        const float mt_new = fmaxf(mt[nb], mxt * c2);
        if (ms_new == kNegInf) continue;  // no valid row seen yet by this lane
        const float fs = fast_exp2(ms[nb] - ms_new);
        const float ft = fast_exp2(mt[nb] - mt_new);
        float sl = 0.f, tl = 0.f, sa = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = zs[mb][nb][r], y = zt[mb][nb][r];
            float es = fast_exp2(fmaf(x, c2, -ms_new));
            float et = fast_exp2(fmaf(y, c2, -mt_new));
            if (!full && !(mb * 32 + acc_row(r, lane) < vlim)) es = et = 0.f;
            sl += es;
            tl += et;
            if (MODE == kModeRKL) sa = fmaf(es, x - y, sa);
            if (MODE == kModeFKL) sa = fmaf(et, y - x, sa);
          }
        ls[nb] = fmaf(ls[nb], fs, sl);
        lt[nb] = fmaf(lt[nb], ft, tl);
        if (MODE == kModeRKL) ac[nb] = fmaf(ac[nb], fs, sa);
        if (MODE == kModeFKL) ac[nb] = fmaf(ac[nb], ft, sa);
        ms[nb] = ms_new;
        mt[nb] = mt_new;
      }
    }
  };
  auto epi = [&](int vt, auto& zs, auto& zt, char*) {
    const int64_t vrow0 = (int64_t)vt * TM + wm * (TM / WM);
    if ((int64_t)(vt + 1) * TM <= a.V)
      epi_tile(std::true_type{}, vrow0, zs, zt);
    else
      epi_tile(std::false_type{}, vrow0, zs, zt);
  };
  sweep<kBf16, TM, TN, WM, WN, NBUF, kLogitRB, true, kR2>(a.ps, a.pt, (int64_t)tt * TN, vt0, vt1, lds, epi);

  // Lanes l and l ^ 32 hold the same tokens (other vocabulary rows).
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (MODE == kModeJSD) {
      ls[nb] += __shfl_xor(ls[nb], 32);
      lt[nb] += __shfl_xor(lt[nb], 32);
    } else {
      const float oms = __shfl_xor(ms[nb], 32), ols = __shfl_xor(ls[nb], 32);
      const float omt = __shfl_xor(mt[nb], 32), olt = __shfl_xor(lt[nb], 32);
      const float oac = __shfl_xor(ac[nb], 32);
      merge_record<MODE>(ms[nb], ls[nb], mt[nb], lt[nb], ac[nb], oms, ols, omt, olt, oac);
    }
  }
  // The WM waves with the same wn hold the vocabulary slices of the same
  // tokens: waves wm > 0 publish their records, wave wm = 0 merges them.
  // The ring is drained: its first buffer holds the records.
  constexpr int kF = MODE == kModeJSD ? kJsdFields : kFwdFields;
  static_assert((WM - 1) * kF * TN * sizeof(float) <= Ring<TM, TN, kLogitRB>::kBytes, "records fit one stage");
  float* red = reinterpret_cast<float*>(lds.b[0]);
  if (wm > 0 && lane < 32) {
    float* r = red + (wm - 1) * kF * TN;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wn * (TN / WN) + nb * 32 + lane;
      if constexpr (MODE == kModeJSD) {
        r[0 * TN + col] = ls[nb];
        r[1 * TN + col] = lt[nb];
      } else {
        r[0 * TN + col] = ms[nb];
        r[1 * TN + col] = ls[nb];
        r[2 * TN + col] = mt[nb];
        r[3 * TN + col] = lt[nb];
        r[4 * TN + col] = ac[nb];
      }
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wn * (TN / WN) + nb * 32 + lane;
      const int64_t n = (int64_t)tt * TN + col;
#pragma unroll
      for (int w = 0; w < WM - 1; ++w) {
        const float* r = red + w * kF * TN;
        if constexpr (MODE == kModeJSD) {
          ls[nb] += r[0 * TN + col];
          lt[nb] += r[1 * TN + col];
        } else {
          merge_record<MODE>(ms[nb], ls[nb], mt[nb], lt[nb], ac[nb], r[0 * TN + col], r[1 * TN + col],
                             r[2 * TN + col], r[3 * TN + col], r[4 * TN + col]);
        }
      }
      if (n < a.N) {
        if constexpr (MODE == kModeJSD) {
          a.part[(0 * (int64_t)a.n_splits + sp) * a.N + n] = ls[nb];
          a.part[(1 * (int64_t)a.n_splits + sp) * a.N + n] = lt[nb];
        } else {
          a.part[(0 * (int64_t)a.n_splits + sp) * a.N + n] = ms[nb];
          a.part[(1 * (int64_t)a.n_splits + sp) * a.N + n] = ls[nb];
          a.part[(2 * (int64_t)a.n_splits + sp) * a.N + n] = mt[nb];
          a.part[(3 * (int64_t)a.n_splits + sp) * a.N + n] = lt[nb];
          a.part[(4 * (int64_t)a.n_splits + sp) * a.N + n] = ac[nb];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-split merge: one thread per token, slices in a fixed order.
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part, int n_splits, int64_t N,
                                                   float inv_tau, float* loss, float* lse_s, float* lse_t,
                                                   float* aux) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const int64_t S = n_splits;
  if constexpr (MODE == kModeJSD) {
    float sl = 0.f, sx = 0.f;
#pragma unroll 8
    for (int s = 0; s < n_splits; ++s) {
      sl += part[(0 * S + s) * N + n];
      sx += part[(1 * S + s) * N + n];
    }
    loss[n] = sl * kLn2;
    if (aux) aux[n] = sx * kLn2;
  } else {
    float ms = kNegInf, ls = 0.f, mt = kNegInf, lt = 0.f, ac = 0.f;
    // unrolled so that the loads of several slices are in flight at once (the
    // merges themselves form a chain)
#pragma unroll 8
    for (int s = 0; s < n_splits; ++s)
      merge_record<MODE>(ms, ls, mt, lt, ac, part[(0 * S + s) * N + n], part[(1 * S + s) * N + n],
                         part[(2 * S + s) * N + n], part[(3 * S + s) * N + n], part[(4 * S + s) * N + n]);
    const float Ls = (ms + log2f(ls)) * kLn2;  // natural-log LSE of the tempered logits
    const float Lt = (mt + log2f(lt)) * kLn2;
    lse_s[n] = Ls;
    lse_t[n] = Lt;
    if (MODE == kModeRKL || MODE == kModeFKL) {
      // RKL: sum_v q (s - t) - Ls + Lt,   FKL: sum_v p (t - s) - Lt + Ls
      const float kl = (MODE == kModeRKL) ? (ac / ls) * inv_tau - Ls + Lt : (ac / lt) * inv_tau - Lt + Ls;
      loss[n] = kl;
      if (aux) aux[n] = kl;
    }
  }
}

// The same merge with one wave per token (four per workgroup), for few tokens,
// where one thread per token leaves the GPU idle: lane l merges slices l,
// l + 64, ..., then a butterfly over the lanes merges the 64 partial records
// in a fixed order.
template <int MODE>
__global__ __launch_bounds__(256) void merge_wave_kernel(const float* __restrict__ part, int n_splits, int64_t N,
                                                        float inv_tau, float* loss, float* lse_s, float* lse_t,
                                                        float* aux) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;  // whole waves only
  const int64_t S = n_splits;
  if constexpr (MODE == kModeJSD) {
    float sl = 0.f, sx = 0.f;
    for (int s = lane; s < n_splits; s += 64) {
      sl += part[(0 * S + s) * N + n];
      sx += part[(1 * S + s) * N + n];
    }
    sl = wave_sum(sl);
    sx = wave_sum(sx);
    if (lane == 0) {
      loss[n] = sl * kLn2;
      if (aux) aux[n] = sx * kLn2;
    }
  } else {
    float ms = kNegInf, ls = 0.f, mt = kNegInf, lt = 0.f, ac = 0.f;
    for (int s = lane; s < n_splits; s += 64)
      merge_record<MODE>(ms, ls, mt, lt, ac, part[(0 * S + s) * N + n], part[(1 * S + s) * N + n],
                         part[(2 * S + s) * N + n], part[(3 * S + s) * N + n], part[(4 * S + s) * N + n]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
      merge_record<MODE>(ms, ls, mt, lt, ac, __shfl_xor(ms, o), __shfl_xor(ls, o), __shfl_xor(mt, o),
                         __shfl_xor(lt, o), __shfl_xor(ac, o));
    if (lane == 0) {
      const float Ls = (ms + log2f(ls)) * kLn2;
      const float Lt = (mt + log2f(lt)) * kLn2;
      lse_s[n] = Ls;
      lse_t[n] = Lt;
      if (MODE == kModeRKL || MODE == kModeFKL) {
        const float kl = (MODE == kModeRKL) ? (ac / ls) * inv_tau - Ls + Lt : (ac / lt) * inv_tau - Lt + Ls;
        loss[n] = kl;
        if (aux) aux[n] = kl;
      }
    }
  }
}

// Launch the merge of the forward's partial records: one thread per token,
// or one wave per token up to kMergeWaveMaxN tokens.
constexpr int64_t kMergeWaveMaxN = 2048;
template <int MODE>
hipError_t launch_merge(const float* part, int n_splits, int64_t N, float inv_tau, float* loss, float* lse_s,
                        float* lse_t, float* aux, hipStream_t st) {
  if (N <= kMergeWaveMaxN)
    hipLaunchKernelGGL((merge_wave_kernel<MODE>), dim3((unsigned)((N + 3) / 4)), dim3(256), 0, st, part, n_splits, N,
                       inv_tau, loss, lse_s, lse_t, aux);
  else
    hipLaunchKernelGGL((merge_kernel<MODE>), dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, part, n_splits, N,
                       inv_tau, loss, lse_s, lse_t, aux);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward, step 1: G[n, v - c0] = grad[n] / tau * dloss_n / ds_v for one chunk.
// ---------------------------------------------------------------------------

// Store 16 consecutive bf16 gradient entries of one token from a 32 x 32 MFMA
// block: rows 16 pr .. 16 pr + 15, where lane l holds rows 0-3 of each 8-row
// group and lane l + 32 rows 4-7 (w2[h]: group 2 pr + h, packed in pairs).
// One permlane32 swap per dword leaves lane l with rows 0-7 and lane l + 32
// with rows 8-15, each written with one 16-byte store. Every lane takes part
// in the swaps; the store is skipped for tokens past N (lanes l and l + 32
// hold the same token).
__device__ __forceinline__ void store_g16(char* G, int64_t ldg, int64_t n, int64_t N, int64_t col0,
                                          const u32x2 (&w2)[2], int lane) {
  const auto sx = __builtin_amdgcn_permlane32_swap(w2[0].x, w2[1].x, false, false);
  const auto sy = __builtin_amdgcn_permlane32_swap(w2[0].y, w2[1].y, false, false);
  if (G && n < N) {
    u32x4 w;
    w.x = sx[0];
    w.y = sy[0];
    w.z = sx[1];
    w.w = sy[1];
    *reinterpret_cast<u32x4*>(G + n * ldg + (col0 + 8 * (lane >> 5)) * 2) = w;
  }
}

// kGT: also write the chunk transposed (a.GT, for dW_s); a compile-time
// switch, so the loss-gradient-only kernel carries none of that code.
template <bool kBf16, int MODE, bool kSmall, int kR2, bool kGT>
__global__ __launch_bounds__(kLogitThreads, 1) void bwdg_kernel(LogitArgs a) {
  constexpr int TM = kTileV, TN = kSmall ? kSmallT : kTileT, WM = kLogitWM, WN = kLogitWN;
  constexpr int NBUF = kSmall ? kSmallBuf : kLogitBuf;
  constexpr int MB = TM / (32 * WM), NB = TN / (32 * WN);
  KD_RING_LDS_N(TM, TN, kLogitRB, NBUF);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  if (L >= a.n_tok_tiles * a.n_splits) return;  // grid padding
  int tt, sp;
  block_coords<kTokGroup>(L, a.n_tok_tiles, a.n_splits, tt, sp);
  const int vt0 = a.vt_offset + sp * a.tiles_per_split;
  const int vt1 = min(vt0 + a.tiles_per_split, a.vt_offset + a.n_vtiles);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave % WM, wn = wave / WM;
  const int64_t tok0 = (int64_t)tt * TN + wn * (TN / WN);
  const float c2 = a.c2, inv_tau = a.inv_tau, beta = a.beta, omb = 1.f - a.beta;

  float Ls2[NB], Lt2[NB], K1[NB], gsc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int64_t n = tok0 + nb * 32 + (lane & 31);
    Ls2[nb] = Lt2[nb] = K1[nb] = gsc[nb] = 0.f;
    if (n < a.N) {
      const float ls = a.lse_s[n], lt = a.lse_t[n];
      Ls2[nb] = ls * kLog2e;
      Lt2[nb] = lt * kLog2e;
      gsc[nb] = (a.grad ? a.grad[n] : 1.f) * inv_tau;
      if (MODE == kModeRKL) K1[nb] = ls - lt + a.aux[n];  // log q - log p - KL = (s - t) - K1
      if (MODE == kModeJSD) K1[nb] = a.aux[n];            // KL(q || m)
    }
  }

  // Sum of this lane's stored G entries per token, over the block's tiles.
  float es[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) es[nb] = 0.f;
  const bool fix = a.esum != nullptr;

  // One vocabulary tile. The epilogue has no per-element row test: in the
  // vocabulary's last tile, the rows past V (read as zeros) first get both
  // logits set to -1e30, so that q = p = 0 there and every gradient formula
  // below gives exactly 0 (and none passes the dominant-entry test). A second,
  // test-free copy of the epilogue for whole tiles spilled registers.
  auto epi = [&](int vt, auto& zs, auto& zt, char*) {
    const int64_t vrow0 = (int64_t)vt * TM + wm * (TM / WM);
    if ((int64_t)(vt + 1) * TM > a.V) {
      const int vlim = (int)max<int64_t>(0, min<int64_t>(a.V - vrow0, TM));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (mb * 32 + acc_row(r, lane) >= vlim) zs[mb][nb][r] = zt[mb][nb][r] = -1e30f;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int64_t n = tok0 + nb * 32 + (lane & 31);
      float lqmax = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          __builtin_amdgcn_sched_barrier(0);  // keep the groups apart: bounds register pressure
          u32x2 w2[2];                        // row groups 2 pr and 2 pr + 1, packed bf16
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int rg = 2 * pr + h;
            float g4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = rg * 4 + e;
              const float x = zs[mb][nb][r], y = zt[mb][nb][r];
              const float lq2 = fmaf(x, c2, -Ls2[nb]);
              lqmax = fmaxf(lqmax, lq2);
              const float q = fast_exp2(lq2);
              float g;
              if constexpr (MODE == kModeRKL) {
                g = q * fmaf(x - y, inv_tau, -K1[nb]);
              } else if constexpr (MODE == kModeFKL) {
                g = q - fast_exp2(fmaf(y, c2, -Lt2[nb]));
              } else {
                const float lp2 = fmaf(y, c2, -Lt2[nb]);
                const float m = beta * fast_exp2(lp2) + omb * q;
                g = (m > 1e-37f) ? omb * q * fmaf(lq2 - fast_log2(m), kLn2, -K1[nb]) : 0.f;
              }
              g4[e] = g * gsc[nb];
            }
            if (kGT && n < a.Np) {
              // transposed copy for the weight gradient: token-contiguous rows;
              // tokens past N carry g = 0, so the padding columns are zeros
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int64_t row = vrow0 + mb * 32 + 8 * rg + 4 * (lane >> 5) + e - a.g_col0;
                char* dst = a.GT + row * a.ldgt;
                if constexpr (kBf16)
                  *reinterpret_cast<uint16_t*>(dst + n * 2) = (uint16_t)f32_to_bf16_bits(g4[e]);
                else
                  *reinterpret_cast<float*>(dst + n * 4) = g4[e];
              }
            }
            if constexpr (kBf16) {
              w2[h].x = pack_bf16x2(g4[0], g4[1]);
              w2[h].y = pack_bf16x2(g4[2], g4[3]);
              // the stored values, widened back to fp32
              es[nb] += (__builtin_bit_cast(float, w2[h].x << 16) + __builtin_bit_cast(float, w2[h].x & 0xFFFF0000u)) +
                        (__builtin_bit_cast(float, w2[h].y << 16) + __builtin_bit_cast(float, w2[h].y & 0xFFFF0000u));
            } else {
              es[nb] += (g4[0] + g4[1]) + (g4[2] + g4[3]);
              if (a.G && n < a.N) {
                const int64_t col = vrow0 + mb * 32 + 8 * rg + 4 * (lane >> 5) - a.g_col0;
                *reinterpret_cast<floatx4*>(a.G + n * a.ldg + col * 4) = floatx4{g4[0], g4[1], g4[2], g4[3]};
              }
            }
          }
          if constexpr (kBf16) store_g16(a.G, a.ldg, n, a.N, vrow0 + mb * 32 + 16 * pr - a.g_col0, w2, lane);
        }
      // The dominant entry (q > 0.6, at most one per token) records its index;
      // the wide threshold keeps the exact test off tiles that cannot hold it.
      if (fix && __ballot(lqmax > kBigLq2Lo) != 0ull) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (n < a.N && fmaf(zs[mb][nb][r], c2, -Ls2[nb]) > kBigLq2)
              a.big[n] = (int32_t)(vrow0 + mb * 32 + acc_row(r, lane));
          }
      }
    }
  };

  sweep<kBf16, TM, TN, WM, WN, NBUF, kLogitRB, true, kR2>(a.ps, a.pt, (int64_t)tt * TN, vt0, vt1, lds, epi);

  if (!fix) return;
  // Per token the block's sum of stored entries: lanes l and l ^ 32 hold the
  // same token; waves wm > 0 publish theirs in the drained ring, wave wm = 0
  // adds them in a fixed order and writes the block's record.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) es[nb] += __shfl_xor(es[nb], 32);
  float* red = reinterpret_cast<float*>(lds.b[0]);
  if (wm > 0 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[(wm - 1) * TN + wn * (TN / WN) + nb * 32 + lane] = es[nb];
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wn * (TN / WN) + nb * 32 + lane;
      float t = es[nb];
#pragma unroll
      for (int w = 0; w < WM - 1; ++w) t += red[w * TN + col];
      const int64_t n = (int64_t)tt * TN + col;
      if (n < a.N) a.esum[(int64_t)sp * a.N + n] = t;
    }
  }
}

// Dominant-entry correction, before the first chunk: no token has one yet.
__global__ __launch_bounds__(256) void big_init_kernel(int32_t* big, int64_t N) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < N; i += (int64_t)gridDim.x * 256) big[i] = -1;
}

// After each chunk: etot[n] (=|+=) the chunk's per-split sums. A block takes
// 64 tokens; wave w sums the splits w, w + 4, w + 8, ... of its lane's token
// (eight loads in flight), then the four partial sums are added in wave
// order: a fixed order, so the result is the same on every run.
constexpr int kEsumTok = 64;
__global__ __launch_bounds__(256) void esum_reduce_kernel(const float* __restrict__ part, int n_split, int64_t N,
                                                          float* __restrict__ etot, int first) {
  __shared__ float red[4][kEsumTok];
  const int tl = threadIdx.x % kEsumTok, w = threadIdx.x / kEsumTok;
  const int64_t n = (int64_t)blockIdx.x * kEsumTok + tl;
  float t = 0.f;
  if (n < N) {
#pragma unroll 8
    for (int s = w; s < n_split; s += 4) t += part[(int64_t)s * N + n];
  }
  red[w][tl] = t;
  __syncthreads();
  if (w == 0 && n < N) {
    const float u = (red[0][tl] + red[1][tl]) + (red[2][tl] + red[3][tl]);
    etot[n] = first ? u : etot[n] + u;
  }
}

// After the last chunk. The gradient entries of a token sum to zero for every
// beta (the beta table of ars-opd-rebuild "03 · 层 2：White-box OPD 基线",
// section 2.3, differentiated), so the dominant entry's exact value is minus
// the sum of all others. Its own formula cancels terms of the size of the
// log-sum-exps, which fp32 cannot resolve when the student is saturated; so
// the stored value g_a is replaced by -(sum of the others as stored): with E
// the sum of every stored entry, dh_s[n] -= E * W_s[a].
template <typename T>
__global__ __launch_bounds__(256) void big_fix_kernel(const int32_t* __restrict__ big, const float* __restrict__ etot,
                                                      const T* __restrict__ W_s, int32_t d_s, int64_t N,
                                                      float* __restrict__ dh) {
  for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
    const int64_t v = big[n];
    if (v < 0) continue;
    const float e = etot[n];
    const T* w = W_s + v * d_s;
    float* o = dh + n * d_s;
    for (int i = threadIdx.x; i < d_s; i += 256) {
      float wi;
      if constexpr (sizeof(T) == 2)
        wi = __builtin_bit_cast(float, (uint32_t)w[i] << 16);
      else
        wi = w[i];
      o[i] = fmaf(-e, wi, o[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, step 2: WsT[d, j] = W_s[c0 + j, d] for j < kcols (zero past V).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ W, T* __restrict__ WT, int64_t V,
                                                        int32_t d, int64_t c0, int64_t pitch) {
  __shared__ T tile[64][65];
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int64_t d0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int jr = i * 4 + ty;
    const int64_t v = c0 + j0 + jr, dd = d0 + tx;
    tile[jr][tx] = (v < V && dd < d) ? W[v * d + dd] : T(0);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int dr = i * 4 + ty;
    const int64_t dd = d0 + dr;
    if (dd < d) WT[dd * pitch + j0 + tx] = tile[tx][dr];
  }
}

// The bf16 transpose with 16-byte global accesses (d is a multiple of 8, so
// every 8-element run of a row is 16-byte aligned): per 64 x 64 tile each
// thread loads two 8-element runs of W rows, the tile goes through LDS with
// a 65-element row pitch (the column reads of a wave then hit 32 distinct
// banks), and each thread writes two 8-element runs of WT rows.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ W, uint16_t* __restrict__ WT,
                                                             int64_t V, int32_t d, int64_t c0, int64_t pitch) {
  __shared__ uint16_t tile[64][65];
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int64_t d0 = (int64_t)blockIdx.y * 64;
  const int c = threadIdx.x & 7, r = threadIdx.x >> 3;  // 8-element run, row (0..31)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int jr = r + 32 * h;
    const int64_t v = c0 + j0 + jr, dd = d0 + 8 * c;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (v < V && dd < d) w = *reinterpret_cast<const u32x4*>(W + v * d + dd);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[jr][8 * c + 2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      tile[jr][8 * c + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int dr = r + 32 * h;
    const int64_t dd = d0 + dr;
    if (dd < d) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)tile[8 * c + 2 * e][dr] | ((uint32_t)tile[8 * c + 2 * e + 1][dr] << 16);
      *reinterpret_cast<u32x4*>(WT + dd * pitch + j0 + 8 * c) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, step 3: dh[n, d] (+)= sum_j G[n, j] WsT[d, j] over one chunk, and
// dW_s[c0 + j, d] = sum_n GT[j, n] hsT[d, n].
// ---------------------------------------------------------------------------
// out[r, d] (+)= sum_k A[r, k] B[d, k]: dh (A = G, token rows; B = the W_s
// chunk transposed) or dW_s (A = G transposed, vocabulary rows of the chunk;
// B = h_s transposed), both operands contracted over contiguous K.
struct DhArgs {
  PairDesc p;
  int64_t N;         // valid output rows
  int32_t d_s;       // output columns (and row pitch)
  int n_tok_tiles, n_d_tiles;
  float* dh;         // output
  int first;         // 1: overwrite, 0: accumulate
  // split contraction (few output tiles): split ks of n_ksplit covers
  // bytes [ks * kspan, (ks + 1) * kspan) of K and writes its own partial
  // tile to part + ks * N * d_s; dh_reduce_kernel then sums the partials
  int n_ksplit;      // 1: no split
  int32_t kspan;
  float* part;
};

template <bool kBf16, bool kSmall>
__global__ __launch_bounds__(kDhThreads, 1) void dh_kernel(DhArgs a) {
  // kSmall (at most 64 output rows): a 64-row tile on 2 x 4 waves with a ring
  // of four 40 KiB stages, three stages of the B operand in flight per CU
  // instead of one.
  constexpr int TM = kSmall ? kSmallT : kTileDhT, TN = kTileDhD;
  constexpr int WM = kSmall ? 2 : kDhWM, WN = kSmall ? 4 : kDhWN;
  constexpr int NBUF = kSmall ? kSmallBuf : kDhBuf;
  constexpr int MB = TM / (32 * WM), NB = TN / (32 * WN);
  KD_RING_LDS_N(TM, TN, kDhRB, NBUF);
  const int L0 = xcd_remap(blockIdx.x, gridDim.x);
  if (L0 >= a.n_tok_tiles * a.n_d_tiles * a.n_ksplit) return;  // grid padding
  const int per_split = a.n_tok_tiles * a.n_d_tiles;
  const int ks = L0 / per_split;  // 0 unless the contraction is split
  int tt, dt;
  block_coords<kTokGroup>(L0 - ks * per_split, a.n_tok_tiles, a.n_d_tiles, tt, dt);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave % WM, wn = wave / WM;
  PairDesc pd = a.p;
  float* out = a.dh;
  int first = a.first;
  if (a.n_ksplit > 1) {
    const int32_t k0 = ks * a.kspan;  // < kbytes: the host sizes the splits
    pd.A += k0;
    pd.B += k0;
    pd.kbytes = min(a.kspan, a.p.kbytes - k0);
    out = a.part + (int64_t)ks * a.N * a.d_s;
    first = 1;
  }
  // Read-modify-write of dh, one 32-row slice at a time: all loads of the
  // slice are issued before its stores, so they overlap instead of forming a
  // chain of dependent round trips.
  auto epi = [&](int tile, auto& acc, auto&, char*) {
    const int64_t d0 = (int64_t)dt * TN + wn * (TN / WN) + (lane & 31);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t n0 = (int64_t)tile * TM + wm * (TM / WM) + mb * 32;
      float old[NB][16];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) old[nb][r] = 0.f;
      if (!first) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t n = n0 + acc_row(r, lane), d = d0 + nb * 32;
            if (n < a.N && d < a.d_s) old[nb][r] = out[n * a.d_s + d];
          }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t n = n0 + acc_row(r, lane), d = d0 + nb * 32;
          if (n < a.N && d < a.d_s) out[n * a.d_s + d] = old[nb][r] + acc[mb][nb][r];
        }
    }
  };
  sweep<kBf16, TM, TN, WM, WN, NBUF, kDhRB, false>(pd, pd, (int64_t)dt * TN, tt, tt + 1, lds, epi);
}

// dh (=|+=) the sum of the split contraction's partial tiles, in split order.
__global__ __launch_bounds__(256) void dh_reduce_kernel(const float* __restrict__ part, int n_split, int64_t count,
                                                        float* __restrict__ dh, int first) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    float v = 0.f;
    for (int s = 0; s < n_split; ++s) v += part[s * count + i];
    dh[i] = first ? v : dh[i] + v;
  }
}

// ---------------------------------------------------------------------------
// Backward of the top-k style losses (the three top-k terms, [Top-K KD] 一.2;
// the tail-bucket divergence, [White-box OPD] 2.4). Gradient reading: the
// selection and the teacher fixed, the bf16 rounding of the student logits
// passed straight through. Either gradient w.r.t. the student logits is
//   dL/dz_v = A q_v + C r_v     for every v outside a short per-token list,
// (q the tempered student softmax, r the untempered one, A and C per token)
// and an arbitrary value on the list (the selected entries and the label).
// A coefficient kernel (one wave per token) computes A, C and the list's
// exact values; per vocabulary chunk a student-only recompute sweep writes
// G = A q + C r in bf16, the list's entries in the chunk overwrite their G
// elements, and the dh GEMM contracts G with the chunk of W_s. Writing the
// listed values whole (rather than adding a correction to A q) keeps the bf16
// rounding of G relative to each entry's own value.
// ---------------------------------------------------------------------------
struct DenseArgs {
  PairDesc ps;  // (W_s, h_s)
  int64_t N, V;
  float c2;     // log2(e) / tau
  const float *lse_s, *lse_s1;  // lse_s1 only when dense_c is set
  const float *dense_a, *dense_c;
  int n_tok_tiles, n_splits, tiles_per_split, n_vtiles, vt_offset;
  char* G;
  int64_t ldg, g_col0;
};

// One operand pair and one accumulator, so the block takes the dh GEMM's
// 256 x 256 tile (256 vocabulary entries x 256 tokens, 64 x 128 per wave) and
// its ring of two 64 KiB stages: half the token-operand bytes per flop of the
// two-accumulator logit tile. kR: the untempered softmax r differs from q
// (a CE term at tau != 1); otherwise C is 0 or r equals q bit for bit (at
// tau = 1 the forward returns the same LSE for both), and one exponential
// per entry serves.
template <bool kR>
__global__ __launch_bounds__(kDenseThreads, 1) void dense_g_kernel(DenseArgs a) {
  constexpr int TM = kTileV, TN = kDenseT, WM = kDhWM, WN = kDhWN;
  constexpr int MB = TM / (32 * WM), NB = TN / (32 * WN);
  KD_RING_LDS_N(TM, TN, kDhRB, kDhBuf);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  if (L >= a.n_tok_tiles * a.n_splits) return;  // grid padding
  int tt, sp;
  block_coords<kTokGroup>(L, a.n_tok_tiles, a.n_splits, tt, sp);
  const int vt0 = a.vt_offset + sp * a.tiles_per_split;
  const int vt1 = min(vt0 + a.tiles_per_split, a.vt_offset + a.n_vtiles);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave % WM, wn = wave / WM;
  const int64_t tok0 = (int64_t)tt * TN + wn * (TN / WN);
  float Ls2[NB], L12[NB], A[NB], C[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int64_t n = tok0 + nb * 32 + (lane & 31);
    Ls2[nb] = L12[nb] = A[nb] = C[nb] = 0.f;
    if (n < a.N) {
      Ls2[nb] = a.lse_s[n] * kLog2e;
      A[nb] = a.dense_a[n];
      if (a.dense_c) {
        L12[nb] = a.lse_s1[n] * kLog2e;
        C[nb] = a.dense_c[n];
      }
    }
  }
  // No per-element row test: in the vocabulary's last tile the rows past V
  // get the logit -1e30 first, so that q = r = 0 and G = 0 there.
  auto epi = [&](int vt, auto& zs, auto&, char*) {
    const int64_t vrow0 = (int64_t)vt * TM + wm * (TM / WM);
    if ((int64_t)(vt + 1) * TM > a.V) {
      const int vlim = (int)max<int64_t>(0, min<int64_t>(a.V - vrow0, TM));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (mb * 32 + acc_row(r, lane) >= vlim) zs[mb][nb][r] = -1e30f;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int64_t n = tok0 + nb * 32 + (lane & 31);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          u32x2 w2[2];  // row groups 2 pr and 2 pr + 1, packed bf16
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float g4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = (2 * pr + h) * 4 + e;
              const float zb = __builtin_bit_cast(float, f32_to_bf16_bits(zs[mb][nb][r]) << 16);
              const float q = fast_exp2(fmaf(zb, a.c2, -Ls2[nb]));
              const float rr = kR ? fast_exp2(fmaf(zb, kLog2e, -L12[nb])) : q;
              g4[e] = fmaf(A[nb], q, C[nb] * rr);
            }
            w2[h].x = pack_bf16x2(g4[0], g4[1]);
            w2[h].y = pack_bf16x2(g4[2], g4[3]);
          }
          store_g16(a.G, a.ldg, n, a.N, vrow0 + mb * 32 + 16 * pr - a.g_col0, w2, lane);
        }
    }
  };
  sweep<true, TM, TN, WM, WN, kDhBuf, kDhRB, false>(a.ps, a.ps, (int64_t)tt * TN, vt0, vt1, lds, epi);
}

// The listed entries of one vocabulary chunk overwrite their G elements: one
// thread per (token, list slot); slots holding -1 or an index outside the
// chunk are skipped.
struct FixArgs {
  const int32_t* idx;  // [N, slots]
  const float* val;    // [N, slots], dL/dz at idx
  int64_t N;
  int slots;
  int64_t c0, ccols;
  char* G;
  int64_t ldg;
};

__global__ __launch_bounds__(256) void g_fix_kernel(FixArgs f) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= f.N * f.slots) return;
  const int64_t n = i / f.slots;
  const int64_t v = f.idx[i];
  if (v < f.c0 || v >= f.c0 + f.ccols) return;
  *reinterpret_cast<uint16_t*>(f.G + n * f.ldg + (v - f.c0) * 2) = (uint16_t)f32_to_bf16_bits(f.val[i]);
}

// Three top-k terms. With Q / P the student / teacher mass on the set K, p^
// the renormalised teacher on K, B = -P/Q + (1-P)/(1-Q) (0 when k == V):
//   A = -w_b B Q / tau,  C = w_ce (when a label and its weight are given)
//   v in K:  A q_v + C r_v + (w_b B q_v + w_c (q_v / Q - p^_v)) / tau - C 1[v = y]
//   v = y outside K:  C (r_y - 1)
// List: the k selected entries, then the label when it is outside K.
struct TopkCoefArgs {
  const uint16_t *h_s, *W_s;
  int64_t N, V;
  int32_t d_s;
  int k;
  float inv_tau;
  const int32_t* labels;
  const int32_t* idx;
  const float *val_t, *val_s, *p_mass, *q_mass, *lse_s, *lse_s1, *gb, *gc, *ge;
  float *dense_a, *dense_c;
  int32_t* list_idx;  // [N, k + 1]
  float* list_val;    // [N, k + 1]
};

__global__ __launch_bounds__(256) void topk_coef_kernel(TopkCoefArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave;
  if (n >= a.N) return;  // whole waves only
  const int K = a.k, slots = K + 1;
  const bool act = lane < K;
  const int32_t v = act ? a.idx[n * K + lane] : -1;
  const bool ok = act && v >= 0 && v < a.V;
  // renormalised teacher on the set, from its bf16 values
  const float t = ok ? a.val_t[n * K + lane] * a.inv_tau : -INFINITY;
  const float mt = wave_max(t);
  const float et = ok ? expf(t - mt) : 0.f;
  const float ph = et / wave_sum(et);
  const float P = a.p_mass[n], Q = a.q_mass[n];
  const float B = (int64_t)K >= a.V ? 0.f : -P / Q + (1.f - P) / (1.f - Q);
  const float wb = a.gb ? a.gb[n] : 0.f, wc = a.gc ? a.gc[n] : 0.f;
  const int32_t y = a.labels ? a.labels[n] : -1;
  const bool has_ce = a.ge && a.lse_s1 && y >= 0 && y < a.V;
  const float C = has_ce ? a.ge[n] : 0.f;
  const float A = -wb * B * Q * a.inv_tau;
  const float L1 = has_ce ? a.lse_s1[n] : 0.f;
  const float zs = ok ? a.val_s[n * K + lane] : 0.f;
  const float q = ok ? expf(zs * a.inv_tau - a.lse_s[n]) : 0.f;
  const float r = (ok && has_ce) ? expf(zs - L1) : 0.f;
  const float total = (wb * B * q * (1.f - Q) + wc * (q / Q - ph)) * a.inv_tau + C * (r - (v == y ? 1.f : 0.f));
  if (act) {
    a.list_idx[n * slots + lane] = ok ? v : -1;
    a.list_val[n * slots + lane] = ok ? total : 0.f;
  }
  const bool y_in_k = __ballot(ok && v == y) != 0ull;
  int32_t yi = -1;
  float yv = 0.f;
  if (has_ce && !y_in_k && C != 0.f) {  // wave-uniform
    const float zy = wave_dot_bf16(a.h_s + n * a.d_s, a.W_s, y, a.d_s, lane);
    yi = y;
    yv = C * (expf(zy - L1) - 1.f);
  }
  if (lane == 0) {
    a.list_idx[n * slots + K] = yi;
    a.list_val[n * slots + K] = yv;
    a.dense_a[n] = A;
    if (a.dense_c) a.dense_c[n] = C;
  }
}

// Tail-bucket divergence. With b(v) the bucket of entry v and a_b = dL/dq_b,
// dL/ds_v = q_v (a_b(v) - c), c = sum_b q_b a_b; beta = 0: q_b a_b = -p_b;
// beta = 1: a_b = log q_b - log p_b + 1; 0 < beta < 1:
// a_b = (1 - beta)(log q_b - log m_b). Outside the support every entry is in
// the tail bucket: A = (a_T - c) w (w = grad_loss / tau), C = 0; the support
// entries get q_v (a_v - c) w. The list is the forward's support as it is.
struct TailCoefArgs {
  int64_t N, V;
  int smax;
  float beta, inv_tau;
  const int32_t* sup_idx;
  const float *sup_t, *sup_s, *lse_s, *lse_t, *grad;
  float *dense_a, *list_val;  // [N], [N, smax]
};

__global__ __launch_bounds__(256) void tail_coef_kernel(TailCoefArgs a) {
  constexpr int kSlots = 3;  // 2 * 64 + 1 support entries at most: three per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave;
  if (n >= a.N) return;  // whole waves only
  const float Ls = a.lse_s[n], Lt = a.lse_t[n];
  float lp[kSlots], lq[kSlots];
  bool okj[kSlots];
  int cnt_l = 0;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int i = lane + 64 * j;
    const int32_t v = i < a.smax ? a.sup_idx[n * a.smax + i] : -1;
    okj[j] = v >= 0 && v < a.V;
    lp[j] = okj[j] ? a.sup_t[n * a.smax + i] * a.inv_tau - Lt : -INFINITY;
    lq[j] = okj[j] ? a.sup_s[n * a.smax + i] * a.inv_tau - Ls : -INFINITY;
    cnt_l += okj[j];
  }
  const int cnt = (int)wave_sum((float)cnt_l);
  const float mp = wave_max(fmaxf(lp[0], fmaxf(lp[1], lp[2])));
  const float mq = wave_max(fmaxf(lq[0], fmaxf(lq[1], lq[2])));
  float ep = 0.f, eq = 0.f;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    ep += okj[j] ? expf(lp[j] - mp) : 0.f;
    eq += okj[j] ? expf(lq[j] - mq) : 0.f;
  }
  const float logP = mp + logf(wave_sum(ep)), logQ = mq + logf(wave_sum(eq));
  // the forward's tail convention: masses below fp32 resolution held at 2^-24
  const bool tail = (int64_t)cnt < a.V;
  const float lpT = log1mexp_f32(fminf(logP, -5.9604645e-8f));
  const float lqT = log1mexp_f32(fminf(logQ, -5.9604645e-8f));
  const float beta = a.beta, lb = logf(beta), l1b = log1pf(-beta);
  // a_b for beta > 0 (log-domain mixture for 0 < beta < 1)
  auto a_of = [&](float p_, float q_) {
    if (beta == 1.f) return q_ - p_ + 1.f;
    const float x = lb + p_, y = l1b + q_;
    const float lm = fmaxf(x, y) + log1pf(expf(-fabsf(x - y)));
    return (1.f - beta) * (q_ - lm);
  };
  const float qT = tail ? expf(lqT) : 0.f;
  const float aT = !tail ? 0.f : beta == 0.f ? -expf(lpT - lqT) : a_of(lpT, lqT);
  float qa[kSlots], q[kSlots], csum = 0.f;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    q[j] = okj[j] ? expf(lq[j]) : 0.f;
    // q_b a_b; for beta = 0 taken as -p_b (no division by a small q_b)
    qa[j] = !okj[j] ? 0.f : beta == 0.f ? -expf(lp[j]) : q[j] * a_of(lp[j], lq[j]);
    csum += qa[j];
  }
  const float c = wave_sum(csum) + qT * aT;
  const float w = (a.grad ? a.grad[n] : 1.f) * a.inv_tau;
  if (lane == 0) a.dense_a[n] = (aT - c) * w;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int i = lane + 64 * j;
    if (i < a.smax) a.list_val[n * a.smax + i] = okj[j] ? (qa[j] - c * q[j]) * w : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Row gather / scatter ([Top-K KD] 二.4: gather the hidden states of the
// positions that carry a loss before the unembedding). One workgroup per row,
// 16-byte words when rows and pointers allow, else 4-byte words. An index
// outside [0, n_other) gathers a row of zeros / is skipped by the scatter.
// ---------------------------------------------------------------------------
template <typename W>
__global__ __launch_bounds__(256) void copy_rows_kernel(const char* __restrict__ src, char* __restrict__ dst,
                                                        const int32_t* __restrict__ rows, int64_t n_rows,
                                                        int64_t n_other, int64_t row_bytes, int scatter) {
  const int64_t words = row_bytes / (int64_t)sizeof(W);
  for (int64_t i = blockIdx.x; i < n_rows; i += gridDim.x) {
    const int64_t r = rows[i];
    const bool ok = r >= 0 && r < n_other;
    if (scatter) {
      if (!ok) continue;
      const W* s = reinterpret_cast<const W*>(src + i * row_bytes);
      W* d = reinterpret_cast<W*>(dst + r * row_bytes);
      for (int64_t w = threadIdx.x; w < words; w += blockDim.x) d[w] = s[w];
    } else {
      W* d = reinterpret_cast<W*>(dst + i * row_bytes);
      if (!ok) {
        for (int64_t w = threadIdx.x; w < words; w += blockDim.x) d[w] = W{};
        continue;
      }
      const W* s = reinterpret_cast<const W*>(src + r * row_bytes);
      for (int64_t w = threadIdx.x; w < words; w += blockDim.x) d[w] = s[w];
    }
  }
}

// One logit-sweep kernel: the 64-token tile, the fp32 tile, or the bf16 tile,
// whose pair 2 starts at ring position 1 when pair 1 (d_s) leaves one stage
// past whole turns of the ring (the 152k-vocabulary workloads' d_s = 1024
// and 2560), and otherwise both pairs run whole turns (the same stages when
// d_s fills whole turns; at most three more per tile when it leaves two:
// with pair 2 starting at position 2, the compiler again drained the ring
// at the head of pair 1's loop).
#define KD_LAUNCH_LOGIT(KERNEL)                                                                                  \
  template <bool kBf16, int MODE>                                                                                \
  hipError_t launch_##KERNEL(bool small, int r2, dim3 grid, const LogitArgs& la, hipStream_t st) {             \
    if (small)                                                                                                   \
      hipLaunchKernelGGL((KERNEL<kBf16, MODE, true, -1>), grid, dim3(kLogitThreads), 0, st, la);                \
    else if (kBf16 && r2 == 1)                                                                                   \
      hipLaunchKernelGGL((KERNEL<kBf16, MODE, false, (kBf16 ? 1 : -1)>), grid, dim3(kLogitThreads), 0, st, la); \
    else                                                                                                         \
      hipLaunchKernelGGL((KERNEL<kBf16, MODE, false, -1>), grid, dim3(kLogitThreads), 0, st, la);               \
    return hipGetLastError();                                                                                    \
  }
KD_LAUNCH_LOGIT(fwd_kernel)
#undef KD_LAUNCH_LOGIT

template <bool kBf16, int MODE, bool kGT>
hipError_t launch_bwdg_gt(bool small, int r2, dim3 grid, const LogitArgs& la, hipStream_t st) {
  if (small)
    hipLaunchKernelGGL((bwdg_kernel<kBf16, MODE, true, -1, kGT>), grid, dim3(kLogitThreads), 0, st, la);
  else if (kBf16 && r2 == 1)
    hipLaunchKernelGGL((bwdg_kernel<kBf16, MODE, false, (kBf16 ? 1 : -1), kGT>), grid, dim3(kLogitThreads), 0, st,
                       la);
  else
    hipLaunchKernelGGL((bwdg_kernel<kBf16, MODE, false, -1, kGT>), grid, dim3(kLogitThreads), 0, st, la);
  return hipGetLastError();
}
template <bool kBf16, int MODE>
hipError_t launch_bwdg_kernel(bool small, int r2, dim3 grid, const LogitArgs& la, hipStream_t st) {
  return la.GT ? launch_bwdg_gt<kBf16, MODE, true>(small, r2, grid, la, st)
               : launch_bwdg_gt<kBf16, MODE, false>(small, r2, grid, la, st);
}

// Pair 2's start position in the ring of the logit sweeps when pair 1 runs
// exactly its stages.
int logit_r2(const Plan& p) { return sweep_r2(p.d_s * p.esz, kLogitRB, kLogitBuf); }

template <bool kBf16>
hipError_t launch_fwd_mode(int mode, bool small, int r2, dim3 grid, const LogitArgs& la, hipStream_t st) {
  switch (mode) {
    case kModeFKL: return launch_fwd_kernel<kBf16, kModeFKL>(small, r2, grid, la, st);
    case kModeRKL: return launch_fwd_kernel<kBf16, kModeRKL>(small, r2, grid, la, st);
    case kModeLSE: return launch_fwd_kernel<kBf16, kModeLSE>(small, r2, grid, la, st);
    default: return launch_fwd_kernel<kBf16, kModeJSD>(small, r2, grid, la, st);
  }
}

template <bool kBf16>
hipError_t launch_bwdg_mode(int mode, bool small, int r2, dim3 grid, const LogitArgs& la, hipStream_t st) {
  switch (mode) {
    case kModeFKL: return launch_bwdg_kernel<kBf16, kModeFKL>(small, r2, grid, la, st);
    case kModeRKL: return launch_bwdg_kernel<kBf16, kModeRKL>(small, r2, grid, la, st);
    default: return launch_bwdg_kernel<kBf16, kModeJSD>(small, r2, grid, la, st);
  }
}

LogitArgs logit_args(const Plan& p, const void* h_s, const void* W_s, const void* h_t, const void* W_t, float tau,
                     float beta) {
  LogitArgs la{};
  la.ps = PairDesc{static_cast<const char*>(W_s), static_cast<const char*>(h_s), (int64_t)p.d_s * p.esz,
                   (int64_t)p.d_s * p.esz, p.V, p.N, (int32_t)(p.d_s * p.esz)};
  la.pt = PairDesc{static_cast<const char*>(W_t), static_cast<const char*>(h_t), (int64_t)p.d_t * p.esz,
                   (int64_t)p.d_t * p.esz, p.V, p.N, (int32_t)(p.d_t * p.esz)};
  la.N = p.N;
  la.V = p.V;
  la.c2 = kLog2e / tau;
  la.inv_tau = 1.f / tau;
  la.beta = beta;
  la.n_tok_tiles = p.n_tok_tiles;
  return la;
}

}  // namespace

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Few token tiles: a logit sweep streams W from HBM and its time is about
// (waves of workgroups over the 256 CUs) x (tiles per workgroup + the fixed
// cost of one, ~1.5 tiles); the tiles per workgroup that minimise it (the
// measured best for the forward at 64..512 tokens).
static int tiles_per_block_few_tokens(int n_tok_tiles, int n_vtiles, int t_min) {
  int tps = t_min;
  double best = 1e30;
  for (int t = t_min; t <= (t_min > 8 ? t_min : 8); ++t) {
    const int64_t blocks = (int64_t)n_tok_tiles * ((n_vtiles + t - 1) / t);
    const double cost = (double)((blocks + 255) / 256) * (t + 1.5);
    if (cost < best) {
      best = cost;
      tps = t;
    }
  }
  return tps;
}

Plan make_plan(int64_t N, int64_t V, int32_t d_s, int32_t d_t, bool bf16) {
  Plan p;
  p.N = N;
  p.V = V;
  p.d_s = d_s;
  p.d_t = d_t;
  p.bf16 = bf16;
  p.esz = bf16 ? 2 : 4;
  p.n_tok_tiles = (int)((N + kTileT - 1) / kTileT);
  p.n_vtiles = (int)((V + kTileV - 1) / kTileV);
  // at most kFwdMaxSplits partial records per token, whatever V
  const int t_min = (p.n_vtiles + kFwdMaxSplits - 1) / kFwdMaxSplits;
  int tps = p.n_tok_tiles <= 4 ? tiles_per_block_few_tokens(p.n_tok_tiles, p.n_vtiles, t_min) : kFwdTilesPerBlock;
  tps = tps > t_min ? tps : t_min;
  p.tiles_per_split = tps < p.n_vtiles ? tps : p.n_vtiles;
  p.n_splits = (p.n_vtiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

size_t fwd_workspace_bytes(const Plan& p, bool jsd) {
  const size_t rec = (size_t)p.n_splits * (size_t)p.N * sizeof(float);
  return align_up(kFwdFields * rec, 256) + (jsd ? align_up(kJsdFields * rec, 256) : 0);
}

// Tokens rounded up to the logit token tile: the token extent (K) of the
// weight-gradient GEMM, zero-padded.
int64_t padded_tokens(const Plan& p) { return (p.N + kTileT - 1) / kTileT * kTileT; }

// Splits of the dh GEMM's contraction (over one chunk) when its output has
// few 256 x 256 tiles (few tokens): enough workgroups for the 256 CUs, each
// split at least 512 vocabulary entries long.
int dh_ksplit(const Plan& p, int32_t chunk_V) {
  const int64_t tiles = ((p.N + kTileDhT - 1) / kTileDhT) * ((p.d_s + kTileDhD - 1) / kTileDhD);
  if (tiles >= 128) return 1;
  int64_t s = (256 + tiles - 1) / tiles;
  const int64_t by_k = chunk_V / 512;
  s = s < by_k ? s : by_k;
  return s > 1 ? (int)s : 1;
}

// The chunk buffers (G, W_s's chunk transposed, and for dW_s their token-major
// counterparts); the dh GEMM's split partial tiles follow them.
static size_t bwd_base_bytes(const Plan& p, int32_t chunk_V, bool with_dW) {
  size_t b = align_up((size_t)p.N * chunk_V * p.esz, 256) + align_up((size_t)p.d_s * chunk_V * p.esz, 256);
  if (with_dW) {
    const size_t np = (size_t)padded_tokens(p);
    b += align_up((size_t)chunk_V * np * p.esz, 256) + align_up((size_t)p.d_s * np * p.esz, 256);
  }
  return b;
}

size_t bwd_workspace_bytes(const Plan& p, int32_t chunk_V, bool with_dW) {
  const int s = dh_ksplit(p, chunk_V);
  return bwd_base_bytes(p, chunk_V, with_dW) +
         (s > 1 ? align_up((size_t)s * p.N * p.d_s * sizeof(float), 256) : 0);
}

// kd_bwd's dominant-entry correction after the chunk buffers: the per-split
// sums of one chunk (at most chunk_V / 256 splits), their running total and
// the dominant index, per token.
static size_t bwd_fix_bytes(const Plan& p, int32_t chunk_V) {
  return align_up((size_t)(chunk_V / kTileV) * p.N * sizeof(float), 256) + 2 * align_up((size_t)p.N * 4, 256);
}

size_t kd_bwd_workspace_bytes(const Plan& p, int32_t chunk_V, bool with_dW) {
  return bwd_workspace_bytes(p, chunk_V, with_dW) + bwd_fix_bytes(p, chunk_V);
}

// dh (+)= G . W_s[chunk] for one chunk (kcols contracted entries), split over
// the contraction when the output has few tiles.
static hipError_t launch_dh(const Plan& p, bool bf16, DhArgs da, int32_t chunk_V, int64_t kcols, float* part,
                            hipStream_t st) {
  const int n_d_tiles = (p.d_s + kTileDhD - 1) / kTileDhD;
  const int n_tok_tiles = (int)((p.N + kTileDhT - 1) / kTileDhT);
  da.n_tok_tiles = n_tok_tiles;
  da.n_d_tiles = n_d_tiles;
  da.n_ksplit = 1;
  const int s_max = dh_ksplit(p, chunk_V);
  if (s_max > 1) {
    // splits of whole 256-entry vocabulary tiles: every split is non-empty
    const int64_t ktiles = kcols / kTileV;
    const int64_t per = (ktiles + s_max - 1) / s_max;
    da.n_ksplit = (int)((ktiles + per - 1) / per);
    da.kspan = (int32_t)(per * kTileV * p.esz);
    da.part = part;
  }
  const dim3 grid((unsigned)xcd_grid(n_tok_tiles * n_d_tiles * da.n_ksplit));
  const bool small = p.N <= kSmallT;  // one token tile either way
  if (bf16 && small)
    hipLaunchKernelGGL((dh_kernel<true, true>), grid, dim3(kDhThreads), 0, st, da);
  else if (bf16)
    hipLaunchKernelGGL((dh_kernel<true, false>), grid, dim3(kDhThreads), 0, st, da);
  else if (small)
    hipLaunchKernelGGL((dh_kernel<false, true>), grid, dim3(kDhThreads), 0, st, da);
  else
    hipLaunchKernelGGL((dh_kernel<false, false>), grid, dim3(kDhThreads), 0, st, da);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || da.n_ksplit == 1) return e;
  const int64_t count = p.N * (int64_t)p.d_s;
  const unsigned rblocks = (unsigned)((count + 255) / 256 < 4096 ? (count + 255) / 256 : 4096);
  hipLaunchKernelGGL(dh_reduce_kernel, dim3(rblocks), dim3(256), 0, st, part, da.n_ksplit, count, da.dh, da.first);
  return hipGetLastError();
}

hipError_t run_fwd(const Plan& p, const FwdIO& io, hipStream_t st) {
  LogitArgs la = logit_args(p, io.h_s, io.W_s, io.h_t, io.W_t, io.tau, io.beta);
  la.n_splits = p.n_splits;
  la.tiles_per_split = p.tiles_per_split;
  la.n_vtiles = p.n_vtiles;
  la.vt_offset = 0;
  la.part = static_cast<float*>(io.workspace);
  const dim3 grid(xcd_grid(p.n_tok_tiles * p.n_splits));
  const bool small = p.N <= kSmallT;  // one token tile either way; the 64-row tile has a deeper ring
  const int r2 = logit_r2(p);
  hipError_t e;
  if (io.beta == 0.f || io.beta == 1.f) {
    const int mode = io.beta == 1.f ? kModeRKL : kModeFKL;
    e = p.bf16 ? launch_fwd_mode<true>(mode, small, r2, grid, la, st) : launch_fwd_mode<false>(mode, small, r2, grid, la, st);
    if (e != hipSuccess) return e;
    return mode == kModeRKL
               ? launch_merge<kModeRKL>(la.part, p.n_splits, p.N, la.inv_tau, io.loss, io.lse_s, io.lse_t, io.aux, st)
               : launch_merge<kModeFKL>(la.part, p.n_splits, p.N, la.inv_tau, io.loss, io.lse_s, io.lse_t, io.aux, st);
  }
  // 0 < beta < 1: sweep 1 -> LSEs, sweep 2 -> mixture sums.
  e = p.bf16 ? launch_fwd_mode<true>(kModeLSE, small, r2, grid, la, st) : launch_fwd_mode<false>(kModeLSE, small, r2, grid, la, st);
  if (e != hipSuccess) return e;
  e = launch_merge<kModeLSE>(la.part, p.n_splits, p.N, la.inv_tau, io.loss, io.lse_s, io.lse_t, io.aux, st);
  if (e != hipSuccess) return e;
  LogitArgs lj = la;
  lj.part = reinterpret_cast<float*>(static_cast<char*>(io.workspace) + align_up(
      kFwdFields * (size_t)p.n_splits * (size_t)p.N * sizeof(float), 256));
  lj.lse_s = io.lse_s;
  lj.lse_t = io.lse_t;
  e = p.bf16 ? launch_fwd_mode<true>(kModeJSD, small, r2, grid, lj, st) : launch_fwd_mode<false>(kModeJSD, small, r2, grid, lj, st);
  if (e != hipSuccess) return e;
  return launch_merge<kModeJSD>(lj.part, p.n_splits, p.N, la.inv_tau, io.loss, io.lse_s, io.lse_t, io.aux, st);
}

static int bwd_tiles_per_block(const Plan& p, int ctiles) {
  if (p.n_tok_tiles <= 4) return tiles_per_block_few_tokens(p.n_tok_tiles, ctiles, 1);
  const int wide = (ctiles + kBwdTilesPerBlock - 1) / kBwdTilesPerBlock;
  return (int64_t)p.n_tok_tiles * wide >= kBwdWideMinBlocks ? kBwdTilesPerBlock : 1;
}

hipError_t run_bwd(const Plan& p, const BwdIO& io, hipStream_t st) {
  const int mode = io.beta == 1.f ? kModeRKL : (io.beta == 0.f ? kModeFKL : kModeJSD);
  const int64_t np = padded_tokens(p);
  char* G = static_cast<char*>(io.workspace);
  char* WsT = G + align_up((size_t)p.N * io.chunk_V * p.esz, 256);
  char* GT = WsT + align_up((size_t)p.d_s * io.chunk_V * p.esz, 256);
  char* hsT = GT + align_up((size_t)io.chunk_V * np * p.esz, 256);
  float* part = reinterpret_cast<float*>(static_cast<char*>(io.workspace) +
                                         bwd_base_bytes(p, io.chunk_V, io.dW != nullptr));
  char* fixw = static_cast<char*>(io.workspace) + bwd_workspace_bytes(p, io.chunk_V, io.dW != nullptr);
  float* esum = reinterpret_cast<float*>(fixw);
  float* etot = reinterpret_cast<float*>(fixw + align_up((size_t)(io.chunk_V / kTileV) * p.N * sizeof(float), 256));
  int32_t* big = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(etot) + align_up((size_t)p.N * 4, 256));
  LogitArgs la = logit_args(p, io.h_s, io.W_s, io.h_t, io.W_t, io.tau, io.beta);
  // Up to 64 tokens the 64-row tile with a deeper ring (one token tile either
  // way); not with dW_s, whose transposed gradient copy must also zero the
  // token columns 64..127 of the 128-padded token extent.
  const bool small = p.N <= kSmallT && io.dW == nullptr;
  const int r2 = logit_r2(p);
  la.lse_s = io.lse_s;
  la.lse_t = io.lse_t;
  la.aux = io.aux;
  la.grad = io.grad;
  la.G = io.dh ? G : nullptr;
  la.ldg = (int64_t)io.chunk_V * p.esz;
  la.GT = io.dW ? GT : nullptr;
  la.ldgt = np * p.esz;
  la.Np = np;
  la.esum = io.dh ? esum : nullptr;
  la.big = io.dh ? big : nullptr;
  const unsigned tok_blocks = (unsigned)((p.N + 255) / 256);
  const int n_d_tiles = (p.d_s + kTileDhD - 1) / kTileDhD;
  hipError_t e;
  auto transpose = [&](const void* src, char* dst, int64_t rows, int64_t c0, int64_t cols, int64_t pitch) {
    const dim3 tgrid((unsigned)(cols / 64), (unsigned)((p.d_s + 63) / 64));
    if (p.bf16)
      hipLaunchKernelGGL(transpose_bf16_kernel, tgrid, dim3(256), 0, st, static_cast<const uint16_t*>(src),
                         reinterpret_cast<uint16_t*>(dst), rows, p.d_s, c0, pitch);
    else
      hipLaunchKernelGGL(transpose_kernel<float>, tgrid, dim3(256), 0, st, static_cast<const float*>(src),
                         reinterpret_cast<float*>(dst), rows, p.d_s, c0, pitch);
    return hipGetLastError();
  };
  auto gemm = [&](const DhArgs& da, int n_row_tiles) {
    const dim3 dgrid(xcd_grid(n_row_tiles * n_d_tiles));
    if (p.bf16)
      hipLaunchKernelGGL((dh_kernel<true, false>), dgrid, dim3(kDhThreads), 0, st, da);
    else
      hipLaunchKernelGGL((dh_kernel<false, false>), dgrid, dim3(kDhThreads), 0, st, da);
    return hipGetLastError();
  };
  // h_s transposed once ([d_s][Np], zero past N): the token-contiguous B operand of dW
  if (io.dW && (e = transpose(io.h_s, hsT, p.N, 0, np, np)) != hipSuccess) return e;
  if (io.dh) {
    hipLaunchKernelGGL(big_init_kernel, dim3(tok_blocks < 1024 ? tok_blocks : 1024), dim3(256), 0, st, big, p.N);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  for (int64_t c0 = 0; c0 < p.V; c0 += io.chunk_V) {
    const int64_t ccols = (p.V - c0 < io.chunk_V) ? p.V - c0 : io.chunk_V;
    const int ctiles = (int)((ccols + kTileV - 1) / kTileV);
    const int64_t kcols = (int64_t)ctiles * kTileV;
    la.vt_offset = (int)(c0 / kTileV);
    la.n_vtiles = ctiles;
    la.tiles_per_split = bwd_tiles_per_block(p, ctiles);
    la.n_splits = (ctiles + la.tiles_per_split - 1) / la.tiles_per_split;
    la.g_col0 = c0;
    const dim3 grid(xcd_grid(p.n_tok_tiles * la.n_splits));
    e = p.bf16 ? launch_bwdg_mode<true>(mode, small, r2, grid, la, st) : launch_bwdg_mode<false>(mode, small, r2, grid, la, st);
    if (e != hipSuccess) return e;
    if (io.dh) {
      // dh_s (+)= G . W_s[chunk], with the chunk of W_s transposed to [d_s][chunk]
      if ((e = transpose(io.W_s, WsT, p.V, c0, kcols, io.chunk_V)) != hipSuccess) return e;
      DhArgs da{};
      da.p = PairDesc{G, WsT, (int64_t)io.chunk_V * p.esz, (int64_t)io.chunk_V * p.esz, p.N, p.d_s,
                      (int32_t)(kcols * p.esz)};
      da.N = p.N;
      da.d_s = p.d_s;
      da.dh = io.dh;
      da.first = c0 == 0;
      if ((e = launch_dh(p, p.bf16, da, io.chunk_V, kcols, part, st)) != hipSuccess) return e;
      hipLaunchKernelGGL(esum_reduce_kernel, dim3((unsigned)((p.N + kEsumTok - 1) / kEsumTok)), dim3(256), 0, st,
                         esum, la.n_splits, p.N, etot, c0 == 0 ? 1 : 0);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (io.dW) {
      // dW_s[chunk] = G^T . h_s: rows of the chunk, contracted over the tokens
      DhArgs dw{};
      dw.p = PairDesc{GT, hsT, np * p.esz, np * p.esz, kcols, p.d_s, (int32_t)(np * p.esz)};
      dw.N = ccols;
      dw.d_s = p.d_s;
      dw.n_tok_tiles = (int)(kcols / kTileDhT);
      dw.n_d_tiles = n_d_tiles;
      dw.dh = io.dW + c0 * p.d_s;
      dw.first = 1;
      dw.n_ksplit = 1;
      if ((e = gemm(dw, dw.n_tok_tiles)) != hipSuccess) return e;
    }
  }
  if (io.dh) {
    const dim3 fgrid((unsigned)(p.N < 4096 ? p.N : 4096));
    if (p.bf16)
      hipLaunchKernelGGL(big_fix_kernel<uint16_t>, fgrid, dim3(256), 0, st, big, etot,
                         static_cast<const uint16_t*>(io.W_s), p.d_s, p.N, io.dh);
    else
      hipLaunchKernelGGL(big_fix_kernel<float>, fgrid, dim3(256), 0, st, big, etot, static_cast<const float*>(io.W_s),
                         p.d_s, p.N, io.dh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Per vocabulary chunk: G = A q + C r (dense_g_kernel), the listed entries
// overwrite their G elements (g_fix_kernel), W_s's chunk is transposed, and
// the dh GEMM writes (first chunk) or accumulates onto dh_s.
static hipError_t run_list_chunks(const Plan& p, DenseArgs a, const int32_t* list_idx, const float* list_val, int slots,
                                  const void* W_s, char* G, char* WsT, float* part, int32_t chunk_V, float* dh,
                                  hipStream_t st) {
  hipError_t e;
  FixArgs f{list_idx, list_val, p.N, slots, 0, 0, G, (int64_t)chunk_V * 2};
  const unsigned fix_blocks = (unsigned)((p.N * slots + 255) / 256);
  for (int64_t c0 = 0; c0 < p.V; c0 += chunk_V) {
    const int64_t ccols = (p.V - c0 < chunk_V) ? p.V - c0 : chunk_V;
    const int ctiles = (int)((ccols + kTileV - 1) / kTileV);
    const int64_t kcols = (int64_t)ctiles * kTileV;
    a.vt_offset = (int)(c0 / kTileV);
    a.n_vtiles = ctiles;
    a.n_splits = ctiles;
    a.g_col0 = c0;
    if (a.dense_c && a.c2 != kLog2e)
      hipLaunchKernelGGL(dense_g_kernel<true>, dim3(xcd_grid(a.n_tok_tiles * ctiles)), dim3(kDenseThreads), 0, st, a);
    else
      hipLaunchKernelGGL(dense_g_kernel<false>, dim3(xcd_grid(a.n_tok_tiles * ctiles)), dim3(kDenseThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    f.c0 = c0;
    f.ccols = ccols;
    hipLaunchKernelGGL(g_fix_kernel, dim3(fix_blocks), dim3(256), 0, st, f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 tgrid((unsigned)(kcols / 64), (unsigned)((p.d_s + 63) / 64));
    hipLaunchKernelGGL(transpose_bf16_kernel, tgrid, dim3(256), 0, st, static_cast<const uint16_t*>(W_s),
                       reinterpret_cast<uint16_t*>(WsT), p.V, p.d_s, c0, (int64_t)chunk_V);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    DhArgs da{};
    da.p = PairDesc{G, WsT, (int64_t)chunk_V * 2, (int64_t)chunk_V * 2, p.N, p.d_s, (int32_t)(kcols * 2)};
    da.N = p.N;
    da.d_s = p.d_s;
    da.dh = dh;
    da.first = c0 == 0 ? 1 : 0;
    if ((e = launch_dh(p, true, da, chunk_V, kcols, part, st)) != hipSuccess) return e;
  }
  return hipSuccess;
}

static DenseArgs dense_args(const Plan& p, const void* h_s, const void* W_s, float tau, char* G, int32_t chunk_V) {
  DenseArgs a{};
  a.ps = PairDesc{static_cast<const char*>(W_s), static_cast<const char*>(h_s), (int64_t)p.d_s * 2,
                  (int64_t)p.d_s * 2, p.V, p.N, (int32_t)(p.d_s * 2)};
  a.N = p.N;
  a.V = p.V;
  a.c2 = kLog2e / tau;
  a.n_tok_tiles = (int)((p.N + kDenseT - 1) / kDenseT);
  a.tiles_per_split = 1;
  a.G = G;
  a.ldg = (int64_t)chunk_V * 2;
  return a;
}

// Workspace after the chunk buffers: dense_a [N], dense_c [N] (top-k only),
// the list's indices [N, slots] (top-k only) and values [N, slots].
size_t topk_bwd_workspace_bytes(const Plan& p, int32_t chunk_V, int32_t k) {
  const size_t slots = (size_t)k + 1;
  return bwd_workspace_bytes(p, chunk_V, false) + 2 * align_up((size_t)p.N * 4, 256) +
         2 * align_up((size_t)p.N * slots * 4, 256);
}

size_t tail_bwd_workspace_bytes(const Plan& p, int32_t chunk_V, int32_t k) {
  const size_t slots = 2 * (size_t)k + 1;  // the largest support
  return bwd_workspace_bytes(p, chunk_V, false) + align_up((size_t)p.N * 4, 256) +
         align_up((size_t)p.N * slots * 4, 256);
}

hipError_t run_topk_bwd(const Plan& p, const TopkBwdIO& io, hipStream_t st) {
  char* G = static_cast<char*>(io.workspace);
  char* WsT = G + align_up((size_t)p.N * io.chunk_V * 2, 256);
  char* rest = static_cast<char*>(io.workspace) + bwd_workspace_bytes(p, io.chunk_V, false);
  const int slots = io.k + 1;
  float* dense_a = reinterpret_cast<float*>(rest);
  float* dense_c = reinterpret_cast<float*>(rest + align_up((size_t)p.N * 4, 256));
  int32_t* list_idx = reinterpret_cast<int32_t*>(rest + 2 * align_up((size_t)p.N * 4, 256));
  float* list_val = reinterpret_cast<float*>(reinterpret_cast<char*>(list_idx) + align_up((size_t)p.N * slots * 4, 256));
  TopkCoefArgs c{};
  c.h_s = static_cast<const uint16_t*>(io.h_s);
  c.W_s = static_cast<const uint16_t*>(io.W_s);
  c.N = p.N;
  c.V = p.V;
  c.d_s = p.d_s;
  c.k = io.k;
  c.inv_tau = 1.f / io.tau;
  c.labels = io.labels;
  c.idx = io.idx;
  c.val_t = io.val_t;
  c.val_s = io.val_s;
  c.p_mass = io.p_mass;
  c.q_mass = io.q_mass;
  c.lse_s = io.lse_s;
  c.lse_s1 = io.lse_s1;
  c.gb = io.grad_binary;
  c.gc = io.grad_cond;
  c.ge = io.grad_ce;
  c.dense_a = dense_a;
  const bool ce = io.grad_ce && io.labels && io.lse_s1;
  c.dense_c = ce ? dense_c : nullptr;
  c.list_idx = list_idx;
  c.list_val = list_val;
  hipLaunchKernelGGL(topk_coef_kernel, dim3((unsigned)((p.N + 3) / 4)), dim3(256), 0, st, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DenseArgs a = dense_args(p, io.h_s, io.W_s, io.tau, G, io.chunk_V);
  a.lse_s = io.lse_s;
  a.lse_s1 = ce ? io.lse_s1 : nullptr;
  a.dense_a = dense_a;
  a.dense_c = ce ? dense_c : nullptr;
  float* part = reinterpret_cast<float*>(static_cast<char*>(io.workspace) + bwd_base_bytes(p, io.chunk_V, false));
  return run_list_chunks(p, a, list_idx, list_val, slots, io.W_s, G, WsT, part, io.chunk_V, io.dh, st);
}

hipError_t run_tail_bwd(const Plan& p, const TailBwdIO& io, hipStream_t st) {
  char* G = static_cast<char*>(io.workspace);
  char* WsT = G + align_up((size_t)p.N * io.chunk_V * 2, 256);
  char* rest = static_cast<char*>(io.workspace) + bwd_workspace_bytes(p, io.chunk_V, false);
  float* dense_a = reinterpret_cast<float*>(rest);
  float* list_val = reinterpret_cast<float*>(rest + align_up((size_t)p.N * 4, 256));
  TailCoefArgs c{};
  c.N = p.N;
  c.V = p.V;
  c.smax = io.smax;
  c.beta = io.beta;
  c.inv_tau = 1.f / io.tau;
  c.sup_idx = io.sup_idx;
  c.sup_t = io.sup_t;
  c.sup_s = io.sup_s;
  c.lse_s = io.lse_s;
  c.lse_t = io.lse_t;
  c.grad = io.grad;
  c.dense_a = dense_a;
  c.list_val = list_val;
  hipLaunchKernelGGL(tail_coef_kernel, dim3((unsigned)((p.N + 3) / 4)), dim3(256), 0, st, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DenseArgs a = dense_args(p, io.h_s, io.W_s, io.tau, G, io.chunk_V);
  a.lse_s = io.lse_s;
  a.dense_a = dense_a;
  float* part = reinterpret_cast<float*>(static_cast<char*>(io.workspace) + bwd_base_bytes(p, io.chunk_V, false));
  return run_list_chunks(p, a, io.sup_idx, list_val, io.smax, io.W_s, G, WsT, part, io.chunk_V, io.dh, st);
}

hipError_t run_copy_rows(const void* src, void* dst, const int32_t* rows, int64_t n_rows, int64_t n_other,
                         int64_t row_bytes, bool scatter, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)(n_rows < 65536 ? n_rows : 65536);
  const bool wide = (row_bytes % 16 == 0) && ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
  if (wide)
    hipLaunchKernelGGL(copy_rows_kernel<u32x4>, dim3(grid), dim3(256), 0, st, static_cast<const char*>(src),
                       static_cast<char*>(dst), rows, n_rows, n_other, row_bytes, scatter ? 1 : 0);
  else
    hipLaunchKernelGGL(copy_rows_kernel<uint32_t>, dim3(grid), dim3(256), 0, st, static_cast<const char*>(src),
                       static_cast<char*>(dst), rows, n_rows, n_other, row_bytes, scatter ? 1 : 0);
  return hipGetLastError();
}

}  // namespace kd
