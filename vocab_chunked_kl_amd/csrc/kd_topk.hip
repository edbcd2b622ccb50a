// kd_topk.hip - top-k three-term decomposition over bf16 logits.
//
// lpnh.cn "Top-K知识蒸馏损失实现详解": section 一.2 splits the top-k KD loss
// into a binary KL (teacher mass inside vs outside the top-k set), a
// conditional KL (the shape inside the set, renormalised) and a CE anchor on
// the true token; section 二.1 keeps the logits in bf16 with fp32 only for
// the log-sum-exp accumulators; section 二.2 gathers the top-64 in bf16 and
// upcasts only those values.
//
// Sweep kernel (one block per token tile and 65536-entry vocabulary split):
// rebuild both logit tiles with bf16 MFMA, round them to bf16 (nearest even),
// fold them into online log-sum-exps of the tempered bf16 logits, and keep a
// running top-k of the teacher's bf16 logits per token in LDS. Candidates are
// ordered by one 32-bit word: (order-preserving bf16 key << 16) | (0xFFFF -
// index within the split), i.e. key descending, then index ascending. Only
// values above the token's current k-th word enter a small candidate buffer;
// a buffer that is nearly full (or overflowed, or at the block's last tile) is
// merged into the running list: by insertion once the list holds k words,
// else by a bitonic sort in registers.
//
// Merge kernel (one wave per token): merge the per-split log-sum-exps and
// top-k lists, recompute the student logits at the selected indices and at
// the label (fp32 dot products, rounded to bf16), and evaluate the terms.
#include <math.h>

#include "kd_internal.h"
#include "kd_sweep.hpp"

namespace kd {

namespace {

constexpr float kNegInf = -INFINITY;
// At most 65536 vocabulary entries per split (the in-split index fits 16
// bits); the vocabulary is cut into ceil(V / 65536) splits of equal tile
// counts, so that no split's blocks run much longer than the others.
constexpr int kTopkSplit = 65536;
constexpr int kCandCap = 16;       // candidate buffer entries per token per round (one list)
constexpr int kCandCap2 = 12;      // the same with two lists (both models ranked at once)
constexpr int kInsertMax = 16;     // a full list takes up to this many candidates by insertion
constexpr int kMergeSlack = 4;     // a buffer is merged once at most this many slots are free
// A block's first tile fills empty lists: every entry passes the test, so with
// one list its candidates go to the idle ring stage, 64 entries per token, and
// the bitonic merge takes up to 128 words at once (4 rounds instead of 16).
constexpr int kCandCapFirst = 64;
constexpr int kTopkFields = 6;     // m_s, l_s, m_t, l_t, m_1, l_1 (untempered student)

struct TopkArgs {
  PairDesc ps, pt;
  int64_t N, V;
  int32_t d_s;
  int k;
  float c2;       // log2(e) / tau
  int n_tok_tiles, n_splits, tiles_per_split, n_vtiles;
  int swap;        // ps / pt hold the teacher / student pair: rank the student
  float* part;     // [kTopkFields][n_splits][N]
  uint32_t* lists; // [n_splits][N][k] packed words, descending
  uint32_t* lists2;  // with two lists: the student-ranked one, same layout
};

// Round to bf16 (nearest, ties to even) and return the rounded value as fp32.
__device__ __forceinline__ float round_bf16(float x) {
  return __builtin_bit_cast(float, f32_to_bf16_bits(x) << 16);
}

// Order-preserving 16-bit key of a bf16 value (given as its rounded fp32);
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t bf16_key(float xb) {
  uint32_t b = __builtin_bit_cast(uint32_t, xb) >> 16;
  if (b == 0x8000u) b = 0;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ float key_to_f32(uint32_t key) {
  const uint32_t b = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
  return __builtin_bit_cast(float, b << 16);
}

__device__ __forceinline__ void merge2(float& m, float& l, float m2, float l2) {
  const float mm = fmaxf(m, m2);
  const float f1 = (m == kNegInf) ? 0.f : fast_exp2(m - mm);
  const float f2 = (m2 == kNegInf) ? 0.f : fast_exp2(m2 - mm);
  l = l * f1 + l2 * f2;
  m = mm;
}

#define KD_RING3_LDS(TM, TN)                                                  \
  __shared__ __attribute__((aligned(16))) char ring0_[Ring<TM, TN>::kBytes]; \
  __shared__ __attribute__((aligned(16))) char ring1_[Ring<TM, TN>::kBytes]; \
  __shared__ __attribute__((aligned(16))) char ring2_[Ring<TM, TN>::kBytes]; \
  const RingLds<3> lds{{ring0_, ring1_, ring2_}}

// Wave grid of the top-k sweep: 4 vocabulary slices x 2 token halves.
constexpr int kTopkWM = 4, kTopkWN = 2, kTopkThreads = 64 * kTopkWM * kTopkWN;
typedef uint32_t u32x16 __attribute__((__vector_size__(16 * sizeof(uint32_t))));

// ---------------------------------------------------------------------------
// Sweep: per (token tile, vocabulary split) top-k lists and LSE partials.
// kSep1: also accumulate the untempered student LSE (tau != 1, for the CE).
// With swap set, the two operand pairs come in exchanged (the ranked model
// is then the student) and the LSE partials are written back in the usual
// field order. kTwo: rank both models at once, the teacher into lists and
// the student into lists2 (smaller candidate buffers, more merge rounds).
// kPt1st: contract the pt pair first, when its stages leave one over whole
// turns of the stage ring (a rank-256 teacher: 4 stages), so that a tile
// needs no padding stages; the epilogue still gets (z_s, z_t).
// ---------------------------------------------------------------------------
template <bool kSep1, bool kTwo, bool kPt1st>
__global__ __launch_bounds__(kTopkThreads, 1) void topk_sweep_kernel(TopkArgs a) {
  constexpr int TM = kTileV, TN = kTopkT, WM = kTopkWM, WN = kTopkWN, NW = WM * WN;
  constexpr int MB = TM / (32 * WM), NB = TN / (32 * WN);
  constexpr int NL = kTwo ? 2 : 1;                // lists: 0 teacher-ranked, 1 student-ranked
  constexpr int CAP = kTwo ? kCandCap2 : kCandCap;
  constexpr int CAPF = kTwo ? kCandCap2 : kCandCapFirst;
  static_assert(NL * TN * CAPF * sizeof(uint32_t) <= Ring<TM, TN>::kBytes, "first-tile buffers fit one stage");
  static_assert(CAPF <= 64, "list and buffer fit the 128-word merge");
  // LDS: a three-stage ring, the candidate buffers and per-token counters.
  // The running top-k lists live in the per-split output rows of the
  // workspace (each token's row is read and written only by the wave that
  // merges it), which leaves LDS room for the third ring stage.
  KD_RING3_LDS(TM, TN);
  __shared__ uint32_t B[NL][TN][CAP];      // candidate buffers
  __shared__ int cntS[NL][TN], cntB[NL][TN];
  __shared__ uint32_t theta[NL][TN];       // k-th word once full, else 0

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  if (L >= a.n_tok_tiles * a.n_splits) return;  // grid padding
  int tt, sp;
  block_coords<kTokGroup>(L, a.n_tok_tiles, a.n_splits, tt, sp);
  const int vt0 = sp * a.tiles_per_split;
  const int vt1 = min(vt0 + a.tiles_per_split, a.n_vtiles);
  const int64_t vbase = (int64_t)vt0 * TM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave % WM, wn = wave / WM;
  const int K = a.k;
  const float c2 = a.c2;

  for (int i = tid; i < NL * TN; i += kTopkThreads) {
    cntS[i / TN][i % TN] = 0;
    cntB[i / TN][i % TN] = 0;
    theta[i / TN][i % TN] = 0u;
  }
  __syncthreads();

  float ms[NB], ls[NB], mt[NB], lt[NB], m1[NB], l1[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    ms[nb] = mt[nb] = m1[nb] = kNegInf;
    ls[nb] = lt[nb] = l1[nb] = 0.f;
  }

  // merge token t's candidate buffer into its state (one wave): the <= 128
  // words (S then B, zero-padded to 128, two per lane: element i = lane + 64 h)
  // are sorted descending by a bitonic network in registers (words are
  // distinct and nonzero, so the zeros sink), and the first min(total, k)
  // become the new state
  // the candidate buffers of the current tile: B (CAP per token and list), or
  // on a block's first tile the idle ring stage (CAPF)
  uint32_t* cbuf = &B[0][0][0];
  int ccap = CAP;
  auto merge_token = [&](int li, int t) {
    const int cs = cntS[li][t];
    const int cap = kTwo ? CAP : ccap;
    const int cb = min(cntB[li][t], cap);
    const uint32_t* Bt = (kTwo ? &B[0][0][0] : cbuf) + (li * TN + t) * cap;
    const int total = cs + cb;
    uint32_t* Sg = (li ? a.lists2 : a.lists) + ((int64_t)sp * a.N + (int64_t)tt * TN + t) * K;  // token < N
    if (cs == K && cb <= kInsertMax) {
      // a full list and a few candidates (the usual case once a split is
      // under way): insert them one at a time. A candidate's rank is the
      // number of list words above it (words are distinct); the words below
      // move down one lane and the last one drops out.
      uint32_t e = lane < K ? Sg[lane] : 0u;
      for (int i = 0; i < cb; ++i) {
        const uint32_t c = Bt[i];
        const int rank = __popcll(__ballot(lane < K && e > c));
        const uint32_t up = __shfl(e, lane > 0 ? lane - 1 : 0);
        e = lane < rank ? e : (lane == rank ? c : up);
      }
      if (lane < K) Sg[lane] = e;
      const uint32_t th = __shfl(e, K - 1);
      if (lane == 0) {
        cntB[li][t] = 0;
        theta[li][t] = th;
      }
      return;
    }
    uint32_t e0 = lane < cs ? Sg[lane] : (lane - cs < cb ? Bt[lane - cs] : 0u);
    const int j1 = lane + 64;
    uint32_t e1 = j1 - cs < cb ? Bt[j1 - cs] : 0u;  // cs <= 64 <= j1
#pragma unroll
    for (int k = 2; k <= 128; k <<= 1) {
#pragma unroll
      for (int j = k >> 1; j > 0; j >>= 1) {
        if (j == 64) {  // partner is the lane's other element; k = 128: descending
          const uint32_t hi = max(e0, e1), lo = min(e0, e1);
          e0 = hi;
          e1 = lo;
        } else {
          const uint32_t p0 = __shfl_xor(e0, j), p1 = __shfl_xor(e1, j);
          const bool lower = (lane & j) == 0;
          const bool desc0 = (lane & k) == 0;
          const bool desc1 = ((lane + 64) & k) == 0;
          e0 = (lower == desc0) ? max(e0, p0) : min(e0, p0);
          e1 = (lower == desc1) ? max(e1, p1) : min(e1, p1);
        }
      }
    }
    const int ns = min(total, K);
    if (lane < K) Sg[lane] = lane < ns ? e0 : 0u;  // the row stays fully defined
    const uint32_t th = __shfl(e0, K - 1);
    if (lane == 0) {
      cntS[li][t] = ns;
      cntB[li][t] = 0;
      theta[li][t] = ns == K ? th : 0u;
    }
  };

  auto epi = [&](int vt, auto& zs, auto& zt, char* idle) {
    const int64_t vrow0 = (int64_t)vt * TM + wm * (TM / WM);
    const bool full = (int64_t)(vt + 1) * TM <= a.V;
    // 1) round both logit tiles to bf16; 2) online LSEs of the tempered values
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mxs = kNegInf, mxt = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = full || (vrow0 + mb * 32 + acc_row(r, lane) < a.V);
          zs[mb][nb][r] = round_bf16(zs[mb][nb][r]);
          zt[mb][nb][r] = round_bf16(zt[mb][nb][r]);
          if (ok) {
            mxs = fmaxf(mxs, zs[mb][nb][r]);
            mxt = fmaxf(mxt, zt[mb][nb][r]);
          }
        }
      const float ms_new = fmaxf(ms[nb], mxs * c2), mt_new = fmaxf(mt[nb], mxt * c2);
      const float m1_new = fmaxf(m1[nb], mxs * kLog2e);
      if (ms_new == kNegInf) continue;
      const float fs = fast_exp2(ms[nb] - ms_new), ft = fast_exp2(mt[nb] - mt_new);
      const float f1 = fast_exp2(m1[nb] - m1_new);
      float sl = 0.f, tl = 0.f, s1 = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = full || (vrow0 + mb * 32 + acc_row(r, lane) < a.V);
          float es = fast_exp2(fmaf(zs[mb][nb][r], c2, -ms_new));
          float et = fast_exp2(fmaf(zt[mb][nb][r], c2, -mt_new));
          float e1 = kSep1 ? fast_exp2(fmaf(zs[mb][nb][r], kLog2e, -m1_new)) : 0.f;
          if (!ok) es = et = e1 = 0.f;
          sl += es;
          tl += et;
          s1 += e1;
        }
      ls[nb] = fmaf(ls[nb], fs, sl);
      lt[nb] = fmaf(lt[nb], ft, tl);
      ms[nb] = ms_new;
      mt[nb] = mt_new;
      if (kSep1) {
        l1[nb] = fmaf(l1[nb], f1, s1);
        m1[nb] = m1_new;
      }
    }
    // with two lists, both 16-bit keys are packed into the teacher's registers
    // (teacher key high, student key low; whole-vector bit casts), so that the
    // student's accumulators are free during the candidate rounds
    if constexpr (kTwo) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          u32x16 kv;
#pragma unroll
          for (int r = 0; r < 16; ++r) kv[r] = (bf16_key(zt[mb][nb][r]) << 16) | bf16_key(zs[mb][nb][r]);
          zt[mb][nb] = __builtin_bit_cast(floatx16, kv);
        }
    }
    // 3) top-k candidates: rounds until no token's buffer overflowed
    constexpr int kDoneWords = (MB * 16 + 31) / 32;
    uint32_t done[NL][NB][kDoneWords];
#pragma unroll
    for (int li = 0; li < NL; ++li)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < kDoneWords; ++i) done[li][nb][i] = 0u;
    const int rel0 = (int)(vrow0 - vbase);
    // (two lists: their registers leave no room for this, B serves throughout)
    bool first = false;
    if constexpr (!kTwo) {
      first = vt == vt0;
      cbuf = first ? reinterpret_cast<uint32_t*>(idle) : &B[0][0][0];
      ccap = first ? CAPF : CAP;
      if (first) __syncthreads();  // every wave is done with its fragments of the idle stage
    }
    while (true) {
      int ov = 0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = wn * (TN / WN) + nb * 32 + (lane & 31);
        const bool tok_ok = (int64_t)tt * TN + col < a.N;  // tokens past N have no list row
#pragma unroll
        for (int li = 0; li < NL; ++li) {
          const uint32_t th = theta[li][col];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int bit = mb * 16 + r;
              const int rel = rel0 + mb * 32 + acc_row(r, lane);
              const bool ok = full || (vbase + rel < a.V);
              uint32_t key;
              if constexpr (kTwo) {
                const uint32_t both = __builtin_bit_cast(u32x16, zt[mb][nb])[r];
                key = li ? (both & 0xFFFFu) : (both >> 16);
              } else {
                key = bf16_key(zt[mb][nb][r]);
              }
              const uint32_t w = (key << 16) | (0xFFFFu - (uint32_t)rel);
              if (ok && tok_ok && w > th && !((done[li][nb][bit >> 5] >> (bit & 31)) & 1u)) {
                const int slot = atomicAdd(&cntB[li][col], 1);
                if constexpr (kTwo) {
                  if (slot < CAP) {
                    B[li][col][slot] = w;
                    done[li][nb][bit >> 5] |= 1u << (bit & 31);
                  } else {
                    ov = 1;
                  }
                } else if (slot < ccap) {
                  cbuf[col * ccap + slot] = w;
                  done[li][nb][bit >> 5] |= 1u << (bit & 31);
                } else {
                  ov = 1;
                }
              }
            }
        }
      }
      const int any = __syncthreads_or(ov);
      // a round that overflowed, and the block's last tile, merge every
      // buffer; otherwise a buffer waits until it holds CAP - kMergeSlack
      // candidates (the threshold lags meanwhile, so a few more entries pass
      // the test, but each list row, long evicted from L2 by the unembedding
      // stream, is read and written once per several candidates)
      const int at = (any || first || vt + 1 == vt1) ? 1 : CAP - kMergeSlack;
      for (int t = wave; t < TN; t += NW)
#pragma unroll
        for (int li = 0; li < NL; ++li)
          if (cntB[li][t] >= at) merge_token(li, t);
      __syncthreads();
      if (!any) break;
    }
  };
  if constexpr (kPt1st)
    sweep<true, TM, TN, WM, WN, 3, 128, true, 1>(a.pt, a.ps, (int64_t)tt * TN, vt0, vt1, lds,
                                                 [&](int vt, auto& z1, auto& z2, char* idle) { epi(vt, z2, z1, idle); });
  else
    sweep<true, TM, TN, WM, WN, 3, 128, true>(a.ps, a.pt, (int64_t)tt * TN, vt0, vt1, lds, epi);
  // the ring is drained: its first buffer holds the cross-wave LSE records
  float* red = reinterpret_cast<float*>(lds.b[0]);
  static_assert((WM - 1) * kTopkFields * TN * sizeof(float) <= Ring<TM, TN>::kBytes, "records fit one stage");

  // LSE partials: lanes l and l^32, then the WM vocabulary-slice waves
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    merge2(ms[nb], ls[nb], __shfl_xor(ms[nb], 32), __shfl_xor(ls[nb], 32));
    merge2(mt[nb], lt[nb], __shfl_xor(mt[nb], 32), __shfl_xor(lt[nb], 32));
    merge2(m1[nb], l1[nb], __shfl_xor(m1[nb], 32), __shfl_xor(l1[nb], 32));
  }
  if (wm > 0 && lane < 32) {
    float* r = red + (wm - 1) * kTopkFields * TN;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wn * (TN / WN) + nb * 32 + lane;
      r[0 * TN + col] = ms[nb];
      r[1 * TN + col] = ls[nb];
      r[2 * TN + col] = mt[nb];
      r[3 * TN + col] = lt[nb];
      r[4 * TN + col] = m1[nb];
      r[5 * TN + col] = l1[nb];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = wn * (TN / WN) + nb * 32 + lane;
#pragma unroll
      for (int w = 0; w < WM - 1; ++w) {
        const float* r = red + w * kTopkFields * TN;
        merge2(ms[nb], ls[nb], r[0 * TN + col], r[1 * TN + col]);
        merge2(mt[nb], lt[nb], r[2 * TN + col], r[3 * TN + col]);
        merge2(m1[nb], l1[nb], r[4 * TN + col], r[5 * TN + col]);
      }
      const int64_t n = (int64_t)tt * TN + col;
      if (n < a.N) {
        const int64_t S_ = a.n_splits;
        const int fs = a.swap ? 2 : 0, ft = 2 - fs;  // fields of the student / teacher records
        a.part[((fs + 0) * S_ + sp) * a.N + n] = ms[nb];
        a.part[((fs + 1) * S_ + sp) * a.N + n] = ls[nb];
        a.part[((ft + 0) * S_ + sp) * a.N + n] = mt[nb];
        a.part[((ft + 1) * S_ + sp) * a.N + n] = lt[nb];
        a.part[(4 * S_ + sp) * a.N + n] = m1[nb];
        a.part[(5 * S_ + sp) * a.N + n] = l1[nb];
      }
    }
  }
  // the lists are in place; a token that never received a candidate (only
  // possible for a split with no valid entry) gets a row of empty words
#pragma unroll
  for (int li = 0; li < NL; ++li)
    for (int i = tid; i < TN * K; i += kTopkThreads) {
      const int t = i / K, j = i - t * K;
      const int64_t n = (int64_t)tt * TN + t;
      if (n < a.N && cntS[li][t] == 0) (li ? a.lists2 : a.lists)[((int64_t)sp * a.N + n) * K + j] = 0u;
    }
}

// ---------------------------------------------------------------------------
// Merge: one wave per token.
// ---------------------------------------------------------------------------
struct MergeArgs {
  const uint16_t *h_s, *W_s;
  int64_t N, V;
  int32_t d_s;
  int k, n_splits, split;  // split: vocabulary entries per split
  float c2;  // log2(e) / tau, the factor the sweep's base-2 maxima were formed with
  const float* part;
  const uint32_t* lists;
  const int32_t* labels;
  int32_t* idx;
  float *val_t, *val_s, *binary, *cond, *ce, *p_mass, *q_mass, *lse_s, *lse_t, *lse_s1;
  int sep1;
};

constexpr int kMaxSplits = 8;  // vocabularies up to 8 * 65536 entries

// Merge token n's per-split lists (S splits of K words) into its global top-K,
// one wave: lane j < K receives the j-th entry's vocabulary index (-1 for an
// empty slot) and its bf16 key value. cw holds S * K words, sel K words (LDS,
// the wave's own).
__device__ __forceinline__ void select_topk(const uint32_t* __restrict__ lists, int64_t N, int64_t V, int64_t n,
                                            int S, int K, int split, unsigned long long* cw, unsigned long long* sel,
                                            int lane, int32_t& vj, float& val) {
  // candidates as 64-bit words: key << 32 | (0xFFFFFFFF - vocabulary index); 0 = empty
  const int C = S * K;
  for (int i = lane; i < C; i += 64) {
    const int s = i / K;
    const uint32_t w = lists[((int64_t)s * N + n) * K + (i - s * K)];
    const uint32_t vidx = (uint32_t)s * (uint32_t)split + (0xFFFFu - (w & 0xFFFFu));
    cw[i] = w == 0u ? 0ull : ((unsigned long long)(w >> 16) << 32) | (0xFFFFFFFFull - vidx);
  }
  if (lane < K) sel[lane] = 0ull;  // slots left empty stay 0 (never read as an index)
  __builtin_amdgcn_wave_barrier();
  // rank every candidate against all others (all words are distinct); rank < K is its slot
  for (int i = lane; i < C; i += 64) {
    const unsigned long long x = cw[i];
    int r = 0;
    for (int j = 0; j < C; ++j) r += cw[j] > x;
    if (x != 0ull && r < K) sel[r] = x;
  }
  __builtin_amdgcn_wave_barrier();
  const unsigned long long xj = lane < K ? sel[lane] : 0ull;
  // an empty slot (only possible with fewer than k finite candidates) or a
  // decoded index outside the vocabulary is never dereferenced
  const uint32_t vdec = 0xFFFFFFFFu - (uint32_t)(xj & 0xFFFFFFFFull);
  vj = (xj != 0ull && (int64_t)vdec < V) ? (int32_t)vdec : -1;
  val = lane < K ? key_to_f32((uint32_t)(xj >> 32)) : 0.f;
  __builtin_amdgcn_wave_barrier();  // cw and sel may be reused after this
}

__global__ __launch_bounds__(256) void topk_merge_kernel(MergeArgs a) {
  __shared__ unsigned long long cand[4][kMaxSplits * KD_TOPK_MAX];
  __shared__ unsigned long long sel[4][KD_TOPK_MAX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave;
  if (n >= a.N) return;  // whole waves only: no block barrier below
  const int K = a.k, S = a.n_splits;
  const int64_t SN = (int64_t)S;

  // log-sum-exps (base 2, tempered; m_1/l_1 untempered when kept apart)
  float ms = kNegInf, ls = 0.f, mt = kNegInf, lt = 0.f, m1 = kNegInf, l1 = 0.f;
  for (int s = lane; s < S; s += 64) {
    merge2(ms, ls, a.part[(0 * SN + s) * a.N + n], a.part[(1 * SN + s) * a.N + n]);
    merge2(mt, lt, a.part[(2 * SN + s) * a.N + n], a.part[(3 * SN + s) * a.N + n]);
    merge2(m1, l1, a.part[(4 * SN + s) * a.N + n], a.part[(5 * SN + s) * a.N + n]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    merge2(ms, ls, __shfl_xor(ms, o), __shfl_xor(ls, o));
    merge2(mt, lt, __shfl_xor(mt, o), __shfl_xor(lt, o));
    merge2(m1, l1, __shfl_xor(m1, o), __shfl_xor(l1, o));
  }
  const float Ls = (ms + log2f(ls)) * kLn2;  // natural LSE of the tempered bf16 logits
  const float Lt = (mt + log2f(lt)) * kLn2;
  const float L1 = a.sep1 ? (m1 + log2f(l1)) * kLn2 : Ls;  // untempered student LSE (tau == 1: the same)

  const bool act = lane < K;
  int32_t vj;
  float tj;
  select_topk(a.lists, a.N, a.V, n, S, K, a.split, cand[wave], sel[wave], lane, vj, tj);
  // student bf16 logits at the selected indices: one wave-wide dot product
  // each, four at a time
  const uint16_t* h = a.h_s + n * a.d_s;
  float sj = 0.f;
  for (int j0 = 0; j0 < K; j0 += 4) {
    int64_t v4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v4[j] = j0 + j < K ? (int64_t)__shfl(vj, j0 + j) : -1;  // wave-uniform
    float z[4];
    wave_dot4_bf16(h, a.W_s, v4, a.d_s, lane, z);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane == j0 + j) sj = v4[j] >= 0 ? z[j] : kNegInf;
  }
  if (act) {
    a.idx[n * K + lane] = vj;
    if (a.val_t) a.val_t[n * K + lane] = tj;
    if (a.val_s) a.val_s[n * K + lane] = sj;
  }
  // The set's log-sum-exps in the sweep's base-2 frame: each selected logit is
  // taken relative to the whole vocabulary's maximum with one fused
  // multiply-add, so log P, log Q and the conditional term are formed from
  // small numbers and a logit offset common to a row costs them no precision
  // (a difference of two fp32 log-sum-exps near 100 is good to only ~1e-5).
  const float dt = act ? fmaf(tj, a.c2, -mt) : kNegInf, ds = act ? fmaf(sj, a.c2, -ms) : kNegInf;
  const float mtK = wave_max(dt), msK = wave_max(ds);
  const float et = act ? exp2f(dt - mtK) : 0.f, es = act ? exp2f(ds - msK) : 0.f;
  const float set = wave_sum(et), ses = wave_sum(es);
  const float LKt = mtK + log2f(set), LKs = msK + log2f(ses);  // base 2, relative to mt and ms
  // Tail masses below fp32 resolution are held at 2^-24 so that their logs stay
  // finite; with the whole vocabulary selected there is no tail at all.
  const bool all = (int64_t)K >= a.V;
  const float logP = fminf((LKt - log2f(lt)) * kLn2, -5.9604645e-8f);
  const float logQ = fminf((LKs - log2f(ls)) * kLn2, -5.9604645e-8f);
  const float cterm = act ? (et / set) * ((dt - LKt) - (ds - LKs)) : 0.f;
  const float condv = wave_sum(cterm) * kLn2;
  if (lane == 0) {
    const float P = expf(logP), Q = expf(logQ);
    const float l1P = log1mexp_f32(logP), l1Q = log1mexp_f32(logQ);
    const float tail = (1.f - P) * (l1P - l1Q);
    a.binary[n] = all ? 0.f : P * (logP - logQ) + tail;
    a.cond[n] = condv;
    a.p_mass[n] = all ? 1.f : P;
    a.q_mass[n] = all ? 1.f : Q;
    a.lse_s[n] = Ls;
    a.lse_t[n] = Lt;
    if (a.lse_s1) a.lse_s1[n] = L1;
  }
  if (a.labels) {
    const int32_t y = a.labels[n];
    if (y >= 0 && y < a.V) {
      // untempered LSE minus the label's logit, both relative to the untempered
      // maximum (with tau = 1 the tempered record is the untempered one)
      const float zy = wave_dot_bf16(h, a.W_s, y, a.d_s, lane);
      const float m1u = a.sep1 ? m1 : ms, l1u = a.sep1 ? l1 : ls;
      if (lane == 0) a.ce[n] = (log2f(l1u) - fmaf(zy, kLog2e, -m1u)) * kLn2;
    } else if (lane == 0) {
      a.ce[n] = NAN;
    }
  }
}

// ---------------------------------------------------------------------------
// Tail-bucket divergence (White-box OPD, section 2.4): the beta-divergence of
// section 2.3 taken over the buckets {each support entry} + {the rest of the
// vocabulary}. The support is the teacher's top-k, the student's top-k, their
// union (duplicates removed) and/or the label, in that order. One wave per
// token: merge the per-split log-sum-exps and lists (one list per ranked
// model), assemble the support in LDS, fill in each entry's missing logit with
// an fp32 dot product (rounded to bf16; the ranked model's value is its key),
// then evaluate the buckets.
// ---------------------------------------------------------------------------
constexpr int kSupMax = 2 * KD_TOPK_MAX + 1;

struct TailArgs {
  const uint16_t *h_s, *W_s, *h_t, *W_t;
  int64_t N, V;
  int32_t d_s, d_t;
  int k, n_splits, split, support, smax;  // split: vocabulary entries per split
  float beta;
  float c2;  // log2(e) / tau, the factor the sweep's base-2 maxima were formed with
  const float* part;
  const uint32_t *lists_t, *lists_s;
  const int32_t* labels;
  int32_t* sup_idx;
  float *sup_t, *sup_s, *loss, *p_mass, *q_mass, *lse_s, *lse_t;
};

__device__ __forceinline__ float logaddexp_f(float x, float y) {
  const float m = fmaxf(x, y);
  return m == kNegInf ? kNegInf : m + log1pf(expf(-fabsf(x - y)));
}

// Wave-wide natural log-sum-exp of up to three values per lane (-inf = none).
__device__ __forceinline__ float wave_lse3(float a, float b, float c) {
  const float m = wave_max(fmaxf(a, fmaxf(b, c)));
  if (m == kNegInf) return kNegInf;
  return m + logf(wave_sum(expf(a - m) + expf(b - m) + expf(c - m)));
}

__global__ __launch_bounds__(256) void tail_merge_kernel(TailArgs a) {
  __shared__ unsigned long long cand[4][kMaxSplits * KD_TOPK_MAX];
  __shared__ unsigned long long sel[4][KD_TOPK_MAX];
  __shared__ int32_t sidx[4][kSupMax];
  __shared__ float sval_t[4][kSupMax], sval_s[4][kSupMax];
  __shared__ int32_t sknown[4][kSupMax];  // bit 0: teacher value known, bit 1: student value known
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave;
  if (n >= a.N) return;  // whole waves only: no block barrier below
  const int K = a.k, S = a.n_splits;
  const int64_t SN = (int64_t)S;
  int32_t* si = sidx[wave];
  float* st = sval_t[wave];
  float* ss = sval_s[wave];
  int32_t* sk = sknown[wave];

  float ms = kNegInf, ls = 0.f, mt = kNegInf, lt = 0.f;
  for (int s = lane; s < S; s += 64) {
    merge2(ms, ls, a.part[(0 * SN + s) * a.N + n], a.part[(1 * SN + s) * a.N + n]);
    merge2(mt, lt, a.part[(2 * SN + s) * a.N + n], a.part[(3 * SN + s) * a.N + n]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    merge2(ms, ls, __shfl_xor(ms, o), __shfl_xor(ls, o));
    merge2(mt, lt, __shfl_xor(mt, o), __shfl_xor(lt, o));
  }
  const float Ls = (ms + log2f(ls)) * kLn2;  // natural LSE of the tempered bf16 logits
  const float Lt = (mt + log2f(lt)) * kLn2;

  // 1) the support
  const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int cnt = 0;
  if (a.support & KD_SUPPORT_TEACHER) {
    int32_t v;
    float key;
    select_topk(a.lists_t, a.N, a.V, n, S, K, a.split, cand[wave], sel[wave], lane, v, key);
    const bool ok = lane < K && v >= 0;  // filled slots form a prefix
    if (ok) {
      si[lane] = v;
      st[lane] = key;
      sk[lane] = 1;
    }
    cnt = __popcll(__ballot(ok));
    __builtin_amdgcn_wave_barrier();
  }
  if (a.support & KD_SUPPORT_STUDENT) {
    int32_t v;
    float key;
    select_topk(a.lists_s, a.N, a.V, n, S, K, a.split, cand[wave], sel[wave], lane, v, key);
    bool keep = lane < K && v >= 0;
    for (int j = 0; j < cnt; ++j) keep = keep && si[j] != v;
    const unsigned long long m = __ballot(keep);
    if (keep) {
      const int pos = cnt + __popcll(m & below);
      si[pos] = v;
      ss[pos] = key;
      sk[pos] = 2;
    }
    cnt += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
  if ((a.support & KD_SUPPORT_LABEL) && a.labels) {
    const int32_t y = a.labels[n];
    if (y >= 0 && y < a.V) {
      bool found = false;
      for (int j = lane; j < cnt; j += 64) found = found || si[j] == y;
      if (__ballot(found) == 0ull) {
        if (lane == 0) {
          si[cnt] = y;
          sk[cnt] = 0;
        }
        ++cnt;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // 2) the missing logits, four consecutive support entries at a time (the
  //    teacher's list, then the student's extras, then the label: runs that
  //    miss the same model's logit), one wave-wide dot product each
  const uint16_t* hs = a.h_s + n * a.d_s;
  const uint16_t* ht = a.h_t + n * a.d_t;
  for (int i0 = 0; i0 < cnt; i0 += 4) {
    int64_t vt[4], vs[4];
    bool any_t = false, any_s = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = i0 + j < cnt;
      const int32_t v = ok ? si[i0 + j] : -1;
      const int kn = ok ? sk[i0 + j] : 3;
      vt[j] = (kn & 1) ? -1 : v;
      vs[j] = (kn & 2) ? -1 : v;
      any_t = any_t || vt[j] >= 0;
      any_s = any_s || vs[j] >= 0;
    }
    float z[4];
    if (any_t) {
      wave_dot4_bf16(ht, a.W_t, vt, a.d_t, lane, z);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane == 0 && vt[j] >= 0) st[i0 + j] = z[j];
    }
    if (any_s) {
      wave_dot4_bf16(hs, a.W_s, vs, a.d_s, lane, z);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane == 0 && vs[j] >= 0) ss[i0 + j] = z[j];
    }
  }
  __builtin_amdgcn_wave_barrier();

  // 3) bucket log-probabilities: three slots per lane cover 2k + 1 <= 129 entries
  //    (each logit relative to the vocabulary's base-2 maximum with one fused
  //    multiply-add, so a logit offset common to a row costs no precision)
  const float l2t = log2f(lt), l2s = log2f(ls);
  float lp[3], lq[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int i = lane + 64 * j;
    const bool ok = i < cnt;
    lp[j] = ok ? (fmaf(st[i], a.c2, -mt) - l2t) * kLn2 : kNegInf;
    lq[j] = ok ? (fmaf(ss[i], a.c2, -ms) - l2s) * kLn2 : kNegInf;
  }
  const float logP = wave_lse3(lp[0], lp[1], lp[2]);
  const float logQ = wave_lse3(lq[0], lq[1], lq[2]);
  // tail masses below fp32 resolution are held at 2^-24 (their logs stay finite);
  // a support that covers the vocabulary leaves no tail bucket
  const bool tail = (int64_t)cnt < a.V;
  const float lpT = log1mexp_f32(fminf(logP, -5.9604645e-8f));
  const float lqT = log1mexp_f32(fminf(logQ, -5.9604645e-8f));
  const float beta = a.beta;
  const float lb = logf(beta), l1b = log1pf(-beta);
  auto term = [&](float p_, float q_) {  // one bucket's share of the divergence
    if (beta == 0.f) return expf(p_) * (p_ - q_);
    if (beta == 1.f) return expf(q_) * (q_ - p_);
    const float lm = logaddexp_f(lb + p_, l1b + q_);
    return beta * expf(p_) * (p_ - lm) + (1.f - beta) * expf(q_) * (q_ - lm);
  };
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (lane + 64 * j < cnt) acc += term(lp[j], lq[j]);
  acc = wave_sum(acc);
  if (lane == 0) {
    a.loss[n] = acc + (tail ? term(lpT, lqT) : 0.f);
    if (a.p_mass) a.p_mass[n] = tail ? expf(logP) : 1.f;
    if (a.q_mass) a.q_mass[n] = tail ? expf(logQ) : 1.f;
    a.lse_s[n] = Ls;
    a.lse_t[n] = Lt;
  }
  // 4) the support rows, padded with index -1 and NaN values
  for (int i = lane; i < a.smax; i += 64) {
    const bool ok = i < cnt;
    a.sup_idx[n * a.smax + i] = ok ? si[i] : -1;
    a.sup_t[n * a.smax + i] = ok ? st[i] : NAN;
    a.sup_s[n * a.smax + i] = ok ? ss[i] : NAN;
  }
}

}  // namespace

size_t topk_workspace_bytes(const Plan& p, int32_t k) {
  const int64_t n_splits = (p.V + kTopkSplit - 1) / kTopkSplit;
  return align_up((size_t)kTopkFields * n_splits * p.N * sizeof(float), 256) +
         align_up((size_t)n_splits * p.N * k * sizeof(uint32_t), 256);
}

// The top-k sweep with the pt pair contracted first when that saves the
// ring's padding stages (see topk_sweep_kernel).
template <bool kSep1, bool kTwo>
static hipError_t launch_topk_sweep(dim3 grid, const TopkArgs& a, hipStream_t st) {
  if (sweep_r2(a.pt.kbytes, 128, 3) == 1)
    hipLaunchKernelGGL((topk_sweep_kernel<kSep1, kTwo, true>), grid, dim3(kTopkThreads), 0, st, a);
  else
    hipLaunchKernelGGL((topk_sweep_kernel<kSep1, kTwo, false>), grid, dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t run_topk(const Plan& p, const TopkIO& io, hipStream_t st) {
  TopkArgs a{};
  a.ps = PairDesc{static_cast<const char*>(io.W_s), static_cast<const char*>(io.h_s), (int64_t)p.d_s * 2,
                  (int64_t)p.d_s * 2, p.V, p.N, p.d_s * 2};
  a.pt = PairDesc{static_cast<const char*>(io.W_t), static_cast<const char*>(io.h_t), (int64_t)p.d_t * 2,
                  (int64_t)p.d_t * 2, p.V, p.N, p.d_t * 2};
  a.N = p.N;
  a.V = p.V;
  a.d_s = p.d_s;
  a.k = io.k;
  a.c2 = kLog2e / io.tau;
  a.n_tok_tiles = (int)((p.N + kTopkT - 1) / kTopkT);
  a.n_vtiles = p.n_vtiles;
  a.n_splits = (int)((p.V + kTopkSplit - 1) / kTopkSplit);
  a.tiles_per_split = (p.n_vtiles + a.n_splits - 1) / a.n_splits;  // <= kTopkSplit / kTileV
  if (a.n_splits > kMaxSplits) return hipErrorInvalidValue;
  a.part = static_cast<float*>(io.workspace);
  a.lists = reinterpret_cast<uint32_t*>(static_cast<char*>(io.workspace) +
                                        align_up((size_t)kTopkFields * a.n_splits * p.N * sizeof(float), 256));
  const bool sep1 = (io.labels != nullptr || io.lse_s1 != nullptr) && io.tau != 1.f;
  const dim3 grid(xcd_grid(a.n_tok_tiles * a.n_splits));
  hipError_t e = sep1 ? launch_topk_sweep<true, false>(grid, a, st) : launch_topk_sweep<false, false>(grid, a, st);
  if (e != hipSuccess) return e;
  MergeArgs m{};
  m.h_s = static_cast<const uint16_t*>(io.h_s);
  m.W_s = static_cast<const uint16_t*>(io.W_s);
  m.N = p.N;
  m.V = p.V;
  m.d_s = p.d_s;
  m.k = io.k;
  m.n_splits = a.n_splits;
  m.split = a.tiles_per_split * kTileV;
  m.c2 = a.c2;
  m.part = a.part;
  m.lists = a.lists;
  m.labels = io.labels;
  m.idx = io.idx;
  m.val_t = io.val;
  m.val_s = io.val_s;
  m.lse_s1 = io.lse_s1;
  m.binary = io.binary;
  m.cond = io.cond;
  m.ce = io.ce;
  m.p_mass = io.p_mass;
  m.q_mass = io.q_mass;
  m.lse_s = io.lse_s;
  m.lse_t = io.lse_t;
  m.sep1 = sep1;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)((p.N + 3) / 4)), dim3(256), 0, st, m);
  return hipGetLastError();
}

int32_t tail_support_slots(int32_t k, int32_t support) {
  return ((support & KD_SUPPORT_TEACHER) ? k : 0) + ((support & KD_SUPPORT_STUDENT) ? k : 0) +
         ((support & KD_SUPPORT_LABEL) ? 1 : 0);
}

size_t tail_workspace_bytes(const Plan& p, int32_t k) {
  // the LSE partials and one list area per ranked model
  return topk_workspace_bytes(p, k) + align_up((size_t)((p.V + kTopkSplit - 1) / kTopkSplit) * p.N * k * 4, 256);
}

hipError_t run_tail(const Plan& p, const TailIO& io, hipStream_t st) {
  TopkArgs a{};
  a.ps = PairDesc{static_cast<const char*>(io.W_s), static_cast<const char*>(io.h_s), (int64_t)p.d_s * 2,
                  (int64_t)p.d_s * 2, p.V, p.N, p.d_s * 2};
  a.pt = PairDesc{static_cast<const char*>(io.W_t), static_cast<const char*>(io.h_t), (int64_t)p.d_t * 2,
                  (int64_t)p.d_t * 2, p.V, p.N, p.d_t * 2};
  a.N = p.N;
  a.V = p.V;
  a.d_s = p.d_s;
  a.k = io.k;
  a.c2 = kLog2e / io.tau;
  a.n_tok_tiles = (int)((p.N + kTopkT - 1) / kTopkT);
  a.n_vtiles = p.n_vtiles;
  a.n_splits = (int)((p.V + kTopkSplit - 1) / kTopkSplit);
  a.tiles_per_split = (p.n_vtiles + a.n_splits - 1) / a.n_splits;  // <= kTopkSplit / kTileV
  if (a.n_splits > kMaxSplits) return hipErrorInvalidValue;
  char* ws = static_cast<char*>(io.workspace);
  a.part = reinterpret_cast<float*>(ws);
  const size_t part_bytes = align_up((size_t)kTopkFields * a.n_splits * p.N * sizeof(float), 256);
  const size_t list_bytes = align_up((size_t)a.n_splits * p.N * io.k * sizeof(uint32_t), 256);
  uint32_t* lists_t = reinterpret_cast<uint32_t*>(ws + part_bytes);
  uint32_t* lists_s = reinterpret_cast<uint32_t*>(ws + part_bytes + list_bytes);
  const dim3 grid(xcd_grid(a.n_tok_tiles * a.n_splits));
  // one sweep: the teacher's list, the student's (the same sweep with the
  // two operand pairs exchanged) or both at once
  const bool rank_t = io.support & KD_SUPPORT_TEACHER, rank_s = io.support & KD_SUPPORT_STUDENT;
  hipError_t e;
  if (rank_t && rank_s) {
    a.lists = lists_t;
    a.lists2 = lists_s;
    e = launch_topk_sweep<false, true>(grid, a, st);
  } else if (rank_t) {
    a.lists = lists_t;
    e = launch_topk_sweep<false, false>(grid, a, st);
  } else {
    TopkArgs b = a;
    b.ps = a.pt;
    b.pt = a.ps;
    b.swap = 1;
    b.lists = lists_s;
    e = launch_topk_sweep<false, false>(grid, b, st);
  }
  if (e != hipSuccess) return e;
  TailArgs m{};
  m.h_s = static_cast<const uint16_t*>(io.h_s);
  m.W_s = static_cast<const uint16_t*>(io.W_s);
  m.h_t = static_cast<const uint16_t*>(io.h_t);
  m.W_t = static_cast<const uint16_t*>(io.W_t);
  m.N = p.N;
  m.V = p.V;
  m.d_s = p.d_s;
  m.d_t = p.d_t;
  m.k = io.k;
  m.n_splits = a.n_splits;
  m.split = a.tiles_per_split * kTileV;
  m.support = io.support;
  m.smax = tail_support_slots(io.k, io.support);
  m.beta = io.beta;
  m.c2 = a.c2;
  m.part = a.part;
  m.lists_t = lists_t;
  m.lists_s = lists_s;
  m.labels = io.labels;
  m.sup_idx = io.sup_idx;
  m.sup_t = io.sup_t;
  m.sup_s = io.sup_s;
  m.loss = io.loss;
  m.p_mass = io.p_mass;
  m.q_mass = io.q_mass;
  m.lse_s = io.lse_s;
  m.lse_t = io.lse_t;
  hipLaunchKernelGGL(tail_merge_kernel, dim3((unsigned)((p.N + 3) / 4)), dim3(256), 0, st, m);
  return hipGetLastError();
}

}  // namespace kd
