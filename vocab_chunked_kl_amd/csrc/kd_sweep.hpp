// kd_sweep.hpp - the pipelined MFMA tile loop shared by the logit-rebuilding
// kernels, the top-k sweep and the dh GEMM.
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
// Pipeline: a ring of NBUF (2 to 4) LDS stage buffers (RB = 128 bytes of K
// per row each) filled by direct-to-LDS buffer loads (no staging registers, no LDS store
// instructions). While stage g is multiplied, the loads of stages g+1 ..
// g+NBUF-2 are in flight and stage g+NBUF-1 is being issued; one barrier per
// stage recycles the buffer read in the previous step. The stage sequence
// (tile by tile: pair 1, then pair 2, each padded to whole turns of the ring)
// runs on continuously through the ring.
#pragma once

#include <type_traits>

#include "kd_device.hpp"

namespace kd {

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

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

// LDS stage layout: [A tile: TM rows][B tile: TN rows], RB bytes per row,
// unpadded, with the 16-byte chunks of row R stored at slot (chunk ^ swz(R)),
// swz(R) = (R & 7) ^ ((R >> 3) & 3). A direct-to-LDS load writes 64 lanes x 16
// bytes contiguously (8 rows); the XOR makes the MFMA fragment reads (16
// consecutive rows at one chunk per 16 lanes) hit 16 distinct 16-byte bank
// groups (consecutive rows sit in alternate halves of the 256-byte bank row).
// (64-byte rows with deeper rings were measured slower: twice the barriers
// and per-stage scalar work for the same bytes in flight.)
template <int RB>
struct RowFmt {
  static_assert(RB == 128, "128-byte stage rows");
  static constexpr int kChunks = RB / 16;         // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 1024 / RB;  // rows per 64-lane direct-to-LDS load
  static constexpr int kSub = RB / 32;            // MFMA k-substeps (32 bytes of K) per stage
  __device__ static __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 3); }
};

// Ring position at which pair 2 starts when pair 1 runs exactly its stages
// (the kR2 argument of sweep, chosen on the host from K1 in bytes).
__host__ __device__ constexpr int sweep_r2(int kbytes1, int rb, int nbuf) { return ((kbytes1 + rb - 1) / rb) % nbuf; }

template <int TM, int TN, int RB = 128>
struct Ring {
  static constexpr int kBytes = (TM + TN) * RB;
};

// Fetch-side state of the stage ring besides its two buffer resources (a
// sizeless type, so they are kept apart): this lane's byte offsets (row *
// pitch + its chunk, at K offset 0) of the stage issued next and the pair's K
// extent. It changes only when the fetch cursor moves to the other operand
// pair or to the next A tile, so it is rebuilt then (once per K extent) and a
// stage's loads cost an add, a compare and a select per lane. Past the last A
// tile both resources are empty and every load writes zeros without reading.
template <int QA, int QB>
struct FetchState {
  int32_t offa[QA], offb[QB];
  int32_t kbytes;
};

// Issue the direct-to-LDS loads of one stage (this wave's share of NW waves:
// QA + QB instructions, one 1024-byte row group each; `qa0` / `qb0`: this
// wave's first row group). `ca` / `cb`: this lane's chunk byte offset per
// load; a lane whose chunk lies at or past the row length reads past the
// resource end and writes zeros.
template <int TM, int RB, int QA, int QB>
__device__ __forceinline__ void dma_stage(char* dst, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          const FetchState<QA, QB>& st, const int32_t (&ca)[QA],
                                          const int32_t (&cb)[QB], int qa0, int qb0, int32_t kbyte0) {
  const int32_t rem = st.kbytes - kbyte0;
#pragma unroll
  for (int i = 0; i < QA; ++i) {
    const int32_t off = ca[i] < rem ? st.offa[i] + kbyte0 : 0x7FFFFFF0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(dst + (qa0 + i) * 1024),
                                             16, off, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < QB; ++i) {
    const int32_t off = cb[i] < rem ? st.offb[i] + kbyte0 : 0x7FFFFFF0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (__attribute__((address_space(3))) void*)(dst + TM * RB + (qb0 + i) * 1024), 16, off, 0, 0, 0);
  }
}

// Pinned instruction order of one stage (sched_group_barrier takes literal
// counts, hence the compile-time recursion over MFMA index M): the LDS reads
// of sub-step 0 first; then each MFMA is followed by at most one LDS read of
// the next sub-step, and the `kLoads` direct-to-LDS loads are spread evenly
// over the first kSpan MFMAs.
template <int kSub, int kMf, int kRd, int kLoads, int kSpan, int M = 0>
__device__ __forceinline__ void pin_stage_order() {
  if constexpr (M == 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kRd, 0);
  if constexpr (M < kSub * kMf) {
    constexpr int lo = M * kLoads / kSpan, hi = (M + 1) * kLoads / kSpan;
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (M < (kSub - 1) * kMf && (M % kMf) < kRd) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    if constexpr (M < kSpan && hi > lo) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, hi - lo, 0);
    pin_stage_order<kSub, kMf, kRd, kLoads, kSpan, M + 1>();
  }
}

// MFMAs of one LDS stage for this wave: kSub k16 sub-steps, fragments double
// buffered in registers so the reads of sub-step j+1 overlap the MFMAs of j.
// a_off / b_off: this lane's row byte offset; colx[j]: its swizzled chunk
// byte offset for sub-step j. `issue` emits the direct-to-LDS loads of a later
// stage; they are spread over the first three quarters of the MFMAs (a burst
// right after the barrier would stall the wave while the address unit drains
// them).
template <bool kBf16, int MB, int NB, int kLoads, int RB, class Issue>
__device__ __forceinline__ void mma_ring_stage(floatx16 (&acc)[MB][NB], const char* cur, int a_off, int b_off,
                                               const int (&colx)[RowFmt<RB>::kSub], Issue&& issue) {
  constexpr int kSub = RowFmt<RB>::kSub;
  u32x4 fa[2][MB], fb[2][NB];
  auto rd = [&](int s, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      fa[s][mb] = *reinterpret_cast<const u32x4*>(cur + a_off + colx[j] + mb * 32 * RB);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      fb[s][nb] = *reinterpret_cast<const u32x4*>(cur + b_off + colx[j] + nb * 32 * RB);
  };
  auto mm = [&](int s) __attribute__((always_inline)) {
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
            // fp32: four 32x32x2 MFMAs per sub-step; lane half g supplies
            // k = 8j + 4g + e on both operands, so every k is summed once.
            // The element is copied out first: a bit_cast of a vector-element
            // lvalue reads element 0 with this compiler.
            const uint32_t ae = fa[s][mb][e], be = fb[s][nb][e];
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, ae),
                                                               __builtin_bit_cast(float, be), acc[mb][nb], 0, 0, 0);
          }
        }
      }
  };
  constexpr int kRd = MB + NB;
  constexpr int kMf = MB * NB * (kBf16 ? 1 : 4);
  constexpr int kSpan = (3 * kSub * kMf) / 4 > 0 ? (3 * kSub * kMf) / 4 : 1;
  rd(0, 0);
  issue();
#pragma unroll
  for (int j = 0; j < kSub; ++j) {
    if (j + 1 < kSub) rd((j + 1) & 1, j + 1);
    mm(j & 1);
  }
  pin_stage_order<kSub, kMf, kRd, kLoads, kSpan>();
}

// Shared LDS of the stage ring: separate objects, so that the compiler sees
// that reads of one stage never alias the loads landing in another.
template <int NBUF>
struct RingLds {
  char* b[NBUF];
};

// WM x WN waves: wave w owns rows (w % WM) * TM / WM .. of the A tile and rows
// (w / WM) * TN / WN .. of the B tile; its accumulators are [MB][NB] 32 x 32
// MFMA blocks, MB = TM / (32 WM), NB = TN / (32 WN).
// kDual = false: one operand pair only (p2 is ignored, the epilogue gets acc1
// twice and no second accumulator is allocated).
// kR2 >= 0 (two pairs only): pair 1 runs exactly its ceil(K1 / RB) stages,
// which the caller guarantees to be kR2 modulo NBUF (sweep_r2 above), and
// pair 2 is padded so that a tile is whole turns of the ring; kR2 = -1 pads
// each pair to whole turns.
template <bool kBf16, int TM, int TN, int WM, int WN, int NBUF, int RB, bool kDual, int kR2 = -1, class Epi>
__device__ __forceinline__ void sweep(const PairDesc& p1, const PairDesc& p2, int64_t b_row0, int a_tile_begin,
                                      int a_tile_end, const RingLds<NBUF>& lds, Epi&& epi) {
  static_assert(NBUF >= 2 && NBUF <= 4, "ring of two to four stage buffers");
  using F = RowFmt<RB>;
  constexpr int NW = WM * WN;
  constexpr int MB = TM / (32 * WM), NB = TN / (32 * WN);
  static_assert(MB * 32 * WM == TM && NB * 32 * WN == TN, "wave tiles must be multiples of 32");
  constexpr int kDma = (TM + TN) / (F::kRowsPerLoad * NW);  // direct-to-LDS loads per wave per stage
  static_assert((NBUF - 2) * kDma < 64, "vmcnt counts up to 63");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is uniform: keep it (and the load addresses built from it) scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int a_off = ((wave % WM) * (TM / WM) + r32) * RB;
  const int b_off = (TM + (wave / WM) * (TN / WN) + r32) * RB;
  int colx[F::kSub];
#pragma unroll
  for (int j = 0; j < F::kSub; ++j) colx[j] = ((2 * j + (lane >> 5)) ^ F::swz(r32)) * 16;

  // Stages per pair. A tile is whole turns of the ring, so every tile starts
  // at ring position 0, and each pair starts at a position fixed at compile
  // time (0, and kR2 for pair 2) with a tail of fixed length: each copy of
  // the step loop has one history of outstanding loads. The stages past a
  // pair's K extent load nothing (every lane past the end writes zeros) and
  // add exact zeros. (With start positions and tail lengths known only at run
  // time, the loop copies per start position were entered from several such
  // histories, and the compiler, unable to tell which stage buffer the loads
  // target, drained them all (vmcnt(0)) before the first fragment read of
  // every ring turn in two of the three copies.)
  static_assert(kR2 < NBUF && (kR2 < 0 || kDual), "pair 2 start position");
  const int n1 = (p1.kbytes + RB - 1) / RB, n2 = kDual ? (p2.kbytes + RB - 1) / RB : 0;
  const int ks1 = kR2 < 0 ? (n1 + NBUF - 1) / NBUF * NBUF : n1;
  const int ks2 = kR2 < 0 ? (n2 + NBUF - 1) / NBUF * NBUF : n2 + (NBUF - (n1 + n2) % NBUF) % NBUF;
  if (a_tile_end <= a_tile_begin || ks1 == 0) return;

  // Load geometry: row group q (8 rows of 128 bytes) of the A tile is load
  // qa0 + i of this wave; the lane moves row q * 8 + rig, swizzled chunk c.
  constexpr int RPL = F::kRowsPerLoad;
  constexpr int QA = TM / (RPL * NW), QB = TN / (RPL * NW);
  static_assert(QA * RPL * NW == TM && QB * RPL * NW == TN, "tile rows must split evenly over the waves");
  const int slot = lane % F::kChunks, rig = lane / F::kChunks;
  const int qa0 = wave * QA, qb0 = wave * QB;
  int32_t ca[QA], cb[QB];
#pragma unroll
  for (int i = 0; i < QA; ++i) ca[i] = (slot ^ F::swz((qa0 + i) * RPL + rig)) * 16;
#pragma unroll
  for (int i = 0; i < QB; ++i) cb[i] = (slot ^ F::swz((qb0 + i) * RPL + rig)) * 16;
  const __amdgpu_buffer_rsrc_t rb1 = make_rsrc(p1.B + b_row0 * p1.ldb, (p1.b_rows - b_row0) * p1.ldb);
  const __amdgpu_buffer_rsrc_t rb2 = make_rsrc(p2.B + b_row0 * p2.ldb, (p2.b_rows - b_row0) * p2.ldb);

  // Fetch cursor: the stage issued next (tile ft, pair fp, stage fs), and the
  // state its loads use, rebuilt whenever the cursor leaves a pair's K extent.
  int ft = a_tile_begin, fp = 0, fs = 0;
  FetchState<QA, QB> st;
  __amdgpu_buffer_rsrc_t fra = rb1, frb = rb1;
  auto refresh = [&]() __attribute__((always_inline)) {
    const bool second = kDual && fp != 0;
    const char* A = second ? p2.A : p1.A;
    const int64_t lda = second ? p2.lda : p1.lda, ldb = second ? p2.ldb : p1.ldb;
    const int64_t a_row0 = (int64_t)ft * TM;
    const bool valid = ft < a_tile_end;
    fra = make_rsrc(A + a_row0 * lda, valid ? ((second ? p2.a_rows : p1.a_rows) - a_row0) * lda : 0);
    frb = valid ? (second ? rb2 : rb1) : make_rsrc(p1.B, 0);
    st.kbytes = second ? p2.kbytes : p1.kbytes;
#pragma unroll
    for (int i = 0; i < QA; ++i) st.offa[i] = ((qa0 + i) * RPL + rig) * (int32_t)lda + ca[i];
#pragma unroll
    for (int i = 0; i < QB; ++i) st.offb[i] = ((qb0 + i) * RPL + rig) * (int32_t)ldb + cb[i];
  };
  auto issue = [&](char* dst) __attribute__((always_inline)) {
    dma_stage<TM, RB, QA, QB>(dst, fra, frb, st, ca, cb, qa0, qb0, fs * RB);
  };
  auto advance = [&]() __attribute__((always_inline)) {
    if (fs + 1 == (fp == 0 ? ks1 : ks2)) {
      const int nfp = (fp == 0 && ks2 > 0) ? 1 : 0;
      ft += nfp == 0 ? 1 : 0;
      fp = nfp;
      fs = 0;
      refresh();
    } else {
      ++fs;
    }
  };

  // One ring step on buffer I: wait for its loads (the NBUF-2 later stages
  // stay in flight), barrier, refill the buffer read one step earlier with
  // the stage NBUF-1 ahead, multiply buffer I.
  auto step = [&](floatx16(&acc)[MB][NB], auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NBUF - 2) * kDma));
    lds_barrier();
    mma_ring_stage<kBf16, MB, NB, kDma, RB>(acc, lds.b[i], a_off, b_off, colx,
                                            [&]() __attribute__((always_inline)) { issue(lds.b[(i + NBUF - 1) % NBUF]); });
    advance();
  };
  // Run `ks` stages into `acc` from ring position R, ending with T single
  // steps (ks = T modulo NBUF); buffer indices are compile-time constants.
  auto run = [&](floatx16(&acc)[MB][NB], int ks, auto R, auto T) __attribute__((always_inline)) {
    constexpr int r = decltype(R)::value, t = decltype(T)::value;
    int s = 0;
    for (; s + NBUF <= ks; s += NBUF)
      static_for<0, NBUF>([&](auto I) __attribute__((always_inline)) {
        step(acc, std::integral_constant<int, (r + I) % NBUF>{});
      });
    static_for<0, t>([&](auto I) __attribute__((always_inline)) {
      step(acc, std::integral_constant<int, (r + I) % NBUF>{});
    });
  };
  using I0 = std::integral_constant<int, 0>;
  using IR2 = std::integral_constant<int, (kR2 < 0 ? 0 : kR2)>;
  using IT2 = std::integral_constant<int, (kR2 < 0 ? 0 : (NBUF - kR2) % NBUF)>;

  floatx16 acc1[MB][NB], acc2[kDual ? MB : 1][kDual ? NB : 1];
  zero_acc(acc1);
  if constexpr (kDual) zero_acc(acc2);
  // prologue: the first NBUF-1 stages
  refresh();
  static_for<0, NBUF - 1>([&](auto I) __attribute__((always_inline)) {
    issue(lds.b[I]);
    advance();
  });
  // The epilogue also gets the stage buffer that the tile's last step read
  // (the ring's last): no load targets it until the next step's barrier, so
  // an epilogue may use it as scratch after a barrier of its own (other waves
  // may still be reading their last fragments from it until then).
  for (int tile = a_tile_begin; tile < a_tile_end; ++tile) {
    run(acc1, ks1, I0{}, IR2{});
    if constexpr (kDual) {
      if (ks2 > 0) run(acc2, ks2, IR2{}, IT2{});
      epi(tile, acc1, acc2, lds.b[NBUF - 1]);
      zero_acc(acc2);
    } else {
      epi(tile, acc1, acc1, lds.b[NBUF - 1]);
    }
    zero_acc(acc1);
  }
  // drain the loads issued past the end before the LDS is reused
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
}

}  // namespace kd
