// kd_internal.h - host-side plan and launcher declarations shared between the
// C-ABI layer (kd_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kd.h"

namespace kd {

// Logit tile: 256 vocabulary rows x kTileT tokens per workgroup, split over
// kLogitWM x kLogitWN waves (vocabulary x tokens), with a ring of kLogitBuf
// LDS stages.
constexpr int kTileV = 256;
#ifndef KD_TILE_T
#define KD_TILE_T 128
#endif
constexpr int kTileT = KD_TILE_T;
#ifndef KD_LOGIT_RB
#define KD_LOGIT_RB 128
#endif
#ifndef KD_LOGIT_BUF
#define KD_LOGIT_BUF 3
#endif
constexpr int kLogitRB = KD_LOGIT_RB;   // bytes of K per LDS stage row
constexpr int kLogitBuf = KD_LOGIT_BUF;
// Token tile of the top-k sweep (its per-token selection state lives in LDS).
constexpr int kTopkT = 128;
#ifndef KD_LOGIT_WM
#define KD_LOGIT_WM 4
#endif
constexpr int kLogitWM = KD_LOGIT_WM;
constexpr int kLogitWN = 2;
constexpr int kLogitThreads = 64 * kLogitWM * kLogitWN;
// dh tile: 256 tokens x kTileDhD hidden units over kDhWM x kDhWN waves, with
// a ring of kDhBuf LDS stages.
constexpr int kTileDhT = 256;
#ifndef KD_DH_TILE_D
#define KD_DH_TILE_D 256
#endif
constexpr int kTileDhD = KD_DH_TILE_D;
#ifndef KD_DH_WM
#define KD_DH_WM 4
#endif
#ifndef KD_DH_WN
#define KD_DH_WN 2
#endif
constexpr int kDhWM = KD_DH_WM;
constexpr int kDhWN = KD_DH_WN;
constexpr int kDhThreads = 64 * kDhWM * kDhWN;
#ifndef KD_DH_RB
#define KD_DH_RB 128
#endif
constexpr int kDhRB = KD_DH_RB;
#ifndef KD_DH_BUF
#define KD_DH_BUF (kTileDhD > 128 ? 2 : 3)
#endif
constexpr int kDhBuf = KD_DH_BUF;
// Number of token tiles grouped together in the block order (L2 reuse).
#ifndef KD_TOK_GROUP
#define KD_TOK_GROUP 8
#endif
constexpr int kTokGroup = KD_TOK_GROUP;
// Vocabulary tiles per forward workgroup (2048 vocabulary entries): blocks
// that run together finish together, which keeps their shared operand rows
// in L2; each writes one partial record per token.
#ifndef KD_FWD_TILES_PER_BLOCK
#define KD_FWD_TILES_PER_BLOCK 8
#endif
constexpr int kFwdTilesPerBlock = KD_FWD_TILES_PER_BLOCK;
// Fields of the forward partial statistics.
constexpr int kFwdFields = 5;  // max_s, sum_s, max_t, sum_t, kl-accumulator
constexpr int kJsdFields = 2;  // loss sum, aux sum

enum Mode { kModeFKL = 0, kModeRKL = 1, kModeLSE = 2, kModeJSD = 3 };

struct Plan {
  int64_t N = 0, V = 0;
  int32_t d_s = 0, d_t = 0;
  int esz = 2;       // bytes per input element
  bool bf16 = true;
  int n_tok_tiles = 0, n_vtiles = 0, n_splits = 0, tiles_per_split = 0;
};

Plan make_plan(int64_t N, int64_t V, int32_t d_s, int32_t d_t, bool bf16);
size_t align_up(size_t x, size_t a);
size_t fwd_workspace_bytes(const Plan& p, bool jsd);
size_t bwd_workspace_bytes(const Plan& p, int32_t chunk_V);

struct FwdIO {
  const void *h_s, *W_s, *h_t, *W_t;
  float beta, tau;
  float *loss, *lse_s, *lse_t, *aux;
  void* workspace;
};
hipError_t run_fwd(const Plan& p, const FwdIO& io, hipStream_t stream);

struct BwdIO {
  const void *h_s, *W_s, *h_t, *W_t;
  float beta, tau;
  int32_t chunk_V;
  const float *lse_s, *lse_t, *aux, *grad;
  float* dh;
  void* workspace;
};
hipError_t run_bwd(const Plan& p, const BwdIO& io, hipStream_t stream);

struct TopkIO {
  const void *h_s, *W_s, *h_t, *W_t;
  int32_t k;
  float tau;
  const int32_t* labels;
  int32_t* idx;
  float *val, *val_s, *binary, *cond, *ce, *p_mass, *q_mass, *lse_s, *lse_t;
  void* workspace;
};
size_t topk_workspace_bytes(const Plan& p, int32_t k);
hipError_t run_topk(const Plan& p, const TopkIO& io, hipStream_t stream);

}  // namespace kd
