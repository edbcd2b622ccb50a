// kd_internal.h - host-side plan and launcher declarations shared between the
// C-ABI layer (kd_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kd.h"

namespace kd {

// Logit tile: 256 vocabulary rows x 128 tokens per workgroup on a 4 x 2 wave
// grid (64 x 64 per wave: two waves per SIMD), with a ring of three LDS
// stages of 128 bytes of K per row (48 KiB each).
constexpr int kTileV = 256;
constexpr int kTileT = 128;
constexpr int kLogitWM = 4;
constexpr int kLogitWN = 2;
constexpr int kLogitThreads = 64 * kLogitWM * kLogitWN;
constexpr int kLogitRB = 128;
constexpr int kLogitBuf = 3;
// Forward sweep for at most 64 tokens: the token tile shrinks to 64 rows, so
// a stage is 40 KiB and a ring of four fills the 160 KiB of LDS: three
// stages of unembedding rows in flight per CU instead of two, where the
// sweep streams W from HBM.
constexpr int kSmallT = 64;
constexpr int kSmallBuf = 4;
// Token tile of the top-k sweep (its per-token selection state lives in LDS).
constexpr int kTopkT = 128;
// dh tile: 256 tokens x 256 hidden units, 4 x 2 waves (64 x 128 per wave, one
// accumulator), ring of two 64 KiB stages.
constexpr int kTileDhT = 256;
constexpr int kTileDhD = 256;
constexpr int kDhWM = 4;
constexpr int kDhWN = 2;
constexpr int kDhThreads = 64 * kDhWM * kDhWN;
constexpr int kDhRB = 128;
constexpr int kDhBuf = 2;
// Token tile of the student-only gradient sweep of the top-k / tail backward
// (one accumulator: the dh GEMM's tile, wave layout and ring).
constexpr int kDenseT = 256;
constexpr int kDenseThreads = kDhThreads;
// Token tiles grouped together in the block order: the 32 blocks that run at
// once on one XCD are 8 token tiles x 4 vocabulary splits, the split that
// minimises the operand bytes its L2 fetches (measured best of 4, 8, 16).
constexpr int kTokGroup = 8;
// Vocabulary tiles per forward workgroup (1024 vocabulary entries; chosen per
// shape for up to 4 token tiles, see make_plan): blocks that run together
// finish together, which keeps their shared operand rows in L2; each writes
// one partial record per token. Measured against 1 to 8: equal to 8 at 32k
// tokens, at or near the best at 1024 to 4096 tokens.
constexpr int kFwdTilesPerBlock = 4;
// Largest number of forward partial records per token: past 256 splits
// (V > 262144 at four tiles per workgroup) the workgroups take more tiles, so
// the forward workspace stays within 7 * 256 floats per token for any V.
constexpr int kFwdMaxSplits = 256;
// Vocabulary tiles per gradient-tile workgroup (bwdg_kernel): two halve the
// pipeline ramps per tile (measured 2 % faster than 1 on the 32k-token
// backward, and 4 no better than 2) as long as the chunk's grid keeps at
// least kBwdWideMinBlocks workgroups; smaller grids (a few hundred tokens)
// keep one tile per workgroup, which measured 4-7 % faster there.
constexpr int kBwdTilesPerBlock = 2;
constexpr int64_t kBwdWideMinBlocks = 2048;
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
size_t bwd_workspace_bytes(const Plan& p, int32_t chunk_V, bool with_dW);
// kd_bwd's workspace: the chunk buffers plus its dominant-entry correction.
size_t kd_bwd_workspace_bytes(const Plan& p, int32_t chunk_V, bool with_dW);

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
  float* dh;  // may be null when dW is not
  float* dW;  // may be null
  void* workspace;
};
hipError_t run_bwd(const Plan& p, const BwdIO& io, hipStream_t stream);

struct TopkIO {
  const void *h_s, *W_s, *h_t, *W_t;
  int32_t k;
  float tau;
  const int32_t* labels;
  int32_t* idx;
  float *val, *val_s, *binary, *cond, *ce, *p_mass, *q_mass, *lse_s, *lse_t, *lse_s1;
  void* workspace;
};
size_t topk_workspace_bytes(const Plan& p, int32_t k);

struct TopkBwdIO {
  const void *h_s, *W_s;
  int32_t k;
  float tau;
  int32_t chunk_V;
  const int32_t* labels;
  const int32_t* idx;
  const float *val_t, *val_s, *p_mass, *q_mass, *lse_s, *lse_s1;
  const float *grad_binary, *grad_cond, *grad_ce;
  float* dh;
  void* workspace;
};
size_t topk_bwd_workspace_bytes(const Plan& p, int32_t chunk_V, int32_t k);
hipError_t run_topk_bwd(const Plan& p, const TopkBwdIO& io, hipStream_t stream);

// dst[i] = src[rows[i]] (gather) or dst[rows[i]] = src[i] (scatter), rows of
// row_bytes bytes; n_other = rows of the indexed array.
hipError_t run_copy_rows(const void* src, void* dst, const int32_t* rows, int64_t n_rows, int64_t n_other,
                         int64_t row_bytes, bool scatter, hipStream_t stream);
hipError_t run_topk(const Plan& p, const TopkIO& io, hipStream_t stream);

// Tail-bucket divergence over a top-k support (support bits KD_SUPPORT_*).
struct TailIO {
  const void *h_s, *W_s, *h_t, *W_t;
  int32_t k, support;
  float beta, tau;
  const int32_t* labels;
  int32_t* sup_idx;  // [N, smax]
  float *sup_t, *sup_s, *loss, *p_mass, *q_mass, *lse_s, *lse_t;
  void* workspace;
};
int32_t tail_support_slots(int32_t k, int32_t support);
size_t tail_workspace_bytes(const Plan& p, int32_t k);
hipError_t run_tail(const Plan& p, const TailIO& io, hipStream_t stream);

struct TailBwdIO {
  const void *h_s, *W_s;
  int32_t smax;
  float beta, tau;
  int32_t chunk_V;
  const int32_t* sup_idx;
  const float *sup_t, *sup_s, *lse_s, *lse_t, *grad;
  float* dh;
  void* workspace;
};
size_t tail_bwd_workspace_bytes(const Plan& p, int32_t chunk_V, int32_t k);
hipError_t run_tail_bwd(const Plan& p, const TailBwdIO& io, hipStream_t stream);

}  // namespace kd
