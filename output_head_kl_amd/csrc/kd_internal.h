// Internal interface between the C-ABI front end (kd_api.hip) and the gfx950
// kernels (kd_kernels.hip).  Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace kd {

// Output tile along tokens (and along everything in fp32): 256.
constexpr int kTile = 256;
// Rows of the A tile of the bf16 GEMMs (vocabulary entries, or hidden units in dh):
// 384, in two wave rows of 192; fp32 keeps 256 (two wave rows of 128).  The forward
// GEMM writes one (max, sum-exp) partial per wave row, i.e. per tile_rows / 2
// vocabulary entries.
constexpr int kTileA16 = 384;
inline int tile_rows(int dtype) { return dtype == 1 ? kTileA16 : kTile; }
// Tokens per dW GEMM launch (bf16): each launch adds its product into the fp32 dW, a
// read and a write of all of dW, so chunks are grouped up to this many tokens (and never
// more chunks than the batch has).  This is the default; a call whose workspace is
// smaller takes the largest group it holds, down to one chunk.
constexpr int kDwGroupTokens = 16384;

// Kernel classes for timing (kd_profile_*).
enum KClass {
  KC_VALIDATE = 0,
  KC_FWD_GEMM,     // logits GEMM + per-tile max / sum-exp
  KC_BUCKET,       // teacher hits sorted by output tile (for the fused gather)
  KC_COMBINE,      // logsumexp + per-token loss
  KC_BWD_GEMM,     // logits recomputed + dense dz
  KC_SCATTER,      // sparse teacher correction of dz
  KC_DH_GEMM,      // dh partials (split over the vocabulary)
  KC_DH_REDUCE,    // dh partials summed and rounded
  KC_DW_GEMM,      // dW accumulation
  KC_TRANSPOSE,    // W and h transposed for the dh and dW GEMMs
  KC_TOPK,         // teacher top-K cache producer
  KC_RESCALE,      // single-sweep backward: exp(z - max) rescaled into dz
  KC_MISC,         // fills, loss accumulation and finalisation
  KC_COUNT
};

// Workspace carve-up; every offset is a multiple of 256 bytes.
struct Layout {
  int64_t C;          // token rows per chunk (min(chunk, N))
  int64_t C_alloc;    // C rounded up to the tile
  int tv;             // tile_rows(dtype)
  int64_t V_pad;      // V rounded up to 256 and to tv (dz holds V_pad / 256 column blocks)
  int64_t d_pad;      // d rounded up to the tile (row pitch of the dh partials)
  int64_t n_lse;      // ceil(V / (tv / 2))
  int nsplit;         // vocabulary splits of the dh GEMM
  int64_t k_split;    // vocabulary rows per split (a multiple of 256)
  int64_t nkeys;      // buckets per chunk: V_pad / tv * C_alloc / 256
  int dw_group;       // chunks per dW GEMM (bf16): dzT and hT hold dw_group chunks side by
                      // side, so fp32 dW is read and written once per dw_group chunks
  size_t off_flags, off_acc, off_partials, off_lse, off_sM, off_s, off_rowterm, off_zg,
      off_dz, off_dhpart, off_bcount, off_bcursor, off_boff, off_bent, off_wt, off_idxloc,
      off_dzt, off_ht, total;
};

// dw_group_tokens caps the dW group (whole chunks, at least one; fp32 always uses one).
bool make_layout(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int dtype,
                 int64_t dw_group_tokens, Layout *L);

// --- launchers (all asynchronous on `s`; return hipSuccess or the launch error) ---
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_clock_stamp(unsigned long long *out, int groups, hipStream_t s);
hipError_t launch_validate(const int32_t *idx, const float *p, int64_t NK, int64_t V,
                           const uint8_t *mask, int64_t N, int *flags,
                           unsigned long long *count, hipStream_t s);
// Teacher hits of a chunk sorted by tv x 256 output tile of the logits GEMM: offsets
// [key..key+1) of entries (c % 256 | (v % tv) << 8 | k << 17), key = (v / tv) *
// ceil(rows / 256) + c / 256, for ntv = V_pad / tv vocabulary tiles.  counts must be
// zero on entry and are left zero.
hipError_t launch_buckets(const int32_t *idx_c, int64_t rows, int32_t K, int tv, int ntv,
                          int *counts, int *cursor, int *offsets, unsigned *entries,
                          hipStream_t s);
// Logits GEMM with the per-tile (max, sum exp) epilogue and the fused gather into zg;
// with u non-null it also writes u = exp(z - max of the token's 128-row group) into the
// dz buffer (rows v < V_pad, tokens c < rows) for launch_rescale_dz.
hipError_t launch_fwd_gemm(int dtype, const void *W, const void *h_c, int64_t rows,
                           int64_t d, int64_t V, float2 *partials, int64_t ld_part,
                           const int *boff, const unsigned *bent, float *zg, int32_t K,
                           void *u, int64_t V_pad, int64_t C_alloc, hipStream_t s);
// Token-blocked layout of the dW GEMM's operands (bf16): element (r, c) of a matrix with
// R rows over the tokens of a dW group at X[(c / 256) * tst + r * 256 + c % 256], with
// tst = R * 256 (R = V_pad for dzT, d for hT).  Pointers passed per chunk point at the
// chunk's first token block.
//
// dz = sM * exp(m_g - lse) * u in place (and dzT for bf16), from the forward's partials.
hipError_t launch_rescale_dz(int dtype, void *dz, void *dzt, int64_t tst, const float2 *partials,
                             const float *lse, const float *sM, int64_t rows, int64_t V,
                             int64_t V_pad, int64_t C_alloc, hipStream_t s);
hipError_t launch_combine(const float2 *partials, int64_t n_lse, int64_t ld_part,
                          const float *zg, const float *p_c, const uint8_t *mask_c,
                          int64_t rows, int32_t K, const float *inv_count, float *lse, float *sM,
                          float *srow, double *rowterm, float *row_loss, float *row_lse,
                          hipStream_t s);
// Backward-only path: sM = g*mask*M/count, s = g*mask/count per token (g on the device).
hipError_t launch_row_scale(const float *p_c, const uint8_t *mask_c, int64_t rows, int32_t K,
                            const float *inv_count, const float *g, float *sM, float *srow,
                            hipStream_t s);
hipError_t launch_accum_loss(const double *rowterm, int64_t rows, double *acc, hipStream_t s);
hipError_t launch_finalize(const double *acc, const unsigned long long *count, float *loss,
                           hipStream_t s);
// count[0] = the mask's count (or N without a mask), inv_count[0] = 1 / count (0 for none)
hipError_t launch_count_prep(const unsigned long long *mask_count, bool has_mask, int64_t N,
                             unsigned long long *count, float *inv_count, hipStream_t s);
// status[0] = bad_code when flags[0] is raised, else 0
hipError_t launch_status_out(const int *flags, int32_t bad_code, int32_t *status, hipStream_t s);
// dh_out = g[0] * dh32 rounded once to dtype (bf16 RNE or fp32), dW *= g[0] in place (dW
// untouched when g[0] == 1); dh32 and dW 16-byte aligned.
hipError_t launch_scale_grads(int dtype, const float *g, const float *dh32, void *dh_out,
                              int64_t n_dh, float *dW, int64_t n_dW, hipStream_t s);
// dz is stored as blocks of 256 vocabulary columns: element (c, v) at
// dz[(v / 256) * C_alloc * 256 + c * 256 + v % 256].
// bf16 also writes dzT, the same values in the token-blocked layout (tst = V_pad * 256)
// for v < V_pad, c < C_alloc (zero for c >= rows).
hipError_t launch_bwd_gemm(int dtype, const void *W, const void *h_c, int64_t rows, int64_t d,
                           int64_t V, const float *lse, const float *sM, void *dz, void *dzt,
                           int64_t tst, int64_t V_pad, int64_t C_alloc, hipStream_t s);
hipError_t launch_scatter(int dtype, void *dz, void *dzt, int64_t tst, int64_t C_alloc,
                          const int32_t *idx_c, const float *p_c, const float *srow, int64_t rows,
                          int32_t K, int64_t V_pad, hipStream_t s);
// h chunk [rows][d] bf16 -> hT in the token-blocked layout (tst = d * 256), columns
// c < C_alloc (zero for c >= rows).
hipError_t launch_transpose_h(const void *h_c, int64_t rows, int64_t d, int64_t C_alloc,
                              void *ht, int64_t tst, hipStream_t s);
// W^T in blocks of 256 vocabulary entries (bf16 only): element (v, j) of W at
// WT[(v / 256) * d * 256 + j * 256 + v % 256], zero for V <= v < V_pad.
hipError_t launch_transpose_w(const void *W, int64_t V, int64_t d, int64_t V_pad, void *WT,
                              hipStream_t s);
// dh partials; bf16 reads W through WT (above), fp32 reads W itself.
hipError_t launch_dh_gemm(int dtype, const void *dz, const void *W, const void *WT, int64_t rows,
                          int64_t d, int64_t V, int64_t V_pad, int nsplit, int64_t k_split,
                          float *part, int64_t d_pad, int64_t C_alloc, hipStream_t s);
hipError_t launch_dh_reduce(int dtype, const float *part, int nsplit, int64_t C_alloc,
                            int64_t d_pad, int64_t rows, int64_t d, void *dh, hipStream_t s);
// dW (+)= dz^T h over k tokens: bf16 reads dzT and hT (token-blocked, k tokens of the
// group), fp32 reads one chunk's dz (k = rows) and h.
hipError_t launch_dw_gemm(int dtype, const void *dz, const void *dzt, const void *h_c,
                          const void *ht, int64_t k, int64_t d, int64_t V,
                          int64_t V_pad, int64_t C_alloc, float *dW, int accumulate,
                          hipStream_t s);

// --- vocabulary shards ---
// loc = idx - v0 inside [v0, v0 + Vs), else -1 (skipped by buckets and scatter); zg of
// the outside entries is set to 0.
hipError_t launch_localize_idx(const int32_t *idx_c, int64_t rows, int32_t K, int64_t v0,
                               int64_t Vs, int32_t *loc, float *zg_c, hipStream_t s);
// Per token of a shard: max, sum exp(z - max) and sum_k p*z (inside the shard).
hipError_t launch_shard_stats(const float2 *partials, int64_t n_lse, int64_t ld_part,
                              const float *zg, const float *p_c, int64_t rows, int32_t K,
                              float *m_out, float *s_out, float *pz_out, hipStream_t s);
// Global logsumexp and per-token loss term from G shards' statistics ([G][N] each).
hipError_t launch_shard_combine(const float *m, const float *sx, const float *pz, int G,
                                int64_t N, const float *p, const uint8_t *mask, int32_t K,
                                float *row_lse, float *row_loss, double *rowterm, hipStream_t s);

// --- teacher top-K cache producer (kd_topk.hip) ---
constexpr int kTopkMaxK = 256;
// Workspace of kd_teacher_topk, and the size of the module scratch that replaces it in
// kd_teacher_topk_noalloc: one validity flag (int), padded to 256 bytes.
constexpr size_t kTopkScratchBytes = 256;
// The current device's copy of the module scratch (kTopkScratchBytes), looked up once per
// device with hipGetSymbolAddress; allocates nothing.
hipError_t topk_scratch(int **out);
// One workgroup per row; flags[0] |= 1 for a row with a NaN or +inf logit or with no
// finite logit.  lse may be null.
hipError_t launch_teacher_topk(int dtype, const void *logits, int64_t N, int64_t V, int32_t K,
                               int32_t *idx, float *p, float *lse, int *flags, hipStream_t s);

// --- timing hooks (kd_api.hip) ---
void prof_begin(int cls, hipStream_t s);
void prof_end(int cls, hipStream_t s);

}  // namespace kd
