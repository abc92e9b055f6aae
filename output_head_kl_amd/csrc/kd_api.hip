// C-ABI front end of the fused, chunked top-K KL loss (declared in include/kdkl.h).
//
// Host-side argument checks run before any HIP call, so a bad call never touches
// the device.  The call then validates the teacher entries and counts the loss mask
// on the device, synchronises the stream once to read the result, and enqueues the
// per-chunk sequence: forward GEMM (per-tile max / sum-exp), gather at the teacher's
// indices, logsumexp + loss, dz, sparse correction of dz, dh GEMM + reduction, dW GEMM.
// The fused call takes dz from the exp(z - max) its forward GEMM kept in the dz buffer
// (one streaming rescale once the logsumexp is known); the backward-only call recomputes
// the logits with a second GEMM.  One chunk's dz is live, plus its token-contiguous copy
// for the chunks of one dW group (as many as the workspace passed holds, 16384 tokens at
// most; one chunk with the smallest workspace).
#include "kd_internal.h"
#include "kdkl.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

inline int64_t rup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// --- timing ---------------------------------------------------------------------
struct Prof {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[kd::KC_COUNT];
  hipEvent_t pending[kd::KC_COUNT] = {};
  // Events are reused rather than created per launch: creating two per launch kept the
  // host busy between launches and let the GPU idle (the profiled pass ran slower).
  std::vector<hipEvent_t> spare;
  hipEvent_t take() {
    hipEvent_t e = nullptr;
    if (!spare.empty()) {
      e = spare.back();
      spare.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
    }
    return e;
  }
};
Prof g_prof;
std::mutex g_prof_mu;

const char *const kClassNames[kd::KC_COUNT] = {
    "validate", "fwd_gemm_lse", "bucket", "combine_lse_loss", "bwd_gemm_dz",
    "scatter",  "dh_gemm",      "dh_reduce", "dw_gemm",      "transpose", "teacher_topk", "dz_rescale", "misc"};

#define HIPCHK(expr)                                                                 \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess)                                                            \
      return fail(KD_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));          \
  } while (0)

#define LAUNCH(cls, expr)                                                            \
  do {                                                                               \
    kd::prof_begin(cls, stream);                                                     \
    hipError_t e_ = (expr);                                                          \
    kd::prof_end(cls, stream);                                                       \
    if (e_ != hipSuccess)                                                            \
      return fail(KD_E_HIP, "launch %s failed: %s", #expr, hipGetErrorString(e_));   \
  } while (0)

int check_sizes(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int32_t dtype) {
  if (dtype != KD_F32 && dtype != KD_BF16) return fail(KD_E_ARG, "dtype %d unknown", dtype);
  if (N < 0) return fail(KD_E_ARG, "N = %lld < 0", (long long)N);
  if (d < 1 || V < 1 || K < 1) return fail(KD_E_ARG, "d, V and K must be >= 1");
  if (chunk < 1) return fail(KD_E_ARG, "chunk = %lld < 1", (long long)chunk);
  if (K > 32768) return fail(KD_E_UNSUPPORTED, "K = %d above 32768", K);
  if (d % 8 != 0) return fail(KD_E_UNSUPPORTED, "d = %lld is not a multiple of 8", (long long)d);
  if (d > (1 << 20) || V > ((int64_t)1 << 24))
    return fail(KD_E_UNSUPPORTED, "d or V too large");
  const int64_t lim = (int64_t)1 << 62;
  if (N > 0 && (N > lim / d || N > lim / K)) return fail(KD_E_ARG, "N too large");
  if (V > lim / d) return fail(KD_E_ARG, "V*d too large");
  // Token offsets inside a chunk (c * 256 in the token-blocked layouts) and the chunk's
  // teacher-hit count (rows * K bucket entries) are 32-bit in the kernels.
  const int64_t rows = chunk < (N > 0 ? N : 1) ? chunk : (N > 0 ? N : 1);
  if (rows > ((int64_t)1 << 22) || rows * K > (int64_t)0x7FFFFFFF)
    return fail(KD_E_UNSUPPORTED,
                "min(chunk, N) = %lld rows per chunk: at most 2^22 rows and 2^31 - 1 teacher "
                "entries per chunk", (long long)rows);
  return KD_OK;
}

}  // namespace

namespace kd {

void prof_begin(int cls, hipStream_t s) {
  if (!g_prof.on) return;
  hipEvent_t a = g_prof.take();
  if (!a) return;
  (void)hipEventRecord(a, s);
  g_prof.pending[cls] = a;
}

void prof_end(int cls, hipStream_t s) {
  if (!g_prof.on || !g_prof.pending[cls]) return;
  hipEvent_t b = g_prof.take();
  if (!b) return;
  (void)hipEventRecord(b, s);
  g_prof.ev[cls].emplace_back(g_prof.pending[cls], b);
  g_prof.pending[cls] = nullptr;
}

bool make_layout(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int dtype,
                 int64_t dw_group_tokens, Layout *L) {
  const int64_t es = dtype == KD_BF16 ? 2 : 4;
  const int64_t Nn = N > 0 ? N : 1;
  L->C = chunk < Nn ? chunk : Nn;
  L->C_alloc = rup(L->C, kTile);
  L->tv = tile_rows(dtype);
  L->V_pad = rup(V, L->tv == kTile ? kTile : 3 * kTile);  // a multiple of 256 and of tv
  L->d_pad = rup(d, kTile);
  L->n_lse = (V + L->tv / 2 - 1) / (L->tv / 2);
  // Split the vocabulary of the dh GEMM so that its workgroups fill whole rounds of the
  // slots that run at once (one workgroup per CU in bf16, three in fp32).  Within one
  // round more splits are more parallel work; past it, a larger split count must fill
  // its rounds 5 % better than the best smaller one, as each split adds a float32
  // partial of dh to reduce.
  const int64_t tiles = ((d + L->tv - 1) / L->tv) * (L->C_alloc / kTile);
  const int64_t slots = dtype == KD_BF16 ? 256 : 768;
  const int64_t max_by_k = L->V_pad / kTile;  // at least one dz column block per split
  int64_t ns = 1;
  double best = 0.0;
  for (int64_t c = 1; c <= 16 && c <= max_by_k; ++c) {
    const int64_t wgs = tiles * c, rounds = (wgs + slots - 1) / slots;
    const double fill = (double)wgs / (double)(rounds * slots);
    if ((rounds == 1 && fill > best) || fill > best + 0.05) {
      best = fill;
      ns = c;
    }
  }
  L->k_split = rup((L->V_pad + ns - 1) / ns, kTile);  // splits start on a dz column block
  L->nsplit = (int)((L->V_pad + L->k_split - 1) / L->k_split);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (size_t)rup((int64_t)bytes, 256);
    return o;
  };
  L->off_flags = take(64);
  L->off_acc = take(64);
  L->off_partials = take((size_t)L->n_lse * L->C_alloc * sizeof(float2));
  L->off_lse = take((size_t)L->C_alloc * 4);
  L->off_sM = take((size_t)L->C_alloc * 4);
  L->off_s = take((size_t)L->C_alloc * 4);
  L->off_rowterm = take((size_t)L->C_alloc * 8);
  L->off_zg = take((size_t)L->C_alloc * K * 4);
  L->off_dz = take((size_t)L->C_alloc * L->V_pad * es);
  L->off_dhpart = take((size_t)L->nsplit * L->C_alloc * L->d_pad * 4);
  L->nkeys = L->V_pad / L->tv * (L->C_alloc / kTile);
  L->off_bcount = take((size_t)L->nkeys * 4);
  L->off_bcursor = take((size_t)L->nkeys * 4);
  L->off_boff = take((size_t)(L->nkeys + 1) * 4);
  L->off_bent = take((size_t)L->C_alloc * K * 4);
  L->off_wt = take(dtype == KD_BF16 ? (size_t)L->V_pad * d * 2 : 0);
  L->off_idxloc = take((size_t)L->C_alloc * K * 4);
  {
    const int64_t nchunks = (Nn + L->C - 1) / L->C;
    int64_t g = dtype == KD_BF16 ? dw_group_tokens / L->C_alloc : 1;
    if (g > nchunks) g = nchunks;
    L->dw_group = (int)(g < 1 ? 1 : g);
  }
  L->off_dzt = take(dtype == KD_BF16 ? (size_t)L->V_pad * L->dw_group * L->C_alloc * 2 : 0);
  L->off_ht = take(dtype == KD_BF16 ? (size_t)d * L->dw_group * L->C_alloc * 2 : 0);
  L->total = off;
  return true;
}

}  // namespace kd

extern "C" {

int kd_version(void) { return 5; }

const char *kd_last_error(void) { return g_err; }

int kd_workspace_bytes_group(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk,
                             int32_t dtype, int64_t dw_group_tokens, size_t *bytes_out) {
  g_err[0] = 0;
  if (!bytes_out) return fail(KD_E_ARG, "bytes_out is NULL");
  int rc = check_sizes(N, d, V, K, chunk, dtype);
  if (rc != KD_OK) return rc;
  if (dw_group_tokens < 0) return fail(KD_E_ARG, "dw_group_tokens is negative");
  if (dw_group_tokens > kd::kDwGroupTokens) dw_group_tokens = kd::kDwGroupTokens;
  kd::Layout L;
  kd::make_layout(N, d, V, K, chunk, dtype, dw_group_tokens, &L);
  *bytes_out = L.total;
  return KD_OK;
}

int kd_workspace_bytes(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int32_t dtype,
                       size_t *bytes_out) {
  return kd_workspace_bytes_group(N, d, V, K, chunk, dtype, kd::kDwGroupTokens, bytes_out);
}

}  // extern "C"

namespace {

// The three entry points share one routine.  FUSED: loss, dh, dW.  FWD: loss and the
// per-token logsumexp (saved for BWD).  BWD: dh and dW from the saved logsumexp and an
// upstream gradient g of the loss, with the logits recomputed chunk by chunk.
// Vocabulary shards (one GPU's share of a tensor-parallel head, W = rows [v0, v0+V) of a
// V_total vocabulary): SFWD exports per-token (max, sum exp, sum p*z) of the shard;
// SBWD writes the shard's float32 dh partial and its dW rows, given the global lse.
enum Mode { M_FUSED, M_FWD, M_BWD, M_SFWD, M_SBWD };

struct ShardArgs {
  int64_t v0 = 0, V_total = 0;
  float *st_m = nullptr, *st_s = nullptr, *st_pz = nullptr;
};

int run(Mode mode, const void *h, const void *W, int32_t dtype, const int32_t *topk_idx,
        const float *topk_p, const uint8_t *loss_mask, int64_t N, int64_t d, int64_t V, int32_t K,
        int64_t chunk, float *loss, void *dh, float *dW, float *row_loss, float *row_lse,
        float *zg, const float *lse_in, const float *grad_loss, void *workspace,
        size_t workspace_bytes, void *stream_v, const ShardArgs &sh = ShardArgs(),
        bool dh_f32 = false, int32_t *status = nullptr) {
  g_err[0] = 0;
  // status given: the one-call form without its host synchronisation (validity reported
  // on the device through *status, the count used on the device only)
  const bool async = status != nullptr;
  int rc = check_sizes(N, d, V, K, chunk, dtype);
  if (rc != KD_OK) return rc;
  const bool shard = mode == M_SFWD || mode == M_SBWD;
  const bool fwd = mode == M_FUSED || mode == M_FWD || mode == M_SFWD;
  const bool bwd = mode == M_FUSED || mode == M_BWD || mode == M_SBWD;
  const int64_t V_idx = shard ? sh.V_total : V;  // range of the teacher indices
  if (shard) {
    if (sh.v0 < 0 || sh.V_total < V || sh.v0 > sh.V_total - V || sh.V_total > ((int64_t)1 << 24))
      return fail(KD_E_ARG, "shard [%lld, %lld) does not lie in a vocabulary of %lld",
                  (long long)sh.v0, (long long)(sh.v0 + V), (long long)sh.V_total);
    if (mode == M_SFWD && N > 0 && (!sh.st_m || !sh.st_s || !sh.st_pz))
      return fail(KD_E_ARG, "shard statistics outputs are required");
  }
  if (!W || !workspace) return fail(KD_E_ARG, "W and workspace are required");
  if (fwd && !shard && !loss) return fail(KD_E_ARG, "loss is required");
  if (bwd && !dW) return fail(KD_E_ARG, "dW is required");
  if ((mode == M_BWD || mode == M_SBWD) && !grad_loss)
    return fail(KD_E_ARG, "grad_loss is required");
  if (N > 0 && (!h || !topk_idx || !topk_p))
    return fail(KD_E_ARG, "h, topk_idx and topk_p are required when N > 0");
  if (N > 0 && bwd && !dh) return fail(KD_E_ARG, "dh is required when N > 0");
  if (N > 0 && mode == M_FWD && !row_lse)
    return fail(KD_E_ARG, "row_lse is required (it is the state the backward call reads)");
  if (N > 0 && (mode == M_BWD || mode == M_SBWD) && !lse_in)
    return fail(KD_E_ARG, "row_lse is required when N > 0");
  auto mis = [](const void *p, uintptr_t a) { return p && ((uintptr_t)p % a) != 0; };
  if (mis(h, 16) || mis(W, 16) || mis(dh, 16) || mis(dW, 16))
    return fail(KD_E_ARG, "h, W, dh and dW must be 16-byte aligned");
  if (mis(topk_idx, 4) || mis(topk_p, 4) || mis(loss, 4) || mis(row_loss, 4) ||
      mis(row_lse, 4) || mis(zg, 4) || mis(lse_in, 4) || mis(grad_loss, 4))
    return fail(KD_E_ARG, "index, probability and float arguments must be 4-byte aligned");
  if (mis(workspace, 256)) return fail(KD_E_ARG, "workspace must be 256-byte aligned");
  // The dW group is the largest (up to kDwGroupTokens tokens) whose copies fit.
  kd::Layout L;
  kd::make_layout(N, d, V, K, chunk, dtype, kd::kDwGroupTokens, &L);
  while (workspace_bytes < L.total && L.dw_group > 1)
    kd::make_layout(N, d, V, K, chunk, dtype, (int64_t)(L.dw_group - 1) * L.C_alloc, &L);
  if (workspace_bytes < L.total)
    return fail(KD_E_WORKSPACE, "workspace has %zu bytes, needs at least %zu", workspace_bytes,
                L.total);

  hipStream_t stream = (hipStream_t)stream_v;
  char *ws = (char *)workspace;
  int *flags = (int *)(ws + L.off_flags);
  unsigned long long *dcount = (unsigned long long *)(ws + L.off_flags + 8);
  unsigned long long *dcount_eff = (unsigned long long *)(ws + L.off_flags + 16);
  float *dinv = (float *)(ws + L.off_flags + 24);
  double *acc = (double *)(ws + L.off_acc);
  float2 *partials = (float2 *)(ws + L.off_partials);
  float *lse = (float *)(ws + L.off_lse);
  float *sM = (float *)(ws + L.off_sM);
  float *srow = (float *)(ws + L.off_s);
  double *rowterm = (double *)(ws + L.off_rowterm);
  float *zg_ws = (float *)(ws + L.off_zg);
  void *dz = ws + L.off_dz;
  void *dzt = dtype == KD_BF16 ? (void *)(ws + L.off_dzt) : nullptr;
  void *ht = dtype == KD_BF16 ? (void *)(ws + L.off_ht) : nullptr;
  float *dhpart = (float *)(ws + L.off_dhpart);
  int *bcount = (int *)(ws + L.off_bcount);
  int *bcursor = (int *)(ws + L.off_bcursor);
  int *boff = (int *)(ws + L.off_boff);
  unsigned *bent = (unsigned *)(ws + L.off_bent);
  int32_t *idxloc = (int32_t *)(ws + L.off_idxloc);
  const int64_t es = dtype == KD_BF16 ? 2 : 4;
  // a shard's dh partial, and dh for an upstream gradient applied later, stay float32
  const int64_t es_dh = (mode == M_SBWD || dh_f32) ? 4 : es;

  if (N == 0) {
    if (fwd && !shard) LAUNCH(kd::KC_MISC, kd::launch_fill_zero(loss, 4, stream));
    if (bwd) LAUNCH(kd::KC_MISC, kd::launch_fill_zero(dW, (size_t)V * d * 4, stream));
    if (async) LAUNCH(kd::KC_MISC, kd::launch_fill_zero(status, 4, stream));
    return KD_OK;
  }

  // Validate the teacher entries and count the mask; the count and its reciprocal stay on
  // the device for the kernels that scale by them.  The synchronising form reads the
  // result back here (its only host synchronisation); the asynchronous one does not, and
  // runs the whole sequence whatever it finds (kernels skip indices outside the padded
  // vocabulary, and a count of zero scales every gradient to zero).
  LAUNCH(kd::KC_MISC, kd::launch_fill_zero(ws + L.off_flags, L.off_acc - L.off_flags + 64, stream));
  LAUNCH(kd::KC_VALIDATE,
         kd::launch_validate(topk_idx, topk_p, N * (int64_t)K, V_idx, loss_mask, N, flags, dcount,
                             stream));
  LAUNCH(kd::KC_MISC, kd::launch_count_prep(dcount, loss_mask != nullptr, N, dcount_eff, dinv,
                                            stream));
  int64_t count = -1;  // unknown on the host in the asynchronous form
  if (!async) {
    struct {
      int flags[2];
      unsigned long long count;
    } hostv;
    HIPCHK(hipMemcpyAsync(&hostv, flags, sizeof hostv, hipMemcpyDeviceToHost, stream));
    HIPCHK(hipStreamSynchronize(stream));
    if (hostv.flags[0])
      return fail(KD_E_INDEX,
                  "a teacher index is outside [0, %lld) or a probability is negative or not finite",
                  (long long)V_idx);
    count = loss_mask ? (int64_t)hostv.count : N;
  }
  const bool want_rows = row_loss || row_lse || zg;

  if (count == 0) {
    if (fwd && !shard) LAUNCH(kd::KC_MISC, kd::launch_fill_zero(loss, 4, stream));
    if (bwd) {
      LAUNCH(kd::KC_MISC, kd::launch_fill_zero(dW, (size_t)V * d * 4, stream));
      LAUNCH(kd::KC_MISC, kd::launch_fill_zero(dh, (size_t)N * d * es_dh, stream));
    }
    if (!fwd || !(want_rows || mode == M_SFWD)) return KD_OK;
  }
  const bool backward = bwd && count != 0;
  if (fwd) LAUNCH(kd::KC_MISC, kd::launch_fill_zero(bcount, (size_t)L.nkeys * 4, stream));
  void *WT = ws + L.off_wt;
  if (backward && dtype == KD_BF16)
    LAUNCH(kd::KC_TRANSPOSE, kd::launch_transpose_w(W, V, d, L.V_pad, WT, stream));

  int chunk_i = 0, dw_launches = 0;
  for (int64_t c0 = 0; c0 < N; c0 += L.C, ++chunk_i) {
    const int64_t rows = (N - c0) < L.C ? (N - c0) : L.C;
    const char *h_c = (const char *)h + c0 * d * es;
    const int32_t *idx_c = topk_idx + c0 * K;
    const float *p_c = topk_p + c0 * K;
    const uint8_t *mask_c = loss_mask ? loss_mask + c0 : nullptr;
    float *zg_c = zg ? zg + c0 * K : zg_ws;
    const float *lse_c = lse;
    const int32_t *idx_k = idx_c;  // indices as the kernels see them (shard-local in a shard)
    if (shard) {
      LAUNCH(kd::KC_BUCKET,
             kd::launch_localize_idx(idx_c, rows, K, sh.v0, V, idxloc, zg_c, stream));
      idx_k = idxloc;
    }

    if (fwd) {
      LAUNCH(kd::KC_BUCKET,
             kd::launch_buckets(idx_k, rows, K, L.tv, (int)(L.V_pad / L.tv), bcount, bcursor,
                                boff, bent, stream));
      // the fused call keeps this chunk's exp(z - max) for its backward (no recompute)
      void *u = (mode == M_FUSED && count != 0) ? dz : nullptr;
      LAUNCH(kd::KC_FWD_GEMM, kd::launch_fwd_gemm(dtype, W, h_c, rows, d, V, partials, L.C_alloc,
                                                  boff, bent, zg_c, K, u, L.V_pad, L.C_alloc,
                                                  stream));
      if (mode == M_SFWD) {
        LAUNCH(kd::KC_COMBINE,
               kd::launch_shard_stats(partials, L.n_lse, L.C_alloc, zg_c, p_c, rows, K,
                                      sh.st_m + c0, sh.st_s + c0, sh.st_pz + c0, stream));
        continue;
      }
      LAUNCH(kd::KC_COMBINE,
             kd::launch_combine(partials, L.n_lse, L.C_alloc, zg_c, p_c, mask_c, rows, K, dinv,
                                lse, sM, srow, rowterm, row_loss ? row_loss + c0 : nullptr,
                                row_lse ? row_lse + c0 : nullptr, stream));
      if (count == 0) continue;  // forward-only sweep for the per-row outputs
      LAUNCH(kd::KC_MISC, kd::launch_accum_loss(rowterm, rows, acc, stream));
    } else {
      lse_c = lse_in + c0;
      LAUNCH(kd::KC_COMBINE, kd::launch_row_scale(p_c, mask_c, rows, K, dinv, grad_loss, sM,
                                                  srow, stream));
    }
    if (!backward) continue;
    // This chunk's columns in the token-contiguous dW operands (dw_group chunks side by
    // side; fp32 has none and multiplies each chunk's dz directly).
    const int slot = chunk_i % L.dw_group;
    // (token-blocked: the slot starts at token block slot * C_alloc / 256)
    const int64_t tst_dz = L.V_pad * 256, tst_h = d * 256;
    void *dzt_c = dzt ? (void *)((char *)dzt + (size_t)slot * L.C_alloc * L.V_pad * 2) : nullptr;
    void *ht_c = ht ? (void *)((char *)ht + (size_t)slot * L.C_alloc * d * 2) : nullptr;
    if (mode == M_FUSED)
      LAUNCH(kd::KC_RESCALE, kd::launch_rescale_dz(dtype, dz, dzt_c, tst_dz, partials, lse_c, sM, rows,
                                                   V, L.V_pad, L.C_alloc, stream));
    else
      LAUNCH(kd::KC_BWD_GEMM, kd::launch_bwd_gemm(dtype, W, h_c, rows, d, V, lse_c, sM, dz, dzt_c,
                                                  tst_dz, L.V_pad, L.C_alloc, stream));
    LAUNCH(kd::KC_SCATTER, kd::launch_scatter(dtype, dz, dzt_c, tst_dz, L.C_alloc, idx_k, p_c, srow,
                                              rows, K, L.V_pad, stream));
    LAUNCH(kd::KC_DH_GEMM, kd::launch_dh_gemm(dtype, dz, W, WT, rows, d, V, L.V_pad, L.nsplit,
                                              L.k_split, dhpart, L.d_pad, L.C_alloc, stream));
    LAUNCH(kd::KC_DH_REDUCE,
           kd::launch_dh_reduce(es_dh == 4 ? (int)KD_F32 : dtype, dhpart, L.nsplit, L.C_alloc,
                                L.d_pad, rows, d, (char *)dh + c0 * d * es_dh, stream));
    if (ht_c)
      LAUNCH(kd::KC_TRANSPOSE,
             kd::launch_transpose_h(h_c, rows, d, L.C_alloc, ht_c, tst_h, stream));
    if (slot == L.dw_group - 1 || c0 + rows >= N) {
      // every earlier chunk of the group is whole: its columns past C are zero
      const int64_t k = (int64_t)slot * L.C_alloc + rows;
      LAUNCH(kd::KC_DW_GEMM, kd::launch_dw_gemm(dtype, dz, dzt, h_c, ht, k, d, V, L.V_pad,
                                                L.C_alloc, dW, dw_launches > 0, stream));
      ++dw_launches;
    }
  }
  if (fwd && !shard && count != 0)
    LAUNCH(kd::KC_MISC, kd::launch_finalize(acc, dcount_eff, loss, stream));
  if (async) LAUNCH(kd::KC_MISC, kd::launch_status_out(flags, KD_E_INDEX, status, stream));
  return KD_OK;
}

}  // namespace

extern "C" {

int kd_chunked_kl_fwd_bwd(const void *h, const void *W, int32_t dtype, const int32_t *topk_idx,
                          const float *topk_p, const uint8_t *loss_mask, int64_t N, int64_t d,
                          int64_t V, int32_t K, int64_t chunk, float *loss, void *dh, float *dW,
                          float *row_loss, float *row_lse, float *zg, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return run(M_FUSED, h, W, dtype, topk_idx, topk_p, loss_mask, N, d, V, K, chunk, loss, dh, dW,
             row_loss, row_lse, zg, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int kd_chunked_kl_fwd_bwd_async(const void *h, const void *W, int32_t dtype,
                                const int32_t *topk_idx, const float *topk_p,
                                const uint8_t *loss_mask, int64_t N, int64_t d, int64_t V,
                                int32_t K, int64_t chunk, float *loss, void *dh, float *dW,
                                float *row_loss, float *row_lse, float *zg, int32_t *status,
                                void *workspace, size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  if (!status) return fail(KD_E_ARG, "status is required");
  if ((uintptr_t)status % 4) return fail(KD_E_ARG, "status must be 4-byte aligned");
  return run(M_FUSED, h, W, dtype, topk_idx, topk_p, loss_mask, N, d, V, K, chunk, loss, dh, dW,
             row_loss, row_lse, zg, nullptr, nullptr, workspace, workspace_bytes, stream,
             ShardArgs(), false, status);
}

int kd_chunked_kl_fwd_bwd_f32dh(const void *h, const void *W, int32_t dtype,
                                const int32_t *topk_idx, const float *topk_p,
                                const uint8_t *loss_mask, int64_t N, int64_t d, int64_t V,
                                int32_t K, int64_t chunk, float *loss, float *dh, float *dW,
                                float *row_loss, float *row_lse, float *zg, void *workspace,
                                size_t workspace_bytes, void *stream) {
  return run(M_FUSED, h, W, dtype, topk_idx, topk_p, loss_mask, N, d, V, K, chunk, loss, dh, dW,
             row_loss, row_lse, zg, nullptr, nullptr, workspace, workspace_bytes, stream,
             ShardArgs(), true);
}

int kd_scale_grads(const float *grad_loss, const float *dh_f32, void *dh, int32_t dtype,
                   int64_t N, int64_t d, float *dW, int64_t V, void *stream_v) {
  g_err[0] = 0;
  if (dtype != KD_F32 && dtype != KD_BF16) return fail(KD_E_ARG, "dtype %d unknown", dtype);
  if (N < 0 || d < 1 || V < 0) return fail(KD_E_ARG, "need N >= 0, d >= 1, V >= 0");
  const int64_t lim = (int64_t)1 << 62;
  if (N > lim / d || V > lim / d) return fail(KD_E_ARG, "N*d or V*d too large");
  if (!grad_loss) return fail(KD_E_ARG, "grad_loss is required");
  if (N > 0 && (!dh_f32 || !dh)) return fail(KD_E_ARG, "dh_f32 and dh are required when N > 0");
  if (V > 0 && !dW) return fail(KD_E_ARG, "dW is required when V > 0");
  auto mis = [](const void *p, uintptr_t a) { return p && ((uintptr_t)p % a) != 0; };
  if (mis(dh_f32, 16) || mis(dh, 16) || mis(dW, 16))
    return fail(KD_E_ARG, "dh_f32, dh and dW must be 16-byte aligned");
  if (mis(grad_loss, 4)) return fail(KD_E_ARG, "grad_loss must be 4-byte aligned");
  if (N * d + V * d == 0) return KD_OK;
  hipStream_t stream = (hipStream_t)stream_v;
  LAUNCH(kd::KC_MISC, kd::launch_scale_grads(dtype, grad_loss, dh_f32, dh, N * d, dW, V * d,
                                             stream));
  return KD_OK;
}

int kd_chunked_kl_fwd(const void *h, const void *W, int32_t dtype, const int32_t *topk_idx,
                      const float *topk_p, const uint8_t *loss_mask, int64_t N, int64_t d,
                      int64_t V, int32_t K, int64_t chunk, float *loss, float *row_lse,
                      float *row_loss, float *zg, void *workspace, size_t workspace_bytes,
                      void *stream) {
  return run(M_FWD, h, W, dtype, topk_idx, topk_p, loss_mask, N, d, V, K, chunk, loss, nullptr,
             nullptr, row_loss, row_lse, zg, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int kd_chunked_kl_bwd(const void *h, const void *W, int32_t dtype, const int32_t *topk_idx,
                      const float *topk_p, const uint8_t *loss_mask, int64_t N, int64_t d,
                      int64_t V, int32_t K, int64_t chunk, const float *row_lse,
                      const float *grad_loss, void *dh, float *dW, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return run(M_BWD, h, W, dtype, topk_idx, topk_p, loss_mask, N, d, V, K, chunk, nullptr, dh, dW,
             nullptr, nullptr, nullptr, row_lse, grad_loss, workspace, workspace_bytes, stream);
}

int kd_vocab_shard_fwd(const void *h, const void *W_shard, int32_t dtype, const int32_t *topk_idx,
                       const float *topk_p, int64_t N, int64_t d, int64_t V_shard,
                       int64_t v_offset, int64_t V_total, int32_t K, int64_t chunk,
                       float *shard_max, float *shard_sumexp, float *shard_pz, float *zg,
                       void *workspace, size_t workspace_bytes, void *stream) {
  ShardArgs sh;
  sh.v0 = v_offset;
  sh.V_total = V_total;
  sh.st_m = shard_max;
  sh.st_s = shard_sumexp;
  sh.st_pz = shard_pz;
  return run(M_SFWD, h, W_shard, dtype, topk_idx, topk_p, nullptr, N, d, V_shard, K, chunk,
             nullptr, nullptr, nullptr, nullptr, nullptr, zg, nullptr, nullptr, workspace,
             workspace_bytes, stream, sh);
}

int kd_vocab_shard_bwd(const void *h, const void *W_shard, int32_t dtype, const int32_t *topk_idx,
                       const float *topk_p, const uint8_t *loss_mask, int64_t N, int64_t d,
                       int64_t V_shard, int64_t v_offset, int64_t V_total, int32_t K,
                       int64_t chunk, const float *row_lse, const float *grad_loss,
                       float *dh_partial, float *dW_shard, void *workspace,
                       size_t workspace_bytes, void *stream) {
  ShardArgs sh;
  sh.v0 = v_offset;
  sh.V_total = V_total;
  return run(M_SBWD, h, W_shard, dtype, topk_idx, topk_p, loss_mask, N, d, V_shard, K, chunk,
             nullptr, dh_partial, dW_shard, nullptr, nullptr, nullptr, row_lse, grad_loss,
             workspace, workspace_bytes, stream, sh);
}

int kd_vocab_shard_combine_workspace_bytes(int64_t N, size_t *bytes_out) {
  g_err[0] = 0;
  if (!bytes_out || N < 0) return fail(KD_E_ARG, "bad arguments");
  *bytes_out = 256 + (size_t)rup(N * 8, 256);
  return KD_OK;
}

int kd_vocab_shard_combine(const float *shard_max, const float *shard_sumexp,
                           const float *shard_pz, int32_t G, const float *topk_p,
                           const uint8_t *loss_mask, int64_t N, int32_t K, float *loss,
                           float *row_lse, float *row_loss, void *workspace,
                           size_t workspace_bytes, void *stream_v) {
  g_err[0] = 0;
  if (G < 1 || N < 0 || K < 1 || K > 65536) return fail(KD_E_ARG, "need G >= 1, N >= 0, 1 <= K <= 65536");
  if (!loss || !workspace) return fail(KD_E_ARG, "loss and workspace are required");
  if (N > 0 && (!shard_max || !shard_sumexp || !shard_pz || !topk_p || !row_lse))
    return fail(KD_E_ARG, "shard statistics, topk_p and row_lse are required when N > 0");
  if (((uintptr_t)shard_max | (uintptr_t)shard_sumexp | (uintptr_t)shard_pz | (uintptr_t)topk_p |
       (uintptr_t)loss | (uintptr_t)row_lse | (uintptr_t)row_loss) % 4)
    return fail(KD_E_ARG, "float arguments must be 4-byte aligned");
  if ((uintptr_t)workspace % 256) return fail(KD_E_ARG, "workspace must be 256-byte aligned");
  const size_t need = 256 + (size_t)rup(N * 8, 256);
  if (workspace_bytes < need)
    return fail(KD_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  hipStream_t stream = (hipStream_t)stream_v;
  char *ws = (char *)workspace;
  int *flags = (int *)ws;
  unsigned long long *dcount = (unsigned long long *)(ws + 8);
  double *acc = (double *)(ws + 64);
  double *rowterm = (double *)(ws + 256);
  LAUNCH(kd::KC_MISC, kd::launch_fill_zero(ws, 256, stream));
  if (N == 0) {
    LAUNCH(kd::KC_MISC, kd::launch_fill_zero(loss, 4, stream));
    return KD_OK;
  }
  LAUNCH(kd::KC_VALIDATE, kd::launch_validate(nullptr, nullptr, 0, 1, loss_mask, N, flags, dcount,
                                              stream));
  // the count divides the loss on the device: no host synchronisation
  unsigned long long *count = (unsigned long long *)(ws + 16);
  float *inv_count = (float *)(ws + 24);
  LAUNCH(kd::KC_MISC, kd::launch_count_prep(dcount, loss_mask != nullptr, N, count, inv_count,
                                            stream));
  LAUNCH(kd::KC_COMBINE, kd::launch_shard_combine(shard_max, shard_sumexp, shard_pz, G, N, topk_p,
                                                  loss_mask, K, row_lse, row_loss, rowterm, stream));
  LAUNCH(kd::KC_MISC, kd::launch_accum_loss(rowterm, N, acc, stream));
  LAUNCH(kd::KC_MISC, kd::launch_finalize(acc, count, loss, stream));
  return KD_OK;
}

int kd_topk_workspace_bytes(size_t *bytes_out) {
  g_err[0] = 0;
  if (!bytes_out) return fail(KD_E_ARG, "bytes_out is NULL");
  *bytes_out = kd::kTopkScratchBytes;
  return KD_OK;
}

}  // extern "C"

namespace {

int topk_check(const void *logits, int32_t dtype, int64_t N, int64_t V, int32_t K,
               int32_t *topk_idx, float *topk_p, float *row_lse) {
  if (dtype != KD_F32 && dtype != KD_BF16) return fail(KD_E_ARG, "dtype %d unknown", dtype);
  if (N < 0 || V < 1 || K < 1) return fail(KD_E_ARG, "need N >= 0, V >= 1, K >= 1");
  if (K > V) return fail(KD_E_ARG, "K = %d exceeds V = %lld", K, (long long)V);
  if (K > kd::kTopkMaxK) return fail(KD_E_UNSUPPORTED, "K = %d above %d", K, kd::kTopkMaxK);
  if (V >= ((int64_t)1 << 29) || N >= ((int64_t)1 << 31))
    return fail(KD_E_UNSUPPORTED, "V must be below 2^29 and N below 2^31");
  if (N > 0 && (!logits || !topk_idx || !topk_p)) return fail(KD_E_ARG, "logits, topk_idx and topk_p are required");
  const size_t es = dtype == KD_BF16 ? 2 : 4;
  if (logits && (uintptr_t)logits % es) return fail(KD_E_ARG, "logits misaligned");
  if (((uintptr_t)topk_idx | (uintptr_t)topk_p | (uintptr_t)row_lse) % 4)
    return fail(KD_E_ARG, "outputs must be 4-byte aligned");
  return KD_OK;
}

// The validity flag at `flags` is cleared by a fill kernel, raised by the producer for a
// bad row, and read back after one stream synchronisation.
int topk_run(const void *logits, int32_t dtype, int64_t N, int64_t V, int32_t K,
             int32_t *topk_idx, float *topk_p, float *row_lse, int *flags, hipStream_t stream) {
  LAUNCH(kd::KC_MISC, kd::launch_fill_zero(flags, sizeof(int), stream));
  LAUNCH(kd::KC_TOPK, kd::launch_teacher_topk(dtype, logits, N, V, K, topk_idx, topk_p, row_lse,
                                              flags, stream));
  int hf = 0;
  HIPCHK(hipMemcpyAsync(&hf, flags, sizeof hf, hipMemcpyDeviceToHost, stream));
  HIPCHK(hipStreamSynchronize(stream));
  if (hf) return fail(KD_E_INDEX, "a row has a NaN or +inf logit or no finite logit; outputs undefined");
  return KD_OK;
}

}  // namespace

extern "C" {

int kd_teacher_topk(const void *logits, int32_t dtype, int64_t N, int64_t V, int32_t K,
                    int32_t *topk_idx, float *topk_p, float *row_lse, void *workspace,
                    size_t workspace_bytes, void *stream_v) {
  g_err[0] = 0;
  int rc = topk_check(logits, dtype, N, V, K, topk_idx, topk_p, row_lse);
  if (rc != KD_OK) return rc;
  if (!workspace) return fail(KD_E_ARG, "workspace is required");
  if ((uintptr_t)workspace % 256) return fail(KD_E_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < kd::kTopkScratchBytes)
    return fail(KD_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                kd::kTopkScratchBytes);
  if (N == 0) return KD_OK;
  return topk_run(logits, dtype, N, V, K, topk_idx, topk_p, row_lse, (int *)workspace,
                  (hipStream_t)stream_v);
}

int kd_teacher_topk_noalloc(const void *logits, int32_t dtype, int64_t N, int64_t V, int32_t K,
                            int32_t *topk_idx, float *topk_p, float *row_lse, void *stream_v) {
  g_err[0] = 0;
  int rc = topk_check(logits, dtype, N, V, K, topk_idx, topk_p, row_lse);
  if (rc != KD_OK) return rc;
  if (N == 0) return KD_OK;
  int *flags = nullptr;
  HIPCHK(kd::topk_scratch(&flags));
  return topk_run(logits, dtype, N, V, K, topk_idx, topk_p, row_lse, flags,
                  (hipStream_t)stream_v);
}

int kd_clock_stamp(uint64_t *stamps, int32_t n_groups, void *stream_v) {
  g_err[0] = 0;
  if (!stamps) return fail(KD_E_ARG, "stamps is null");
  if ((uintptr_t)stamps % 8) return fail(KD_E_ARG, "stamps must be 8-byte aligned");
  if (n_groups < 1 || n_groups > 65536)
    return fail(KD_E_ARG, "n_groups = %d outside [1, 65536]", n_groups);
  HIPCHK(kd::launch_clock_stamp((unsigned long long *)stamps, n_groups, (hipStream_t)stream_v));
  return KD_OK;
}

int kd_wall_clock_khz(int32_t *khz_out) {
  g_err[0] = 0;
  if (!khz_out) return fail(KD_E_ARG, "khz_out is null");
  int dev = 0, khz = 0;
  HIPCHK(hipGetDevice(&dev));
  HIPCHK(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev));
  *khz_out = khz;
  return KD_OK;
}

int kd_profile_enable(int on) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof.on = on != 0;
  return KD_OK;
}

int kd_profile_num_classes(void) { return kd::KC_COUNT; }

const char *kd_profile_class_name(int cls) {
  return (cls >= 0 && cls < kd::KC_COUNT) ? kClassNames[cls] : "";
}

int kd_profile_read(int cls, double *total_ms, int64_t *launches) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  if (cls < 0 || cls >= kd::KC_COUNT || !total_ms || !launches)
    return fail(KD_E_ARG, "bad profile class or null output");
  double tot = 0.0;
  int64_t n = 0;
  for (auto &pr : g_prof.ev[cls]) {
    float ms = 0.f;
    if (hipEventSynchronize(pr.second) == hipSuccess &&
        hipEventElapsedTime(&ms, pr.first, pr.second) == hipSuccess) {
      tot += ms;
      ++n;
    }
    g_prof.spare.push_back(pr.first);
    g_prof.spare.push_back(pr.second);
  }
  g_prof.ev[cls].clear();
  *total_ms = tot;
  *launches = n;
  return KD_OK;
}

}  // extern "C"
