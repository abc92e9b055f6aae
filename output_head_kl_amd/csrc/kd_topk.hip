// Teacher top-K cache producer on gfx950: for every row of teacher logits, the K
// most likely tokens with their probabilities under the full softmax, and the
// row's logsumexp.  The offline step runs the teacher once and keeps its top 100
// tokens and scores per position (thorstenmeyerai.com article, TL;DR and infographic
// "Select top 100"); the loss reads them as probabilities (aimodeling.com article,
// "First cut").
//
// One workgroup (2 waves) per row reads the row from HBM exactly once.  Small
// workgroups with a small candidate buffer (12 KB of LDS) keep about 10 rows in flight
// per CU, which is what keeps HBM busy; their barriers are cheap.
//  * streaming pass: 16-byte loads per lane; an online (max, sum exp) per lane for the
//    logsumexp; every element whose order-preserving key reaches the running
//    threshold is appended to an LDS candidate buffer (one LDS atomic per wave per
//    chunk);
//  * after every GROUP chunks (one chunk of 1024 bf16 or two of 512 fp32), if the
//    buffer could overflow on the next group, a radix select
//    over the buffer keeps exactly the K best candidates and raises the threshold;
//  * the selection key is unique: (value key << 32) | ~index, so equal logits are
//    ordered by increasing token index and the result does not depend on timing;
//  * at the end a last radix select leaves exactly K entries, each finds its rank
//    among them, and the outputs are written in decreasing order.
#include "kd_internal.h"

#include <cstdint>
#include <mutex>

namespace kd {

// Scratch of the allocation-free entry point (kd_teacher_topk_noalloc): the validity flag
// the kernel raises, in module memory that exists on every device the library runs on
// from module load until the process ends.  Host code never passes `scratch` itself (on
// the host it names a stand-in, not the device copy): topk_scratch() looks up each
// device's address once and every launch takes that.
static __device__ __align__(256) int scratch[kTopkScratchBytes / sizeof(int)];
static_assert(sizeof(int) <= kTopkScratchBytes, "the flag fits the scratch");

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t topk_scratch(int **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (int *)p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

constexpr float kTkLog2e = 1.4426950408889634f;
constexpr float kTkLn2 = 0.6931471805599453f;
constexpr int kTkThreads = 128;

// Workgroup barrier that orders LDS accesses only: every exchange between threads in
// this kernel goes through LDS, and a full __syncthreads would also wait for the
// global loads in flight (the prefetch ring).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Order-preserving 32-bit key of a float (larger float -> larger key); -0.0 is +0.0.
__device__ __forceinline__ uint32_t f_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int DT> struct TkT;
template <> struct TkT<1> {  // bf16 logits: 16-bit value keys, 8 elements per load
  static constexpr int VB = 16, EPL = 8;
  static __device__ __forceinline__ uint32_t vkey(float x) { return f_key(x) >> 16; }
  static __device__ __forceinline__ float value(uint32_t k) {
    const uint32_t u = (k & 0x8000u) ? ((k & 0x7FFFu) << 16) : ((~k & 0xFFFFu) << 16);
    return __uint_as_float(u);
  }
  // the float x with "x >= result" <=> "vkey(x) >= k" for every non-NaN x
  static __device__ __forceinline__ float threshold(uint64_t k) {
    if (k <= 0x007Fu) return -INFINITY;     // at or below the key of -inf
    if (k >= 0xFF80u) return INFINITY;      // at or above the key of +inf
    return value((uint32_t)k);
  }
};
template <> struct TkT<0> {  // fp32 logits: 32-bit value keys, 4 elements per load
  static constexpr int VB = 32, EPL = 4;
  static __device__ __forceinline__ uint32_t vkey(float x) { return f_key(x); }
  static __device__ __forceinline__ float value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
  }
  static __device__ __forceinline__ float threshold(uint64_t k) {
    if (k <= 0x007FFFFFu) return -INFINITY;
    if (k >= 0xFF800000u) return INFINITY;
    return value((uint32_t)k);
  }
};

// Composite selection key: value key, then the complemented index (smaller index wins).
__device__ __forceinline__ uint64_t comp_key(uint32_t vk, uint32_t idx) {
  return ((uint64_t)vk << 32) | (uint32_t)~idx;
}

// Block-wide: among s_ck[0..n) (unique composite keys of TB significant bits), find
// (P, D) such that exactly `need` entries have (key >> (TB - D)) >= P.  Digits of 8
// bits from the top; stops as soon as the selected digit's whole bin is needed.
template <int TB>
__device__ void radix_select(const uint64_t *s_ck, int n, int need, uint32_t *s_hist,
                             uint64_t *s_res, int t) {
  constexpr int NB = 256 / kTkThreads;  // bins per thread: t owns bins NB*t .. NB*t+NB-1
  constexpr int NWV = kTkThreads / 64;
  static_assert(NB * kTkThreads == 256 && NWV >= 1 && NWV <= 4, "block shape");
  uint64_t P = 0;
  int D = 0;
  __shared__ int s_bin, s_above, s_inbin;
  __shared__ uint32_t s_wtot[4];
  for (int level = 0; level < TB / 8; ++level) {
    const int shift = TB - 8 * (level + 1);
#pragma unroll
    for (int j = 0; j < NB; ++j) s_hist[NB * t + j] = 0u;
    lds_sync();
    // entries whose digits above this level equal the prefix (at the first level of a
    // 64-bit key every entry matches: a shift by 64 would be undefined)
    const bool all = shift + 8 >= 64;
    for (int i = t; i < n; i += kTkThreads) {
      const uint64_t c = s_ck[i];
      if (all || (c >> (shift + 8)) == P) atomicAdd(&s_hist[(c >> shift) & 255u], 1u);
    }
    lds_sync();
    // suffix sums over the 256 bins, from the top: this thread's bins, then the threads
    // above it (lanes above in the wave, then the waves above)
    const int lane = t & 63, w = t >> 6;
    uint32_t h[NB], own = 0;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      h[j] = s_hist[NB * t + j];
      own += h[j];
    }
    uint32_t sfx = own;  // inclusive suffix of the thread totals within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_down(sfx, o, 64);
      if (lane + o < 64) sfx += y;
    }
    if (NWV > 1) {
      if (lane == 0) s_wtot[w] = sfx;
      lds_sync();
    }
    uint32_t later = sfx - own;  // threads above this one
    for (int w2 = w + 1; w2 < NWV; ++w2) later += s_wtot[w2];
    uint32_t S = later;  // entries of this prefix with digit >= the bin, accumulated down
#pragma unroll
    for (int j = NB - 1; j >= 0; --j) {
      S += h[j];
      if (S >= (uint32_t)need && S - h[j] < (uint32_t)need) {
        s_bin = NB * t + j;
        s_above = (int)(S - h[j]);
        s_inbin = (int)h[j];
      }
    }
    lds_sync();
    const int bin = s_bin, above = s_above, inbin = s_inbin;
    need -= above;
    P = (P << 8) | (uint64_t)bin;
    D += 8;
    lds_sync();  // s_bin and friends are rewritten by the next level
    if (inbin == need) break;
  }
  if (t == 0) {
    s_res[0] = P;
    s_res[1] = (uint64_t)D;
  }
  lds_sync();
}

// Keeps the entries selected by (P, D) at the front of the buffer (order arbitrary).
// Every thread first takes its entries into registers, so the rewrite cannot
// overwrite an entry not yet read.
template <int TB, int CAP>
__device__ int compact(uint64_t *s_ck, int n, uint64_t P, int D, int *s_cnt, int t) {
  constexpr int PER = (CAP + kTkThreads - 1) / kTkThreads;
  uint64_t mine[PER];
  bool sel[PER];
  int nm = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int i = t + r * kTkThreads;
    mine[r] = i < n ? s_ck[i] : 0ull;
    sel[r] = i < n && (mine[r] >> (TB - D)) >= P;
    nm += sel[r] ? 1 : 0;
  }
  lds_sync();
  if (t == 0) *s_cnt = 0;
  lds_sync();
  int slot = nm ? atomicAdd(s_cnt, nm) : 0;
#pragma unroll
  for (int r = 0; r < PER; ++r)
    if (sel[r]) s_ck[slot++] = mine[r];
  lds_sync();
  return *s_cnt;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kTkThreads) void k_teacher_topk(const void *logits, long long V,
                                                             int K, int32_t *idx_out,
                                                             float *p_out, float *lse_out,
                                                             int *flags) {
  using T = TkT<DT>;
  constexpr int EPL = VEC ? T::EPL : 1;
  constexpr int CHUNK = kTkThreads * EPL;
  constexpr int GROUP = DT == 1 ? 1 : 2;                 // chunks between checkpoints
  constexpr int CAP = kTopkMaxK + GROUP * CHUNK;         // never overflows (see below)
  constexpr int TB = T::VB + 32;
  __shared__ uint64_t s_ck[CAP];
  __shared__ uint32_t s_hist[256];
  __shared__ uint64_t s_res[2];
  __shared__ int s_cnt;
  __shared__ float s_m[kTkThreads / 64];
  __shared__ double s_s[kTkThreads / 64];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const long long row = blockIdx.x;
  const char *rp = (const char *)logits + row * V * (DT == 1 ? 2 : 4);
  if (t == 0) s_cnt = 0;
  lds_sync();

  // Candidate test: x >= tf, a float threshold equivalent to "value key >= tge" (the key
  // order is the float order, +0.0 and -0.0 alike); -inf lets everything through.
  uint64_t tge = 0;
  float tf = -INFINITY;
  // running max m and sum of exp(x - max) per lane, in base 2: with m2 = m * log2(e)
  // rounded once, each term is exp2(x * log2(e) - m2) from one fused multiply-add, and
  // the same m2 is the reference of every later use of the sum (the rescale when the
  // max rises, the combine across lanes and the probabilities), so its rounding cancels.
  // The sum is kept in float64 (a row has ~V/256 terms per lane), each term is a
  // float32 exp2.  A NaN or +inf logit makes the final sum NaN or the maximum +inf,
  // which is how bad rows are found.
  float m = -INFINITY, m2 = -INFINITY;
  double s = 0.0;
  int bad = 0;
  const int nchunks = (int)((V + CHUNK - 1) / CHUNK);
  const int Vi = (int)V;
  // Raw 16-byte (or one-element) loads run PF chunks ahead of their use, so that a
  // row's chunks are not each a full memory round trip.  Buffer loads with the row as
  // the resource's range: offsets past the row read zero without a branch (a load
  // under a branch would make the compiler wait for it at the join).
  constexpr int PF = 4;
  constexpr int ES = DT == 1 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)rp, (short)0, Vi * ES, 0x00020000);
  auto load_raw = [&](int ci) {
    uint4 r = {0u, 0u, 0u, 0u};
    const int e0 = ci * CHUNK + t * EPL;
    const int o = e0 < Vi ? e0 * ES : (int)0x7FFFFFFF;   // past the row: reads zero
    if constexpr (VEC) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
      r = uint4{v[0], v[1], v[2], v[3]};
    } else if constexpr (DT == 1) {
      r.x = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, o, 0, 0);
    } else {
      r.x = __builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0);
    }
    return r;
  };
  uint4 ring[PF];
  // issued in slot order (the loop waits for them in that order)
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    ring[u] = load_raw(u);
    __builtin_amdgcn_sched_barrier(0);
  }
  // The trip count is a whole number of ring turns (chunks past the row read nothing
  // and add nothing), so each slot keeps its registers: a slot is decoded, then
  // reloaded in place, and only its own load is waited for.
  const int nch_pad = (nchunks + PF - 1) / PF * PF;
  for (int c0 = 0; c0 < nch_pad; c0 += PF)
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    const int ci = c0 + u;
    const int e0 = ci * CHUNK + t * EPL;
    // all EPL elements of a lane are in the row or none is (V % EPL == 0 when VEC); a
    // lane past the row (loaded zeros) is masked as a whole, never element by element
    const bool in = e0 < Vi;
    float x[EPL];
    {
      const uint32_t wd[4] = {ring[u].x, ring[u].y, ring[u].z, ring[u].w};
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        uint32_t b;
        if (DT == 1) b = VEC ? ((j & 1) ? (wd[j >> 1] & 0xFFFF0000u) : (wd[j >> 1] << 16))
                             : (wd[0] << 16);
        else b = VEC ? wd[j] : wd[0];
        x[j] = __uint_as_float(b);
      }
    }
    ring[u] = load_raw(ci + PF);
    // online logsumexp of this lane
    float lm = -INFINITY;
    if (in) {
      lm = x[0];
#pragma unroll
      for (int j = 1; j < EPL; ++j) lm = fmaxf(lm, x[j]);
      if (lm > m) {
        asm volatile("");  // rare: keep it a branch rather than computed every chunk
        const float lm2 = lm * kTkLog2e;
        s = (m == -INFINITY) ? 0.0 : s * (double)__builtin_amdgcn_exp2f(m2 - lm2);
        m = lm;
        m2 = lm2;
      }
      if (m != -INFINITY) {
        float part = __builtin_amdgcn_exp2f(fmaf(x[0], kTkLog2e, -m2));  // <= 8 terms
#pragma unroll
        for (int j = 1; j < EPL; ++j) part += __builtin_amdgcn_exp2f(fmaf(x[j], kTkLog2e, -m2));
        s += (double)part;
      }
    }
    // candidates (rare once the threshold has risen): skipped when no lane of the wave
    // has one, which the lane maximum alone tells (a NaN is never a candidate)
    if (__builtin_amdgcn_ballot_w64(lm >= tf)) {  // lanes past the row count nothing below
      int mycnt = 0;
#pragma unroll
      for (int j = 0; j < EPL; ++j) mycnt += (in && x[j] >= tf) ? 1 : 0;
      int incl = mycnt;  // inclusive prefix over the wave
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const int wtot = __shfl(incl, 63, 64);
      int wbase = 0;
      if (lane == 63) wbase = atomicAdd(&s_cnt, wtot);
      wbase = __shfl(wbase, 63, 64);
      int slot = wbase + incl - mycnt;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (in && x[j] >= tf) {
          if (slot < CAP) s_ck[slot] = comp_key(T::vkey(x[j]), (uint32_t)(e0 + j));
          else bad = 1;  // cannot happen (see the checkpoint); kept as a guard
          ++slot;
        }
    }

    // checkpoint: the buffer holds at most kTopkMaxK + GROUP * CHUNK entries because it
    // is cut back to K <= kTopkMaxK whenever fewer than GROUP * CHUNK slots remain
    if ((ci + 1) % GROUP == 0 && ci + 1 < nchunks) {
      lds_sync();
      const int n = min(s_cnt, CAP);
      if (n > CAP - GROUP * CHUNK && n > K) {
        radix_select<TB>(s_ck, n, K, s_hist, s_res, t);
        const uint64_t P = s_res[0];
        const int D = (int)s_res[1];
        compact<TB, CAP>(s_ck, n, P, D, &s_cnt, t);
        // later elements have larger indices than every buffered one, so with the
        // value part of the threshold resolved a later element needs a larger value
        if (D >= T::VB) tge = (P >> (D - T::VB)) + 1;
        else tge = P << (T::VB - D);
        tf = T::threshold(tge);
      }
      lds_sync();
    }
  }
  lds_sync();
  // final selection: exactly K entries
  int n = min(s_cnt, CAP);
  if (n > K) {
    radix_select<TB>(s_ck, n, K, s_hist, s_res, t);
    n = compact<TB, CAP>(s_ck, n, s_res[0], (int)s_res[1], &s_cnt, t);
  }
  // logsumexp of the row, in base 2 (M, Mb: the largest m2)
  float M = m2;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  double sl = (m2 == -INFINITY) ? 0.0 : s * (double)__builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sl += __shfl_xor(sl, o, 64);
  if (lane == 0) {
    s_m[w] = M;
    s_s[w] = sl;
  }
  const int anybad = __syncthreads_or(bad);
  float Mb = s_m[0];
  for (int i = 1; i < kTkThreads / 64; ++i) Mb = fmaxf(Mb, s_m[i]);
  double Sd = 0.0;
  for (int i = 0; i < kTkThreads / 64; ++i)
    if (s_m[i] != -INFINITY) Sd += s_s[i] * (double)__builtin_amdgcn_exp2f(s_m[i] - Mb);
  const float Sb = (float)Sd;
  const bool finite = Mb > -INFINITY && Mb < INFINITY && Sd == Sd && Sd < (double)INFINITY;
  if (t == 0 && (anybad || !finite || n != K)) atomicOr(flags, 1);
  if (t == 0 && lse_out) lse_out[row] = (Mb + __builtin_amdgcn_logf(Sb)) * kTkLn2;
  // rank of each selected entry among the K (keys are unique), then write in order
  const float invS = 1.f / Sb;
  for (int i = t; i < n; i += kTkThreads) {
    const uint64_t c = s_ck[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += s_ck[j] > c ? 1 : 0;
    const uint32_t ix = ~(uint32_t)c;
    const float xv = T::value((uint32_t)(c >> 32));
    if (rank < K) {
      idx_out[row * K + rank] = (int32_t)ix;
      p_out[row * K + rank] = __builtin_amdgcn_exp2f(fmaf(xv, kTkLog2e, -Mb)) * invS;
    }
  }
}

}  // namespace

hipError_t launch_teacher_topk(int dtype, const void *logits, int64_t N, int64_t V, int32_t K,
                               int32_t *idx, float *p, float *lse, int *flags, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int es = dtype == 1 ? 2 : 4;
  const bool vec = ((uintptr_t)logits % 16 == 0) && ((V * es) % 16 == 0);
  const dim3 grid((unsigned)N), block(kTkThreads);
  if (dtype == 1) {
    if (vec)
      hipLaunchKernelGGL((k_teacher_topk<1, true>), grid, block, 0, s, logits, (long long)V, K,
                         idx, p, lse, flags);
    else
      hipLaunchKernelGGL((k_teacher_topk<1, false>), grid, block, 0, s, logits, (long long)V, K,
                         idx, p, lse, flags);
  } else {
    if (vec)
      hipLaunchKernelGGL((k_teacher_topk<0, true>), grid, block, 0, s, logits, (long long)V, K,
                         idx, p, lse, flags);
    else
      hipLaunchKernelGGL((k_teacher_topk<0, false>), grid, block, 0, s, logits, (long long)V, K,
                         idx, p, lse, flags);
  }
  return hipGetLastError();
}

}  // namespace kd
