// gfx950 kernels of the fused, chunked top-K KL loss.
//
// Per token chunk (kd_api.hip enqueues the sequence):
//   buckets        the chunk's teacher hits sorted by output tile of the logits GEMM;
//   forward GEMM   z^T tile = W_tile . h_tile^T on MFMA, epilogue: per-token max and
//                  sum of exp over each 192-row vocabulary group, z gathered at the
//                  tile's teacher hits, and (one-call form) u = exp(z - max) kept as
//                  bf16 in the chunk's dz buffer; no logits are stored;
//   combine        logsumexp over the groups, per-token loss;
//   dz             one-call form: a streaming rescale of u into dz = (mask/count) * M *
//                  exp(z - lse), as each chunk's backward follows its forward; the
//                  backward-only call recomputes z with a second GEMM whose epilogue
//                  forms the same dz (thorstenmeyerai.com infographic, "Recompute
//                  backward");
//   scatter        dz -= (mask/count) * p at the teacher's indices;
//   dh GEMM        dh = dz . W (split over the vocabulary, fp32 partials, then reduced);
//   dW GEMM        dW += dz^T . h over a group of chunks (fp32 read-modify-write).
// The dz buffer holds one chunk; its token-contiguous copy for the dW GEMM holds the
// chunks of one dW group (one chunk with the smallest workspace).
#include "kd_internal.h"

#include <cstdint>
#include <type_traits>

namespace kd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
  return __uint_as_float(((unsigned int)b) << 16);
}
// Round to nearest, ties to even: gfx950's v_cvt_pk_bf16_f32 converts two floats in one
// instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  return (unsigned short)(pack_bf16x2(f, 0.f) & 0xFFFFu);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes l and l^32 hold the two halves of a token's values; combine them.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Workgroups are dispatched round-robin over the 8 XCDs (bid % 8).  Give each XCD a
// contiguous range of tile ids so that tiles sharing operands share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int T) {
  const int q = T >> 3, r = T & 7, x = bid & 7, j = bid >> 3;
  return x * q + (x < r ? x : r) + j;
}

// ---------------------------------------------------------------------------------
// MFMA GEMM core
//
// D[m][n] = sum_k A[m][k] * B[k][n] over one 256 x 256 tile, K in steps of one
// 128-byte row chunk per operand row (64 bf16 or 32 fp32).  An operand is either
//   KC: stored [mn][k] (k contiguous) -> LDS [256 rows][128 B], 16-B chunks XOR
//       swizzled by row, fragments read with ds_read_b128;
//   MC: stored [k][mn] (mn contiguous) -> LDS [k rows][256 mn] padded rows,
//       fragments read transposed (ds_read_b64_tr_b16 for bf16).
// Each wave owns 128 x 128 of the tile as 4 x 4 blocks of the 32x32 MFMA;
// accumulator element i of lane l in block (rb, cb) is row
// rb*32 + (i/4)*8 + (l/32)*4 + i%4 and column cb*32 + l%32 of the wave's square.
// ---------------------------------------------------------------------------------
enum { OP_KC = 0, OP_MC = 1 };

// Element (mn, k) of an operand lives at
//   KC: ptr[(k / 256) * ts + k % 256 + mn * ld],  MC: ptr[(mn / 256) * ts + mn % 256 + k * ld].
// A plain row-major matrix has ts = 256; a matrix stored as blocks of 256 contiguous
// columns (each block [rows][256]) has ld = 256 and ts = rows * 256.
struct Operand {
  const void *ptr;
  long long ld;     // elements between rows
  int mn_ext;       // rows/cols with mn >= mn_ext read as zero
  int k_ext;        // k >= k_ext read as zero
  long long ts;     // elements between 256-column blocks
};

__device__ __forceinline__ long long op_index(const Operand &op, int kind, int mn, int k) {
  return kind == 0 ? (long long)(k >> 8) * op.ts + (k & 255) + (long long)mn * op.ld
                   : (long long)(mn >> 8) * op.ts + (mn & 255) + (long long)k * op.ld;
}

struct GemmGrid {
  int ntm, ntn, nsplit;
  int k_len;    // k range of one split (multiple of the k-step)
  int k_total;  // loop bound
  int order;    // 0: n-tile index fastest, 1: m-tile index fastest
  int ngrp;     // order 0 (bf16 pipe kernel): n tiles taken in groups of ngrp, all m
                // tiles of a group before the next group (0: one group)
};

template <int DT> struct Elem;
template <> struct Elem<1> {  // bf16
  static constexpr int CH = 8, BK = 64, ES = 2, MC_PITCH = 576, MC_ROWS = 64;
};
template <> struct Elem<0> {  // fp32
  static constexpr int CH = 4, BK = 32, ES = 4, MC_PITCH = 1088, MC_ROWS = 32;
};

template <int DT, int KIND> struct OpLds {
  static constexpr int BYTES = KIND == OP_KC ? 256 * 128 : Elem<DT>::MC_ROWS * Elem<DT>::MC_PITCH;
};

template <int DT, int KIND>
__device__ __forceinline__ void load_stage(u32x4 (&r)[8], const Operand &op, int mn0, int k0,
                                           int t) {
  constexpr int CH = Elem<DT>::CH, ES = Elem<DT>::ES;
  const char *base = (const char *)op.ptr;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = t + 256 * i;
    int mn, k;
    if (KIND == OP_KC) {
      mn = mn0 + (q >> 3);
      k = k0 + (q & 7) * CH;
    } else if (DT == 1) {
      k = k0 + (q >> 5);
      mn = mn0 + (q & 31) * CH;
    } else {
      k = k0 + (q >> 6);
      mn = mn0 + (q & 63) * CH;
    }
    const bool ok = mn < op.mn_ext && k < op.k_ext;
    const long long e = op_index(op, KIND, mn, k);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *(const u32x4 *)(base + e * ES);
    r[i] = v;
  }
}

template <int DT, int KIND>
__device__ __forceinline__ void store_stage(char *lds, const u32x4 (&r)[8], int t) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = t + 256 * i;
    int off;
    if (KIND == OP_KC) {
      const int row = q >> 3, kc = q & 7;
      off = row * 128 + ((kc ^ (row & 7)) << 4);
    } else if (DT == 1) {
      off = (q >> 5) * Elem<1>::MC_PITCH + (q & 31) * 16;
    } else {
      off = (q >> 6) * Elem<0>::MC_PITCH + (q & 63) * 16;
    }
    *(LDS_AS u32x4 *)((LDS_AS char *)lds + off) = r[i];
  }
}

// Fragment of 32 rows r0..r0+31 for k-substep ks (16 bf16 or 8 fp32 of k).
template <int DT, int KIND> struct Frag;

template <> struct Frag<1, OP_KC> {
  typedef bf16x8 type;
  static __device__ __forceinline__ type load(const char *lds, int r0, int ks, int lane) {
    const int row = r0 + (lane & 31), kc = ks * 2 + (lane >> 5);
    return *(const LDS_AS bf16x8 *)((const LDS_AS char *)lds + row * 128 + ((kc ^ (row & 7)) << 4));
  }
};
template <> struct Frag<1, OP_MC> {
  typedef bf16x8 type;
  // ds_read_b64_tr_b16: in each 16-lane group, lane j receives element j%4 of the
  // 8 bytes loaded by lanes j/4 + 4r, r = 0..3.  Lane s of the group loads the 4
  // values at [k = kb + s/4][m = mb + 4*(s%4) ..], so lane j gets [kb..kb+3][mb + j].
  static __device__ __forceinline__ type load(const char *lds, int r0, int ks, int lane) {
    const int s = lane & 15, g = lane >> 4;
    const int m = r0 + (g & 1) * 16 + 4 * (s & 3);
    const int k = ks * 16 + (g >> 1) * 8 + (s >> 2);
    const LDS_AS char *b = (const LDS_AS char *)lds;
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_AS s16x4 *)(b + k * Elem<1>::MC_PITCH + m * 2));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (LDS_AS s16x4 *)(b + (k + 4) * Elem<1>::MC_PITCH + m * 2));
    s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
};
template <> struct Frag<0, OP_KC> {
  typedef f32x4 type;
  static __device__ __forceinline__ type load(const char *lds, int r0, int ks, int lane) {
    const int row = r0 + (lane & 31), kc = ks * 2 + (lane >> 5);
    return *(const LDS_AS f32x4 *)((const LDS_AS char *)lds + row * 128 + ((kc ^ (row & 7)) << 4));
  }
};
template <> struct Frag<0, OP_MC> {
  typedef f32x4 type;
  static __device__ __forceinline__ type load(const char *lds, int r0, int ks, int lane) {
    const int m = r0 + (lane & 31), k = ks * 8 + (lane >> 5) * 4;
    const LDS_AS char *b = (const LDS_AS char *)lds;
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = *(const LDS_AS float *)(b + (k + e) * Elem<0>::MC_PITCH + m * 4);
    return v;
  }
};

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// fp32: the 16-byte fragment holds 4 k values per lane; k-slot l/32 of MFMA e uses
// element e, so four 32x32x2 MFMAs cover the same 8 k as one bf16 fragment pair.
__device__ __forceinline__ f32x16 mma(f32x4 a, f32x4 b, f32x16 c) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
  return c;
}

template <int DT, int AK, int BKIND, class Epi>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(Operand A, Operand B, GemmGrid G, Epi epi) {
  constexpr int A_BYTES = OpLds<DT, AK>::BYTES, B_BYTES = OpLds<DT, BKIND>::BYTES;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int BK = Elem<DT>::BK;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int T = gridDim.x;
  const int lin = xcd_remap(blockIdx.x, T);
  const int per_split = G.ntm * G.ntn;
  const int split = lin / per_split;
  const int rem = lin - split * per_split;
  int tm, tn;
  if (G.order == 0) {
    tm = rem / G.ntn;
    tn = rem - tm * G.ntn;
  } else {
    tn = rem / G.ntm;
    tm = rem - tn * G.ntm;
  }
  const int m0 = tm * kTile, n0 = tn * kTile;
  const int kb = split * G.k_len;
  const int ke = min(G.k_total, kb + G.k_len);
  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wr = w >> 1, wc = w & 1;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  u32x4 ra[8], rbuf[8];
  if (nk > 0) {
    load_stage<DT, AK>(ra, A, m0, kb, t);
    load_stage<DT, BKIND>(rbuf, B, n0, kb, t);
    store_stage<DT, AK>(smem, ra, t);
    store_stage<DT, BKIND>(smem + A_BYTES, rbuf, t);
  }
  __syncthreads();

  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nk;
    if (more) {
      load_stage<DT, AK>(ra, A, m0, kb + (it + 1) * BK, t);
      load_stage<DT, BKIND>(rbuf, B, n0, kb + (it + 1) * BK, t);
    }
    const char *la = smem + cur * STAGE;
    const char *lb = la + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      typename Frag<DT, AK>::type fa[4];
      typename Frag<DT, BKIND>::type fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = Frag<DT, AK>::load(la, wr * 128 + i * 32, ks, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = Frag<DT, BKIND>::load(lb, wc * 128 + j * 32, ks, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma(fa[i], fb[j], acc[i][j]);
    }
    if (more) {
      char *nxt = smem + (cur ^ 1) * STAGE;
      store_stage<DT, AK>(nxt, ra, t);
      store_stage<DT, BKIND>(nxt + A_BYTES, rbuf, t);
    }
    __syncthreads();
  }
  epi(acc, m0 + wr * 128, n0 + wc * 128, lane, split, smem);
}

// Accumulator number s = (rb * NCB + cb) * 16 + i of a lane.  s is wave-uniform, so the
// switch becomes a tree of scalar branches that ends in one register move.
template <int NRB, int NCB, int S>
__device__ __forceinline__ float acc_at(const f32x16 (&acc)[NRB][NCB]) {
  if constexpr (S < NRB * NCB * 16) return acc[S / (16 * NCB)][(S / 16) % NCB][S % 16];
  else return 0.f;
}
template <int NRB, int NCB>
__device__ __forceinline__ float pick_acc(const f32x16 (&acc)[NRB][NCB], int s) {
  static_assert(NRB * NCB * 16 <= 256, "at most 256 accumulators per lane");
  switch (s) {
#define KD_ACC1(n) case n: return acc_at<NRB, NCB, n>(acc);
#define KD_ACC4(n) KD_ACC1(n) KD_ACC1(n + 1) KD_ACC1(n + 2) KD_ACC1(n + 3)
#define KD_ACC16(n) KD_ACC4(n) KD_ACC4(n + 4) KD_ACC4(n + 8) KD_ACC4(n + 12)
#define KD_ACC64(n) KD_ACC16(n) KD_ACC16(n + 16) KD_ACC16(n + 32) KD_ACC16(n + 48)
    KD_ACC64(0) KD_ACC64(64) KD_ACC64(128) KD_ACC64(192)
#undef KD_ACC64
#undef KD_ACC16
#undef KD_ACC4
#undef KD_ACC1
    default: return 0.f;
  }
}

// ---------------------------------------------------------------------------------
// Epilogues
// ---------------------------------------------------------------------------------
// Forward: tile rows are vocabulary entries v, columns are tokens c.  A wave holds
// WR = 32 * NRB rows (128, or 192 in the 384-row bf16 tile) of each of its tokens: each
// lane half of them, lane l^32 the rest.
//  * per (token, WR vocabulary rows): max and sum of exp(z - max) -> part, at index
//    (first row of the wave) / WR;
//  * gather: the tile's teacher hits (bucket key = vocabulary tile * token tiles + token
//    tile, entries packed c_local | v_local << 8 | k << 17) read z from the tile: up to
//    64 hits straight from the owning lane's accumulator, more through LDS in slices of
//    64 vocabulary rows ([256 tokens][68] fp32, 68 KB);
//  * optionally (u != null) u = exp(z - max) itself, in dz's layout, for the single-sweep
//    backward (launch_rescale_dz turns it into dz once the logsumexp is known).
template <int DT>
struct EpiFwdLse {
  static constexpr bool kPrefetch = true;
  // Tiles with at most this many teacher hits take them straight from the accumulators
  // (every wave holds the tile's entries, one per lane); others stage z through LDS.
  static constexpr int kDirect = 64;
  float2 *part;   // [n_lse][ld] (max, sum exp(z - max)) per wave row of the tile
  long long ld;
  int V, rows;
  const int *boff;        // bucket offsets, [ntm * ntn + 1]
  const unsigned *bent;   // bucket entries
  int ntn;                // token tiles in the chunk
  float *zg;              // [rows][K] logits at the teacher's indices
  int K;
  void *u;                // null, or dz's buffer: [V_pad/256][C_alloc][256]
  long long ts;           // C_alloc * 256
  int V_pad;
  // The tile's bucket of teacher hits: [beg, end) of the entries, and when the tile has
  // at most one hit per thread, this thread's entry (else ~0); with at most kDirect hits,
  // entry `lane` in every wave.  The pipelined core loads it before its k-loop, so that
  // the loads' latency hides behind the loop.
  struct Pre {
    int beg, end;
    unsigned ent1;
  };
  template <int NRB>
  __device__ __forceinline__ Pre prefetch(int m0, int n0) const {
    constexpr int TR = 64 * NRB;
    const int key = (m0 / TR) * ntn + (n0 >> 8);
    Pre pr;
    pr.beg = boff[key];
    pr.end = boff[key + 1];
    const int n = pr.end - pr.beg;
    const int j = n <= kDirect ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
    pr.ent1 = n <= (int)blockDim.x && j < n ? bent[pr.beg + j] : 0xFFFFFFFFu;
    return pr;
  }
  // Each wave walks the tile's n entries (held one per lane) and takes those in its own
  // rows and columns: the owning lane holds z in accumulator
  // (rb, cb, i) for wave-local row r = 32 rb + 8 (i / 4) + 4 (lane / 32) + i % 4 and
  // column c = 32 cb + lane % 32.
  template <int NRB, int NCB>
  __device__ __forceinline__ void gather_direct(const f32x16 (&acc)[NRB][NCB], int m0, int n0,
                                                int lane, int tn, int n, unsigned ent1) const {
    constexpr int WR = 32 * NRB, WNC = 32 * NCB;
    const int rlo = m0 % (2 * WR), clo = n0 & 255;
    for (int e = 0; e < n; ++e) {
      const unsigned ent = (unsigned)__builtin_amdgcn_readlane((int)ent1, e);
      const int cl = (int)(ent & 255), k = (int)(ent >> 17);
      const int r = (int)((ent >> 8) & 511) - rlo, c = cl - clo;
      if ((unsigned)r >= (unsigned)WR || (unsigned)c >= (unsigned)WNC) continue;
      const int rr = r & 31;
      const float v = pick_acc(acc, ((r >> 5) * NCB + (c >> 5)) * 16 + ((rr >> 3) << 2) + (rr & 3));
      if (lane == (c & 31) + (((rr >> 2) & 1) << 5)) zg[(long long)(tn * 256 + cl) * K + k] = v;
    }
  }
  template <int NRB, int NCB>
  __device__ __forceinline__ void operator()(f32x16 (&acc)[NRB][NCB], int m0, int n0, int lane,
                                             int split, char *smem) const {
    (*this)(acc, m0, n0, lane, split, smem, prefetch<NRB>(m0, n0));
  }
  template <int NRB, int NCB>
  __device__ __forceinline__ void operator()(f32x16 (&acc)[NRB][NCB], int m0, int n0, int lane,
                                             int, char *smem, const Pre &pr) const {
    constexpr int WR = 32 * NRB, TR = 2 * WR, SPW = WR / 64;  // slices of 64 rows per wave row
    // Fused gather first, while no other temporaries are live (the same branch for every
    // wave of the workgroup).  The tile's z goes through LDS SPP slices of 64 vocabulary
    // rows at a time ([256 tokens][68] fp32 each, 68 KB); when the tile has at most one
    // hit per thread, each thread's entry was loaded once (prefetch) for every pass.
    const int tm = m0 / TR, tn = n0 >> 8;
    const int beg = pr.beg, end = pr.end;
    if (beg != end && end - beg <= kDirect) {
      gather_direct(acc, m0, n0, lane, tn, end - beg, pr.ent1);
    } else if (beg != end) {
      const int t = threadIdx.x, wr = (m0 - tm * TR) / WR;
      constexpr int P = 68, SLB = 256 * P * 4;      // slice pitch (floats), slice bytes
      constexpr int NS = 2 * SPW;                   // 64-row slices in the tile
      constexpr int SPP = DT == 1 ? 2 : 1;          // slices per pass (bf16 core: 160 KB LDS)
      static_assert(NS % SPP == 0, "whole passes");
      const int cl0 = (n0 & 255) + (lane & 31);
      const bool one = end - beg <= (int)blockDim.x;
      const unsigned ent1 = pr.ent1;
#pragma unroll
      for (int q = 0; q < NS / SPP; ++q) {
        __syncthreads();
#pragma unroll
        for (int hs = 0; hs < SPP; ++hs) {
          const int sl = q * SPP + hs;
          if (wr == sl / SPW) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int rb = (sl % SPW) * 2 + h;
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  const int vloc = h * 32 + g * 8 + (lane >> 5) * 4;
                  const f32x4 v4 = {acc[rb][cb][g * 4], acc[rb][cb][g * 4 + 1],
                                    acc[rb][cb][g * 4 + 2], acc[rb][cb][g * 4 + 3]};
                  *(LDS_AS f32x4 *)((LDS_AS char *)smem + hs * SLB +
                                    ((cl0 + cb * 32) * P + vloc) * 4) = v4;
                }
            }
          }
        }
        __syncthreads();
        auto take = [&](unsigned ent) {
          const int cl = ent & 255, vloc = (ent >> 8) & 511, k = ent >> 17;
          if ((vloc >> 6) / SPP == q)
            zg[(long long)(tn * 256 + cl) * K + k] = *(const LDS_AS float *)(
                (const LDS_AS char *)smem + ((vloc >> 6) % SPP) * SLB + (cl * P + (vloc & 63)) * 4);
        };
        if (one) {
          if (ent1 != 0xFFFFFFFFu) take(ent1);
        } else {
          for (int e = beg + t; e < end; e += blockDim.x) take(bent[e]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // (max, sum exp) per wave row and token, and u
    const int vl = m0 + (lane >> 5) * 4;
    if constexpr (DT == 1 && NRB % 2 == 0 && NRB >= 4) {
      staged_u(acc, m0, n0, lane, smem);
      return;
    }
    if (m0 < V) {
      const bool full = m0 + WR <= V;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        float mx = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int v = vl + rb * 32 + (i >> 2) * 8 + (i & 3);
            if (full || v < V) mx = fmaxf(mx, acc[rb][cb][i]);
          }
        mx = halves_max(mx);
        const float mx2 = mx * kLog2e;
        const int c = n0 + cb * 32 + (lane & 31);
        const bool keep = u != nullptr && c < rows;
        float s = 0.f;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int v0 = vl + rb * 32 + g * 8;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[e] = (full || v0 + e < V) ? fast_exp2(fmaf(acc[rb][cb][g * 4 + e], kLog2e, -mx2))
                                          : 0.f;
              s += x[e];
            }
            if (keep && v0 < V_pad) {
              if (DT == 1) {
                const u32x2 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                *(u32x2 *)((unsigned short *)u + (long long)(v0 >> 8) * ts + c * 256 +
                           (v0 & 255)) = pk;
              } else {
                *(f32x4 *)((float *)u + (long long)(v0 >> 8) * ts + c * 256 + (v0 & 255)) =
                    f32x4{x[0], x[1], x[2], x[3]};
              }
            }
          }
        s = halves_sum(s);
        if (lane < 32 && c < rows) part[(long long)(m0 / WR) * ld + c] = make_float2(mx, s);
      }
    } else if (u != nullptr) {
      // rows V <= v < V_pad of a wave wholly past V: u = 0
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int c = n0 + cb * 32 + (lane & 31);
        if (c >= rows) continue;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int v0 = vl + rb * 32 + g * 8;
            if (v0 >= V_pad) continue;
            if (DT == 1)
              *(u32x2 *)((unsigned short *)u + (long long)(v0 >> 8) * ts + c * 256 + (v0 & 255)) =
                  u32x2{0u, 0u};
            else
              *(f32x4 *)((float *)u + (long long)(v0 >> 8) * ts + c * 256 + (v0 & 255)) =
                  f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
  }

  // bf16, 192-row waves: as above, but u (when wanted) goes out through LDS so that the
  // stores are whole 16-byte pieces of a token's vocabulary run instead of 8-byte pieces
  // for 32 tokens at once.  A pass covers 64 rows, so each token's run is one aligned
  // 128-byte line (wave rows start at multiples of 192 rows, three lines) and no line is
  // written in parts by two passes.  The stores are non-temporal: u is streamed once into
  // the rescale, and the GEMM's operands keep L2.  Each wave stages its own 64 rows x
  // 32*NCB tokens per pass in a private slice of LDS (9 KB); the workgroup barrier first
  // lets every wave finish with the gather's staging buffer.
  template <int NRB, int NCB>
  __device__ __forceinline__ void staged_u(f32x16 (&acc)[NRB][NCB], int m0, int n0, int lane,
                                           char *smem) const {
    constexpr int WR = 32 * NRB, RP = 2, NP = NRB / RP;  // 32-row blocks per pass, passes
    constexpr int TOK = 32 * NCB, PITCH = RP * 32 + 8;    // tokens per wave, bf16 per row
    constexpr int QPR = RP * 32 / 8;                      // 16-byte pieces per token row
    const bool keep = u != nullptr;                       // the same for the workgroup
    if (keep) __syncthreads();
    LDS_AS unsigned short *stg =
        (LDS_AS unsigned short *)smem + (threadIdx.x >> 6) * TOK * PITCH;
    const int vl = m0 + (lane >> 5) * 4;
    const bool live = m0 < V;                 // the wave has rows below V
    if (live && m0 + WR > V) {
      // rows v >= V of the last vocabulary tile drop out of the max and the sum as -inf
      // (exp2(-inf) = 0), so that whole waves need no per-element bound test below
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (vl + rb * 32 + (i >> 2) * 8 + (i & 3) >= V) acc[rb][cb][i] = -INFINITY;
    }
    float mx[NCB], sum[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float m = -INFINITY;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, acc[rb][cb][i]);
      mx[cb] = halves_max(m);
      // a wave wholly past V: every u is 0 (and the max stays -inf, so avoid inf - inf)
      if (!live) mx[cb] = INFINITY;
      sum[cb] = 0.f;
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float mx2 = mx[cb] * kLog2e;
        const int cl = cb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          const int rb = p * RP + r;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[e] = fast_exp2(fmaf(acc[rb][cb][g * 4 + e], kLog2e, -mx2));
              sum[cb] += x[e];
            }
            if (keep) {
              const u32x2 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
              *(LDS_AS u32x2 *)(stg + cl * PITCH + r * 32 + g * 8 + (lane >> 5) * 4) = pk;
            }
          }
        }
      }
      if (!keep) continue;
#pragma unroll
      for (int it = 0; it < TOK * QPR / 64; ++it) {
        const int q = it * 64 + lane, cl = q / QPR, pc = q - cl * QPR;
        const int c = n0 + cl, v = m0 + p * RP * 32 + pc * 8;
        const u32x4 val = *(const LDS_AS u32x4 *)(stg + cl * PITCH + pc * 8);
        if (c < rows)
          __builtin_nontemporal_store(
              val, (u32x4 *)((unsigned short *)u + (long long)(v >> 8) * ts + c * 256 + (v & 255)));
      }
    }
    if (!live) return;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const float sm = halves_sum(sum[cb]);
      const int c = n0 + cb * 32 + (lane & 31);
      if (lane < 32 && c < rows) part[(long long)(m0 / WR) * ld + c] = make_float2(mx[cb], sm);
    }
  }
};

// Backward: dz[c][v] = sM[c] * exp(z - lse[c]) for v < V, 0 for V <= v < V_pad.
// bf16 also writes dzT (token-contiguous in blocks of 256 tokens, for the dW GEMM):
// lanes c and c ^ 1 swap halves of their packed values so that each writes two tokens
// of two rows.
template <int DT>
struct EpiBwdDz {
  static constexpr bool kPrefetch = false;
  struct Pre {};
  void *dz;      // blocks of 256 vocabulary columns: [V_pad/256][C_alloc][256]
  long long ts;  // C_alloc * 256
  const float *lse, *sM;
  int V, rows, V_pad;
  unsigned short *dzt;  // (v, c) at dzt[(c / 256) * tst + v * 256 + c % 256] (bf16 only)
  long long tst;
  template <int NRB, int NCB>
  __device__ __forceinline__ void operator()(f32x16 (&acc)[NRB][NCB], int m0, int n0, int lane,
                                             int, char *smem) const {
    if constexpr (DT == 1 && NRB % 2 == 0 && NRB >= 4) {
      staged(acc, m0, n0, lane, smem);
      return;
    }
    const int vl = m0 + (lane >> 5) * 4;
    const bool odd = lane & 1;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      // tokens rows <= c < C_alloc get zeros: the dW GEMM reads dzT in 8-token chunks
      const int c = n0 + cb * 32 + (lane & 31);
      const bool cv = c < rows;
      float l2 = 0.f, a = 0.f;
      if (cv) {
        l2 = lse[c] * kLog2e;
        a = sM[c];
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int v0 = vl + rb * 32 + g * 8;
          if (v0 >= V_pad) continue;  // V_pad is a multiple of 4
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[e] = (cv && v0 + e < V) ? a * fast_exp2(fmaf(acc[rb][cb][g * 4 + e], kLog2e, -l2))
                                      : 0.f;
          if (DT == 1) {
            u32x2 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
            *(u32x2 *)((unsigned short *)dz + (long long)(v0 >> 8) * ts + c * 256 + (v0 & 255)) = pk;
            // even lane: rows v0, v0+1 at tokens (c, c+1); odd lane: rows v0+2, v0+3 at
            // tokens (c-1, c)
            const unsigned got = __shfl_xor(odd ? pk[0] : pk[1], 1, 64);
            const unsigned mine = odd ? pk[1] : pk[0];
            const unsigned lo = odd ? got : mine, hi = odd ? mine : got;
            const unsigned r0 = (lo & 0xFFFFu) | (hi << 16);
            const unsigned r1 = (lo >> 16) | (hi & 0xFFFF0000u);
            unsigned short *q = dzt + (long long)(c >> 8) * tst +
                                (long long)(v0 + (odd ? 2 : 0)) * 256 + ((c & 255) & ~1);
            *(unsigned *)q = r0;
            *(unsigned *)(q + 256) = r1;
          } else {
            *(f32x4 *)((float *)dz + (long long)(v0 >> 8) * ts + c * 256 + (v0 & 255)) =
                f32x4{x[0], x[1], x[2], x[3]};
          }
        }
    }
  }

  // bf16, 192-row waves: dz and dzT leave through a per-wave LDS slice ([64 tokens][64
  // rows] per pass, 9 KB), dz as 16-byte pieces of each token's 64-row run (one aligned
  // 128-byte line), dzT as 16-byte pieces (8 tokens) of each row's 64-token run, instead
  // of 8-byte and 4-byte scattered stores.  dzT is read only by the group's dW GEMM:
  // non-temporal stores.
  template <int NRB, int NCB>
  __device__ __forceinline__ void staged(f32x16 (&acc)[NRB][NCB], int m0, int n0, int lane,
                                         char *smem) const {
    constexpr int RP = 2, NP = NRB / RP;                 // 32-row blocks per pass, passes
    constexpr int TOK = 32 * NCB, PITCH = RP * 32 + 8;   // tokens per wave, bf16 per row
    constexpr int QPR = RP * 32 / 8;                     // 16-byte pieces per token row
    constexpr int TG = TOK / 8;                          // 8-token groups per vocabulary row
    __syncthreads();  // every wave is done with the k-loop's LDS ring
    LDS_AS unsigned short *stg =
        (LDS_AS unsigned short *)smem + (threadIdx.x >> 6) * TOK * PITCH;
    const int vl = m0 + (lane >> 5) * 4;
    float l2[NCB], a[NCB];
    bool cv[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      // tokens rows <= c < C_alloc get zeros: the dW GEMM reads dzT in 8-token chunks
      const int c = n0 + cb * 32 + (lane & 31);
      cv[cb] = c < rows;
      l2[cb] = cv[cb] ? lse[c] * kLog2e : 0.f;
      a[cb] = cv[cb] ? sM[c] : 0.f;
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int cl = cb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          const int rb = p * RP + r;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int v0 = vl + rb * 32 + g * 8;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[e] = (cv[cb] && v0 + e < V)
                         ? a[cb] * fast_exp2(fmaf(acc[rb][cb][g * 4 + e], kLog2e, -l2[cb]))
                         : 0.f;
            const u32x2 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
            *(LDS_AS u32x2 *)(stg + cl * PITCH + r * 32 + g * 8 + (lane >> 5) * 4) = pk;
          }
        }
      }
      const int vp = m0 + p * RP * 32;  // first vocabulary row of the pass
      // dz: token runs
#pragma unroll
      for (int it = 0; it < TOK * QPR / 64; ++it) {
        const int q = it * 64 + lane, cl = q / QPR, pc = q - cl * QPR;
        const int c = n0 + cl, v = vp + pc * 8;
        const u32x4 val = *(const LDS_AS u32x4 *)(stg + cl * PITCH + pc * 8);
        if (c < rows && v < V_pad)
          *(u32x4 *)((unsigned short *)dz + (long long)(v >> 8) * ts + c * 256 + (v & 255)) = val;
      }
      // dzT: row runs of 64 tokens (n0 and the wave's 64 tokens lie in one 256-token block)
      const int c0 = n0;
#pragma unroll
      for (int it = 0; it < RP * 32 * TG / 64; ++it) {
        const int q = it * 64 + lane, r = q / TG, tg = q - r * TG;
        const int v = vp + r;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = (unsigned)stg[(tg * 8 + 2 * e) * PITCH + r] |
                 ((unsigned)stg[(tg * 8 + 2 * e + 1) * PITCH + r] << 16);
        const int c = c0 + tg * 8;
        if (v < V_pad)
          __builtin_nontemporal_store(
              o, (u32x4 *)(dzt + (long long)(c >> 8) * tst + (long long)v * 256 + (c & 255)));
      }
    }
  }
};

// dh split: tile rows are hidden units j, columns tokens c; fp32 partial per split.
struct EpiDhPart {
  static constexpr bool kPrefetch = false;
  struct Pre {};
  float *part;
  long long split_stride, ld;  // C_alloc*d_pad, d_pad
  int rows;
  template <int NRB, int NCB>
  __device__ __forceinline__ void operator()(f32x16 (&acc)[NRB][NCB], int m0, int n0, int lane,
                                             int split, char *) const {
    float *base = part + split * split_stride;
    const int jl = m0 + (lane >> 5) * 4;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = n0 + cb * 32 + (lane & 31);
      if (c >= rows) continue;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int j = jl + rb * 32 + g * 8;
          if (j >= ld) continue;  // d_pad is a multiple of 4
          const f32x4 v = {acc[rb][cb][g * 4], acc[rb][cb][g * 4 + 1], acc[rb][cb][g * 4 + 2],
                           acc[rb][cb][g * 4 + 3]};
          *(f32x4 *)(base + (long long)c * ld + j) = v;
        }
    }
  }
};

// dW: tile rows are vocabulary entries v, columns hidden units j, so each accumulator
// register holds 32 consecutive floats of two dW rows (one per half-wave).  The first
// chunk group stores; later groups add.  Each element gets exactly one addition per
// launch and launches are ordered, so the result does not depend on timing: the bf16
// kernel reads the old values through LDS and stores the sums, the fp32 kernel adds with
// one fire-and-forget atomic per element.
struct EpiDw {
  static constexpr bool kPrefetch = false;
  struct Pre {};
  float *dW;
  int d, V, accumulate;
  int lds_rmw;  // accumulate by reading the old values through LDS (bf16 pipe kernel only)
  template <int NRB, int NCB>
  __device__ __forceinline__ void operator()(f32x16 (&acc)[NRB][NCB], int m0, int n0, int lane,
                                             int, char *smem) const {
    // One buffer resource per wave, from its first row to the end of dW: elements of
    // rows v >= V lie outside its range and the hardware drops them; lanes with
    // j >= d get an offset outside every range.  Offsets stay below 32 * NRB * d * 4 bytes.
    if (NCB == 2 && NRB % 2 == 0 && accumulate && lds_rmw)
      __syncthreads();  // (every wave) all have left the k-loop: the operand ring is free
    const long long rem = (long long)(V - m0) * d * 4;
    if (rem <= 0) return;
    const int nrec = rem > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)rem;
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(dW + (long long)m0 * d), (short)0, nrec, 0x00020000);
    int vo[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int j = n0 + cb * 32 + (lane & 31);
      vo[cb] = j < d ? (((lane >> 5) * 4 * d + j) * 4) : (int)0x80000000;
    }
    if constexpr (NCB == 2 && NRB % 2 == 0) {
      if (accumulate && lds_rmw) {
        // Read-modify-write through the wave's own LDS slice (the tile belongs to one
        // workgroup per launch, so plain loads and stores suffice): 64 rows of the wave's
        // 64 columns per pass, copied by the buffer unit as 16 loads of 4 rows x 256 B,
        // each placed 1088 B apart so that rows r and r + 4 (the two half-waves of a read)
        // fall in different banks; then each lane adds and stores its own elements.
        // Rows v >= V read zero and are not stored; columns j >= d are not stored.
        constexpr int PITCH = 1088;
        LDS_AS char *slice = (LDS_AS char *)smem + (threadIdx.x >> 6) * (16 * PITCH);
#pragma unroll
        for (int ps = 0; ps < NRB / 2; ++ps) {
          if (ps > 0) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): last pass's reads
#pragma unroll
          for (int k = 0; k < 16; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (LDS_AS void *)(slice + k * PITCH), 16,
                ((ps * 64 + 4 * k + (lane >> 4)) * d + n0 + (lane & 15) * 4) * 4, 0, 0,
                16 /* cache policy sc1: through L2 only */);
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
#pragma unroll
          for (int r2 = 0; r2 < 2; ++r2) {
            const int rb = ps * 2 + r2;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int rp = r2 * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);  // row in pass
              const int roff = (rb * 32 + (i >> 2) * 8 + (i & 3)) * d * 4;
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb) {
                const float old = *(const LDS_AS float *)(slice + (rp >> 2) * PITCH +
                                                          (rp & 3) * 256 +
                                                          (cb * 32 + (lane & 31)) * 4);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[rb][cb][i] + old), rs,
                                                      vo[cb] + roff, 0, 0);
              }
            }
          }
        }
        return;
      }
    }
    if (accumulate) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int roff = (rb * 32 + (i >> 2) * 8 + (i & 3)) * d * 4;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[rb][cb][i], rs, vo[cb] + roff, 0, 0);
        }
    } else {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int roff = (rb * 32 + (i >> 2) * 8 + (i & 3)) * d * 4;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[rb][cb][i]), rs,
                                                  vo[cb] + roff, 0, 0);
        }
    }
  }
};

// ---------------------------------------------------------------------------------
// bf16 MFMA GEMM core, pipelined
//
// Same tile, wave layout, operand kinds and epilogues as gemm_kernel, with:
//  * operands copied global -> LDS by the buffer unit (buffer_load_dwordx4 ... lds),
//    so no staging registers; lanes whose element lies outside the operand get an
//    offset past the buffer's range and read zero;
//  * a ring of NST LDS stages of BK k, every slot loading: the slot of the stage just
//    consumed is refilled at once, NST stages ahead;
//  * one barrier per stage, placed before the last 16-k substep, so that the fragment
//    reads for the next substep always overlap 16 MFMAs in flight.
// KC stage tile: [256 rows][2*BK B], 16-B chunk kc of row r at kc ^ swz(r).
// MC stage tile: [BK k][512 B], 16-B chunk mc of row k at chunk mc ^ ((k&3)<<2).
// The LDS serves 256 B per clock (64 banks of 4 B): a ds_read_b128 in four phases of
// 16 lanes, a ds_read_b64_tr_b16 in two phases of 32 lanes.  With these swizzles
// every phase of a fragment read touches 16 distinct 16-B bank groups.
// ---------------------------------------------------------------------------------
namespace pipe {
constexpr int OOB = (int)0x80000000;   // offset outside every buffer: reads zero
constexpr int kLoadSc1 = 16;           // buffer-load cache-policy bit SC1

// Stage geometry for a k-depth of BK bf16 (32 or 64) and ROWS tile rows (256 or 384).
template <int BK, int ROWS = 256> struct Geo {
  static constexpr int OPB = ROWS * BK * 2;  // bytes per operand per stage
  static constexpr int ROWB = BK * 2;        // KC row bytes
  static constexpr int CPR = BK / 8;         // KC 16-B chunks per row
  static constexpr int LOADS = OPB / 1024;   // 1-KB buffer loads per operand per stage
  // KC swizzle: a 16-lane LDS phase reads 16 rows of one logical chunk; rows that share
  // a 256-B bank window (same row % (256/ROWB)) get distinct chunks.
  static __device__ __forceinline__ int kc_swz(int row) {
    return BK == 32 ? ((row >> 2) & 3) : ((row >> 1) & 7);
  }
};

// Per-lane description of the NI chunks (of 16 B) one lane moves per operand per stage.
// Chunk j of wave w sits at LDS position q = (w*NI + j)*64 + lane (16-B units).
//   KC: row q / CPR, 16-B column (q % CPR) ^ swz(row);
//   MC: k row q / 32, 16-B column (q % 32) ^ ((k & 3) << 2).
// With BK = 64 (CPR = 8) and NI even, both reduce to a part shared by all chunks of one
// parity of j plus a wave-uniform part linear in g = w*NI + j, so a lane keeps two
// offsets and two k (or mn) values instead of three numbers per chunk.
template <int KIND, int BK, int NI> struct LaneChunks {
  static_assert(BK == 64 && NI % 2 == 0, "chunk parity layout");
  int rel[2];   // per-lane byte offset (even, odd j)
  int var[2];   // KC: k offset; MC: mn offset (even, odd j)
  int fix;      // KC: row within a group of 8; MC: k within a pair
  long long ld;
  __device__ __forceinline__ void init(long long ld_, int lane) {
    ld = ld_;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (KIND == OP_KC) {
        // row = 8 g + (lane >> 3); swz(row) = (row >> 1) & 7 = (4 (g & 1) + (lane >> 4)) & 7
        const int kc = (lane & 7) ^ ((4 * p + (lane >> 4)) & 7);
        fix = lane >> 3;
        var[p] = kc * 8;
        rel[p] = (int)(((long long)fix * ld + kc * 8) * 2);
      } else {
        // k = 2 g + (lane >> 5); (k & 3) = 2 (g & 1) + (lane >> 5)
        const int mc = (lane & 31) ^ ((2 * p + (lane >> 5)) << 2);
        fix = lane >> 5;
        var[p] = mc * 8;
        rel[p] = (int)(((long long)fix * ld + mc * 8) * 2);
      }
    }
  }
  // chunk g = w*NI + j of the stage: mn, k offsets within the tile / stage and the
  // byte offset from the stage base
  __device__ __forceinline__ void at(int g, int &mn, int &k, int &off) const {
    const int p = g & 1;
    if (KIND == OP_KC) {
      mn = 8 * g + fix;
      k = var[p];
      off = (int)(16LL * g * ld) + rel[p];
    } else {
      mn = var[p];
      k = 2 * g + fix;
      off = (int)(4LL * g * ld) + rel[p];
    }
  }
};

// Cache policy sc1 (device scope) on every operand load: the lines go through L2 only;
// each CU reads a line once per stage, so the vector L1 holds nothing it would reuse.
template <int KIND, int BK, int NI> struct Loader {
static __device__ __forceinline__ void issue(const Operand &op, const LaneChunks<KIND, BK, NI> &c,
                                             int mn0, int k0, char *lds, int w) {
  const unsigned short *base = (const unsigned short *)op.ptr;
  base += op_index(op, KIND, mn0, k0);   // a stage never crosses a 256-column block
  if (KIND == OP_KC && k0 + BK <= op.k_ext) {
    // The whole stage lies inside k.  The resource ends at row mn_ext, so the hardware
    // drops rows past the operand; chunk g = w*NI + j (rows 8g .. 8g+7 of the tile) is at
    // rel[g & 1] + 16 g ld bytes.  The two lane offsets are made opaque here so that the
    // per-chunk offsets are formed at each stage instead of being held in registers.
    const long long rows = (long long)op.mn_ext - mn0;
    const long long bytes = rows * op.ld * 2;
    const int nrec = rows <= 0 ? 0 : bytes > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes;
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, nrec, 0x00020000);
    int r0 = c.rel[0], r1 = c.rel[1];
    asm volatile("" : "+v"(r0), "+v"(r1));
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int g = w * NI + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (LDS_AS void *)((LDS_AS char *)lds + g * 1024), 16,
          ((j & 1) ? r1 : r0) + (int)(16LL * g * op.ld), 0, 0, kLoadSc1);
    }
    return;
  }
  // general case (the last, partial stage of k, or an MC operand): per-lane tests
  __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    int mn, k, off;
    c.at(w * NI + j, mn, k, off);
    const bool ok = (mn0 + mn < op.mn_ext) && (k0 + k < op.k_ext);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (LDS_AS void *)((LDS_AS char *)lds + (w * NI + j) * 1024), 16, ok ? off : OOB, 0, 0,
        kLoadSc1);
  }
}
};

template <int KIND, int BK> struct PFrag;
template <int BK> struct PFrag<OP_KC, BK> {
  static __device__ __forceinline__ bf16x8 load(const char *lds, int r0, int ks, int lane) {
    using GG = Geo<BK>;
    const int row = r0 + (lane & 31), kc = ks * 2 + (lane >> 5);
    return *(const LDS_AS bf16x8 *)((const LDS_AS char *)lds + row * GG::ROWB +
                                    ((kc ^ GG::kc_swz(row)) << 4));
  }
};
template <int BK> struct PFrag<OP_MC, BK> {
  static __device__ __forceinline__ bf16x8 load(const char *lds, int r0, int ks, int lane) {
    const int s = lane & 15, g = lane >> 4;
    const int m = r0 + (g & 1) * 16 + 4 * (s & 3);
    const int k = ks * 16 + (g >> 1) * 8 + (s >> 2);
    const int col = (((m >> 3) ^ ((k & 3) << 2)) << 4) + (m & 7) * 2;
    const LDS_AS char *b = (const LDS_AS char *)lds;
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(b + k * 512 + col));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)(b + (k + 4) * 512 + col));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

// s_waitcnt with vmcnt <= N and, with LGKM0, lgkmcnt == 0.  Immediate: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 (left at their maxima unless LGKM0).
template <int N, bool LGKM0>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((LGKM0 ? 0x0070 : 0x0F70) | (N & 15) | ((N >> 4) << 14));
}
}  // namespace pipe

// Scheduling hints: sched_group_barrier(mask, n, id) asks the scheduler for the next
// n instructions of a class; the sequence below places one load or LDS read in the
// shadow of each MFMA, so that with one wave per SIMD the matrix core never waits for
// the wave to issue its memory traffic.
#define KD_SG_MFMA 0x008
#define KD_SG_VALU 0x002
#define KD_SG_SALU 0x004
#define KD_SG_VMEM 0x020
#define KD_SG_DSRD 0x100

// WN = waves along n: 2 gives 4 waves of (TMA/2) x 128 (one per SIMD), 4 gives 8 waves
// of (TMA/2) x 64 (two per SIMD, so one wave's MFMAs cover the other's waits).  TMA =
// rows of the A tile: 256, or 384 for a k-contiguous A, which cuts the operand bytes
// per flop by a sixth; with TMA = 384 the A fragments are single-buffered (each one is
// re-read for the next substep as soon as its MFMAs have issued) so that the 192
// accumulators per lane and the fragments fit in 256 registers.  NSTA / NSTB = LDS
// slots of the A / B rings; A may have one slot more than B.
template <int AK, int BKIND, class Epi, int NSTA, int NSTB, int BK, int WN, int TMA = 256>
__global__ __attribute__((amdgpu_flat_work_group_size(128 * WN, 128 * WN),
                          amdgpu_waves_per_eu(WN / 2, WN / 2)))
void gemm_pipe_kernel(Operand A, Operand B, GemmGrid G, Epi epi) {
  using namespace pipe;
  using GA = Geo<BK, TMA>;
  using GB = Geo<BK, 256>;
  constexpr int NW = 2 * WN;            // waves
  constexpr int NCB = 8 / WN;           // 32-column MFMA blocks per wave
  constexpr int WNC = 32 * NCB;         // columns per wave
  constexpr int WMR = TMA / 2;          // rows per wave
  constexpr int NRB = WMR / 32;         // 32-row MFMA blocks per wave
  constexpr int NIA = GA::LOADS / NW;   // buffer loads per wave per stage, A
  constexpr int NIB = GB::LOADS / NW;   // buffer loads per wave per stage, B
  constexpr int S = BK / 16;            // 16-k substeps per stage
  constexpr int LPS = NIA + NIB;        // buffer loads per wave per stage
  constexpr int NMF = NRB * NCB;        // MFMAs per wave per substep
  constexpr bool FA1 = TMA > 256;       // single-buffered A fragments
  // LDS reads per substep: one per fragment, two per transposed (MC) fragment
  constexpr int NRD = NRB * (AK == OP_MC ? 2 : 1) + NCB * (BKIND == OP_MC ? 2 : 1);
  static_assert(NSTB >= 2 && (NSTA == NSTB || NSTA == NSTB + 1), "ring shapes");
  static_assert(TMA == 256 || (TMA == 384 && AK == OP_KC), "a 384-row A tile must be k-contiguous");
  static_assert(GA::LOADS % NW == 0 && GB::LOADS % NW == 0, "whole loads per wave");
  __shared__ __attribute__((aligned(1024))) char smem[NSTA * GA::OPB + NSTB * GB::OPB];
  char *const smemB = smem + NSTA * GA::OPB;

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per_split = G.ntm * G.ntn;
  const int split = lin / per_split;
  const int rem = lin - split * per_split;
  int tm, tn;
  if (G.order == 0) {
    if (G.ngrp > 0 && G.ngrp < G.ntn) {
      const int span = G.ntm * G.ngrp, grp = rem / span;
      const int gs = min(G.ngrp, G.ntn - grp * G.ngrp), r = rem - grp * span;
      tm = r / gs;
      tn = grp * G.ngrp + (r - tm * gs);
    } else {
      tm = rem / G.ntn;
      tn = rem - tm * G.ntn;
    }
  } else {
    tn = rem / G.ntm;
    tm = rem - tn * G.ntm;
  }
  const int m0 = tm * TMA, n0 = tn * kTile;
  const int kb = split * G.k_len;
  const int ke = min(G.k_total, kb + G.k_len);
  const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = w / WN, wc = w % WN;
  LaneChunks<AK, BK, NIA> ca;
  LaneChunks<BKIND, BK, NIB> cb;
  ca.init(A.ld, lane);
  cb.init(B.ld, lane);
  // k beyond this split's range reads zero (and moves no data)
  Operand Ak = A, Bk = B;
  Ak.k_ext = min(A.k_ext, ke);
  Bk.k_ext = min(B.k_ext, ke);

  f32x16 acc[NRB][NCB];
#pragma unroll
  for (int i = 0; i < NRB; ++i)
#pragma unroll
    for (int j = 0; j < NCB; ++j) acc[i][j] = f32x16{};

  // Prologue: every slot loading, in the order A0 B0 A1 B1 [A2] (stages past the end
  // are all-zero loads, so the count of loads in flight is the same in every
  // iteration); then stage 0 landed.
  for (int s = 0; s < NSTA; ++s) {
    Loader<AK, BK, NIA>::issue(Ak, ca, m0, kb + s * BK, smem + s * GA::OPB, w);
    if (s < NSTB) Loader<BKIND, BK, NIB>::issue(Bk, cb, n0, kb + s * BK, smemB + s * GB::OPB, w);
  }
  // epilogue inputs that do not depend on the product, loaded behind the first stages
  typename Epi::Pre pre{};
  if constexpr (Epi::kPrefetch) pre = epi.template prefetch<NRB>(m0 + wr * WMR, n0 + wc * WNC);
  wait_vm<NIA * (NSTA - 1) + NIB * (NSTB - 1), false>();
  __syncthreads();

  constexpr int NFA = FA1 ? 1 : 2;
  bf16x8 fa[NFA][NRB], fb[2][NCB];
#pragma unroll
  for (int i = 0; i < NRB; ++i) fa[0][i] = PFrag<AK, BK>::load(smem, wr * WMR + i * 32, 0, lane);
#pragma unroll
  for (int j = 0; j < NCB; ++j) fb[0][j] = PFrag<BKIND, BK>::load(smemB, wc * WNC + j * 32, 0, lane);

  int acur = 0, bcur = 0;  // ring slots of stage it
  for (int it = 0; it < nk; ++it) {
    const int anext = acur + 1 == NSTA ? 0 : acur + 1;
    const int bnext = bcur + 1 == NSTB ? 0 : bcur + 1;
    char *cura = smem + acur * GA::OPB;
    char *curb = smemB + bcur * GB::OPB;
#pragma unroll
    for (int ss = 0; ss < S - 1; ++ss) {
      // substep ss on registers [ss&1]; read substep ss+1 meanwhile
#pragma unroll
      for (int j = 0; j < NCB; ++j)
        fb[(ss + 1) & 1][j] = PFrag<BKIND, BK>::load(curb, wc * WNC + j * 32, ss + 1, lane);
      if constexpr (FA1) {
#pragma unroll
        for (int i = 0; i < NRB; ++i) {
#pragma unroll
          for (int j = 0; j < NCB; ++j) acc[i][j] = mma(fa[0][i], fb[ss & 1][j], acc[i][j]);
          fa[0][i] = PFrag<AK, BK>::load(cura, wr * WMR + i * 32, ss + 1, lane);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NRB; ++i)
          fa[(ss + 1) & 1][i] = PFrag<AK, BK>::load(cura, wr * WMR + i * 32, ss + 1, lane);
#pragma unroll
        for (int i = 0; i < NRB; ++i)
#pragma unroll
          for (int j = 0; j < NCB; ++j) acc[i][j] = mma(fa[ss & 1][i], fb[ss & 1][j], acc[i][j]);
      }
      // one or two LDS reads in the shadow of each MFMA
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(KD_SG_DSRD, (NRD + NMF - 1) / NMF, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // Stage it+1 must have landed for every wave, and every wave must hold the whole of
    // stage it in registers or accumulators, since its slots are refilled next.  Loads
    // are issued B(j+NSTB) then A(j+NSTA) in iteration j, so what may still be in
    // flight here is A(it+2) when A has the extra slot, else nothing.
    wait_vm<NIA * (NSTA - NSTB), true>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // last substep on registers [(S-1)&1]; meanwhile read substep 0 of stage it+1 and
    // refill this stage's slots with B(it+NSTB) and A(it+NSTA)
    const char *nxa = smem + anext * GA::OPB;
    const char *nxb = smemB + bnext * GB::OPB;
#pragma unroll
    for (int j = 0; j < NCB; ++j) fb[0][j] = PFrag<BKIND, BK>::load(nxb, wc * WNC + j * 32, 0, lane);
    if constexpr (FA1) {
#pragma unroll
      for (int i = 0; i < NRB; ++i) {
#pragma unroll
        for (int j = 0; j < NCB; ++j) acc[i][j] = mma(fa[0][i], fb[(S - 1) & 1][j], acc[i][j]);
        fa[0][i] = PFrag<AK, BK>::load(nxa, wr * WMR + i * 32, 0, lane);
      }
      Loader<BKIND, BK, NIB>::issue(Bk, cb, n0, kb + (it + NSTB) * BK, curb, w);
      Loader<AK, BK, NIA>::issue(Ak, ca, m0, kb + (it + NSTA) * BK, cura, w);
    } else {
#pragma unroll
      for (int i = 0; i < NRB; ++i) fa[0][i] = PFrag<AK, BK>::load(nxa, wr * WMR + i * 32, 0, lane);
      Loader<BKIND, BK, NIB>::issue(Bk, cb, n0, kb + (it + NSTB) * BK, curb, w);
      Loader<AK, BK, NIA>::issue(Ak, ca, m0, kb + (it + NSTA) * BK, cura, w);
#pragma unroll
      for (int i = 0; i < NRB; ++i)
#pragma unroll
        for (int j = 0; j < NCB; ++j)
          acc[i][j] = mma(fa[(S - 1) & 1][i], fb[(S - 1) & 1][j], acc[i][j]);
    }
    // reads for the next stage in the first half of the MFMAs (they gate the next
    // iteration), loads in the second half
#pragma unroll
    for (int q = 0; q < NMF / 2; ++q) {
      __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 1, 1);
      __builtin_amdgcn_sched_group_barrier(KD_SG_DSRD, (2 * NRD + NMF - 1) / NMF, 1);
    }
#pragma unroll
    for (int q = 0; q < NMF / 2; ++q) {
      __builtin_amdgcn_sched_group_barrier(KD_SG_MFMA, 1, 1);
      __builtin_amdgcn_sched_group_barrier(KD_SG_VMEM, (2 * LPS + NMF - 1) / NMF, 1);
      __builtin_amdgcn_sched_group_barrier(KD_SG_VALU, 2, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    acur = anext;
    bcur = bnext;
  }
  wait_vm<0, false>();  // the zero loads issued past the end
  if constexpr (Epi::kPrefetch)
    epi(acc, m0 + wr * WMR, n0 + wc * WNC, lane, split, smem, pre);
  else
    epi(acc, m0 + wr * WMR, n0 + wc * WNC, lane, split, smem);
}

template <int DT, int AK, int BKIND, class Epi>
static hipError_t run_gemm(const Operand &A, const Operand &B, const GemmGrid &G, const Epi &epi,
                           hipStream_t s) {
  const long long T = (long long)G.ntm * G.ntn * G.nsplit;
  if (T <= 0) return hipSuccess;
  // 8 waves (two per SIMD), two LDS stages of 64 k: a KC operand row is then one
  // 128-byte segment per stage, which halves the memory requests of k-contiguous operands
  if constexpr (DT == 1)
    hipLaunchKernelGGL((gemm_pipe_kernel<AK, BKIND, Epi, 2, 2, 64, 4, kTileA16>), dim3((unsigned)T),
                       dim3(512), 0, s, A, B, G, epi);
  else
    hipLaunchKernelGGL((gemm_kernel<DT, AK, BKIND, Epi>), dim3((unsigned)T), dim3(256), 0, s, A,
                       B, G, epi);
  return hipGetLastError();
}

static inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// ---------------------------------------------------------------------------------
// GEMM launchers
// ---------------------------------------------------------------------------------
hipError_t launch_fwd_gemm(int dtype, const void *W, const void *h_c, int64_t rows, int64_t d,
                           int64_t V, float2 *partials, int64_t ld_part, const int *boff,
                           const unsigned *bent, float *zg, int32_t K, void *u, int64_t V_pad,
                           int64_t C_alloc, hipStream_t s) {
  // vocabulary tiles cover V_pad (a multiple of the tile), so u is written for every row
  Operand A{W, d, (int)V, (int)d, 256};
  Operand B{h_c, d, (int)rows, (int)d, 256};
  // Eight token tiles per raster group: an XCD's 32 concurrent workgroups then cover
  // four vocabulary tiles x eight token tiles, the fewest distinct operand rows per stage
  // (more token tiles per chunk would otherwise spread them over two vocabulary tiles).
  GemmGrid G{(int)(V_pad / tile_rows(dtype)), cdiv(rows, kTile), 1, (int)d, (int)d, 0, 8};
  if (dtype == 1) {
    EpiFwdLse<1> e{partials, ld_part, (int)V, (int)rows, boff, bent, G.ntn, zg, (int)K, u,
                   C_alloc * 256, (int)V_pad};
    return run_gemm<1, OP_KC, OP_KC>(A, B, G, e, s);
  }
  EpiFwdLse<0> e{partials, ld_part, (int)V, (int)rows, boff, bent, G.ntn, zg, (int)K, u,
                 C_alloc * 256, (int)V_pad};
  return run_gemm<0, OP_KC, OP_KC>(A, B, G, e, s);
}

// Single-sweep backward: u = exp(z - m_g) from the forward epilogue (m_g the max of the
// token's group g of gr = tile_rows / 2 vocabulary rows) becomes dz = sM * exp(z - lse) =
// sM * exp(m_g - lse) * u, in place.
//
// bf16 also writes dzT, the same values in the token-blocked layout of the dW GEMM's A
// operand (element (v, c) at dzT[(c / 256) * tst + v * 256 + c % 256], zeros for tokens
// rows <= c < C_alloc).  A block takes one 256-column block of dz (256 vocabulary rows:
// two 192-row groups, or three) x TC tokens: the u it reads and rewrites is TC x 512
// contiguous bytes, and its dzT rows are TC x 2 bytes at a 512-byte pitch.  Each thread
// first issues all its loads of u (NQ chunks of 8 elements), then the factors are formed.
// The transpose goes through LDS as [token][256], 16-byte chunk q of token row c stored
// at q ^ (c / 8 % 32), so that the column reads (8 tokens of one vocabulary row per
// thread, 16 threads per row) hit distinct banks.
template <int TC, int NT>
__global__ __launch_bounds__(NT) void k_rescale_dz_bf16(unsigned short *dz, long long ts,
                                                        unsigned short *dzt, long long tst,
                                                        const float2 *part, long long ld,
                                                        const float *lse, const float *sM,
                                                        int rows, int V, int gr) {
  constexpr int NQ = TC * 32 / NT;  // 16-byte chunks per thread
  static_assert(NQ * NT == TC * 32 && TC % 8 == 0 && 256 % TC == 0, "block shape");
  __shared__ float f[3][TC];
  __shared__ __attribute__((aligned(16))) unsigned short t[TC * 256];
  auto tix = [](int c, int v) { return c * 256 + ((((v >> 3) ^ (c >> 3)) & 31) << 3) + (v & 7); };
  const int v0 = blockIdx.x * 256, c0 = blockIdx.y * TC, tid = threadIdx.x;
  unsigned short *ub = dz + (long long)blockIdx.x * ts;  // this column block, [C_alloc][256]
  u32x4 in[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int q = tid + j * NT, c = c0 + (q >> 5);
    in[j] = u32x4{0u, 0u, 0u, 0u};
    if (c < rows) in[j] = *(const u32x4 *)(ub + (long long)c * 256 + (q & 31) * 8);
  }
  const int g0 = v0 / gr;  // 256 rows span at most three groups of gr >= 128
  for (int i = tid; i < 3 * TC; i += NT) {
    const int gl = i / TC, cl = i - gl * TC, c = c0 + cl, g = g0 + gl;
    float fc = 0.f;
    if (c < rows && g * gr < V)
      fc = sM[c] * fast_exp2((part[(long long)g * ld + c].x - lse[c]) * kLog2e);
    f[gl][cl] = fc;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int q = tid + j * NT, r = q >> 5, vq = (q & 31) * 8, c = c0 + r;
    const float a = f[(v0 + vq) / gr - g0][r];  // gr is a multiple of 8
    u32x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      val[e] = pack_bf16x2(a * bf16_to_f32((unsigned short)(in[j][e] & 0xFFFFu)),
                           a * bf16_to_f32((unsigned short)(in[j][e] >> 16)));
    if (c < rows) *(u32x4 *)(ub + (long long)c * 256 + vq) = val;
    *(u32x4 *)&t[tix(r, vq)] = val;  // zero for c >= rows (a = 0, u = 0)
  }
  __syncthreads();
  // dzT is read only by the dW GEMM, after the rest of its group: streamed out with
  // non-temporal stores, so that it does not displace the operands of the kernels between
  unsigned short *tb = dzt + (long long)(c0 >> 8) * tst + (long long)v0 * 256 + (c0 & 255);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int q = tid + j * NT, vr = q / (TC / 8), c8 = (q % (TC / 8)) * 8;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (unsigned)t[tix(c8 + 2 * e, vr)] | ((unsigned)t[tix(c8 + 2 * e + 1, vr)] << 16);
    __builtin_nontemporal_store(o, (u32x4 *)(tb + (long long)vr * 256 + c8));
  }
}

// fp32: a block takes 64 vocabulary rows (inside one group, as 64 divides gr) x 64 tokens.
__global__ __launch_bounds__(256) void k_rescale_dz_f32(float *dz, long long ts, const float2 *part,
                                                        long long ld, const float *lse,
                                                        const float *sM, int rows, int V, int gr) {
  constexpr int TC = 64, NQ = TC * 8 / 256;
  __shared__ float f[TC];
  const int v0 = blockIdx.x * 64, c0 = blockIdx.y * TC, tid = threadIdx.x;
  f32x8 in[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int q = tid + j * 256, r = q >> 3, v = v0 + (q & 7) * 8, c = c0 + r;
    in[j] = f32x8{};
    if (c < rows) in[j] = *(const f32x8 *)(dz + (long long)(v >> 8) * ts + c * 256 + (v & 255));
  }
  if (tid < TC) {
    const int c = c0 + tid;
    float fc = 0.f;
    if (c < rows && v0 < V)
      fc = sM[c] * fast_exp2((part[(long long)(v0 / gr) * ld + c].x - lse[c]) * kLog2e);
    f[tid] = fc;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int q = tid + j * 256, r = q >> 3, v = v0 + (q & 7) * 8, c = c0 + r;
    if (c >= rows) continue;
    f32x8 x = in[j];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= f[r];
    *(f32x8 *)(dz + (long long)(v >> 8) * ts + c * 256 + (v & 255)) = x;
  }
}

constexpr int kRescTC = 128, kRescNT = 256;  // bf16 rescale block: tokens, threads

hipError_t launch_rescale_dz(int dtype, void *dz, void *dzt, int64_t tst, const float2 *partials,
                             const float *lse, const float *sM, int64_t rows, int64_t V,
                             int64_t V_pad, int64_t C_alloc, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 1)  // C_alloc and V_pad are multiples of 256
    hipLaunchKernelGGL((k_rescale_dz_bf16<kRescTC, kRescNT>),
                       dim3((unsigned)(V_pad / 256), (unsigned)(C_alloc / kRescTC)), dim3(kRescNT),
                       0, s, (unsigned short *)dz, (long long)C_alloc * 256, (unsigned short *)dzt,
                       (long long)tst, partials, (long long)C_alloc, lse, sM, (int)rows, (int)V,
                       tile_rows(1) / 2);
  else
    hipLaunchKernelGGL(k_rescale_dz_f32, dim3((unsigned)(V_pad / 64), (unsigned)(C_alloc / 64)),
                       dim3(256), 0, s, (float *)dz, (long long)C_alloc * 256, partials,
                       (long long)C_alloc, lse, sM, (int)rows, (int)V, tile_rows(0) / 2);
  return hipGetLastError();
}

hipError_t launch_bwd_gemm(int dtype, const void *W, const void *h_c, int64_t rows, int64_t d,
                           int64_t V, const float *lse, const float *sM, void *dz, void *dzt,
                           int64_t tst, int64_t V_pad, int64_t C_alloc, hipStream_t s) {
  Operand A{W, d, (int)V, (int)d, 256};
  Operand B{h_c, d, (int)rows, (int)d, 256};
  GemmGrid G{(int)(V_pad / tile_rows(dtype)), cdiv(rows, kTile), 1, (int)d, (int)d, 0, 8};
  if (dtype == 1) {
    EpiBwdDz<1> e{dz, C_alloc * 256, lse, sM, (int)V, (int)rows, (int)V_pad,
                  (unsigned short *)dzt, tst};
    return run_gemm<1, OP_KC, OP_KC>(A, B, G, e, s);
  }
  EpiBwdDz<0> e{dz, C_alloc * 256, lse, sM, (int)V, (int)rows, (int)V_pad, nullptr, 0};
  return run_gemm<0, OP_KC, OP_KC>(A, B, G, e, s);
}

hipError_t launch_dh_gemm(int dtype, const void *dz, const void *W, const void *WT, int64_t rows,
                          int64_t d, int64_t V, int64_t V_pad, int nsplit, int64_t k_split,
                          float *part, int64_t d_pad, int64_t C_alloc, hipStream_t s) {
  // D[j][c] = sum_v W[v][j] dz[c][v]; B = dz as KC ([c][v] in 256-column blocks).
  Operand B{dz, 256, (int)rows, (int)V_pad, C_alloc * 256};
  GemmGrid G{cdiv(d, tile_rows(dtype)), cdiv(rows, kTile), nsplit, (int)k_split, (int)V_pad, 0};
  EpiDhPart e{part, C_alloc * d_pad, d_pad, (int)rows};
  if (dtype == 1) {
    // A = W^T as KC: [j][v] in blocks of 256 v, zero-padded to V_pad, so both operands
    // are read with plain 16-byte LDS reads
    Operand A{WT, 256, (int)d, (int)V_pad, d * 256};
    return run_gemm<1, OP_KC, OP_KC>(A, B, G, e, s);
  }
  Operand A{W, d, (int)d, (int)V, 256};  // A = W as MC ([v][j])
  return run_gemm<0, OP_MC, OP_KC>(A, B, G, e, s);
}

// W [V][d] bf16 -> WT blocks: element (v, j) at (v / 256) * d * 256 + j * 256 + v % 256,
// zero for V <= v < V_pad.  A block moves a 64 (v) x 64 (j) tile through LDS so that
// both the reads of W rows and the writes of WT rows are 128-byte segments.
__global__ __launch_bounds__(256) void k_transpose_w(const unsigned short *W, int V, int d,
                                                     int V_pad, unsigned short *WT) {
  __shared__ __attribute__((aligned(16))) unsigned short t[64][72];
  const int v0 = blockIdx.x * 64, j0 = blockIdx.y * 64, tid = threadIdx.x;
#pragma unroll
  for (int q = tid; q < 512; q += 256) {
    const int r = q >> 3, c8 = (q & 7) * 8;
    const int v = v0 + r, j = j0 + c8;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (v < V && j < d) val = *(const u32x4 *)(W + (long long)v * d + j);  // d % 8 == 0
    *(u32x4 *)&t[r][c8] = val;
  }
  __syncthreads();
#pragma unroll
  for (int q = tid; q < 512; q += 256) {
    const int jr = q >> 3, v8 = (q & 7) * 8;
    const int j = j0 + jr, v = v0 + v8;
    if (j >= d || v >= V_pad) continue;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (unsigned)t[v8 + 2 * e][jr] | ((unsigned)t[v8 + 2 * e + 1][jr] << 16);
    *(u32x4 *)(WT + (long long)(v >> 8) * d * 256 + (long long)j * 256 + (v & 255)) = o;
  }
}

hipError_t launch_transpose_w(const void *W, int64_t V, int64_t d, int64_t V_pad, void *WT,
                              hipStream_t s) {
  const dim3 grid((unsigned)(V_pad / 64), (unsigned)((d + 63) / 64));
  hipLaunchKernelGGL(k_transpose_w, grid, dim3(256), 0, s, (const unsigned short *)W, (int)V,
                     (int)d, (int)V_pad, (unsigned short *)WT);
  return hipGetLastError();
}

hipError_t launch_dw_gemm(int dtype, const void *dz, const void *dzt, const void *h_c,
                          const void *ht, int64_t k, int64_t d, int64_t V,
                          int64_t V_pad, int64_t C_alloc, float *dW, int accumulate,
                          hipStream_t s) {
  // D[v][j] = sum_c dz[c][v] h[c][j] over k tokens
  GemmGrid G{cdiv(V, tile_rows(dtype)), cdiv(d, kTile), 1, (int)k, (int)k, 0};
  EpiDw e{dW, (int)d, (int)V, accumulate, dtype == 1};
  if (dtype == 1) {
    // A = dzT ([v][c]), B = hT ([j][c]): both token-contiguous (KC), in blocks of 256
    // tokens ([V_pad][256] and [d][256] each)
    Operand A{dzt, 256, (int)V, (int)k, V_pad * 256};
    Operand B{ht, 256, (int)d, (int)k, d * 256};
    return run_gemm<1, OP_KC, OP_KC>(A, B, G, e, s);
  }
  // A = dz as MC ([c][v] in 256-column blocks), B = h as MC ([c][j])
  Operand A{dz, 256, (int)V_pad, (int)k, C_alloc * 256};
  Operand B{h_c, d, (int)d, (int)k, 256};
  return run_gemm<0, OP_MC, OP_MC>(A, B, G, e, s);
}

// h chunk [rows][d] -> hT (bf16), token-contiguous in blocks of 256 tokens: element (j, c)
// at ht[(c / 256) * tst + j * 256 + c % 256], columns c < ncols (zero for c >= rows),
// through a 64 x 64 LDS tile.
__global__ __launch_bounds__(256) void k_transpose_h(const unsigned short *h, int rows, int ncols,
                                                     int d, long long tst, unsigned short *ht) {
  __shared__ __attribute__((aligned(16))) unsigned short t[64][72];
  const int c0 = blockIdx.x * 64, j0 = blockIdx.y * 64, tid = threadIdx.x;
#pragma unroll
  for (int q = tid; q < 512; q += 256) {
    const int r = q >> 3, j8 = (q & 7) * 8;
    const int c = c0 + r, j = j0 + j8;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (c < rows && j < d) val = *(const u32x4 *)(h + (long long)c * d + j);  // d % 8 == 0
    *(u32x4 *)&t[r][j8] = val;
  }
  __syncthreads();
#pragma unroll
  for (int q = tid; q < 512; q += 256) {
    const int jr = q >> 3, c8 = (q & 7) * 8;
    const int j = j0 + jr, c = c0 + c8;
    if (j >= d || c >= ncols) continue;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (unsigned)t[c8 + 2 * e][jr] | ((unsigned)t[c8 + 2 * e + 1][jr] << 16);
    *(u32x4 *)(ht + (long long)(c >> 8) * tst + (long long)j * 256 + (c & 255)) = o;  // ncols % 8 == 0
  }
}

hipError_t launch_transpose_h(const void *h_c, int64_t rows, int64_t d, int64_t C_alloc,
                              void *ht, int64_t tst, hipStream_t s) {
  if (C_alloc <= 0) return hipSuccess;
  const dim3 grid((unsigned)(C_alloc / 64), (unsigned)((d + 63) / 64));
  hipLaunchKernelGGL(k_transpose_h, grid, dim3(256), 0, s, (const unsigned short *)h_c, (int)rows,
                     (int)C_alloc, (int)d, (long long)tst, (unsigned short *)ht);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------------
__global__ void k_fill_zero(unsigned int *p, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
  const long long n = (long long)(bytes / 4);
  if (n == 0) return hipSuccess;
  const int blocks = (int)(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, s, (unsigned int *)p, n);
  return hipGetLastError();
}

// Clock measurement (benchmarks only): lane 0 of each one-wave workgroup writes the
// identity of its compute unit (XCC_ID in bits 35:32, HW_ID in bits 31:0: its SE, SH and
// CU numbers are bits 15:8), the unit's shader cycle counter and the device's
// constant-rate counter.  The cycle counters of different units are not aligned, so two
// stamps are compared unit by unit.
constexpr int kHwRegXccId = 20 | ((4 - 1) << 11);   // hwreg(XCC_ID, 0, 4)
constexpr int kHwRegHwId = 4 | ((32 - 1) << 11);    // hwreg(HW_ID, 0, 32)
__global__ __launch_bounds__(64) void k_clock_stamp(unsigned long long *out) {
  if (threadIdx.x != 0) return;
  const unsigned xcc = __builtin_amdgcn_s_getreg(kHwRegXccId) & 15u;
  const unsigned hw = __builtin_amdgcn_s_getreg(kHwRegHwId);
  unsigned long long *o = out + 3 * (long long)blockIdx.x;
  o[0] = ((unsigned long long)xcc << 32) | hw;
  o[1] = clock64();
  o[2] = wall_clock64();
}

hipError_t launch_clock_stamp(unsigned long long *out, int groups, hipStream_t s) {
  hipLaunchKernelGGL(k_clock_stamp, dim3((unsigned)groups), dim3(64), 0, s, out);
  return hipGetLastError();
}

// flags[0] |= 1 for an index outside [0, V) or a probability that is negative or not
// finite; count += number of nonzero mask bytes.
__global__ void k_validate(const int32_t *idx, const float *p, long long NK, int V,
                           const uint8_t *mask, long long N, int *flags,
                           unsigned long long *count) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long g = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  int bad = 0;
  for (long long i = g; i < NK; i += stride) {
    const int v = idx[i];
    const float q = p[i];
    if (v < 0 || v >= V || !(q >= 0.f) || q == INFINITY) bad = 1;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flags, 1);
  unsigned long long c = 0;
  if (mask)
    for (long long i = g; i < N; i += stride) c += mask[i] != 0;
  __shared__ unsigned long long sh[4];
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long tot = sh[0] + sh[1] + sh[2] + sh[3];
    if (tot) atomicAdd(count, tot);
  }
}

hipError_t launch_validate(const int32_t *idx, const float *p, int64_t NK, int64_t V,
                           const uint8_t *mask, int64_t N, int *flags,
                           unsigned long long *count, hipStream_t s) {
  long long work = NK > N ? NK : N;
  int blocks = (int)((work + 255) / 256);
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_validate, dim3(blocks), dim3(256), 0, s, idx, p, (long long)NK, (int)V,
                     mask, (long long)N, flags, count);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Buckets of teacher hits per output tile of the logits GEMMs (a counting sort).
// Key of entry (row r, k) of a chunk: (idx / tv) * ntn + (r >> 8).  A block takes 8 rows,
// which share one token tile, and aggregates its keys in LDS before touching global
// counters (the Zipf head puts about half of all hits in the first vocabulary tile).
// With more than kBucketLdsBins vocabulary tiles the blocks count in global memory.
// ---------------------------------------------------------------------------------
constexpr int kBucketLdsBins = 8192;

__global__ void k_bucket_count(const int32_t *idx, int rows, int K, int tv, int ntm, int ntn,
                               int *counts) {
  extern __shared__ int hist[];
  const int t = threadIdx.x;
  const bool lds = ntm <= kBucketLdsBins;
  const int r0 = blockIdx.x * 8;
  const int n = min(8, rows - r0) * K;
  const int32_t *ip = idx + (long long)r0 * K;
  const int tn = r0 >> 8;
  if (lds) {
    for (int i = t; i < ntm; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int e = t; e < n; e += blockDim.x)
      if ((unsigned)ip[e] < (unsigned)(ntm * tv)) atomicAdd(&hist[ip[e] / tv], 1);
    __syncthreads();
    for (int i = t; i < ntm; i += blockDim.x)
      if (hist[i]) atomicAdd(&counts[i * ntn + tn], hist[i]);
  } else {
    for (int e = t; e < n; e += blockDim.x)
      if ((unsigned)ip[e] < (unsigned)(ntm * tv)) atomicAdd(&counts[(ip[e] / tv) * ntn + tn], 1);
  }
}

// One block of 1024 threads: offsets = exclusive scan of counts; counts and cursors are
// cleared for the next chunk.
__global__ void k_bucket_scan(int *counts, int nkeys, int *offsets, int *cursor) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (nkeys + 1023) / 1024;
  const int b = min(nkeys, t * per), e = min(nkeys, b + per);
  int s = 0;
  for (int i = b; i < e; ++i) s += counts[i];
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - s;
  for (int i = b; i < e; ++i) {
    offsets[i] = run;
    run += counts[i];
    counts[i] = 0;
    cursor[i] = 0;
  }
  if (t == 1023) offsets[nkeys] = part[1023];
}

__global__ void k_bucket_fill(const int32_t *idx, int rows, int K, int tv, int ntm, int ntn,
                              const int *offsets, int *cursor, unsigned *entries) {
  extern __shared__ int sh[];
  const int t = threadIdx.x;
  const bool lds = ntm <= kBucketLdsBins;
  int *hist = sh, *base = sh + ntm;
  const int r0 = blockIdx.x * 8;
  const int n = min(8, rows - r0) * K;
  const int32_t *ip = idx + (long long)r0 * K;
  const int tn = r0 >> 8;
  if (lds) {
    for (int i = t; i < ntm; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int e = t; e < n; e += blockDim.x)
      if ((unsigned)ip[e] < (unsigned)(ntm * tv)) atomicAdd(&hist[ip[e] / tv], 1);
    __syncthreads();
    for (int i = t; i < ntm; i += blockDim.x)
      if (hist[i]) {
        base[i] = offsets[i * ntn + tn] + atomicAdd(&cursor[i * ntn + tn], hist[i]);
        hist[i] = 0;
      }
    __syncthreads();
  }
  for (int e = t; e < n; e += blockDim.x) {
    const int v = ip[e];
    // negative: outside this vocabulary shard; past the padded vocabulary: an invalid entry
    // that the validation scan reports (never bucketed, so never addressed)
    if ((unsigned)v >= (unsigned)(ntm * tv)) continue;
    const int bin = v / tv, q = e / K, r = r0 + q, k = e - q * K;
    const int pos = lds ? base[bin] + atomicAdd(&hist[bin], 1)
                        : offsets[bin * ntn + tn] + atomicAdd(&cursor[bin * ntn + tn], 1);
    entries[pos] = (unsigned)(r & 255) | ((unsigned)(v - bin * tv) << 8) | ((unsigned)k << 17);
  }
}

hipError_t launch_buckets(const int32_t *idx_c, int64_t rows, int32_t K, int tv, int ntv,
                          int *counts, int *cursor, int *offsets, unsigned *entries,
                          hipStream_t s) {
  const int ntm = ntv, ntn = (int)((rows + kTile - 1) / kTile);
  const int blocks = (int)((rows + 7) / 8);
  const bool lds = ntm <= kBucketLdsBins;
  hipLaunchKernelGGL(k_bucket_count, dim3(blocks), dim3(256), lds ? ntm * 4 : 0, s, idx_c,
                     (int)rows, (int)K, tv, ntm, ntn, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(1024), 0, s, counts, ntm * ntn, offsets, cursor);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bucket_fill, dim3(blocks), dim3(256), lds ? 2 * ntm * 4 : 0, s, idx_c,
                     (int)rows, (int)K, tv, ntm, ntn, offsets, cursor, entries);
  return hipGetLastError();
}

// 64 token rows per block of 16 waves; lane = row.  Wave w folds the (max, sum-exp)
// partials t = w, w+16, ... (eight loads in flight per lane) and the teacher entries
// k = w, w+16, ...; wave 0 then folds the 16 results in a fixed order.
constexpr int kCombWaves = 16;
__global__ __launch_bounds__(64 * kCombWaves) void k_combine(
    const float2 *part, int n_lse, long long ld, const float *zg, const float *p,
    const uint8_t *mask, int rows, int K, const float *inv_count_p, float *lse_out, float *sM_out,
    float *s_out, double *rowterm, float *row_loss, float *row_lse) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = blockIdx.x * 64 + lane;
  const bool live = r < rows;
  float m = -INFINITY, sum = 0.f;
  if (live) {
    for (int t0 = w; t0 < n_lse; t0 += 8 * kCombWaves) {
      float2 q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = t0 + kCombWaves * u;
        q[u] = t < n_lse ? part[(long long)t * ld + r] : make_float2(-INFINITY, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (q[u].y == 0.f) continue;
        if (q[u].x > m) {
          sum = sum * fast_exp2((m - q[u].x) * kLog2e) + q[u].y;
          m = q[u].x;
        } else {
          sum += q[u].y * fast_exp2((q[u].x - m) * kLog2e);
        }
      }
    }
  }
  __shared__ float sm[kCombWaves][64], ss[kCombWaves][64];
  __shared__ double sd[3][kCombWaves][64];
  sm[w][lane] = m;
  ss[w][lane] = sum;
  double H = 0.0, PZ = 0.0, Ms = 0.0;
  if (live) {
    for (int k = w; k < K; k += kCombWaves) {
      const double q = p[(long long)r * K + k];
      Ms += q;
      PZ += q * (double)zg[(long long)r * K + k];
      if (q > 0.0) H += q * log(q);
    }
  }
  sd[0][w][lane] = H;
  sd[1][w][lane] = PZ;
  sd[2][w][lane] = Ms;
  __syncthreads();
  if (w == 0 && live) {
    float M = sm[0][lane];
    for (int i = 1; i < kCombWaves; ++i) M = fmaxf(M, sm[i][lane]);
    float S = 0.f;
    for (int i = 0; i < kCombWaves; ++i)
      if (ss[i][lane] != 0.f) S += ss[i][lane] * fast_exp2((sm[i][lane] - M) * kLog2e);
    const float lse = M + logf(S);
    double h = 0.0, pz = 0.0, ms = 0.0;
    for (int i = 0; i < kCombWaves; ++i) {
      h += sd[0][i][lane];
      pz += sd[1][i][lane];
      ms += sd[2][i][lane];
    }
    const double ell = h - pz + ms * (double)lse;
    const bool on = mask ? mask[r] != 0 : true;
    lse_out[r] = lse;
    const float inv_count = inv_count_p[0];
    sM_out[r] = on ? (float)(ms * (double)inv_count) : 0.f;
    s_out[r] = on ? inv_count : 0.f;
    rowterm[r] = on ? ell : 0.0;
    if (row_loss) row_loss[r] = on ? (float)ell : 0.f;
    if (row_lse) row_lse[r] = lse;
  }
}

hipError_t launch_combine(const float2 *partials, int64_t n_lse, int64_t ld_part,
                          const float *zg, const float *p_c, const uint8_t *mask_c,
                          int64_t rows, int32_t K, const float *inv_count, float *lse, float *sM,
                          float *srow, double *rowterm, float *row_loss, float *row_lse,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3(cdiv(rows, 64)), dim3(64 * kCombWaves), 0, s, partials,
                     (int)n_lse,
                     (long long)ld_part, zg, p_c, mask_c, (int)rows, (int)K, inv_count, lse, sM,
                     srow, rowterm, row_loss, row_lse);
  return hipGetLastError();
}

// Backward-only path: per token, sM = g * mask * M / count and s = g * mask / count,
// with M = sum_k p summed in float64 in exactly the order k_combine uses (wave w takes
// k = w, w+16, ...; the 16 wave sums are added in wave order), so that with g = 1 the
// backward matches the fused call bit for bit.  g is read from device memory.
__global__ __launch_bounds__(64 * kCombWaves) void k_row_scale(const float *p,
                                                               const uint8_t *mask, int rows,
                                                               int K, const float *inv_count_p,
                                                               const float *g, float *sM_out,
                                                               float *s_out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = blockIdx.x * 64 + lane;
  const bool live = r < rows;
  double Ms = 0.0;
  if (live)
    for (int k = w; k < K; k += kCombWaves) Ms += (double)p[(long long)r * K + k];
  __shared__ double sd[kCombWaves][64];
  sd[w][lane] = Ms;
  __syncthreads();
  if (w == 0 && live) {
    double ms = 0.0;
    for (int i = 0; i < kCombWaves; ++i) ms += sd[i][lane];
    const bool on = mask ? mask[r] != 0 : true;
    const float gg = g[0], inv_count = inv_count_p[0];
    sM_out[r] = on ? (float)(ms * (double)inv_count) * gg : 0.f;
    s_out[r] = on ? inv_count * gg : 0.f;
  }
}

hipError_t launch_row_scale(const float *p_c, const uint8_t *mask_c, int64_t rows, int32_t K,
                            const float *inv_count, const float *g, float *sM, float *srow,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_row_scale, dim3(cdiv(rows, 64)), dim3(64 * kCombWaves), 0, s, p_c, mask_c,
                     (int)rows, (int)K, inv_count, g, sM, srow);
  return hipGetLastError();
}

// acc[0] += sum of rowterm[0..rows) in a fixed order (deterministic).
__global__ void k_accum_loss(const double *rowterm, int rows, double *acc) {
  __shared__ double sh[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < rows; i += 256) s += rowterm[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) acc[0] += sh[0];
}

hipError_t launch_accum_loss(const double *rowterm, int64_t rows, double *acc, hipStream_t s) {
  hipLaunchKernelGGL(k_accum_loss, dim3(1), dim3(256), 0, s, rowterm, (int)rows, acc);
  return hipGetLastError();
}

__global__ void k_finalize(const double *acc, const unsigned long long *count_p, float *loss) {
  if (threadIdx.x == 0) {
    const unsigned long long count = count_p[0];
    loss[0] = count > 0 ? (float)(acc[0] / (double)count) : 0.f;
  }
}

hipError_t launch_finalize(const double *acc, const unsigned long long *count, float *loss,
                           hipStream_t s) {
  hipLaunchKernelGGL(k_finalize, dim3(1), dim3(64), 0, s, acc, count, loss);
  return hipGetLastError();
}

// The number of counted tokens (the mask's nonzero bytes, or every token without a mask)
// and its reciprocal, on the device, for the kernels that scale by them: with them there,
// the sequence after the validation scan needs nothing back on the host.
__global__ void k_count_prep(const unsigned long long *mask_count, int has_mask, long long N,
                             unsigned long long *count, float *inv_count) {
  if (threadIdx.x == 0) {
    const unsigned long long c = has_mask ? mask_count[0] : (unsigned long long)N;
    count[0] = c;
    inv_count[0] = c > 0 ? (float)(1.0 / (double)c) : 0.f;
  }
}

hipError_t launch_count_prep(const unsigned long long *mask_count, bool has_mask, int64_t N,
                             unsigned long long *count, float *inv_count, hipStream_t s) {
  hipLaunchKernelGGL(k_count_prep, dim3(1), dim3(64), 0, s, mask_count, has_mask ? 1 : 0,
                     (long long)N, count, inv_count);
  return hipGetLastError();
}

// status[0] = bad_code if the validation scan raised its flag, else 0.
__global__ void k_status_out(const int *flags, int bad_code, int32_t *status) {
  if (threadIdx.x == 0) status[0] = flags[0] ? bad_code : 0;
}

hipError_t launch_status_out(const int *flags, int32_t bad_code, int32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(k_status_out, dim3(1), dim3(64), 0, s, flags, (int)bad_code, status);
  return hipGetLastError();
}

// Upstream gradient of the loss applied to gradients computed for g = 1: dh_out =
// g * dh32 rounded once to the output type, and dW *= g in place.  g is read on the device;
// with g == 1 the product is exact, so dW is left alone (no traffic) and dh_out is dh32
// rounded.  Four elements per thread (16-byte loads; the tail element by element).
template <int DT>
__global__ __launch_bounds__(256) void k_scale_grads(const float *g, const float *dh32,
                                                     void *dh_out, long long n_dh, float *dW,
                                                     long long n_dW) {
  const float gv = g[0];
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long t0 = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  for (long long q = t0; q * 4 < n_dh; q += stride) {
    const long long i = q * 4;
    if (i + 4 <= n_dh) {
      const f32x4 x = *(const f32x4 *)(dh32 + i);
      if (DT == 1) {
        *(u32x2 *)((unsigned short *)dh_out + i) =
            u32x2{pack_bf16x2(gv * x[0], gv * x[1]), pack_bf16x2(gv * x[2], gv * x[3])};
      } else {
        *(f32x4 *)((float *)dh_out + i) = f32x4{gv * x[0], gv * x[1], gv * x[2], gv * x[3]};
      }
    } else {
      for (long long j = i; j < n_dh; ++j) {
        if (DT == 1) ((unsigned short *)dh_out)[j] = f32_to_bf16(gv * dh32[j]);
        else ((float *)dh_out)[j] = gv * dh32[j];
      }
    }
  }
  if (gv == 1.f) return;
  for (long long q = t0; q * 4 < n_dW; q += stride) {
    const long long i = q * 4;
    if (i + 4 <= n_dW) {
      f32x4 x = *(const f32x4 *)(dW + i);
      *(f32x4 *)(dW + i) = f32x4{gv * x[0], gv * x[1], gv * x[2], gv * x[3]};
    } else {
      for (long long j = i; j < n_dW; ++j) dW[j] *= gv;
    }
  }
}

hipError_t launch_scale_grads(int dtype, const float *g, const float *dh32, void *dh_out,
                              int64_t n_dh, float *dW, int64_t n_dW, hipStream_t s) {
  const long long q = ((n_dh > n_dW ? n_dh : n_dW) + 3) / 4;
  int blocks = (int)((q + 255) / 256);
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  if (dtype == 1)
    hipLaunchKernelGGL(k_scale_grads<1>, dim3(blocks), dim3(256), 0, s, g, dh32, dh_out,
                       (long long)n_dh, dW, (long long)n_dW);
  else
    hipLaunchKernelGGL(k_scale_grads<0>, dim3(blocks), dim3(256), 0, s, g, dh32, dh_out,
                       (long long)n_dh, dW, (long long)n_dW);
  return hipGetLastError();
}

// dz[r][idx[r][k]] -= s[r] * (sum of p over the row's entries with that index).
// One wave per row.  The row's indices first go into a per-wave hash table in LDS: when
// none repeats (the usual case), every entry updates its own element.  Otherwise lane k
// compares its index with every entry of the row (64 at a time through shuffles): the
// first entry of each distinct index sums the probabilities of its later duplicates in
// order and does the update, so no two threads touch the same element.
constexpr int kScatTab = 512;  // hash slots per wave (rows of up to 256 entries use it)

template <int DT>
__device__ __forceinline__ void scatter_one(void *dz, long long ts, unsigned short *dzt,
                                            long long tst, int r, int v, float delta) {
  if (DT == 1) {
    unsigned short *q = (unsigned short *)dz + (long long)(v >> 8) * ts + r * 256 + (v & 255);
    const unsigned short nv = f32_to_bf16(bf16_to_f32(*q) - delta);
    *q = nv;
    dzt[(long long)(r >> 8) * tst + (long long)v * 256 + (r & 255)] = nv;
  } else {
    float *q = (float *)dz + (long long)(v >> 8) * ts + r * 256 + (v & 255);
    *q = *q - delta;
  }
}

template <int DT>
__global__ __launch_bounds__(256) void k_scatter(void *dz, long long ts, unsigned short *dzt,
                                                 long long tst, const int32_t *idx,
                                                 const float *p, const float *srow, int rows,
                                                 int K, int vlim) {
  __shared__ int tab[4][kScatTab];
  const int w = threadIdx.x >> 6;
  const int r = blockIdx.x * 4 + w, lane = threadIdx.x & 63;
  if (r >= rows) return;
  const float sr = srow[r];
  if (sr == 0.f) return;
  const int32_t *ir = idx + (long long)r * K;
  const float *pr = p + (long long)r * K;
  // repeated index test; an index outside [0, vlim) is skipped everywhere (negative: outside
  // this vocabulary shard; vlim or more: an invalid entry that the validation scan reports)
  bool dup = K > kScatTab / 2;
  if (!dup) {
    for (int i = lane; i < kScatTab; i += 64) tab[w][i] = -1;
    for (int k = lane; k < K; k += 64) {
      const int v = ir[k];
      if ((unsigned)v >= (unsigned)vlim) continue;
      unsigned hs = ((unsigned)v * 2654435761u) >> 23;  // 9 bits
      for (int probe = 0; probe < kScatTab; ++probe) {  // a free slot always exists
        const int old = atomicCAS(&tab[w][hs], -1, v);
        if (old == -1) break;
        if (old == v) {
          dup = true;
          break;
        }
        hs = (hs + 1) & (kScatTab - 1);
      }
    }
    dup = __ballot(dup) != 0;
  }
  if (!dup) {
    for (int k = lane; k < K; k += 64) {
      const int v = ir[k];
      if ((unsigned)v < (unsigned)vlim) scatter_one<DT>(dz, ts, dzt, tst, r, v, sr * pr[k]);
    }
    return;
  }
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int k = k0 + lane;
    const bool has = k < K;
    const int v = has ? ir[k] : -1;
    float tot = has ? pr[k] : 0.f;
    bool first = has && (unsigned)v < (unsigned)vlim;
    for (int j0 = 0; j0 < K; j0 += 64) {
      const int jl = j0 + lane;
      const int vjl = jl < K ? ir[jl] : -1;
      const float pjl = jl < K ? pr[jl] : 0.f;
      const int n = min(64, K - j0);
      for (int t = 0; t < n; ++t) {
        const int vj = __shfl(vjl, t, 64);
        const float pj = __shfl(pjl, t, 64);
        const int j = j0 + t;
        if (vj == v) {
          if (j < k) first = false;
          else if (j > k) tot += pj;
        }
      }
    }
    if (first) scatter_one<DT>(dz, ts, dzt, tst, r, v, sr * tot);
  }
}

hipError_t launch_scatter(int dtype, void *dz, void *dzt, int64_t tst, int64_t C_alloc,
                          const int32_t *idx_c, const float *p_c, const float *srow, int64_t rows,
                          int32_t K, int64_t V_pad, hipStream_t s) {
  const int blocks = (int)((rows + 3) / 4);
  if (dtype == 1)
    hipLaunchKernelGGL(k_scatter<1>, dim3(blocks), dim3(256), 0, s, dz, (long long)C_alloc * 256,
                       (unsigned short *)dzt, (long long)tst, idx_c, p_c, srow, (int)rows,
                       (int)K, (int)V_pad);
  else
    hipLaunchKernelGGL(k_scatter<0>, dim3(blocks), dim3(256), 0, s, dz, (long long)C_alloc * 256,
                       (unsigned short *)nullptr, 0LL, idx_c, p_c, srow, (int)rows, (int)K,
                       (int)V_pad);
  return hipGetLastError();
}

// dh[r][j..j+3] = sum over splits of part[s][r][j..j+3], rounded once to the output type.
template <int DT>
__global__ void k_dh_reduce(const float *part, int nsplit, long long split_stride, long long ld,
                            int rows, int d, void *dh) {
  const long long g = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  const int q = d / 4;
  if (g >= (long long)rows * q) return;
  const int r = (int)(g / q), j = (int)(g - (long long)r * q) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < nsplit; ++sp) acc += *(const f32x4 *)(part + sp * split_stride + r * ld + j);
  if (DT == 1) {
    u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *(u32x2 *)((unsigned short *)dh + (long long)r * d + j) = pk;
  } else {
    *(f32x4 *)((float *)dh + (long long)r * d + j) = acc;
  }
}

hipError_t launch_dh_reduce(int dtype, const float *part, int nsplit, int64_t C_alloc,
                            int64_t d_pad, int64_t rows, int64_t d, void *dh, hipStream_t s) {
  const long long n = rows * (d / 4);
  const int blocks = (int)((n + 255) / 256);
  if (dtype == 1)
    hipLaunchKernelGGL(k_dh_reduce<1>, dim3(blocks), dim3(256), 0, s, part, nsplit,
                       (long long)(C_alloc * d_pad), (long long)d_pad, (int)rows, (int)d, dh);
  else
    hipLaunchKernelGGL(k_dh_reduce<0>, dim3(blocks), dim3(256), 0, s, part, nsplit,
                       (long long)(C_alloc * d_pad), (long long)d_pad, (int)rows, (int)d, dh);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Vocabulary shards (one GPU's share of a tensor-parallel output head)
// ---------------------------------------------------------------------------------
// loc[r][k] = idx - v0 when v0 <= idx < v0 + Vs, else -1; zg of outside entries = 0.
__global__ void k_localize_idx(const int32_t *idx, long long n, int v0, int Vs, int32_t *loc,
                               float *zg) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    const int v = idx[i] - v0;
    const bool in = v >= 0 && v < Vs;
    loc[i] = in ? v : -1;
    if (!in) zg[i] = 0.f;
  }
}

hipError_t launch_localize_idx(const int32_t *idx_c, int64_t rows, int32_t K, int64_t v0,
                               int64_t Vs, int32_t *loc, float *zg_c, hipStream_t s) {
  const long long n = rows * (long long)K;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(k_localize_idx, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s, idx_c, n,
                     (int)v0, (int)Vs, loc, zg_c);
  return hipGetLastError();
}

// Per token of a shard: max and sum exp(z - max) over the shard's logits (folded from
// the forward GEMM's per-slice partials, as in k_combine) and sum_k p * z over the
// teacher entries inside the shard (zg is 0 for the others).
__global__ __launch_bounds__(64 * kCombWaves) void k_shard_stats(
    const float2 *part, int n_lse, long long ld, const float *zg, const float *p, int rows,
    int K, float *m_out, float *s_out, float *pz_out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = blockIdx.x * 64 + lane;
  const bool live = r < rows;
  float m = -INFINITY, sum = 0.f;
  if (live) {
    for (int t = w; t < n_lse; t += kCombWaves) {
      const float2 q = part[(long long)t * ld + r];
      if (q.y == 0.f) continue;
      if (q.x > m) {
        sum = sum * fast_exp2((m - q.x) * kLog2e) + q.y;
        m = q.x;
      } else {
        sum += q.y * fast_exp2((q.x - m) * kLog2e);
      }
    }
  }
  __shared__ float sm[kCombWaves][64], ss[kCombWaves][64];
  __shared__ double sd[kCombWaves][64];
  sm[w][lane] = m;
  ss[w][lane] = sum;
  double PZ = 0.0;
  if (live)
    for (int k = w; k < K; k += kCombWaves)
      PZ += (double)p[(long long)r * K + k] * (double)zg[(long long)r * K + k];
  sd[w][lane] = PZ;
  __syncthreads();
  if (w == 0 && live) {
    float M = sm[0][lane];
    for (int i = 1; i < kCombWaves; ++i) M = fmaxf(M, sm[i][lane]);
    float S = 0.f;
    for (int i = 0; i < kCombWaves; ++i)
      if (ss[i][lane] != 0.f) S += ss[i][lane] * fast_exp2((sm[i][lane] - M) * kLog2e);
    double pz = 0.0;
    for (int i = 0; i < kCombWaves; ++i) pz += sd[i][lane];
    m_out[r] = M;
    s_out[r] = S;
    pz_out[r] = (float)pz;
  }
}

hipError_t launch_shard_stats(const float2 *partials, int64_t n_lse, int64_t ld_part,
                              const float *zg, const float *p_c, int64_t rows, int32_t K,
                              float *m_out, float *s_out, float *pz_out, hipStream_t s) {
  hipLaunchKernelGGL(k_shard_stats, dim3(cdiv(rows, 64)), dim3(64 * kCombWaves), 0, s, partials,
                     (int)n_lse, (long long)ld_part, zg, p_c, (int)rows, (int)K, m_out, s_out,
                     pz_out);
  return hipGetLastError();
}

// Combine of G shards' statistics per token: lse = M + log sum_g s_g exp(m_g - M),
// l = sum_k p log p - sum_g pz_g + (sum_k p) lse; rowterm = mask ? l : 0.
__global__ void k_shard_combine(const float *m, const float *sx, const float *pz, int G,
                                long long N, const float *p, const uint8_t *mask, int K,
                                float *row_lse, float *row_loss, double *rowterm) {
  const long long r = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (r >= N) return;
  float M = -INFINITY;
  for (int g = 0; g < G; ++g) M = fmaxf(M, m[g * N + r]);
  double S = 0.0, PZ = 0.0;
  for (int g = 0; g < G; ++g) {
    if (sx[g * N + r] != 0.f) S += (double)sx[g * N + r] * (double)fast_exp2((m[g * N + r] - M) * kLog2e);
    PZ += (double)pz[g * N + r];
  }
  const float lse = M + logf((float)S);
  double H = 0.0, Ms = 0.0;
  for (int k = 0; k < K; ++k) {
    const double q = p[r * K + k];
    Ms += q;
    if (q > 0.0) H += q * log(q);
  }
  const double ell = H - PZ + Ms * (double)lse;
  const bool on = mask ? mask[r] != 0 : true;
  if (row_lse) row_lse[r] = lse;
  if (row_loss) row_loss[r] = on ? (float)ell : 0.f;
  rowterm[r] = on ? ell : 0.0;
}

hipError_t launch_shard_combine(const float *m, const float *sx, const float *pz, int G,
                                int64_t N, const float *p, const uint8_t *mask, int32_t K,
                                float *row_lse, float *row_loss, double *rowterm, hipStream_t s) {
  hipLaunchKernelGGL(k_shard_combine, dim3(cdiv(N, 256)), dim3(256), 0, s, m, sx, pz, G,
                     (long long)N, p, mask, (int)K, row_lse, row_loss, rowterm);
  return hipGetLastError();
}

}  // namespace kd
