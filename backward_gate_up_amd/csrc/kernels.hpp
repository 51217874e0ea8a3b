// kernels.hpp -- the kernels of the fused SwiGLU MLP for gfx950, their
// launchers and the per-dtype drivers run_fwd / run_bwd / run_infer.
// Included by swiglu_mlp.hip (the C ABI, which only declares the drivers)
// and by instantiate.hip, which is compiled once per (dtype, entry point)
// and defines one driver each, so the kernels build in parallel.
//
// The method is the one of "[RFC] Full-pipeline SwiGLU MLP with
// forward/backward co-optimization" (Liger-Kernel issue #1347), section
// "Summary". Its steps map onto launches of one MFMA tile engine
// (gemm_tile.hpp), each with its own operand layouts and epilogue:
//
//  stage  computes                                  M x N x K    A op / B op
//  0      G = X Wg, U = X Wu, A = SiLU(G) U         T x H x D    KC / MC (two B sources)
//  1      Y = A Wd                                  T x D x H    KC / MC
//  2      dA = dY Wd^T -> dG, dU over G, U          T x H x D    KC / KC
//  3      dWd = A^T dY                              H x D x T    MC / MC
//  4      [dWg | dWu] = X^T [dG | dU]               D x H x T    MC / MC (grid z = 2)
//  5      dI = dG Wg^T + dU Wu^T                    T x D x 2H   KC / KC (two K halves)
//  6,7    no-grad: stage 0 writing only A, then stage 1
//
// Numerics: fp32 accumulation; each stored value is rounded once to the
// storage type. The forward epilogue is the one-round program of "Scope
// one-round FP32 SwiGLU to the exact Qwen3.5 contract" (xorl PR #51, review
// thread), applied to the stored (already rounded) g and u so that the saved
// A, G and U are mutually consistent; the backward epilogue likewise works in
// fp32 from the fp32 dA accumulator and the stored g and u, rounding dG and
// dU once.
#pragma once
#include <hip/hip_runtime.h>
#include <atomic>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "gemm_tile.hpp"
#include "gemm_ring.hpp"
#include "gemm_skinny.hpp"
#include "gemm_stream.hpp"
#include "swiglu_mlp.h"

namespace swiglu {

enum Kind { GATEUP = 0, PLAIN = 1, DSWIGLU = 2, DX = 3 };

struct KArgs {
  Operand a0, a1;  // A operand; a1 = second K half (DX)
  Operand b0, b1;  // B operand; b1 = second N half (GATEUP), second K half (DX), z = 1 (PLAIN)
  char* c0;        // PLAIN/DX: C; GATEUP: A plane; DSWIGLU: G plane (in/out)
  char* c1;        // PLAIN: C for z = 1; GATEUP: G plane; DSWIGLU: U plane (in/out)
  char* c2;        // GATEUP: U plane
  int64_t ldc;     // elements
  int M, N;        // output extent (GATEUP: N = H)
  int tiles_m, tiles_n;
  int store_gu;    // GATEUP: write the G and U planes (training) or A only (no-grad)
  int planes;      // PLAIN: number of (B source, output) planes (1 or 2)
  int plane_a;     // PLAIN, two planes: plane 1 takes its A operand from a1 (B shared) instead of B from b1
  int group_m;     // M-tiles per group of the tile walk (tile_coords); 0 = 8
  int two_round;   // GATEUP: A = rnd(rnd(SiLU(g)) * u) instead of rnd(SiLU(g) * u)
  float* P;        // PLAIN, split K: fp32 partial tiles, 256 x 256 each (else nullptr)
  int kchunk;      // PLAIN, split K: K stages per piece
  int n_full;      // weight-gradient launch: items (plane-major tiles) run whole
  int ksplit;      // weight-gradient launch: pieces per split tile
  int n_split;     // weight-gradient launch: tiles split over K (items n_full ..)
  unsigned* zero_ctr;  // no-grad gate/up: arrival counters of the down launch to clear (or nullptr)
  int n_zero;          // ... and how many
};

// Workgroup 0 of a no-grad gate/up launch clears the arrival counters that
// the down launch after it on the stream counts on (see stream_gemm).
__device__ __forceinline__ void clear_counters(const KArgs& g) {
  if (g.zero_ctr && blockIdx.x == 0)
    for (int i = threadIdx.x; i < g.n_zero; i += blockDim.x) g.zero_ctr[i] = 0u;
}

// Logistic function sigma(g) = 1 / (1 + exp(-g)) in fp32, from a stored gate
// value. IEEE form: expf from the device math library and IEEE division
// (fp32 mode). Fast form (bf16/fp16 storage): exp(-g) = 2^(-g log2 e) with
// the hardware base-2 exponential, then the hardware reciprocal; both are
// about 1 fp32 ulp, far below half an ulp of the 16-bit result, so the value
// rounded to bf16/fp16 is the correctly rounded one except within ~1e-5
// relative of a rounding tie (then 1 ulp away). For g <= -80 the reciprocal
// would near the fp32 denormal range, where the hardware approximations
// flush; there sigma(g) equals e^g to fp32 precision (e^g < 2e-35), taken as
// 2^(g log2 e + 64) * 2^-64: the exponential stays in the normal range and
// the exact power-of-two scaling rounds once, into the denormals where the
// value lies there. Both forms share one exponential and a select, with no
// branch (the epilogues evaluate this for every element of a tile).
__device__ __forceinline__ float sigmoid_ieee(float g) { return 1.0f / (1.0f + expf(-g)); }
__device__ __forceinline__ float sigmoid_fast(float g) {
  const float x = g * 1.44269504088896341f;  // g log2 e
  const bool lo = g <= -80.0f;
  const float e = __builtin_amdgcn_exp2f(lo ? x + 64.0f : -x);
  return lo ? e * 0x1p-64f : __builtin_amdgcn_rcpf(1.0f + e);
}
// The fast form for g > -80 (and g = -Inf, NaN) only.
__device__ __forceinline__ float sigmoid_fast_hi(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
}
template <class E>
__device__ __forceinline__ float sigmoid_f32(float g) {
  if constexpr (E::kBytes == 4) return sigmoid_ieee(g);
  else return sigmoid_fast(g);
}

// A from the stored gate and up values g, u. One-round program: SiLU(g) * u
// evaluated in fp32 and rounded once to the storage type ("Scope one-round
// FP32 SwiGLU to the exact Qwen3.5 contract", review thread). Two-round
// (historical) program of the same page: SiLU(g) rounded to the storage type
// first, then the product rounded again. In fp32 storage the two coincide.
template <class E>
__device__ __forceinline__ typename E::elem swiglu_a(float gf, float uf, int two_round) {
  const float silu = gf * sigmoid_f32<E>(gf);
  if (two_round) return E::from_f32(E::to_f32(E::from_f32(silu)) * uf);
  return E::from_f32(silu * uf);
}

// sigma of four gate values of one lane. 16-bit storage: the branch-free fast
// form, except that the g <= -80 range is taken only when some lane of the
// wave has such a value among its four (a wave-uniform branch, almost never
// taken), so the common case skips that range's instructions.
template <class E>
__device__ __forceinline__ void sigmoid4(const float (&g)[4], float (&sg)[4]) {
  if constexpr (E::kBytes == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sg[e] = sigmoid_ieee(g[e]);
  } else {
    const float gmin = fminf(fminf(g[0], g[1]), fminf(g[2], g[3]));
    if (__any(gmin <= -80.0f)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sg[e] = sigmoid_fast(g[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) sg[e] = sigmoid_fast_hi(g[e]);
    }
  }
}

// A from g, sigma(g) and u: the one-round (TWO = false) or two-round program
// of swiglu_a, with the program fixed at compile time.
template <class E, bool TWO>
__device__ __forceinline__ typename E::elem swiglu_a_s(float gf, float sg, float uf) {
  const float silu = gf * sg;
  if constexpr (TWO) return E::from_f32(E::to_f32(E::from_f32(silu)) * uf);
  else return E::from_f32(silu * uf);
}

// dG and dU from the fp32 dA and the stored gate and up values g, u, in fp32
// (the caller rounds each once): dU = dA SiLU(g), dG = dA u SiLU'(g), with
// SiLU'(g) = sigma (1 + g (1 - sigma)) = sigma + SiLU(g) (1 - sigma).
template <class E>
__device__ __forceinline__ void dswiglu(float da, float gf, float uf, float& dg, float& du) {
  const float sg = sigmoid_f32<E>(gf);
  const float silu = gf * sg;
  du = da * silu;
  dg = (da * uf) * fmaf(silu, 1.0f - sg, sg);
}
// The same for four elements of one lane, with sigmoid4.
template <class E>
__device__ __forceinline__ void dswiglu4(const float (&da)[4], const float (&gf)[4], const float (&uf)[4],
                                         float (&dg)[4], float (&du)[4]) {
  float sg[4];
  sigmoid4<E>(gf, sg);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float silu = gf[e] * sg[e];
    du[e] = da[e] * silu;
    dg[e] = (da[e] * uf[e]) * fmaf(silu, 1.0f - sg[e], sg[e]);
  }
}

// Epilogue of one tile. acc[i][j][r] holds output
//   m = m0 + a_rows[i] + (lane & 31),
//   n = (column base of subtile j) + (r / 4) * 8 + (lane / 32) * 4 + r % 4,
// so each lane stores runs of 4 consecutive n (8 bytes in bf16).
template <class E, int BM, int BN, int KIND, int TM, int TN>
__device__ __forceinline__ void epilogue(const KArgs& g, char* C, f32x16_t (&acc)[TM][TN], int m0, int n0,
                                         const int (&a_rows)[TM], const int (&b_rows)[TN], int wn, int lane) {
  constexpr int EB = E::kBytes;
  using V4 = typename E::vec4;
  const int ml = lane & 31;
  const int nl = (lane >> 5) * 4;
  if constexpr (KIND == GATEUP) {
    constexpr int H2 = TN / 2;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + a_rows[i] + ml;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < H2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * (BN / 4) + j * 32 + q * 8 + nl;
          if (n >= g.N) continue;
          V4 gv, uv, av;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            typename E::elem gs = E::from_f32(acc[i][j][q * 4 + e]);
            typename E::elem us = E::from_f32(acc[i][j + H2][q * 4 + e]);
            float gf = E::to_f32(gs), uf = E::to_f32(us);
            gv[e] = gs;
            uv[e] = us;
            av[e] = swiglu_a<E>(gf, uf, g.two_round);
          }
          const int64_t off = ((int64_t)m * g.ldc + n) * EB;
          *(V4*)(g.c0 + off) = av;
          if (g.store_gu) {
            *(V4*)(g.c1 + off) = gv;
            *(V4*)(g.c2 + off) = uv;
          }
        }
      }
    }
  } else if constexpr (KIND == DSWIGLU) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + a_rows[i] + ml;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + b_rows[j] + q * 8 + nl;
          if (n >= g.N) continue;
          const int64_t off = ((int64_t)m * g.ldc + n) * EB;
          V4 gv = *(const V4*)(g.c0 + off);
          V4 uv = *(const V4*)(g.c1 + off);
          V4 dg, du;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float dgf, duf;
            dswiglu<E>(acc[i][j][q * 4 + e], E::to_f32(gv[e]), E::to_f32(uv[e]), dgf, duf);
            dg[e] = E::from_f32(dgf);
            du[e] = E::from_f32(duf);
          }
          *(V4*)(g.c0 + off) = dg;
          *(V4*)(g.c1 + off) = du;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + a_rows[i] + ml;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + b_rows[j] + q * 8 + nl;
          if (n >= g.N) continue;
          V4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = E::from_f32(acc[i][j][q * 4 + e]);
          *(V4*)(C + ((int64_t)m * g.ldc + n) * EB) = v;
        }
      }
    }
  }
}

// One output tile: the K loop and the epilogue. bid is the tile's index in
// its launch group, bz the plane (PLAIN with two B sources / outputs).
template <class E, int BM, int BN, int AL, int BL, int KIND>
__device__ __forceinline__ void gemm_tile(const KArgs& g, char* smem, int bid, int bz) {
  using Geo = Geometry<E, BM, BN, AL, BL>;
  constexpr int EB = E::kBytes;
  constexpr int BK = E::kBK;
  constexpr int TM = Geo::TM, TN = Geo::TN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(bid, g.tiles_m, g.tiles_n, g.group_m > 0 ? g.group_m : 8, tm, tn);
  const int m0 = tm * BM;
  const int n0 = (KIND == GATEUP) ? tn * (BN / 2) : tn * BN;

  Operand A = g.a0, B = g.b0;
  char* C = g.c0;
  if (KIND == PLAIN && bz == 1) {
    if (g.plane_a) A = g.a1;
    else B = g.b1;
    C = g.c1;
  }

  int a_rows[TM], b_rows[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_rows[i] = wm * Geo::WTM + i * 32;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if constexpr (KIND == GATEUP) {
      // G columns in LDS rows [0, BN/2), U columns in [BN/2, BN); wave wn
      // owns the same BN/4 hidden units of both.
      constexpr int H2 = TN / 2;
      b_rows[j] = (j < H2 ? 0 : BN / 2) + wn * (BN / 4) + (j % H2) * 32;
    } else {
      b_rows[j] = wn * Geo::WTN + j * 32;
    }
  }

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

  TileLoader<E, BM, AL> la;
  // GATEUP fills the B tile from two sources of BN/2 rows each.
  constexpr int RB = (KIND == GATEUP) ? BN / 2 : BN;
  TileLoader<E, RB, BL, BN> lb0;
  TileLoader<E, RB, BL, BN> lb1;

  const int nk1 = (A.k + BK - 1) / BK;
  const int nk = (KIND == DX) ? 2 * nk1 : nk1;

  if constexpr (KIND == DX) {
    la.init(g.a0, m0, tid);  // both K halves share the layout and extents
    lb0.init(g.b0, n0, tid);
  } else {
    la.init(A, m0, tid);
    lb0.init(B, n0, tid);
    if constexpr (KIND == GATEUP) lb1.init(g.b1, n0, tid);
  }
  auto load = [&](int kt) {
    if constexpr (KIND == DX) {
      bool second = kt >= nk1;
      int k0 = (second ? kt - nk1 : kt) * BK;
      la.load(second ? g.a1 : g.a0, m0, k0, tid);
      lb0.load(second ? g.b1 : g.b0, n0, k0, tid);
    } else {
      int k0 = kt * BK;
      la.load(A, m0, k0, tid);
      lb0.load(B, n0, k0, tid);
      if constexpr (KIND == GATEUP) lb1.load(g.b1, n0, k0, tid);
    }
  };
  auto store = [&](int stage) {
    char* sa = smem + stage * Geo::STAGE;
    char* sb = sa + Geo::A_BYTES;
    la.store(sa, tid);
    lb0.store(sb, tid, 0);
    if constexpr (KIND == GATEUP) lb1.store(sb, tid, BN / 2);
  };

  // Software pipeline (per K stage kt, LDS stage cur, other stage nxt):
  //   sub-step 0..3 each issue the MFMAs of one sub-step while the operand
  //   fragments of the following sub-step are read from LDS; during sub-step
  //   2 the registers holding tile kt+1 are written to stage nxt; one barrier
  //   then publishes stage nxt, the global loads of tile kt+2 are issued, and
  //   sub-step 3 runs while the first fragments of stage nxt are read.
  // Every LDS stage is read only between the barrier that follows its
  // writes and the barrier that precedes its next overwrite.
  using F = Frags<E, BM, BN, AL, BL, TM, TN>;
  constexpr int NM = F::kMfma, NR = F::kReads;
  constexpr int NW = TileLoader<E, BM, AL>::PER_THREAD + TileLoader<E, RB, BL, BN>::PER_THREAD *
                                                             (KIND == GATEUP ? 2 : 1);
  F f0, f1;
  // One K stage; ST: write tile kt+1 to the other LDS stage, LD: issue the
  // global loads of tile kt+2, NX: read the first fragments of tile kt+1.
  // The flags are compile-time so that the steady-state body has no branch
  // (branches would split the MFMA/DS interleave into separate blocks).
  auto body = [&](int kt, auto ST, auto LD, auto NX) {
    const int cur = kt & 1;
    const char* sa = smem + cur * Geo::STAGE;
    const char* sb = sa + Geo::A_BYTES;
    const char* na = smem + (cur ^ 1) * Geo::STAGE;
    const char* nb = na + Geo::A_BYTES;
    f1.read(sa, sb, a_rows, b_rows, 1, lane);
    f0.mma(acc);
    interleave_mfma_ds<NM, NR>();
    f0.read(sa, sb, a_rows, b_rows, 2, lane);
    f1.mma(acc);
    interleave_mfma_ds<NM, NR>();
    f1.read(sa, sb, a_rows, b_rows, 3, lane);
    if constexpr (decltype(ST)::value) store(cur ^ 1);
    f0.mma(acc);
    interleave_mfma_ds<NM, NR + (decltype(ST)::value ? NW : 0)>();
    if constexpr (decltype(ST)::value) __syncthreads();
    if constexpr (decltype(LD)::value) load(kt + 2);
    if constexpr (decltype(NX)::value) f0.read(na, nb, a_rows, b_rows, 0, lane);
    f1.mma(acc);
    interleave_mfma_ds<NM, decltype(NX)::value ? NR : 0>();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (nk > 0) {
    load(0);
    store(0);
    if (nk > 1) load(1);
    __syncthreads();
    f0.read(smem, smem + Geo::A_BYTES, a_rows, b_rows, 0, lane);
    int kt = 0;
    for (; kt + 2 < nk; ++kt) body(kt, T_{}, T_{}, T_{});
    if (kt + 1 < nk) body(kt++, T_{}, F_{}, T_{});
    body(kt, F_{}, F_{}, F_{});
  }

  epilogue<E, BM, BN, KIND, TM, TN>(g, C, acc, m0, n0, a_rows, b_rows, wn, lane);
}

// One launch = one stage. STAGE only names the kernel (one symbol per
// stage in profiles). Grid: x = tiles, z = planes.
template <class E, int BM, int BN, int AL, int BL, int KIND, int STAGE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mlp_gemm(const KArgs g) {
  __shared__ __attribute__((aligned(16))) char smem[Geometry<E, BM, BN, AL, BL>::LDS];
  if constexpr (KIND == GATEUP) clear_counters(g);
  gemm_tile<E, BM, BN, AL, BL, KIND>(g, smem, blockIdx.x, blockIdx.z);
}

// Two independent stages in one launch: the first group's tiles (g1, with
// g1.planes planes) take the lowest workgroup ids, so long-K tiles can be
// dispatched first and the second group's short tiles fill in behind them;
// this removes the wave-quantization tail of launches with few tiles.
template <class E, int AL1, int BL1, int KIND1, int AL2, int BL2, int KIND2, int STAGE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mlp_gemm_pair(const KArgs g1, const KArgs g2) {
  constexpr int L1 = Geometry<E, 256, 256, AL1, BL1>::LDS, L2 = Geometry<E, 256, 256, AL2, BL2>::LDS;
  __shared__ __attribute__((aligned(16))) char smem[L1 > L2 ? L1 : L2];
  const int nt1 = g1.tiles_m * g1.tiles_n;
  const int n1 = nt1 * g1.planes;
  const int b = blockIdx.x;
  if (b < n1)
    gemm_tile<E, 256, 256, AL1, BL1, KIND1>(g1, smem, b % nt1, b / nt1);
  else
    gemm_tile<E, 256, 256, AL2, BL2, KIND2>(g2, smem, b - n1, 0);
}



// ---------------------------------------------------------------------------
// Epilogue of the ring kernels: results go through LDS so that every global
// access is 16 bytes per lane over whole rows (each store instruction covers
// full 128-byte lines). Each wave uses its own 32 KiB ring array, so after
// one barrier (all waves done with the K loop) no further synchronisation is
// needed: LDS operations of one wave complete in order.
// A wave's output block is `rows` x W elements (W = 64 or 128); in LDS row r
// holds W*2 bytes and its 16-byte chunk c sits at chunk c ^ (r % (W/8)).
// ---------------------------------------------------------------------------
// Cache-policy operand of the buffer store builtins that selects the
// non-temporal (nt) hint on gfx950.
constexpr int kNonTemporalPolicy = 2;

template <class E, int W>
struct WaveBlock {
  static constexpr int NC = W / 8;       // 16-byte chunks per row
  static constexpr int RB = W * 2;       // bytes per row
  char* buf;
  __device__ __forceinline__ int off(int r, int col) const {
    return r * RB + (((col >> 3) ^ (r & (NC - 1))) << 4) + (col & 7) * 2;
  }
  // four consecutive elements at (r, col), col % 4 == 0
  __device__ __forceinline__ void put4(int r, int col, typename E::vec4 v) const {
    *(typename E::vec4*)(buf + off(r, col)) = v;
  }
  __device__ __forceinline__ typename E::vec4 get4(int r, int col) const {
    return *(const typename E::vec4*)(buf + off(r, col));
  }
  // Row chunks i = b .. b + NB - 1 of this lane (chunk i covers 16-byte
  // chunk (i * 64 + lane) % NC of row (i * 64 + lane) / NC), read from LDS
  // back to back so that one LDS latency covers the batch.
  template <int NB>
  __device__ __forceinline__ void read_chunks(u32x4_t (&v)[NB], int b, int lane) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int g = (b + i) * 64 + lane, r = g / NC, c = g % NC;
      v[i] = *(const u32x4_t*)(buf + r * RB + ((c ^ (r & (NC - 1))) << 4));
    }
  }
  // Store those chunks to dst(row0 + r, col0 + c), masked to M x N. One
  // store instruction per chunk, whatever the mask: chunks outside the
  // matrix take an offset past the descriptor, which drops them, so a
  // caller can count the stores in vmcnt. Non-temporal: results are not
  // re-read by this kernel, and streaming them past L2 leaves it to the
  // operand tiles (gate/up writes three [T, H] planes: measured 2.5-4 %
  // faster, the other stages unchanged).
  template <int NB>
  __device__ __forceinline__ void write_chunks(const u32x4_t (&v)[NB], int b, char* dst, int64_t ld, int row0,
                                               int col0, int M, int N, int lane) const {
    const int64_t first = (int64_t)row0 * ld + col0;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(dst + first * 2, ((int64_t)M * ld - first) * 2);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int g = (b + i) * 64 + lane, r = g / NC, c = g % NC;
      const bool in = row0 + r < M && col0 + c * 8 < N;
      const uint32_t off = in ? (uint32_t)((r * (int)ld + c * 8) * 2) : kOOB;
      __builtin_amdgcn_raw_buffer_store_b128(v[i], rs, off, 0, kNonTemporalPolicy);
    }
  }
  // store rows [0, ROWS) to dst(row0 + r, col0 + c), masked to M x N:
  // ROWS * NC / 64 store instructions, in batches of up to eight chunks
  template <int ROWS>
  __device__ __forceinline__ void store(char* dst, int64_t ld, int row0, int col0, int M, int N, int lane) const {
    constexpr int NI = ROWS * NC / 64;
    constexpr int NB = NI < 8 ? NI : 8;
    static_assert(NI % NB == 0, "whole batches");
#pragma unroll
    for (int b = 0; b < NI; b += NB) {
      u32x4_t v[NB];
      read_chunks<NB>(v, b, lane);
      write_chunks<NB>(v, b, dst, ld, row0, col0, M, N, lane);
    }
  }
  // load rows [0, rows) from src(row0 + r, col0 + c) with direct-to-LDS
  // loads (1 KiB per instruction: RB-byte rows, swizzle applied on the global
  // side). Rows past M read as zeros; columns past N feed unstored outputs.
  // Non-temporal: each element is read once (dA's G/U blocks), so the loads
  // need not displace the operand panels other CUs share in L2 (dA 2.3 %
  // faster, same-box A/B).
  __device__ __forceinline__ void load(const char* src, int64_t ld, int64_t plane_bytes, int row0, int col0,
                                       int rows, int lane) const {
    const char* base = src + ((int64_t)row0 * ld + col0) * 2;
    const int64_t avail = plane_bytes - ((int64_t)row0 * ld + col0) * 2;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, avail);
    constexpr int RPI = 1024 / RB;  // rows per instruction
    const int rl = lane / NC, p = lane % NC;
#pragma unroll 4
    for (int t = 0; t < rows / RPI; ++t) {
      const int r = t * RPI + rl;
      const int c = p ^ (r & (NC - 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ring::lds_void_t*)(buf + t * 1024), 16,
                                               (uint32_t)(r * (int)ld * 2 + c * 16), 0, 0, kNonTemporalPolicy);
    }
  }
};

template <class E, int KIND>
__device__ __forceinline__ void ring_epilogue(const KArgs& g, char* C, f32x4_t (&acc)[8][8], int m0, int n0,
                                              int wm, int wn, int lane, char* wbuf) {
  using V4 = typename E::vec4;
  // acc[i][j] holds this wave's row 16 i + ml, columns 16 j + nl .. + 3
  const int ml = lane & 15;
  const int nl = (lane >> 4) * 4;
  ring::lds_barrier();  // every wave is done reading the K-loop stages
  if constexpr (KIND == GATEUP) {
    // wave block: 128 rows (t) x 64 hidden units, planes A, G, U
    WaveBlock<E, 64> pa{wbuf}, pg{wbuf + 16384};
    const int r0 = m0 + wm * 128, c0 = n0 + wn * 64;
    // A and G into LDS; the program (one- or two-round) is fixed per launch
    // (column blocks 0-3 of the wave are G, 4-7 the matching U)
    auto stage_ag = [&](auto two) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          V4 gv, av;
          float gf[4], uf[4], sg[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gv[e] = E::from_f32(acc[i][j][e]);
            gf[e] = E::to_f32(gv[e]);
            uf[e] = E::to_f32(E::from_f32(acc[i][j + 4][e]));
          }
          sigmoid4<E>(gf, sg);
#pragma unroll
          for (int e = 0; e < 4; ++e) av[e] = swiglu_a_s<E, decltype(two)::value>(gf[e], sg[e], uf[e]);
          pa.put4(i * 16 + ml, j * 16 + nl, av);
          pg.put4(i * 16 + ml, j * 16 + nl, gv);
        }
    };
    if (g.two_round) stage_ag(std::true_type{});
    else stage_ag(std::false_type{});
    pa.template store<128>(g.c0, g.ldc, r0, c0, g.M, g.N, lane);
    if (g.store_gu) {
      pg.template store<128>(g.c1, g.ldc, r0, c0, g.M, g.N, lane);
      WaveBlock<E, 64> pu{wbuf};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          V4 uv;
#pragma unroll
          for (int e = 0; e < 4; ++e) uv[e] = E::from_f32(acc[i][j + 4][e]);
          pu.put4(i * 16 + ml, j * 16 + nl, uv);
        }
      pu.template store<128>(g.c2, g.ldc, r0, c0, g.M, g.N, lane);
    }
  } else if constexpr (KIND == DSWIGLU) {
    // wave block: 128 rows x 128 hidden units, in eight parts of 16 rows
    // (one MFMA row block each). The G and U rows of a part are loaded into
    // LDS, turned into dG and dU in place (this tile's own (t, h) block only)
    // and stored back. Four LDS slots of 8 KiB: while part q is computed and
    // stored the loads of parts q + 1 .. q + 3 are in flight, and those of
    // q + 4 go into q's slot as soon as q's results have been read back into
    // registers, before q's stores (the loads wait on memory latency, so
    // more of them in flight). A part is 8 loads (4 per plane) and 8 stores
    // (4 per plane, out-of-range chunks dropped by the descriptor rather than
    // skipped), and vmcnt counts this wave's loads and stores in issue order:
    // L0 L1 L2 L3 | L4 S0 | L5 S1 | L6 S2 | L7 S3 | S4 | S5 | S6 | S7. So
    // waiting for the loads of part q never waits for a store: 24, 32, 40,
    // 48, 56, 48, 40 and 32 operations issued after them may stay
    // outstanding.
    const int64_t plane_bytes = (int64_t)g.M * g.ldc * 2;
    const int c0 = n0 + wn * 128;
    auto issue = [&](int q) {
      char* slot = wbuf + (q & 3) * 8192;
      const int r0 = m0 + wm * 128 + q * 16;
      WaveBlock<E, 128>{slot}.load(g.c0, g.ldc, plane_bytes, r0, c0, 16, lane);
      WaveBlock<E, 128>{slot + 4096}.load(g.c1, g.ldc, plane_bytes, r0, c0, 16, lane);
    };
    issue(0);
    issue(1);
    issue(2);
    issue(3);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q == 0) ring::wait_vmcnt<24>();
      else if (q == 1 || q == 7) ring::wait_vmcnt<32>();
      else if (q == 2 || q == 6) ring::wait_vmcnt<40>();
      else if (q == 3 || q == 5) ring::wait_vmcnt<48>();
      else ring::wait_vmcnt<56>();
      WaveBlock<E, 128> pg{wbuf + (q & 3) * 8192}, pu{wbuf + (q & 3) * 8192 + 4096};
      // every G and U value of the part first (one LDS latency), then the
      // math
      V4 gv[8], uv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        gv[j] = pg.get4(ml, j * 16 + nl);
        uv[j] = pu.get4(ml, j * 16 + nl);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = j * 16 + nl;
        V4 dg, du;
        float da[4], gf[4], uf[4], dgf[4], duf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          da[e] = acc[q][j][e];
          gf[e] = E::to_f32(gv[j][e]);
          uf[e] = E::to_f32(uv[j][e]);
        }
        dswiglu4<E>(da, gf, uf, dgf, duf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dg[e] = E::from_f32(dgf[e]);
          du[e] = E::from_f32(duf[e]);
        }
        pg.put4(ml, c, dg);
        pu.put4(ml, c, du);
      }
      u32x4_t vg[4], vu[4];
      pg.template read_chunks<4>(vg, 0, lane);
      pu.template read_chunks<4>(vu, 0, lane);
      // the slot's contents are in registers: part q + 4 may load into it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (q + 4 < 8) issue(q + 4);
      const int r0 = m0 + wm * 128 + q * 16;
      pg.template write_chunks<4>(vg, 0, g.c0, g.ldc, r0, c0, g.M, g.N, lane);
      pu.template write_chunks<4>(vu, 0, g.c1, g.ldc, r0, c0, g.M, g.N, lane);
    }
  } else {
    // PLAIN / DX: 128 x 128 block of C
    WaveBlock<E, 128> pc{wbuf};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        V4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = E::from_f32(acc[i][j][e]);
        pc.put4(i * 16 + ml, j * 16 + nl, v);
      }
    pc.template store<128>(C, g.ldc, m0 + wm * 128, n0 + wn * 128, g.M, g.N, lane);
  }
}

// One 256 x 256 output tile on the direct-to-LDS ring (16-bit types; see
// gemm_ring.hpp). st0..st3 are the four stage arrays; separate arrays let the
// compiler wait for exactly the stage a read needs.
// A piece of a split weight-gradient tile: the dense 256 x 256 fp32 partial
// tile `piece` (rows and columns past the matrix hold sums of zero operands;
// the reduction skips them); each lane holds 4 consecutive columns.
__device__ __forceinline__ void ring_partial_store(const KArgs& g, const f32x4_t (&acc)[8][8], int piece,
                                                   const int (&a_rows)[8], const int (&b_rows)[8], int lane) {
  float* P = g.P + (int64_t)piece * 65536;
  const int ml = lane & 15, nl = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) *(f32x4_t*)(P + (a_rows[i] + ml) * 256 + b_rows[j] + nl) = acc[i][j];
}

template <class E, int AL, int BL, int KIND>
__device__ __forceinline__ void ring_tile(const KArgs& g, char* st0, char* st1, char* st2, char* st3, int bid,
                                          int bz, int ks = 0, int piece = -1) {
  using namespace ring;
  static_assert(E::kBytes == 2, "the ring pipeline is for bf16/fp16");
  // the wave index is uniform within a wave; readfirstlane lets the compiler
  // keep it (and the DMA destinations and descriptors derived from it) in
  // scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(bid, g.tiles_m, g.tiles_n, g.group_m > 0 ? g.group_m : 8, tm, tn);
  const int m0 = tm * 256;
  const int n0 = (KIND == GATEUP) ? tn * 128 : tn * 256;
  Operand A = g.a0, B = g.b0;
  char* C = g.c0;
  if (KIND == PLAIN && bz == 1) {
    if (g.plane_a) A = g.a1;
    else B = g.b1;
    C = g.c1;
  }
  // this wave's 16-row blocks of A and 16-column blocks of B (gate/up:
  // four of Wg, then the same four of Wu)
  int a_rows[8], b_rows[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a_rows[i] = wm * 128 + i * 16;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    b_rows[j] = (KIND == GATEUP) ? (j < 4 ? 0 : 128) + wn * 64 + (j & 3) * 16 : wn * 128 + j * 16;

  // zeroed inside the K loop, after its prologue: the fence makes the zeros
  // opaque, and live across the prologue they were spilled, not rebuilt
  f32x4_t acc[8][8];
  auto zero_acc = [&] {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{};
    acc_fence<true>(acc);
  };

  Dma<AL> da;
  Dma<BL> db;
  da.init(A, m0, wave, lane);
  // gate/up with K-major weights: B rows [0, 128) from Wg, [128, 256) from Wu
  db.init(B, n0, wave, lane, KIND == GATEUP && BL == KC);
  const int nk1 = (A.k + BK - 1) / BK;
  // split K (a piece of a weight-gradient tile): stages [sb, sb + nk) of
  // the K loop, written as fp32 partial tile `piece`
  const bool split = KIND == PLAIN && piece >= 0;
  const int sb = split ? ks * g.kchunk : 0;
  const int nk = (KIND == DX) ? 2 * nk1 : (split ? (nk1 - sb < g.kchunk ? nk1 - sb : g.kchunk) : nk1);
  char* st[4] = {st0, st1, st2, st3};

  // descriptors (K-major) and M/N-major sources built once per tile: [0]
  // the operand (DX: its first half, (dG, Wg)), [1] DX's second half
  using DA = Dma<AL>;
  using DB = Dma<BL>;
  __amdgpu_buffer_rsrc_t ra[2], rb[2];
  typename DA::McSrc ma[2];
  typename DB::McSrc mb[2];
  if constexpr (AL == KC) {
    ra[0] = DA::kc_rsrc(KIND == DX ? g.a0 : A, m0);
    ra[1] = KIND == DX ? DA::kc_rsrc(g.a1, m0) : ra[0];
  } else {
    ma[0] = DA::mc_src(A, m0, A, m0 + 128, wave);
  }
  if constexpr (BL == KC) {
    // gate/up: B rows [0, 128) from Wg (waves 0-1), [128, 256) from Wu
    const Operand& b0 = (KIND == GATEUP && wave >= 2) ? g.b1 : (KIND == DX ? g.b0 : B);
    rb[0] = DB::kc_rsrc(b0, n0);
    rb[1] = KIND == DX ? DB::kc_rsrc(g.b1, n0) : rb[0];
  } else if constexpr (KIND == GATEUP) {
    mb[0] = DB::mc_src(g.b0, n0, g.b1, n0, wave);
  } else if constexpr (KIND == DX) {
    mb[0] = DB::mc_src(g.b0, n0, g.b0, n0 + 128, wave);
    mb[1] = DB::mc_src(g.b1, n0, g.b1, n0 + 128, wave);
  } else {
    mb[0] = DB::mc_src(B, n0, B, n0 + 128, wave);
  }

  auto slot = [&](int i) -> char* {
    i &= 3;
    return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : st3;
  };
  // The K loop, compiled with (KT) and without the K-tail checks of K-major
  // loads; the epilogue after it exists once.
  auto kloop = [&](auto KTc) {
    constexpr bool KT = decltype(KTc)::value;
    constexpr int PW = Geo<BK>::PPW;  // loads per wave per operand tile
    // this wave's loads [j0, j1) of A / B of stage s into stage array stg
    auto issue_a = [&](int s, char* stg, int j0, int j1) {
      if constexpr (KIND == DX) {
        const bool h = s >= nk1;
        da.template issue_kcr<KT>(h ? ra[1] : ra[0], h ? g.a1.k : g.a0.k, (h ? s - nk1 : s) * BK, stg, wave, lane,
                                  j0, j1);
      } else if constexpr (AL == KC) {
        da.template issue_kcr<KT>(ra[0], A.k, (sb + s) * BK, stg, wave, lane, j0, j1);
      } else {
        da.issue_mcs(ma[0], (sb + s) * BK, stg, wave, j0, j1);
      }
    };
    auto issue_b = [&](int s, char* stg, int j0, int j1) {
      if constexpr (KIND == DX) {
        const bool h = s >= nk1;
        if constexpr (BL == KC)
          db.template issue_kcr<KT>(h ? rb[1] : rb[0], h ? g.b1.k : g.b0.k, (h ? s - nk1 : s) * BK, stg + OPB, wave,
                                    lane, j0, j1);
        else db.issue_mcs(h ? mb[1] : mb[0], (h ? s - nk1 : s) * BK, stg + OPB, wave, j0, j1);
      } else if constexpr (BL == KC) {
        db.template issue_kcr<KT>(rb[0], KIND == GATEUP ? (wave >= 2 ? g.b1.k : g.b0.k) : B.k, (sb + s) * BK,
                                  stg + OPB, wave, lane, j0, j1);
      } else {
        db.issue_mcs(mb[0], (sb + s) * BK, stg + OPB, wave, j0, j1);
      }
    };
    auto issue = [&](int s, char* stg) {
      issue_a(s, stg, 0, PW);
      issue_b(s, stg, 0, PW);
    };
    // M/N-major sources: the first K row of the stage a step loads (s + 4),
    // carried from step to step (a 64-bit add, not a multiply, per stage)
    constexpr bool MA = AL == MC && KIND != DX, MB = BL == MC && KIND != DX;
    const char* pa = nullptr;
    const char* pb = nullptr;
    if constexpr (MA) pa = ma[0].base + (int64_t)((sb + 4) * BK) * ma[0].rowb;
    if constexpr (MB) pb = mb[0].base + (int64_t)((sb + 4) * BK) * mb[0].rowb;
    auto issue_a4 = [&](int s, char* stg, int j0, int j1) {
      if constexpr (MA) da.issue_mcp(ma[0], pa, (sb + s) * BK, stg, wave, j0, j1);
      else issue_a(s, stg, j0, j1);
    };
    auto issue_b4 = [&](int s, char* stg, int j0, int j1) {
      if constexpr (MB) db.issue_mcp(mb[0], pb, (sb + s) * BK, stg + OPB, wave, j0, j1);
      else issue_b(s, stg, j0, j1);
    };
    auto advance = [&] {
      if constexpr (MA) pa += DA::stride(ma[0]);
      if constexpr (MB) pb += DB::stride(mb[0]);
    };
    using F = RingFrags<E, AL, BL>;
    F fr;
    // Stage s is one step. Its fragments are read from Q2 of stage s - 1 to
    // Q1 of stage s; between Q1 and Q2 this wave's loads of stage s + 1 have
    // landed (those of s + 2 and s + 3 may be in flight) and a barrier
    // publishes every wave's. Every wave is then done with stage s's slot,
    // so Q2 and Q3 issue the loads of stage s + 4 into it.
    if (nk > 0) {
      issue(0, st0);
      if (nk > 1) issue(1, st1);
      if (nk > 2) issue(2, st2);
      if (nk > 3) issue(3, st3);
      if (nk > 3) wait_vmcnt<3 * L>();
      else if (nk > 2) wait_vmcnt<2 * L>();
      else if (nk > 1) wait_vmcnt<L>();
      else wait_vmcnt<0>();
      lds_barrier();
      fr.template read_a<0>(st0, a_rows, 0, lane);
      fr.template read_b<0>(st0 + OPB, b_rows, 0, lane);
    }
    zero_acc();
    // steady state (stage s + 4 exists): static slots and parities
    auto step = [&](int s, auto J) {
      constexpr int j = decltype(J)::value;
      char* cur = st[j];
      char* nx = st[(j + 1) & 3];
      fr.template step<(j & 1), PW, true>(
          acc, cur, cur + OPB, 0, nx, nx + OPB, 0, a_rows, b_rows, lane,
          [&] {
            wait_vmcnt<2 * L>();
            lds_barrier();
          },
          [&](int q, int k) {
            if (q == 2) issue_a4(s + 4, cur, k, k + 1);
            else if (q == 3) issue_b4(s + 4, cur, k, k + 1);
          });
      advance();
    };
    int s = 0;
    for (; s + 8 <= nk; s += 4) {
      step(s, std::integral_constant<int, 0>{});
      step(s + 1, std::integral_constant<int, 1>{});
      step(s + 2, std::integral_constant<int, 2>{});
      step(s + 3, std::integral_constant<int, 3>{});
    }
    // Last stages: the same order with run-time slot selection and counts,
    // two at a time so that each step keeps a fixed parity (one copy of the
    // MFMA sequence per parity). The last step also reads the fragments of
    // a step that does not come; its slot holds an older stage and no load
    // writes it any more.
    auto tail = [&](int s, auto P) {
      char* cur = slot(s);
      char* nx = slot(s + 1);
      const bool more = s + 4 < nk;
      auto mid = [&] {
        if (s + 1 < nk) {
          const int last = nk - 1 < s + 3 ? nk - 1 : s + 3;  // last stage issued so far
          if (last - (s + 1) >= 2) wait_vmcnt<2 * L>();
          else if (last - (s + 1) == 1) wait_vmcnt<L>();
          else wait_vmcnt<0>();
          lds_barrier();
        }
      };
      auto iss = [&](int q, int k) {
        if (more) {
          if (q == 2) issue_a4(s + 4, cur, k, k + 1);
          else if (q == 3) issue_b4(s + 4, cur, k, k + 1);
        }
      };
      fr.template step<decltype(P)::value, PW, true>(acc, cur, cur + OPB, 0, nx, nx + OPB, 0, a_rows, b_rows, lane,
                                                      mid, iss);
      advance();
    };
    for (; s + 2 <= nk; s += 2) {
      tail(s, std::integral_constant<int, 0>{});
      tail(s + 1, std::integral_constant<int, 1>{});
    }
    if (s < nk) tail(s, std::integral_constant<int, 0>{});
  };
  constexpr bool kc = AL == KC || BL == KC;
  if (kc && A.k % BK == 0) kloop(std::false_type{});
  else kloop(std::integral_constant<bool, kc>{});
  acc_fence<false>(acc);
  if constexpr (KIND == PLAIN) {
    if (split) {
      ring_partial_store(g, acc, piece, a_rows, b_rows, lane);
      return;
    }
  }
  ring_epilogue<E, KIND>(g, C, acc, m0, n0, wm, wn, lane, slot(wave));
}

// 64 values of K per stage with the operand tiles in a ring of five 32 KiB
// LDS arrays: operand tile t (A of stage s is t = 2s, B is t = 2s + 1) lives
// in array t % 5. While stage s is multiplied, its two arrays are busy, A of
// stage s + 1 is already on its way, and the two arrays stage s - 1 used take
// B of stage s + 1 and A of stage s + 2: every K-major row is still one whole
// 128-byte line per request, and the loads of A run a stage and a half ahead.
// Before the last sub-step of stage s this wave's loads up to B of stage s + 1
// are waited for (vmcnt counts this wave's loads in issue order), then a
// barrier publishes stage s + 1.
template <class E, int AL, int BL, int KIND>
__device__ __forceinline__ void ring5_tile(const KArgs& g, char* const (&R)[5], int bid, int bz, int ks = 0,
                                           int piece = -1) {
  using namespace ring;
  constexpr int BK2 = 64;
  static_assert(E::kBytes == 2, "the ring pipeline is for bf16/fp16");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(bid, g.tiles_m, g.tiles_n, g.group_m > 0 ? g.group_m : 8, tm, tn);
  const int m0 = tm * 256;
  const int n0 = (KIND == GATEUP) ? tn * 128 : tn * 256;
  Operand A = g.a0, B = g.b0;
  char* C = g.c0;
  if (KIND == PLAIN && bz == 1) {
    if (g.plane_a) A = g.a1;
    else B = g.b1;
    C = g.c1;
  }
  int a_rows[8], b_rows[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a_rows[i] = wm * 128 + i * 16;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    b_rows[j] = (KIND == GATEUP) ? (j < 4 ? 0 : 128) + wn * 64 + (j & 3) * 16 : wn * 128 + j * 16;

  // zeroed inside the K loop, after its prologue: the fence makes the zeros
  // opaque, and live across the prologue they were spilled, not rebuilt
  f32x4_t acc[8][8];
  auto zero_acc = [&] {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{};
    acc_fence<true>(acc);
  };

  Dma<AL, BK2> da;
  Dma<BL, BK2> db;
  da.init(A, m0, wave, lane);
  db.init(B, n0, wave, lane, KIND == GATEUP && BL == KC);
  const int nk1 = (A.k + BK2 - 1) / BK2;
  // split K (a piece of a weight-gradient tile): stages [sb, sb + nk) of
  // the K loop, written as fp32 partial tile `piece`
  const bool split = KIND == PLAIN && piece >= 0;
  const int sb = split ? ks * g.kchunk : 0;
  const int nk = (KIND == DX) ? 2 * nk1 : (split ? (nk1 - sb < g.kchunk ? nk1 - sb : g.kchunk) : nk1);
  constexpr int NT = Geo<BK2>::PPW;  // loads per wave per operand tile
  // descriptors (K-major) and M/N-major sources built once per tile: [0]
  // the operand (DX: its first half, (dG, Wg)), [1] DX's second half (dU, Wu)
  using DA = Dma<AL, BK2>;
  using DB = Dma<BL, BK2>;
  __amdgpu_buffer_rsrc_t ra[2], rb[2];
  typename DA::McSrc ma[1];
  typename DB::McSrc mb[2];
  if constexpr (AL == KC) {
    ra[0] = DA::kc_rsrc(KIND == DX ? g.a0 : A, m0);
    ra[1] = KIND == DX ? DA::kc_rsrc(g.a1, m0) : ra[0];
  } else {
    ma[0] = DA::mc_src(A, m0, A, m0 + 128, wave);
  }
  if constexpr (BL == KC) {
    // gate/up: B rows [0, 128) from Wg (waves 0-1), [128, 256) from Wu
    const Operand& b0 = (KIND == GATEUP && wave >= 2) ? g.b1 : (KIND == DX ? g.b0 : B);
    rb[0] = DB::kc_rsrc(b0, n0);
    rb[1] = KIND == DX ? DB::kc_rsrc(g.b1, n0) : rb[0];
  } else if constexpr (KIND == GATEUP) {
    mb[0] = DB::mc_src(g.b0, n0, g.b1, n0, wave);
  } else if constexpr (KIND == DX) {
    mb[0] = DB::mc_src(g.b0, n0, g.b0, n0 + 128, wave);
    mb[1] = DB::mc_src(g.b1, n0, g.b1, n0 + 128, wave);
  } else {
    mb[0] = DB::mc_src(B, n0, B, n0 + 128, wave);
  }

  auto reg = [&](int t) -> char* {
    t %= 5;
    return t == 0 ? R[0] : t == 1 ? R[1] : t == 2 ? R[2] : t == 3 ? R[3] : R[4];
  };
  // The K loop, compiled with (KT) and without the K-tail checks of K-major
  // loads; the epilogue after it exists once.
  auto kloop = [&](auto KTc) {
    constexpr bool KT = decltype(KTc)::value;
    // pieces [j0, j1) of this wave's share of A of stage s
    auto issue_a = [&](int s, char* t, int j0 = 0, int j1 = NT) {
      if constexpr (KIND == DX) {
        const bool h = s >= nk1;
        da.template issue_kcr<KT>(h ? ra[1] : ra[0], h ? g.a1.k : g.a0.k, (h ? s - nk1 : s) * BK2, t, wave, lane, j0, j1);
      } else if constexpr (AL == KC) {
        da.template issue_kcr<KT>(ra[0], A.k, (sb + s) * BK2, t, wave, lane, j0, j1);
      } else {
        da.issue_mcs(ma[0], (sb + s) * BK2, t, wave, j0, j1);
      }
    };
    auto issue_b = [&](int s, char* t, int j0 = 0, int j1 = NT) {
      if constexpr (KIND == DX) {
        const bool h = s >= nk1;
        if constexpr (BL == KC)
          db.template issue_kcr<KT>(h ? rb[1] : rb[0], h ? g.b1.k : g.b0.k, (h ? s - nk1 : s) * BK2, t, wave, lane, j0,
                                    j1);
        else db.issue_mcs(h ? mb[1] : mb[0], (h ? s - nk1 : s) * BK2, t, wave, j0, j1);
      } else if constexpr (BL == KC) {
        db.template issue_kcr<KT>(rb[0], KIND == GATEUP ? (wave >= 2 ? g.b1 : g.b0).k : B.k, (sb + s) * BK2, t, wave,
                                  lane, j0, j1);
      } else {
        db.issue_mcs(mb[0], (sb + s) * BK2, t, wave, j0, j1);
      }
    };

    // M/N-major sources: the first K row of the stage each operand loads
    // next (B: s + 1, A: s + 2), carried from stage to stage (a 64-bit add,
    // not a multiply, per stage)
    constexpr bool MA = AL == MC && KIND != DX, MB = BL == MC && KIND != DX;
    const char* pa = nullptr;
    const char* pb = nullptr;
    if constexpr (MA) pa = ma[0].base + (int64_t)((sb + 2) * BK2) * ma[0].rowb;
    if constexpr (MB) pb = mb[0].base + (int64_t)((sb + 1) * BK2) * mb[0].rowb;
    auto issue_a2 = [&](int s, char* t, int j0, int j1) {
      if constexpr (MA) da.issue_mcp(ma[0], pa, (sb + s) * BK2, t, wave, j0, j1);
      else issue_a(s, t, j0, j1);
    };
    auto issue_b1 = [&](int s, char* t, int j0, int j1) {
      if constexpr (MB) db.issue_mcp(mb[0], pb, (sb + s) * BK2, t, wave, j0, j1);
      else issue_b(s, t, j0, j1);
    };

    using F = RingFrags<E, AL, BL, BK2>;
    F fr;
    if (nk > 0) {
      issue_a(0, R[0]);
      issue_b(0, R[1]);
      if (nk > 1) {
        issue_a(1, R[2]);
        wait_vmcnt<NT>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();
      fr.template read_a<0>(R[0], a_rows, 0, lane);
      fr.template read_b<0>(R[1], b_rows, 0, lane);
    }
    zero_acc();
    // One stage: two 32-K steps, the first of even parity, the second odd.
    // `full`: stages s + 1 and s + 2 exist (known at compile time in the
    // unrolled loop); otherwise the tail checks at run time. The first step
    // issues B of stage s + 1 (Q0, Q1) and A of stage s + 2 (Q2, Q3); its
    // successor is the same stage at K 32..63, so it needs no barrier. The
    // second step's barrier (between its Q1 and Q2) publishes stage s + 1,
    // whose first fragments its Q2 and Q3 read.
    auto stage = [&](int s, char* ca, char* cb, char* na, char* nb, char* na2, bool full) {
      const bool more = full || s + 1 < nk;
      const bool more2 = full || s + 2 < nk;
      // stages scheduled one at a time: without this fence the scheduler
      // gathered up to 14 loads of neighbouring stages into one burst
      // (dA + dSwiGLU 4 % slower); dI measured no better with it
      if constexpr (KIND != DX) __builtin_amdgcn_sched_barrier(0);
      static_assert(NT == 8, "four loads per quadrant");
      fr.template step<0, 4, true>(acc, ca, cb, 0, ca, cb, 1, a_rows, b_rows, lane, [] {}, [&](int q, int k) {
        if (q < 2) {
          if (more) issue_b1(s + 1, nb, 4 * q + k, 4 * q + k + 1);
        } else if (more2) {
          issue_a2(s + 2, na2, 4 * (q - 2) + k, 4 * (q - 2) + k + 1);
        }
      });
      auto mid = [&] {
        if (more2) wait_vmcnt<NT>();
        else wait_vmcnt<0>();
        lds_barrier();
      };
      // (the last stage reads fragments of a stage that does not come, from
      // arrays no load writes any more)
      fr.template step<1, 4, true>(acc, ca, cb, 1, na, nb, 0, a_rows, b_rows, lane, mid, [](int, int) {});
      if constexpr (MA) pa += DA::stride(ma[0]);
      if constexpr (MB) pb += DB::stride(mb[0]);
    };
    int s = 0;
    for (; s + 7 <= nk; s += 5) {
      stage(s + 0, R[0], R[1], R[2], R[3], R[4], true);
      stage(s + 1, R[2], R[3], R[4], R[0], R[1], true);
      stage(s + 2, R[4], R[0], R[1], R[2], R[3], true);
      stage(s + 3, R[1], R[2], R[3], R[4], R[0], true);
      stage(s + 4, R[3], R[4], R[0], R[1], R[2], true);
    }
    for (; s < nk; ++s) stage(s, reg(2 * s), reg(2 * s + 1), reg(2 * s + 2), reg(2 * s + 3), reg(2 * s + 4), false);
  };
  constexpr bool kc = AL == KC || BL == KC;
  if (kc && A.k % BK2 == 0) kloop(std::false_type{});
  else kloop(std::integral_constant<bool, kc>{});
  acc_fence<false>(acc);
  if constexpr (KIND == PLAIN) {
    if (split) {
      ring_partial_store(g, acc, piece, a_rows, b_rows, lane);
      return;
    }
  }
  // (a select, not R[wave]: indexing R at run time would keep it in scratch)
  ring_epilogue<E, KIND>(g, C, acc, m0, n0, wm, wn, lane, reg(wave));
}

// Pipeline per operand layouts: 4 = four stages of 32 K (ring_tile), 5 =
// five-array ring of 64 K stages (ring5_tile). Measured at D = 4096,
// H = 11008, T = 65536 (bf16): with a K-major A operand the 64 K stages are
// the faster (gate/up 4 %, down 7 %: half the stage barriers per K).
template <int AL, int BL>
constexpr int ring_variant() {
  return AL == KC ? 5 : 4;
}
// The weight gradients (both operands M/N-major, split over K at the edge):
// the five-array ring for [dWg | dWu] (stage 4), the four-stage ring for
// dWd (stage 3), each the faster on its shapes at D = 4096, H = 11008,
// T = 65536.
template <int STAGE>
constexpr int wgrad_variant() {
  return STAGE == 3 ? 4 : 5;
}
template <int STAGE>
constexpr int wgrad_bk() {
  return wgrad_variant<STAGE>() == 5 ? 64 : ring::BK;
}

template <class E, int AL, int BL, int KIND>
__device__ __forceinline__ void any_ring_tile(const KArgs& g, char* const (&R)[5], int bid, int bz) {
  if constexpr (ring_variant<AL, BL>() == 5) ring5_tile<E, AL, BL, KIND>(g, R, bid, bz);
  else ring_tile<E, AL, BL, KIND>(g, R[0], R[1], R[2], R[3], bid, bz);
}

// A K range of a tile (piece `piece` of a split weight-gradient tile, K
// stages [ks * kchunk, ...) of the ring's own stage depth).
template <class E, int AL, int BL, int STAGE>
__device__ __forceinline__ void ring_tile_piece(const KArgs& g, char* const (&R)[5], int bid, int bz, int ks,
                                                int piece) {
  if constexpr (wgrad_variant<STAGE>() == 5) ring5_tile<E, AL, BL, PLAIN>(g, R, bid, bz, ks, piece);
  else ring_tile<E, AL, BL, PLAIN>(g, R[0], R[1], R[2], R[3], bid, bz, ks, piece);
}

// Four 32 KiB LDS arrays, and a fifth when a five-array ring runs.
#define SWIGLU_RING_LDS(NEED5)                                                        \
  __shared__ __attribute__((aligned(16))) char s0[ring::STAGE];                       \
  __shared__ __attribute__((aligned(16))) char s1[ring::STAGE];                       \
  __shared__ __attribute__((aligned(16))) char s2[ring::STAGE];                       \
  __shared__ __attribute__((aligned(16))) char s3[ring::STAGE];                       \
  __shared__ __attribute__((aligned(16))) char s4[(NEED5) ? ring::STAGE : 16];        \
  char* R[5];                                                                         \
  R[0] = s0;                                                                          \
  R[1] = s1;                                                                          \
  R[2] = s2;                                                                          \
  R[3] = s3;                                                                          \
  R[4] = s4;

template <class E, int AL, int BL, int KIND, int STAGE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
ring_gemm(const KArgs g) {
  SWIGLU_RING_LDS((ring_variant<AL, BL>() == 5))
  any_ring_tile<E, AL, BL, KIND>(g, R, blockIdx.x, blockIdx.z);
}

// Tile and plane of weight-gradient item `item` (nt tiles per plane). Two
// planes ([dWg | dWu], which share the A operand X) alternate within each
// XCD's run of items: items x + 8 (2j) and x + 8 (2j + 1) are the two planes
// of tile x + 8j, dispatched to the same XCD, so the two read each X panel
// through one L2. Past the last full run of 8 tiles the two planes of a
// tile are consecutive items.
__device__ __forceinline__ void wgrad_item(int item, int nt, int planes, int& bid, int& bz) {
  if (planes == 1) {
    bid = item;
    bz = 0;
    return;
  }
  const int nt8 = nt & ~7;
  if (item < 2 * nt8) {
    const int j = item >> 3;
    bz = j & 1;
    bid = ((j >> 1) << 3) | (item & 7);
  } else {
    const int r = item - 2 * nt8;
    bz = r & 1;
    bid = nt8 + (r >> 1);
  }
}

// Weight-gradient launch (PLAIN, K = T): items are (tile, plane) pairs in
// wgrad_item's order. Items [0, n_full) run whole; each of the n_split items after them is
// split into ksplit pieces over K (workgroup n_full + r * ksplit + s is piece
// s of item n_full + r), which write fp32 partial tiles for
// splitk_reduce_tiles. The split covers only the last, partly filled round of
// tiles on the GPU's CUs.
template <class E, int AL, int BL, int STAGE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
ring_wgrad(const KArgs g) {
  SWIGLU_RING_LDS((wgrad_variant<STAGE>() == 5))
  const int nt = g.tiles_m * g.tiles_n;
  const int b = blockIdx.x;
  int item = b, ks = 0, piece = -1;
  if (b >= g.n_full) {
    piece = b - g.n_full;
    item = g.n_full + piece / g.ksplit;
    ks = piece % g.ksplit;
  }
  int bid, bz;
  wgrad_item(item, nt, g.planes, bid, bz);
  ring_tile_piece<E, AL, BL, STAGE>(g, R, bid, bz, ks, piece);
}



// ---------------------------------------------------------------------------
// Few-token kernels (T <= 64; gemm_skinny.hpp). KIND GATEUP: unit = 16 hidden
// units, computes G and U for them and writes A (and G, U when store_gu).
// KIND PLAIN: unit = 16 output columns of C = A_op * B.
// g.a0: activations [T, K] (K-contiguous); g.b0 (g.b1): weights [K, N]
// (N-contiguous). MT = number of 16-row token tiles (T <= 16 * MT).
// ---------------------------------------------------------------------------
template <class E, int KIND, int MT, int WAVES, int NS>
__device__ __forceinline__ void skinny_unit(const KArgs& g, char* lds, int unit) {
  using skinny::KS;
  using skinny::act_frag;
  using skinny::mfma16;
  using skinny::slab_frag;
  static_assert(NS >= 2 && (NS - 2) * (MT + 2) <= 63, "vmcnt range");
  constexpr int NW = (KIND == GATEUP) ? 2 : 1;  // weight matrices streamed
  constexpr int C = NW + MT;                    // 1-KiB loads per step
  constexpr int SLOT = C * 1024;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = unit * 16;
  const Operand& X = g.a0;
  const int K = X.k;
  const int steps = (K + KS - 1) / KS;
  const int per = (steps + WAVES - 1) / WAVES;
  const int sbeg = wave * per;
  const int nst = steps - sbeg < per ? (steps - sbeg > 0 ? steps - sbeg : 0) : per;

  char* ring = lds + wave * NS * SLOT;  // this wave's NS slots
  const uint32_t ring_addr = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  const int64_t ldw = g.b0.ld;
  const char* wb1 = NW == 2 ? g.b1.base : g.b0.base;
  const i32x4_t rx = rsrc_words(X.base, (int64_t)X.rows * X.ld * 2);
  // weight slab: lane -> (K row lane / 2, columns n0 + 8 (lane % 2) .. + 7)
  const uint32_t voff_w = (uint32_t)((lane >> 1) * (int)ldw * 2 + (n0 + (lane & 1) * 8) * 2);
  // activation tile: lane -> (token row lane / 4, logical chunk of its slot)
  const int am = lane >> 2;
  const int ac = (lane & 3) ^ ((am >> 2) & 3);

  auto issue = [&](int i, int sl) {
    // the slot being refilled was read by this wave one step earlier; make
    // sure those LDS reads have completed before the new data can land
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const bool live = i < nst;
    const int k0 = (sbeg + i) * KS;
    const uint32_t base = ring_addr + sl * SLOT;
    // descriptors start at K row k0 and end at row K, so the rows of a
    // ragged last step past K fall outside them and read as zeros (all
    // masking is in the lane offset; the scalar offset stays 0)
    const int kk = live ? k0 : 0;
    const int64_t wbytes = (int64_t)(K - kk) * ldw * 2;
    dma16(base, rsrc_words(g.b0.base + (int64_t)kk * ldw * 2, wbytes), live ? voff_w : kOOB, 0u);
    if constexpr (NW == 2) dma16(base + 1024, rsrc_words(wb1 + (int64_t)kk * ldw * 2, wbytes), live ? voff_w : kOOB, 0u);
    const int k = k0 + ac * 8;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + am;
      const bool ok = live && k < K && m < X.rows;
      dma16(base + (NW + t) * 1024, rx, ok ? (uint32_t)((m * K + k) * 2) : kOOB, 0u);
    }
  };

  f32x4_t acc[NW][MT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[w][t] = f32x4_t{};

  // NS - 1 steps in flight. Step i reads slot i % NS after waiting for its
  // loads (the NS - 2 later steps' loads may still be in flight), then issues
  // step i + NS - 1 into the slot read at step i - 1 (those reads completed:
  // their values fed step i - 1's MFMAs).
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(p, p);
  for (int i = 0; i < nst; i += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      ring::wait_vmcnt<(NS - 2) * C>();
      const char* sl = ring + j * SLOT;
      u32x4_t p[NW], qv[MT];
#pragma unroll
      for (int w = 0; w < NW; ++w) p[w] = slab_frag(sl + w * 1024, lane);
#pragma unroll
      for (int t = 0; t < MT; ++t) qv[t] = act_frag(sl + (NW + t) * 1024, lane);
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[w][t] = mfma16<E>(p[w], qv[t], acc[w][t]);
      issue(i + j + NS - 1, (j + NS - 1) % NS);
    }
  }
  ring::wait_vmcnt<0>();  // the surplus steps' loads (zeros) have landed too

  // sum the four waves' partials through LDS
  ring::lds_barrier();
  char* part = lds + wave * (NW * MT * 1024);
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int t = 0; t < MT; ++t) *(f32x4_t*)(part + ((w * MT + t) * 64 + lane) * 16) = acc[w][t];
  ring::lds_barrier();

  using V4 = typename E::vec4;
  const int ncol = n0 + (lane >> 4) * 4;  // 4 consecutive output columns
  for (int t = wave; t < MT; t += WAVES) {
    f32x4_t sum[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sum[w] = f32x4_t{};
#pragma unroll
      for (int v = 0; v < WAVES; ++v)
        sum[w] += *(const f32x4_t*)(lds + v * (NW * MT * 1024) + ((w * MT + t) * 64 + lane) * 16);
    }
    const int m = t * 16 + (lane & 15);
    if (m >= g.M || ncol >= g.N) continue;
    const int64_t off = ((int64_t)m * g.ldc + ncol) * E::kBytes;
    if constexpr (KIND == GATEUP) {
      V4 gv, uv, av;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        typename E::elem gs = E::from_f32(sum[0][e]);
        typename E::elem us = E::from_f32(sum[1][e]);
        const float gf = E::to_f32(gs), uf = E::to_f32(us);
        gv[e] = gs;
        uv[e] = us;
        av[e] = swiglu_a<E>(gf, uf, g.two_round);
      }
      *(V4*)(g.c0 + off) = av;
      if (g.store_gu) {
        *(V4*)(g.c1 + off) = gv;
        *(V4*)(g.c2 + off) = uv;
      }
    } else {
      V4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = E::from_f32(sum[0][e]);
      *(V4*)(g.c0 + off) = v;
    }
  }
}

// Waves per workgroup and ring slots per wave for the few-token kernels:
// the most waves (up to 16) whose rings fit in LDS with 4, else 3, slots. More waves split K finer, which shortens each wave's
// serial chain of loads: with few output units (D = 1024: 64 units in the
// down projection) that chain, not bandwidth, sets the time.
template <int KIND, int MT>
struct SkinnyCfg {
  static constexpr int C = (KIND == GATEUP ? 2 : 1) + MT;  // KiB per slot
  static constexpr bool fits(int w, int ns) { return w <= 16 && w * ns * C <= 160; }
  static constexpr int W = fits(16, 4) || fits(16, 3) ? 16 : (fits(8, 4) || fits(8, 3) ? 8 : 4);
  static constexpr int NS = fits(W, 4) ? 4 : 3;
};

template <class E, int KIND, int MT, int STAGE>
__global__ void __launch_bounds__((64 * SkinnyCfg<KIND, MT>::W)) skinny_gemm(const KArgs g) {
  constexpr int NW = (KIND == GATEUP) ? 2 : 1;
  constexpr int W = SkinnyCfg<KIND, MT>::W, NS = SkinnyCfg<KIND, MT>::NS;
  constexpr int BYTES = W * NS * (NW + MT) * 1024;
  static_assert(BYTES <= 160 * 1024, "LDS");
  static_assert(BYTES >= W * NW * MT * 1024, "partial sums must fit");
  __shared__ __attribute__((aligned(1024))) char lds[BYTES];
  // consecutive units on one XCD (the hardware deals workgroups round-robin
  // over the 8 XCDs)
  if constexpr (KIND == GATEUP) clear_counters(g);
  const int nb = gridDim.x, nb8 = nb & ~7;
  int b = blockIdx.x;
  if (b < nb8) b = (b & 7) * (nb8 >> 3) + (b >> 3);
  skinny_unit<E, KIND, MT, W, NS>(g, lds, b);
}

// ---------------------------------------------------------------------------
// Weight streaming for the no-grad forward, T <= 128 (gemm_stream.hpp).
// KIND GATEUP: weights g.b0 = Wg, g.b1 = Wu; writes A (and G, U when
// store_gu). KIND PLAIN: weights g.b0; writes C.
// g.a0: activations [T, K] (K-contiguous); weights [K, N] (N-contiguous).
// Workgroup b = unit * splits + split streams K steps of its split for the
// unit's 64 columns. splits == 1: the workgroup owns whole outputs and
// applies the epilogue itself. splits > 1: each workgroup writes an fp32
// partial (P: [splits][NW][T][N]) and counts its arrival on ctr[unit]; the
// last of a unit's workgroups to arrive adds the unit's partials in split
// order (deterministic), applies the epilogue and leaves the counter at
// zero. The counters must be zero when the launch starts: the gate/up
// launch of the same call clears those of the down launch (zero_ctr).
// ---------------------------------------------------------------------------
template <int KIND, int MT>
struct StreamCfg {
  static constexpr int NW = KIND == GATEUP ? 2 : 1;
  static constexpr int C = NW * 4 + MT;  // 1-KiB loads per step (= KiB per slot)
  static constexpr int W = 4;            // waves
  static constexpr int NS = W * 4 * C <= 160 ? 4 : (W * 3 * C <= 160 ? 3 : 2);
  static constexpr int BYTES = W * NS * C * 1024;
};

// The epilogue of four consecutive outputs (m, n .. n + 3) from their fp32
// sums: GATEUP rounds g and u, writes A (and G, U when store_gu); PLAIN
// writes C.
template <class E, int KIND>
__device__ __forceinline__ void stream_store(const KArgs& g, int m, int n, const f32x4_t (&sum)[KIND == GATEUP ? 2 : 1]) {
  using V4 = typename E::vec4;
  const int64_t off = ((int64_t)m * g.ldc + n) * E::kBytes;
  if constexpr (KIND == GATEUP) {
    V4 gv, uv, av;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      typename E::elem gs = E::from_f32(sum[0][e]);
      typename E::elem us = E::from_f32(sum[1][e]);
      gv[e] = gs;
      uv[e] = us;
      av[e] = swiglu_a<E>(E::to_f32(gs), E::to_f32(us), g.two_round);
    }
    *(V4*)(g.c0 + off) = av;
    if (g.store_gu) {
      *(V4*)(g.c1 + off) = gv;
      *(V4*)(g.c2 + off) = uv;
    }
  } else {
    V4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = E::from_f32(sum[0][e]);
    *(V4*)(g.c0 + off) = v;
  }
}

// fp32 partials of the split no-grad down projection: 16 bytes per lane with
// the device-scope cache policy (sc1: the access bypasses this XCD's
// non-coherent caches, as the compiler's own agent-scope atomic loads and
// stores do), so one workgroup's stores are visible to the workgroup of
// another XCD that adds them up. `plane` is one [T, N] plane; offsets stay
// below 2^31 for T <= 128 and N within the shape limit.
constexpr int kCoherentPolicy = 16;
__device__ __forceinline__ void store_partial(const float* plane, int T, int N, int m, int n, f32x4_t v) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(plane, (int64_t)T * N * 4);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, ((uint32_t)m * N + n) * 4u, 0,
                                         kCoherentPolicy);
}
__device__ __forceinline__ f32x4_t load_partial(const float* plane, int T, int N, int m, int n) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(plane, (int64_t)T * N * 4);
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, ((uint32_t)m * N + n) * 4u, 0,
                                                                           kCoherentPolicy));
}

template <class E, int KIND, int MT>
__global__ void __launch_bounds__(256) stream_gemm(const KArgs g, float* P, int splits, unsigned* ctr) {
  using namespace stream;
  using skinny::act_frag;
  using skinny::mfma16;
  using Cfg = StreamCfg<KIND, MT>;
  constexpr int NW = Cfg::NW, C = Cfg::C, W = Cfg::W, NS = Cfg::NS;
  constexpr int SLOT = C * 1024;
  static_assert(Cfg::BYTES <= 160 * 1024, "LDS");
  static_assert(Cfg::BYTES >= W * NW * MT * 1024, "one column block of partial sums must fit");
  static_assert((NS - 2) * C <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x / splits, split = blockIdx.x - unit * splits;
  if constexpr (KIND == GATEUP) clear_counters(g);
  const int n0 = unit * NC;
  const Operand& X = g.a0;
  const int K = X.k, N = g.N, T = g.M;
  const int steps = (K + KS - 1) / KS;
  const int psplit = (steps + splits - 1) / splits;
  const int s0 = split * psplit;
  const int s1 = s0 + psplit < steps ? s0 + psplit : steps;
  const int per = (s1 - s0 + W - 1) / W;
  const int sbeg = s0 + wave * per;
  const int nst = s1 - sbeg < per ? (s1 - sbeg > 0 ? s1 - sbeg : 0) : per;

  char* ring = lds + wave * NS * SLOT;
  const uint32_t ring_addr = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  const int64_t ldw = g.b0.ld;
  const char* wb1 = NW == 2 ? g.b1.base : g.b0.base;
  const i32x4_t rx = rsrc_words(X.base, (int64_t)X.rows * X.ld * 2);
  // weight load q covers slab rows 8q .. 8q + 7: lane -> row 8q + lane / 8,
  // physical chunk lane % 8, which holds logical chunk (lane % 8) ^ wswz(row)
  uint32_t voff_w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = q * 8 + (lane >> 3);
    const int col = n0 + (((lane & 7) ^ wswz(row)) << 3);
    voff_w[q] = col < N ? (uint32_t)(row * (int)ldw * 2 + col * 2) : kOOB;
  }
  // activation tile: lane -> (token row lane / 4, logical chunk of its slot)
  const int am = lane >> 2;
  const int ac = (lane & 3) ^ ((am >> 2) & 3);

  auto issue = [&](int i, int sl) {
    // the slot being refilled was read by this wave one step earlier
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const bool live = i < nst;
    const int k0 = (sbeg + i) * KS;
    const uint32_t base = ring_addr + sl * SLOT;
    // descriptors from K row k0 to row K: rows of a ragged last step past K
    // read as zeros; all masking is in the lane offsets
    const int kk = live ? k0 : 0;
    const int64_t wbytes = (int64_t)(K - kk) * ldw * 2;
    const i32x4_t r0 = rsrc_words(g.b0.base + (int64_t)kk * ldw * 2, wbytes);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(base + q * 1024, r0, live ? voff_w[q] : kOOB, 0u);
    if constexpr (NW == 2) {
      const i32x4_t r1 = rsrc_words(wb1 + (int64_t)kk * ldw * 2, wbytes);
#pragma unroll
      for (int q = 0; q < 4; ++q) dma16(base + WSLAB + q * 1024, r1, live ? voff_w[q] : kOOB, 0u);
    }
    const int k = k0 + ac * 8;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + am;
      const bool ok = live && k < K && m < X.rows;
      dma16(base + (NW * 4 + t) * 1024, rx, ok ? (uint32_t)((m * K + k) * 2) : kOOB, 0u);
    }
  };

  f32x4_t acc[NW][4][MT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[w][c][t] = f32x4_t{};

  // NS - 1 steps in flight, as in the few-token kernels: step i waits for its
  // own loads, reads slot i % NS, then refills the slot read at step i - 1.
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(p, p);
  for (int i = 0; i < nst; i += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      ring::wait_vmcnt<(NS - 2) * C>();
      const char* sl = ring + j * SLOT;
      u32x4_t qv[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) qv[t] = act_frag(sl + (NW * 4 + t) * 1024, lane);
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4_t p = wfrag(sl + w * WSLAB, c, lane);
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[w][c][t] = mfma16<E>(p, qv[t], acc[w][c][t]);
        }
      issue(i + j + NS - 1, (j + NS - 1) % NS);
    }
  }
  ring::wait_vmcnt<0>();  // the surplus steps' loads (zeros) have landed too

  // add the waves' sums through LDS, one 16-column block at a time; then
  // either apply the epilogue (whole K here) or write this workgroup's
  // partial
  constexpr int NB = NW * MT;  // 1-KiB blocks of f32x4 per wave and column block
  char* part = lds + wave * (NB * 1024);
  const bool direct = splits == 1;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    ring::lds_barrier();  // the ring (or the previous block's sums) is no longer read
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int t = 0; t < MT; ++t) *(f32x4_t*)(part + ((w * MT + t) * 64 + lane) * 16) = acc[w][c][t];
    ring::lds_barrier();
    // 16x16 output block of token tile t: token t * 16 + lane % 16, columns
    // 16 c + 4 (lane / 16) .. + 3
    const int n = n0 + c * 16 + (lane >> 4) * 4;
    if (direct) {
      for (int t = wave; t < MT; t += W) {
        f32x4_t sum[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          sum[w] = f32x4_t{};
#pragma unroll
          for (int v = 0; v < W; ++v) sum[w] += *(const f32x4_t*)(lds + v * (NB * 1024) + ((w * MT + t) * 64 + lane) * 16);
        }
        const int m = t * 16 + (lane & 15);
        if (m < T && n < N) stream_store<E, KIND>(g, m, n, sum);
      }
    } else {
      for (int blk = wave; blk < NB; blk += W) {
        f32x4_t sum = f32x4_t{};
#pragma unroll
        for (int v = 0; v < W; ++v) sum += *(const f32x4_t*)(lds + v * (NB * 1024) + (blk * 64 + lane) * 16);
        const int w = blk / MT, t = blk % MT;
        const int m = t * 16 + (lane & 15);
        if (m < T && n < N) store_partial(P + ((int64_t)split * NW + w) * T * N, T, N, m, n, sum);
      }
    }
  }
  if (direct) return;

  // Arrival. The partials went out as device-coherent stores
  // (store_partial); each wave waits until its own have completed, the
  // barrier then orders all of them before thread 0's atomic add on the
  // unit's counter. The workgroup that brings the count to `splits` is the
  // last: it reads the partials with device-coherent loads, so no cache of
  // its CU or XCD can serve stale data, and no cache write-back or
  // invalidation is needed anywhere.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // (also: every wave is done reading the LDS sums)
  int* last_arrival = (int*)lds;
  if (threadIdx.x == 0)
    *last_arrival = __hip_atomic_fetch_add(ctr + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    (unsigned)(splits - 1);
  __syncthreads();
  if (!*last_arrival) return;
  if (threadIdx.x == 0) __hip_atomic_store(ctr + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the unit's T x 64 outputs, four consecutive columns per thread
  for (int i = threadIdx.x; i < T * (NC / 4); i += 256) {
    const int m = i / (NC / 4), n = n0 + (i % (NC / 4)) * 4;
    if (n >= N) continue;
    f32x4_t sum[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sum[w] = f32x4_t{};
      for (int sp = 0; sp < splits; ++sp) sum[w] += load_partial(P + ((int64_t)sp * NW + w) * T * N, T, N, m, n);
    }
    stream_store<E, KIND>(g, m, n, sum);
  }
}

// ---------------------------------------------------------------------------
// Weight streaming with a workgroup-shared ring, no-grad forward with
// 32 < T <= 256 (MT = 4, 8 or 16 token tiles of 16). The per-wave ring of
// stream_gemm holds each wave's own activation tiles, so with many tokens
// only two slots fit and every step waits on its own loads. Here one stage
// (32 K) is the unit's weight slabs (NW x 4 KiB) and the activation tiles
// (MT KiB), loaded once for the workgroup and read by all four waves, which
// split the 64 columns x MT token tiles 2 x 2; NSTG stages (6 or 8) are in
// flight. Each wave then owns whole outputs: splits == 1 applies the
// epilogue from registers, splits > 1 writes partials and counts arrivals
// as stream_gemm does.
// ---------------------------------------------------------------------------
template <int KIND, int MT>
struct RingStreamCfg {
  static constexpr int NW = KIND == GATEUP ? 2 : 1;
  static constexpr int C = NW * 4 + MT;  // 1-KiB loads per stage (= KiB per stage)
  static_assert(C % 4 == 0, "every wave issues the same number of loads");
  static constexpr int LW = C / 4;        // loads per wave per stage
  static constexpr int NSTG = 160 / C > 8 ? 8 : 160 / C;
  static constexpr int BYTES = NSTG * C * 1024;
};

template <class E, int KIND, int MT>
__global__ void __launch_bounds__(256) stream_ring(const KArgs g, float* P, int splits, unsigned* ctr) {
  using namespace stream;
  using skinny::act_frag;
  using skinny::mfma16;
  using Cfg = RingStreamCfg<KIND, MT>;
  constexpr int NW = Cfg::NW, C = Cfg::C, LW = Cfg::LW, NSTG = Cfg::NSTG;
  constexpr int SLOT = C * 1024;
  constexpr int TW = MT / 2;  // token tiles per wave
  static_assert(MT >= 2 && MT % 2 == 0, "two token halves");
  static_assert(Cfg::BYTES <= 160 * 1024, "LDS");
  static_assert((NSTG - 2) * LW <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ch = wave & 1, th = wave >> 1;  // column half (32 columns), token half (TW tiles)
  const int unit = blockIdx.x / splits, split = blockIdx.x - unit * splits;
  if constexpr (KIND == GATEUP) clear_counters(g);
  const int n0 = unit * NC;
  const Operand& X = g.a0;
  const int K = X.k, N = g.N, T = g.M;
  const int steps = (K + KS - 1) / KS;
  const int psplit = (steps + splits - 1) / splits;
  const int s0 = split * psplit;
  const int s1 = s0 + psplit < steps ? s0 + psplit : steps;
  const int nst = s1 > s0 ? s1 - s0 : 0;

  const uint32_t ring_addr = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  const int64_t ldw = g.b0.ld;
  const char* wb1 = NW == 2 ? g.b1.base : g.b0.base;
  // T <= 256 rows of at most 4194296 elements: every offset below 2^31
  const i32x4_t rx = rsrc_words(X.base, (int64_t)X.rows * X.ld * 2);
  // This wave's loads of a stage: load q = wave * LW + j of the C loads;
  // q < NW * 4: weight slab q / 4, rows 8 (q % 4) .. + 7 (lane -> row
  // 8 (q % 4) + lane / 8, physical chunk lane % 8 holding logical chunk
  // (lane % 8) ^ wswz(row)); else activation tile q - NW * 4 (lane ->
  // token row lane / 4 of the tile, logical chunk of its slot).
  uint32_t voff[LW];
  int kind[LW];  // 0, 1: weight plane; 2: activation
  const int am = lane >> 2;
  const int ac = (lane & 3) ^ ((am >> 2) & 3);
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int q = wave * LW + j;
    if (q < NW * 4) {
      const int row = (q & 3) * 8 + (lane >> 3);
      const int col = n0 + (((lane & 7) ^ wswz(row)) << 3);
      kind[j] = q >> 2;
      voff[j] = col < N ? (uint32_t)row * (uint32_t)ldw * 2u + (uint32_t)col * 2u : kOOB;
    } else {
      const int m = (q - NW * 4) * 16 + am;
      kind[j] = 2;
      voff[j] = m < T ? (uint32_t)m * (uint32_t)X.ld * 2u + (uint32_t)ac * 16u : kOOB;
    }
  }

  // loads of stage i (K rows [k0, k0 + 32)) into slot sl; past the end they
  // fetch nothing (out-of-range offsets: zeros) and only keep the counts
  auto issue = [&](int i, int sl) {
    const bool live = i < nst;
    const int k0 = (s0 + i) * KS;
    const int kk = live ? k0 : 0;
    const uint32_t base = ring_addr + sl * SLOT;
    // weight descriptors from K row k0 to K: rows of a ragged last stage
    // past K read as zeros
    const int64_t wbytes = (int64_t)(K - kk) * ldw * 2;
    const i32x4_t r0 = rsrc_words(g.b0.base + (int64_t)kk * ldw * 2, wbytes);
    const i32x4_t r1 = rsrc_words(wb1 + (int64_t)kk * ldw * 2, wbytes);
    const bool kin = kk + ac * 8 < K;
#pragma unroll
    for (int j = 0; j < LW; ++j) {
      const uint32_t dst = base + (wave * LW + j) * 1024;
      if (kind[j] == 2) dma16(dst, rx, (live && kin) ? voff[j] + (uint32_t)kk * 2u : kOOB, 0u);
      else dma16(dst, kind[j] ? r1 : r0, live ? voff[j] : kOOB, 0u);
    }
  };

  f32x4_t acc[NW][2][TW];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < TW; ++t) acc[w][c][t] = f32x4_t{};

#pragma unroll
  for (int p = 0; p < NSTG - 1; ++p) issue(p, p);
  for (int i = 0; i < nst; i += NSTG) {
#pragma unroll
    for (int jj = 0; jj < NSTG; ++jj) {
      // own loads of stage i + jj have landed; the barrier publishes every
      // wave's, and every wave is done reading the slot refilled next
      ring::wait_vmcnt<(NSTG - 2) * LW>();
      ring::lds_barrier();
      issue(i + jj + NSTG - 1, (jj + NSTG - 1) % NSTG);
      const char* sl = lds + jj * SLOT;
      u32x4_t qv[TW];
#pragma unroll
      for (int t = 0; t < TW; ++t) qv[t] = act_frag(sl + (NW * 4 + th * TW + t) * 1024, lane);
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4_t p = wfrag(sl + w * WSLAB, ch * 2 + c, lane);
#pragma unroll
          for (int t = 0; t < TW; ++t) acc[w][c][t] = mfma16<E>(p, qv[t], acc[w][c][t]);
        }
      if (i + jj + 1 >= nst) break;
    }
  }
  ring::wait_vmcnt<0>();  // the surplus stages' loads (zeros) have landed too

  // outputs of this wave: token tile th * TW + t, columns
  // n0 + 16 (2 ch + c) + 4 (lane / 16) .. + 3, token (lane % 16)
  auto out_at = [&](int c, int t, int& m, int& n) {
    m = (th * TW + t) * 16 + (lane & 15);
    n = n0 + (ch * 2 + c) * 16 + (lane >> 4) * 4;
  };
  if (splits == 1) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        int m, n;
        out_at(c, t, m, n);
        if (m >= T || n >= N) continue;
        f32x4_t sum[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) sum[w] = acc[w][c][t];
        stream_store<E, KIND>(g, m, n, sum);
      }
    return;
  }
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        int m, n;
        out_at(c, t, m, n);
        if (m >= T || n >= N) continue;
        store_partial(P + ((int64_t)split * NW + w) * T * N, T, N, m, n, acc[w][c][t]);
      }
  // arrival, as in stream_gemm: device-coherent partials, each wave waits
  // for its own stores, the barrier orders them before the atomic add
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* last_arrival = (int*)lds;
  if (threadIdx.x == 0)
    *last_arrival = __hip_atomic_fetch_add(ctr + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    (unsigned)(splits - 1);
  __syncthreads();
  if (!*last_arrival) return;
  if (threadIdx.x == 0) __hip_atomic_store(ctr + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = threadIdx.x; i < T * (NC / 4); i += 256) {
    const int m = i / (NC / 4), n = n0 + (i % (NC / 4)) * 4;
    if (n >= N) continue;
    f32x4_t sum[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sum[w] = f32x4_t{};
      for (int sp = 0; sp < splits; ++sp) sum[w] += load_partial(P + ((int64_t)sp * NW + w) * T * N, T, N, m, n);
    }
    stream_store<E, KIND>(g, m, n, sum);
  }
}

// Sum of the partial tiles of the split items of a weight-gradient launch, in
// piece order (deterministic): C = rnd(sum over s of P[r * ksplit + s]) for
// split item n_full + r, written to plane c0 or c1. One thread per 4
// consecutive outputs of a tile row.
template <class E>
__global__ void __launch_bounds__(256) splitk_reduce_tiles(const KArgs g, const float* P) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)g.n_split * 16384) return;
  const int r = (int)(i >> 14), rr = (int)(i >> 6) & 255, cq = (int)i & 63;
  const int nt = g.tiles_m * g.tiles_n, item = g.n_full + r;
  int bid, bz, tm, tn;
  wgrad_item(item, nt, g.planes, bid, bz);
  tile_coords(bid, g.tiles_m, g.tiles_n, g.group_m > 0 ? g.group_m : 8, tm, tn);
  const int m = tm * 256 + rr, n = tn * 256 + cq * 4;
  if (m >= g.M || n >= g.N) return;
  const float* p = P + (int64_t)r * g.ksplit * 65536 + rr * 256 + cq * 4;
  f32x4_t sum = f32x4_t{};
  for (int s = 0; s < g.ksplit; ++s) sum += *(const f32x4_t*)(p + (int64_t)s * 65536);
  typename E::vec4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = E::from_f32(sum[e]);
  *(typename E::vec4*)((bz ? g.c1 : g.c0) + ((int64_t)m * g.ldc + n) * E::kBytes) = v;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Stage timing (profiling aid).
struct Timer {
  bool on = false;
  int cap = 0;
  int count[SWIGLU_NUM_STAGES] = {};
  hipEvent_t* ev[SWIGLU_NUM_STAGES] = {};  // 2 * cap events per stage
};
extern Timer g_timer;  // defined once, in swiglu_mlp.hip

struct StageScope {
  int s;
  hipStream_t st;
  bool rec = false;
  StageScope(int stage, hipStream_t stream) : s(stage), st(stream) {
    if (g_timer.on && g_timer.count[s] < g_timer.cap) {
      rec = true;
      (void)hipEventRecord(g_timer.ev[s][2 * g_timer.count[s]], st);
    }
  }
  ~StageScope() {
    if (rec) {
      (void)hipEventRecord(g_timer.ev[s][2 * g_timer.count[s] + 1], st);
      g_timer.count[s]++;
    }
  }
};

static inline Operand opnd(const void* p, int64_t ld, int64_t rows, int64_t k) {
  return Operand{(const char*)p, ld, (int)rows, (int)k};
}

template <class E, int BM, int BN, int AL, int BL, int KIND, int STAGE>
static int launch(KArgs a, int grid_z, hipStream_t stream) {
  const int nb = a.tiles_m * a.tiles_n;
  a.planes = grid_z;
  if (nb <= 0) return SWIGLU_OK;
  StageScope scope(STAGE, stream);
  hipLaunchKernelGGL((mlp_gemm<E, BM, BN, AL, BL, KIND, STAGE>), dim3(nb, 1, grid_z), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_LAUNCH;
}

template <class E, int AL1, int BL1, int K1, int AL2, int BL2, int K2, int STAGE>
static int launch_pair(KArgs a1, KArgs a2, hipStream_t stream) {
  const int nb = a1.tiles_m * a1.tiles_n * a1.planes + a2.tiles_m * a2.tiles_n;
  if (nb <= 0) return SWIGLU_OK;
  StageScope scope(STAGE, stream);
  hipLaunchKernelGGL((mlp_gemm_pair<E, AL1, BL1, K1, AL2, BL2, K2, STAGE>), dim3(nb), dim3(256), 0, stream, a1, a2);
  return hipGetLastError() == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_LAUNCH;
}

// Tile walk of the ring kernels (tile_coords): each XCD runs group_m M-tiles
// x (32 / group_m) N-tiles at a time, so that its concurrent tiles share
// operand rows through its L2. Per stage and weight layout (BL: the B
// operand's), measured over 1, 2, 4 and 8 at D = 4096, H = 11008,
// T = 65536 (the differences are 0.5-10 %): 2 for gate/up, down (stage 1)
// and dA + dSwiGLU; for dI 4 with K-major weights, 1 with the nn.Linear
// layout's N-major ones; for the weight gradients 4, except the nn.Linear
// layout's [dWg | dWu] (planes switching the A operand): 1 (wgrad_group_m).
template <int KIND, int STAGE, int BL>
constexpr int ring_group_m() {
  return KIND == DX ? (BL == MC ? 1 : 4) : KIND == GATEUP || KIND == DSWIGLU || STAGE == 1 ? 2 : 4;
}
static inline int wgrad_group_m(bool plane_a) { return plane_a ? 1 : 4; }

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Compute units of the current device (launch plans size work per CU);
// cached per device, 256 when the runtime cannot say.
static int dev_ncu() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    int v = 0;
    n = (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ? v : 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Modelled time of one 256 x 256 ring tile with K values of K on one CU
// (about 5 TFLOP/s per CU), used only to size launch plans.
static inline double ring_tile_us(int64_t K) { return 2.0 * 256 * 256 * (double)K / 5.0e6; }

template <class E, int AL, int BL, int KIND, int STAGE>
static int launch_ring(KArgs a, int grid_z, hipStream_t stream) {
  a.group_m = ring_group_m<KIND, STAGE, BL>();
  const int nb = a.tiles_m * a.tiles_n;
  a.planes = grid_z;
  if (nb <= 0) return SWIGLU_OK;
  StageScope scope(STAGE, stream);
  hipLaunchKernelGGL((ring_gemm<E, AL, BL, KIND, STAGE>), dim3(nb, 1, grid_z), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_LAUNCH;
}

// Work split of a weight-gradient ring launch (K = T; nt tiles over all
// planes). Whole rounds of tiles (one per CU) run unsplit. The remaining
// rem = nt % ncu tiles would leave the last round partly idle, so each is
// split into s pieces over K, s chosen by a model: ceil(rem s / ncu) rounds
// of 1/s of a tile, plus writing and reading the fp32 partial tiles (256 KiB
// each), plus the reduction launch. With no remainder, or no gain, nothing
// is split.
struct WgradPlan {
  int n_full, n_split, ksplit, kchunk;
};
static WgradPlan wgrad_plan(int nt, int64_t K, int ncu, int bk) {
  const int nk = cdiv(K, bk);  // K stages of the ring that runs the tiles
  WgradPlan p{nt, 0, 1, nk};
  const int rem = nt % ncu;
  if (rem == 0) return p;
  const double tile = ring_tile_us(K);
  double best = tile;
  int bs = 1;
  for (int s = 2; s <= 16 && nk / s >= 16; ++s) {
    const double t = cdiv((int64_t)rem * s, ncu) * tile / s + (double)rem * s * 65536 * 4 * 2 / 4.0e6 + 5.0;
    if (t < 0.97 * best) {
      best = t;
      bs = s;
    }
  }
  if (bs == 1) return p;
  p.n_full = nt - rem;
  p.n_split = rem;
  p.kchunk = cdiv(nk, bs);
  p.ksplit = cdiv(nk, p.kchunk);
  return p;
}

// Weight-gradient ring launch (PLAIN, 1 or 2 planes) following wgrad_plan:
// whole tiles write the outputs; split tiles write fp32 partials into P,
// then splitk_reduce_tiles adds them; timed as one stage.
template <class E, int AL, int BL, int STAGE>
static int launch_ring_wgrad(KArgs a, int grid_z, float* P, hipStream_t stream) {
  const int nt = a.tiles_m * a.tiles_n;
  if (nt <= 0) return SWIGLU_OK;
  const WgradPlan pl = wgrad_plan(nt * grid_z, a.a0.k, dev_ncu(), wgrad_bk<STAGE>());
  a.planes = grid_z;
  a.group_m = wgrad_group_m(a.plane_a != 0);
  a.P = pl.n_split ? P : nullptr;
  a.kchunk = pl.kchunk;
  a.n_full = pl.n_full;
  a.ksplit = pl.ksplit;
  a.n_split = pl.n_split;
  StageScope scope(STAGE, stream);
  hipLaunchKernelGGL((ring_wgrad<E, AL, BL, STAGE>), dim3(pl.n_full + pl.n_split * pl.ksplit), dim3(256), 0, stream,
                     a);
  if (hipGetLastError() != hipSuccess) return SWIGLU_ERR_LAUNCH;
  if (pl.n_split == 0) return SWIGLU_OK;
  hipLaunchKernelGGL((splitk_reduce_tiles<E>), dim3(pl.n_split * 64), dim3(256), 0, stream, a, (const float*)P);
  return hipGetLastError() == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_LAUNCH;
}

// fp32 partial bytes of the weight-gradient launches (bf16/fp16, T > 512):
// the larger of dWd ([H, D]) and [dWg | dWu] (2 x [D, H]).
static inline size_t splitk_bytes(int64_t T, int64_t D, int64_t H) {
  const int ncu = dev_ncu();
  const WgradPlan pd = wgrad_plan(cdiv(H, 256) * cdiv(D, 256), T, ncu, wgrad_bk<3>());
  const WgradPlan pg = wgrad_plan(cdiv(D, 256) * cdiv(H, 256) * 2, T, ncu, wgrad_bk<4>());
  const size_t bd = (size_t)pd.n_split * pd.ksplit * 65536 * 4, bg = (size_t)pg.n_split * pg.ksplit * 65536 * 4;
  return bd > bg ? bd : bg;
}

// Few-token launch: one workgroup per 16 output columns.
template <class E, int KIND, int STAGE>
static int launch_skinny(KArgs a, int64_t T, int64_t ncols, hipStream_t stream) {
  const int nb = cdiv(ncols, 16);
  if (nb <= 0 || T <= 0) return SWIGLU_OK;
  StageScope scope(STAGE, stream);
  if (T <= 16)
    hipLaunchKernelGGL((skinny_gemm<E, KIND, 1, STAGE>), dim3(nb), dim3(64 * SkinnyCfg<KIND, 1>::W), 0, stream, a);
  else if (T <= 32)
    hipLaunchKernelGGL((skinny_gemm<E, KIND, 2, STAGE>), dim3(nb), dim3(64 * SkinnyCfg<KIND, 2>::W), 0, stream, a);
  else
    hipLaunchKernelGGL((skinny_gemm<E, KIND, 4, STAGE>), dim3(nb), dim3(64 * SkinnyCfg<KIND, 4>::W), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_LAUNCH;
}

// Streaming launch (no-grad, 16-bit, T <= 128): `splits` workgroups per
// 64-column unit; see stream_gemm. One launch per stage.
struct StreamArgs {
  int splits;     // K splits per unit (1: no partials)
  float* P;       // fp32 partials (splits > 1)
  unsigned* ctr;  // arrival counters, one per unit (splits > 1), zero at launch
};

// No-grad weight streaming: up to kStreamMaxT tokens; above kStreamRingMinT
// tokens the workgroup-shared ring (stream_ring), else the per-wave rings
// (stream_gemm). Measured gate/up at D = 4096, H = 11008: S = 128 70 us
// (per-wave rings 84), S = 256 103 us (64-row tile engine 148).
constexpr int kStreamMaxT = 256;
constexpr int kStreamRingMinT = 32;

template <class E, int KIND, int MT>
static void launch_stream_mt(const KArgs& a, int grid, const StreamArgs& st, hipStream_t stream) {
  hipLaunchKernelGGL((stream_gemm<E, KIND, MT>), dim3(grid), dim3(256), 0, stream, a, st.P, st.splits, st.ctr);
}
template <class E, int KIND, int STAGE>
static int launch_stream(KArgs a, int64_t T, int64_t ncols, const StreamArgs& st, hipStream_t stream) {
  const int units = cdiv(ncols, stream::NC);
  if (units <= 0 || T <= 0) return SWIGLU_OK;
  StageScope scope(STAGE, stream);
  const int grid = units * st.splits;
  if (T <= 16) launch_stream_mt<E, KIND, 1>(a, grid, st, stream);
  else if (T <= 32) launch_stream_mt<E, KIND, 2>(a, grid, st, stream);
  else if (T <= kStreamRingMinT) {
    if (T <= 64) launch_stream_mt<E, KIND, 4>(a, grid, st, stream);
    else launch_stream_mt<E, KIND, 8>(a, grid, st, stream);
  } else if (T <= 64) {
    hipLaunchKernelGGL((stream_ring<E, KIND, 4>), dim3(grid), dim3(256), 0, stream, a, st.P, st.splits, st.ctr);
  } else if (T <= 128) {
    hipLaunchKernelGGL((stream_ring<E, KIND, 8>), dim3(grid), dim3(256), 0, stream, a, st.P, st.splits, st.ctr);
  } else {
    hipLaunchKernelGGL((stream_ring<E, KIND, 16>), dim3(grid), dim3(256), 0, stream, a, st.P, st.splits, st.ctr);
  }
  return hipGetLastError() == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_LAUNCH;
}

// Tokens up to which the forward runs on the weight-streaming kernels
// (training: few_t; no-grad, which has a workspace: stream_t).
static inline bool few_t(int64_t T) { return T <= 64; }
static inline bool stream_t(int64_t T) { return T <= kStreamMaxT; }
static inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// No-grad gate/up with few tokens and a narrow hidden dimension: the
// few-token kernel (16-column units, up to 16 waves splitting K) gives more,
// shorter weight streams than 64-column units would.
constexpr int kInferSkinnyMaxH = 4096;
static inline bool infer_gateup_skinny(int64_t T, int64_t H) { return few_t(T) && H <= kInferSkinnyMaxH; }

// Largest fp32 partial buffer of the no-grad down projection, as a multiple
// of the call's A + Y bytes: the split count is capped so that the
// intermediate memory of a call (workspace + Y) stays within 3 (A + Y).
// Measured at D = 4096, H = 11008 (3 splits): the down projection takes
// 24-59 us for S = 1-128 against 45-110 us unsplit; more splits were no
// faster at S = 1 and slower from S = 64 on (the last arrival's reduction
// grows with them).
constexpr int kInferPartialCap = 2;
// Above this many tokens the down projection is not split over K (it runs
// on the 64-row tile engine), so the call's intermediate memory is exactly
// A + Y there (the pages' table at S = 256 measures A + Y). Measured at
// D = 4096, H = 11008, S = 256: 124 us there, 184 us unsplit streaming,
// 104 us split three ways (with 2.6 (A + Y) of memory).
constexpr int kInferSplitMaxT = 128;
// Tokens up to which the no-grad gate/up streams whatever H (few tokens:
// the few-token kernel or the per-wave rings).
constexpr int kInferGateSkinnyT = 128;

// No-grad workspace. The A plane [T, H]; for 16-bit with T <= kInferSplitMaxT
// also the down projection's arrival counters (one per 64 columns) and, when
// its K is split, its fp32 partials, each 256-byte aligned after A. The
// gate/up stage never splits K: the hidden dimension alone gives enough
// 64-column units. stream: gate/up (and, with down_stream, down) run on the
// weight-streaming kernels.
struct InferPlan {
  size_t a_bytes = 0, ctr_off = 0, p_off = 0, total = 0;
  bool stream = false, down_stream = false;  // gate/up, down on the weight-streaming kernels
  int down_units = 0, down_splits = 1;
};
static inline InferPlan infer_plan(int64_t T, int64_t D, int64_t H, size_t e) {
  InferPlan p;
  p.a_bytes = (size_t)T * H * e;
  p.total = p.a_bytes;
  if (e != 2 || T <= 0 || !stream_t(T)) return p;
  // above kInferGateSkinnyT tokens the gate/up streams only with at least
  // 128 units of 64 hidden units (H = 2816, S = 256: 33 us streaming on 44
  // units, 24 us on the 64-row tile engine; H = 11008: 103 us against 148)
  p.stream = T <= kInferGateSkinnyT || cdiv(H, stream::NC) >= 128;
  if (T > kInferSplitMaxT) return p;
  p.down_stream = true;
  p.down_units = cdiv(D, stream::NC);
  int sp = stream::splits_for(p.down_units, cdiv(H, stream::KS), StreamCfg<PLAIN, 1>::W);
  const size_t per = (size_t)T * D * 4;                                    // one split's partials
  const size_t cap = (size_t)kInferPartialCap * (size_t)T * (H + D) * e;  // x (A + Y)
  const int sp_mem = (int)(cap / per);
  if (sp > sp_mem) sp = sp_mem < 1 ? 1 : sp_mem;
  p.down_splits = sp;
  p.ctr_off = align256(p.a_bytes);
  p.p_off = align256(p.ctr_off + (size_t)p.down_units * 4);
  p.total = sp > 1 ? p.p_off + (size_t)sp * per : p.ctr_off + (size_t)p.down_units * 4;
  return p;
}

// Rows of X per workgroup tile for the T-indexed GEMMs. Small token counts
// (the no-grad shapes) use short tiles so that more workgroups share the
// weight stream.
static inline bool small_t(int64_t T) { return T <= 512; }

// The weights come in one of two layouts (the LIN template argument):
//   kernel layout (LIN = false): Wg, Wu [D, H], Wd [H, D], row-major, so the
//     forward reads them N-major and the backward (dA, dI) K-major;
//   linear layout (LIN = true): the nn.Linear weights, gate_proj and
//     up_proj [H, D], down_proj [D, H], row-major, so the forward reads them
//     K-major and the backward N-major; the weight gradients are written in
//     the same layout (dWg, dWu [H, D], dWd [D, H]).
// Either way no weight is copied or transposed: each GEMM reads its operand
// in the layout it is given (FW: the forward's weight operand layout, BW:
// the backward's). The weight-streaming kernels assume N-contiguous weights,
// so the linear layout runs few-token shapes on the 64-row tile engine.
template <class E, bool LIN>
struct Path {
  static constexpr int EB = E::kBytes;
  static constexpr int FW = LIN ? KC : MC;
  static constexpr int BW = LIN ? MC : KC;

  template <int STAGE>
  static int gateup(const void* X, const void* Wg, const void* Wu, char* Ap, char* Gp, char* Up,
                    int64_t T, int64_t D, int64_t H, bool store_gu, bool two_round, const StreamArgs* st,
                    hipStream_t s, unsigned* zero_ctr = nullptr, int n_zero = 0) {
    KArgs a{};
    a.a0 = opnd(X, D, T, D);
    if constexpr (LIN) {
      a.b0 = opnd(Wg, D, H, D);  // Bop[k=d][n=h] = Wg[h][d]: K-contiguous rows
      a.b1 = opnd(Wu, D, H, D);
    } else {
      a.b0 = opnd(Wg, H, H, D);  // Bop[k=d][n=h] = Wg[d][h]: N-contiguous rows
      a.b1 = opnd(Wu, H, H, D);
    }
    a.c0 = Ap;
    a.c1 = Gp;
    a.c2 = Up;
    a.ldc = H;
    a.M = (int)T;
    a.N = (int)H;
    a.store_gu = store_gu ? 1 : 0;
    a.two_round = two_round ? 1 : 0;
    a.zero_ctr = zero_ctr;
    a.n_zero = n_zero;
    if constexpr (E::kBytes == 2 && !LIN) {
      // (the streaming kernels are instantiated for the no-grad stage only)
      if constexpr (STAGE == 6)
        if (st) {
          if (infer_gateup_skinny(T, H)) return launch_skinny<E, GATEUP, STAGE>(a, T, H, s);
          return launch_stream<E, GATEUP, STAGE>(a, T, H, *st, s);
        }
      if (few_t(T)) return launch_skinny<E, GATEUP, STAGE>(a, T, H, s);
    }
    if (small_t(T)) {
      a.tiles_m = cdiv(T, 64);
      a.tiles_n = cdiv(H, 128);
      return launch<E, 64, 256, KC, FW, GATEUP, STAGE>(a, 1, s);
    }
    a.tiles_m = cdiv(T, 256);
    a.tiles_n = cdiv(H, 128);
    if constexpr (E::kBytes == 2) {
      // few ring tiles: 64-row tiles when those fit one round (as the down
      // projection)
      if (cdiv(T, 64) * a.tiles_n <= 256) {
        a.tiles_m = cdiv(T, 64);
        return launch<E, 64, 256, KC, FW, GATEUP, STAGE>(a, 1, s);
      }
      return launch_ring<E, KC, FW, GATEUP, STAGE>(a, 1, s);
    }
    else return launch<E, 256, 256, KC, FW, GATEUP, STAGE>(a, 1, s);
  }

  template <int STAGE>
  static int down(const char* Ap, const void* Wd, void* Y, int64_t T, int64_t D, int64_t H,
                  const StreamArgs* st, hipStream_t s) {
    KArgs a{};
    a.a0 = opnd(Ap, H, T, H);
    if constexpr (LIN) a.b0 = opnd(Wd, H, D, H);  // Bop[k=h][n=d] = Wd[d][h]
    else a.b0 = opnd(Wd, D, D, H);                // Bop[k=h][n=d] = Wd[h][d]
    a.c0 = (char*)Y;
    a.ldc = D;
    a.M = (int)T;
    a.N = (int)D;
    if constexpr (E::kBytes == 2 && !LIN) {
      if constexpr (STAGE == 7)
        if (st) return launch_stream<E, PLAIN, STAGE>(a, T, D, *st, s);
      if (few_t(T)) return launch_skinny<E, PLAIN, STAGE>(a, T, D, s);
    }
    if (small_t(T)) {
      // 64-row tiles; the widest N tile that still gives 256 workgroups (the
      // down projection has only D / 256 tiles of 256 columns per row block)
      a.tiles_m = cdiv(T, 64);
      if (a.tiles_m * cdiv(D, 256) >= 256) {
        a.tiles_n = cdiv(D, 256);
        return launch<E, 64, 256, KC, FW, PLAIN, STAGE>(a, 1, s);
      }
      if (a.tiles_m * cdiv(D, 128) >= 256) {
        a.tiles_n = cdiv(D, 128);
        return launch<E, 64, 128, KC, FW, PLAIN, STAGE>(a, 1, s);
      }
      a.tiles_n = cdiv(D, 64);
      return launch<E, 64, 64, KC, FW, PLAIN, STAGE>(a, 1, s);
    }
    a.tiles_m = cdiv(T, 256);
    a.tiles_n = cdiv(D, 256);
    if constexpr (E::kBytes == 2) {
      // few 256-column tiles (small D): when the 64-row tiles of the same
      // rows still fit one round on the CUs, they beat one round of ring
      // tiles on a quarter of them (T = 4096, D = 1024: 50 against 63 us;
      // at two rounds of 64-row tiles the ring wins)
      if (cdiv(T, 64) * a.tiles_n <= 256) {
        a.tiles_m = cdiv(T, 64);
        return launch<E, 64, 256, KC, FW, PLAIN, STAGE>(a, 1, s);
      }
      return launch_ring<E, KC, FW, PLAIN, STAGE>(a, 1, s);
    }
    else {
      // fp32: with fewer 256 x 256 tiles than CUs (D / 256 per row block),
      // 64-row tiles fill the chip (D = 2048, T = 4096: 128 tiles leave half
      // the CUs idle; 512 64-row tiles made the step 6.5 % faster)
      if (a.tiles_m * a.tiles_n < 256) {
        a.tiles_m = cdiv(T, 64);
        return launch<E, 64, 256, KC, FW, PLAIN, STAGE>(a, 1, s);
      }
      return launch<E, 256, 256, KC, FW, PLAIN, STAGE>(a, 1, s);
    }
  }

  // Backward stage arguments (tiles_m/tiles_n filled by the launchers).
  static KArgs args_dgu(const void* dY, const void* Wd, char* Gp, char* Up, int64_t T, int64_t D, int64_t H) {
    KArgs a{};
    a.a0 = opnd(dY, D, T, D);
    if constexpr (LIN) a.b0 = opnd(Wd, H, H, D);  // Bop[k=d][n=h] = Wd[d][h]: N-contiguous rows
    else a.b0 = opnd(Wd, D, H, D);                // Bop[k=d][n=h] = Wd[h][d]: K-contiguous rows
    a.c0 = Gp;
    a.c1 = Up;
    a.ldc = H;
    a.M = (int)T;
    a.N = (int)H;
    a.planes = 1;
    return a;
  }
  static KArgs args_dwd(const char* Ap, const void* dY, void* dWd, int64_t T, int64_t D, int64_t H) {
    KArgs a{};
    if constexpr (LIN) {
      // dWd [D, H] = dY^T A
      a.a0 = opnd(dY, D, D, T);  // Aop[m=d][k=t] = dY[t][d]
      a.b0 = opnd(Ap, H, H, T);  // Bop[k=t][n=h] = A[t][h]
      a.ldc = H;
      a.M = (int)D;
      a.N = (int)H;
    } else {
      // dWd [H, D] = A^T dY
      a.a0 = opnd(Ap, H, H, T);  // Aop[m=h][k=t] = A[t][h]
      a.b0 = opnd(dY, D, D, T);  // Bop[k=t][n=d] = dY[t][d]
      a.ldc = D;
      a.M = (int)H;
      a.N = (int)D;
    }
    a.c0 = (char*)dWd;
    a.tiles_m = cdiv(a.M, 256);
    a.tiles_n = cdiv(a.N, 256);
    a.planes = 1;
    return a;
  }
  static KArgs args_dwgu(const void* X, const char* dGp, const char* dUp, void* dWg, void* dWu, int64_t T,
                         int64_t D, int64_t H) {
    KArgs a{};
    if constexpr (LIN) {
      // dWg, dWu [H, D] = dG^T X, dU^T X: the planes switch the A operand
      a.a0 = opnd(dGp, H, H, T);  // Aop[m=h][k=t] = dG[t][h]
      a.a1 = opnd(dUp, H, H, T);
      a.b0 = opnd(X, D, D, T);    // Bop[k=t][n=d] = X[t][d]
      a.plane_a = 1;
      a.ldc = D;
      a.M = (int)H;
      a.N = (int)D;
    } else {
      // [dWg | dWu] [D, H] = X^T [dG | dU]: the planes switch the B operand
      a.a0 = opnd(X, D, D, T);    // Aop[m=d][k=t] = X[t][d]
      a.b0 = opnd(dGp, H, H, T);  // Bop[k=t][n=h] = dG[t][h]
      a.b1 = opnd(dUp, H, H, T);
      a.ldc = H;
      a.M = (int)D;
      a.N = (int)H;
    }
    a.c0 = (char*)dWg;
    a.c1 = (char*)dWu;
    a.tiles_m = cdiv(a.M, 256);
    a.tiles_n = cdiv(a.N, 256);
    a.planes = 2;
    return a;
  }
  static KArgs args_dx(const char* dGp, const char* dUp, const void* Wg, const void* Wu, void* dX, int64_t T,
                       int64_t D, int64_t H) {
    KArgs a{};
    a.a0 = opnd(dGp, H, T, H);
    a.a1 = opnd(dUp, H, T, H);
    if constexpr (LIN) {
      a.b0 = opnd(Wg, D, D, H);  // Bop[k=h][n=d] = Wg[h][d]: N-contiguous rows
      a.b1 = opnd(Wu, D, D, H);
    } else {
      a.b0 = opnd(Wg, H, D, H);  // Bop[k=h][n=d] = Wg[d][h]: K-contiguous rows
      a.b1 = opnd(Wu, H, D, H);
    }
    a.c0 = (char*)dX;
    a.ldc = D;
    a.M = (int)T;
    a.N = (int)D;
    a.planes = 1;
    return a;
  }

  // Separate launches (stages 2, 3, 4, 5).
  static int bwd_separate(KArgs dgu, KArgs dwd, KArgs dwgu, KArgs dx, int64_t T, int64_t D, int64_t H,
                          hipStream_t s) {
    int rc;
    if (small_t(T)) {
      dgu.tiles_m = cdiv(T, 64);
      dgu.tiles_n = cdiv(H, 256);
      rc = launch<E, 64, 256, KC, BW, DSWIGLU, 2>(dgu, 1, s);
    } else {
      dgu.tiles_m = cdiv(T, 256);
      dgu.tiles_n = cdiv(H, 256);
      rc = launch<E, 256, 256, KC, BW, DSWIGLU, 2>(dgu, 1, s);
    }
    if (rc) return rc;
    if ((rc = launch<E, 256, 256, MC, MC, PLAIN, 3>(dwd, 1, s))) return rc;
    if ((rc = launch<E, 256, 256, MC, MC, PLAIN, 4>(dwgu, 2, s))) return rc;
    if (small_t(T)) {
      dx.tiles_m = cdiv(T, 64);
      dx.tiles_n = cdiv(D, 256);
      return launch<E, 64, 256, KC, BW, DX, 5>(dx, 1, s);
    }
    dx.tiles_m = cdiv(T, 256);
    dx.tiles_n = cdiv(D, 256);
    return launch<E, 256, 256, KC, BW, DX, 5>(dx, 1, s);
  }

  // T > 512. bf16/fp16: the four ring launches (stages 2, 3, 4, 5). fp32 on
  // the register-staged engine: paired launches, {dWd (long K = T), dA +
  // dSwiGLU} as stage 8, then {dWg | dWu (long K = T), dI} as stage 9.
  static int bwd_large(KArgs dgu, KArgs dwd, KArgs dwgu, KArgs dx, int64_t T, int64_t D, int64_t H, float* P,
                       hipStream_t s) {
    dgu.tiles_m = cdiv(T, 256);
    dgu.tiles_n = cdiv(H, 256);
    dx.tiles_m = cdiv(T, 256);
    dx.tiles_n = cdiv(D, 256);
    if constexpr (E::kBytes == 2) {
      // one ring launch per step: measured 0.5 % faster than pairing the
      // short-K stages with the long-K weight gradients on the ring engine
      int rc;
      // dA + dSwiGLU on 64-row tiles when those fit one round (as the down
      // projection; T = 1024, D = 1024, H = 2816: 29 against 43 us)
      if (cdiv(T, 64) * dgu.tiles_n <= 256) {
        KArgs d64 = dgu;
        d64.tiles_m = cdiv(T, 64);
        rc = launch<E, 64, 256, KC, BW, DSWIGLU, 2>(d64, 1, s);
      } else {
        rc = launch_ring<E, KC, BW, DSWIGLU, 2>(dgu, 1, s);
      }
      if (rc) return rc;
      if ((rc = launch_ring_wgrad<E, MC, MC, 3>(dwd, 1, P, s))) return rc;
      if ((rc = launch_ring_wgrad<E, MC, MC, 4>(dwgu, 2, P, s))) return rc;
      // dI as the down projection above (T = 4096, D = 1024: 86 against
      // 100 us)
      if (cdiv(T, 64) * dx.tiles_n <= 256) {
        dx.tiles_m = cdiv(T, 64);
        return launch<E, 64, 256, KC, BW, DX, 5>(dx, 1, s);
      }
      return launch_ring<E, KC, BW, DX, 5>(dx, 1, s);
    } else {
      int rc = launch_pair<E, MC, MC, PLAIN, KC, BW, DSWIGLU, 8>(dwd, dgu, s);
      if (rc) return rc;
      return launch_pair<E, MC, MC, PLAIN, KC, BW, DX, 9>(dwgu, dx, s);
    }
  }
};

template <class E, bool LIN>
int run_fwd(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y, void* saved, int64_t T,
            int64_t D, int64_t H, bool two_round, hipStream_t s) {
  const size_t plane = (size_t)T * H * E::kBytes;
  char* Ap = (char*)saved;
  int rc = Path<E, LIN>::template gateup<0>(X, Wg, Wu, Ap, Ap + plane, Ap + 2 * plane, T, D, H, true, two_round,
                                            nullptr, s);
  if (rc) return rc;
  return Path<E, LIN>::template down<1>(Ap, Wd, Y, T, D, H, nullptr, s);
}

template <class E, bool LIN>
int run_bwd(const void* dY, const void* X, const void* Wg, const void* Wu, const void* Wd, void* saved, void* dX,
            void* dWg, void* dWu, void* dWd, float* P, int64_t T, int64_t D, int64_t H, hipStream_t s) {
  using Pa = Path<E, LIN>;
  const size_t plane = (size_t)T * H * E::kBytes;
  char* Ap = (char*)saved;
  char* Gp = Ap + plane;
  char* Up = Ap + 2 * plane;
  KArgs dgu = Pa::args_dgu(dY, Wd, Gp, Up, T, D, H);
  KArgs dwd = Pa::args_dwd(Ap, dY, dWd, T, D, H);
  KArgs dwgu = Pa::args_dwgu(X, Gp, Up, dWg, dWu, T, D, H);
  KArgs dx = Pa::args_dx(Gp, Up, Wg, Wu, dX, T, D, H);
  if (small_t(T)) return Pa::bwd_separate(dgu, dwd, dwgu, dx, T, D, H, s);
  return Pa::bwd_large(dgu, dwd, dwgu, dx, T, D, H, P, s);
}

template <class E, bool LIN>
int run_infer(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y, void* ws, int64_t T,
              int64_t D, int64_t H, bool two_round, hipStream_t s) {
  using Pa = Path<E, LIN>;
  char* Ap = (char*)ws;
  const InferPlan pl = infer_plan(T, D, H, E::kBytes);
  const StreamArgs sg{1, nullptr, nullptr};
  const bool gs = !LIN && pl.stream, ds = !LIN && pl.down_stream;
  // the gate/up launch (streaming or not) clears the down launch's counters
  unsigned* ctr = ds ? (unsigned*)(Ap + pl.ctr_off) : nullptr;
  int rc = Pa::template gateup<6>(X, Wg, Wu, Ap, nullptr, nullptr, T, D, H, false, two_round, gs ? &sg : nullptr, s,
                                  ctr, ds ? pl.down_units : 0);
  if (rc) return rc;
  // above kInferSplitMaxT tokens an unsplit streaming down projection reads
  // all of A once per 64 columns: the 64-row tile engine is faster there
  const StreamArgs sd{pl.down_splits, pl.down_splits > 1 ? (float*)(Ap + pl.p_off) : nullptr, ctr};
  return Pa::template down<7>(Ap, Wd, Y, T, D, H, ds ? &sd : nullptr, s);
}


}  // namespace swiglu
