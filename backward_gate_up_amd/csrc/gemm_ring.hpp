// gemm_ring.hpp -- direct-to-LDS, 4-stage pipeline for the 16-bit training
// GEMMs (256 x 256 output tiles, 4 waves), gfx950.
//
// Why: with operands staged through registers, a 256 x 256 x 64 stage can
// only be fetched one stage (about 1 us) ahead -- the accumulators and the
// staging registers fill the register file -- and every barrier then waits
// for the slowest L2 miss. Here global memory is copied straight into LDS by
// buffer_load ... lds (no registers, no ds_write), into a ring of four 32 KiB
// stages, three stages ahead of the matrix cores.
//
// Stage s of the K loop lives in LDS array (s & 3). Each stage holds the A
// tile and the B tile (16 KiB each):
//   K-major (KC) tile: 256 rows x 32 K = 64 B per row; the 16-byte chunk c of
//     row r sits at chunk c ^ ((r >> 2) & 3), so the 16 rows that one
//     16-lane group of a ds_read_b128 reads fall on 16 distinct bank quads.
//   M/N-major (MC) tile: two 128-column sub-tiles of 32 K rows x 256 B; chunk
//     c (0..15) of K row kr sits at c ^ mc_swz(kr), so the two 16-lane
//     groups of a half-wave of ds_read_b64_tr_b16 (4 K rows each, 8 rows
//     apart, 32 bytes per row) read 8 distinct 32-byte bank ranges.
//
// The matrix cores run v_mfma_f32_16x16x32: measured on all CUs under the
// chip's power limit, back-to-back 16x16x32 MFMAs sustain 2041 TFLOP/s
// against 1780 for 32x32x16 (the wider instruction reads and writes a
// 16-register accumulator per 16 K, the narrower 4 registers per 32 K).
// One buffer_load_dwordx4 ... lds writes 1 KiB of consecutive LDS (lane i at
// M0 + 16 i, measured on the device), so the swizzle is applied on the global
// side: each lane fetches the logical chunk that belongs at its slot.
//
// Synchronisation per stage s: issue the loads of stage s + 3 (into the slot
// of stage s - 1, which every wave finished reading before the previous
// barrier); run sub-step 0 of stage s while reading sub-step 1's fragments;
// wait until this wave's own loads of stage s + 1 have landed (vmcnt counts
// this wave's loads in issue order), then a barrier publishes stage s + 1 to
// all waves; run sub-step 1 while reading stage s + 1's first fragments. The
// barrier only waits for LDS traffic (lgkmcnt), never for the loads still in
// flight for later stages.
#pragma once
#include "gemm_tile.hpp"

namespace swiglu {
namespace ring {

constexpr int BK = 32;               // K per stage of the four-stage ring
constexpr int OPB = 256 * BK * 2;    // one operand tile per stage: 16 KiB
constexpr int STAGE = 2 * OPB;       // 32 KiB
constexpr int L = 8;                 // loads per wave per stage (4 for A, 4 for B)

typedef __attribute__((address_space(3))) void lds_void_t;

// Geometry of one 256-row (KC) or 256-column (MC) operand tile holding BKT
// values of K.
template <int BKT>
struct Geo {
  static_assert(BKT == 32 || BKT == 64, "stage depth");
  static constexpr int ROWB = BKT * 2;            // bytes of a K-major row
  static constexpr int LPR = ROWB / 16;           // lanes per K-major row in one load
  static constexpr int RPI = 64 / LPR;            // K-major rows per 1-KiB load
  static constexpr int OPB = 256 * ROWB;          // bytes per operand tile
  static constexpr int PPW = OPB / 1024 / 4;      // 1-KiB loads per wave and operand
  static constexpr int SUB = OPB / 2;             // MC: bytes per 128-column sub-tile
};

// K-major tile: chunk c of row r. 64-byte rows: c ^ ((r >> 2) & 3); 128-byte
// rows: c ^ ((r >> 1) & 7). Either way the 16 rows read by one 16-lane group
// of a ds_read_b128 land on distinct bank quads.
template <int BKT>
__device__ __forceinline__ int kc_swz(int r) {
  return BKT == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}
template <int BKT>
__device__ __forceinline__ int kc_off(int r, int c) {
  return r * Geo<BKT>::ROWB + ((c ^ kc_swz<BKT>(r)) << 4);
}

// MC chunk swizzle of K row kr: bits 2-3 from kr & 3, bit 1 from kr & 8.
__device__ __forceinline__ int mc_swz(int kr) { return ((kr & 3) << 2) | (((kr >> 3) & 1) << 1); }

template <int BKT>
__device__ __forceinline__ int mc_off(int kr, int col) {
  const int sub = col >> 7, cc = col & 127;
  return sub * Geo<BKT>::SUB + kr * 256 + (((cc >> 3) ^ mc_swz(kr)) << 4) + (cc & 7) * 2;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Barrier that waits for this wave's LDS traffic only (not for loads in
// flight to later stages); the memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The loads of one operand tile for one stage: this wave issues PPW of the
// 1-KiB pieces (pieces PPW*w .. PPW*w + PPW - 1).
template <int LAYOUT, int BKT = BK>
struct Dma {
  using G = Geo<BKT>;
  uint32_t voff[G::PPW];

  // Per-tile lane offsets. r0 is the first row (KC) or, for MC, unused here:
  // MC sub-tiles are positioned through the descriptor. KC with `halves`:
  // the tile's rows [0, 128) and [128, 256) are rows [r0, r0 + 128) of two
  // operands of the same shape (waves 0-1 load the first, waves 2-3 the
  // second; the caller passes each wave its operand).
  __device__ __forceinline__ void init(const Operand& op, int r0, int wave, int lane, bool halves = false) {
#pragma unroll
    for (int j = 0; j < G::PPW; ++j) {
      if constexpr (LAYOUT == KC) {
        const int r = (wave * G::PPW + j) * G::RPI + lane / G::LPR;  // row of the LDS tile
        const int rr = halves ? (r & 127) : r;                       // row of the operand, from r0
        const int c = (lane % G::LPR) ^ kc_swz<BKT>(r);
        voff[j] = (r0 + rr < op.rows) ? (uint32_t)(rr * (int)op.ld * 2 + c * 16) : kOOB;
      } else {
        const int kr = ((wave & 1) * G::PPW + j) * 4 + (lane >> 4);
        const int c = (lane & 15) ^ mc_swz(kr);
        voff[j] = (uint32_t)(kr * (int)op.ld * 2 + c * 16);
      }
    }
  }

  // Descriptor of a KC operand's rows [r0, op.rows). It does not change
  // along K, so a tile builds it once, not at every stage.
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t kc_rsrc(const Operand& op, int r0) {
    return make_rsrc(op.base + (int64_t)r0 * op.ld * 2, ((int64_t)(op.rows - r0)) * op.ld * 2);
  }

  // KC: rows [r0, r0 + 256), K columns [k0, k0 + BKT) into `tile`; this
  // wave's pieces j0 .. j1 - 1.
  __device__ __forceinline__ void issue_kc(const Operand& op, int r0, int k0, char* tile, int wave, int lane,
                                           int j0 = 0, int j1 = G::PPW) {
    issue_kcr<true>(kc_rsrc(op, r0), op.k, k0, tile, wave, lane, j0, j1);
  }
  // The same from the tile's descriptor `rs` of an operand with K = kk.
  // KT = false: K is a multiple of BKT, so no stage has a K tail and the
  // per-chunk check is compiled out.
  template <bool KT>
  __device__ __forceinline__ void issue_kcr(const __amdgpu_buffer_rsrc_t rs, int kk, int k0, char* tile, int wave,
                                            int lane, int j0 = 0, int j1 = G::PPW) {
    const bool tail = KT && k0 + BKT > kk;
#pragma unroll
    for (int j = 0; j < G::PPW; ++j) {
      if (j < j0 || j >= j1) continue;
      const int q = wave * G::PPW + j;
      uint32_t vo = voff[j];
      if (tail) {
        const int r = q * G::RPI + lane / G::LPR;
        const int c = (lane % G::LPR) ^ kc_swz<BKT>(r);
        if (k0 + c * 8 >= kk) vo = kOOB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + q * 1024), 16, vo, k0 * 2, 0, 0);
    }
  }

  // An M/N-major operand as this wave reads it (waves 0-1: columns from c0
  // of op0, waves 2-3: from c1 of op1), built once per tile. The K loops
  // carry the first row of the next stage to load from stage to stage (one
  // 64-bit add of stride()); only the stage that reaches the last K row has a
  // descriptor of its own size.
  struct McSrc {
    const char* base;  // K row 0, column cs
    int64_t rowb;      // bytes per K row
    int kk;            // K rows
    int cs2;           // cs in bytes
  };
  __device__ __forceinline__ static McSrc mc_src(const Operand& op0, int c0, const Operand& op1, int c1,
                                                 int wave) {
    const bool second = wave >= 2;
    const Operand& op = second ? op1 : op0;
    const int cs = second ? c1 : c0;
    return McSrc{op.base + (int64_t)cs * 2, op.ld * 2, op.k, cs * 2};
  }
  // K rows [k0, k0 + BKT) of the wave's sub-tile. A stage that ends before
  // the last K row gets BKT rows of descriptor (its reads past column N, if
  // any, land in the next row, which exists); the stage that reaches it gets
  // exactly the bytes up to the end of K row kk - 1, so rows past K read as
  // zeros and nothing past the matrix is touched. BKT rows of the leading
  // dimension stay below 2^31 bytes (the shape limit), so the size is int32.
  __device__ __forceinline__ void issue_mcs(const McSrc& m, int k0, char* tile, int wave, int j0 = 0,
                                           int j1 = G::PPW) {
    issue_mcp(m, m.base + (int64_t)k0 * m.rowb, k0, tile, wave, j0, j1);
  }
  // Bytes per stage of BKT K rows.
  __device__ __forceinline__ static int64_t stride(const McSrc& m) { return BKT * m.rowb; }
  // The same with the stage's first row at hand: row = base + k0 * rowb. The
  // last stage's size depends only on the operand (loop-invariant), so a
  // stage costs two compares and selects for it; a stage past K (k0 >= kk)
  // gets an empty descriptor.
  __device__ __forceinline__ void issue_mcp(const McSrc& m, const char* row, int k0, char* tile, int wave,
                                           int j0 = 0, int j1 = G::PPW) {
    const int rb = (int)m.rowb;
    const int klast = ((m.kk - 1) / BKT) * BKT;  // first K row of the last stage
    int tail = (m.kk - klast) * rb - m.cs2;
    tail = tail < 0 ? 0 : tail;
    const int n = k0 + BKT < m.kk ? BKT * rb : (k0 < m.kk ? tail : 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc32(row, n);
#pragma unroll
    for (int j = 0; j < G::PPW; ++j) {
      if (j < j0 || j >= j1) continue;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + (wave * G::PPW + j) * 1024), 16, voff[j],
                                               0, 0, 0);
    }
  }

  // MC: sub-tile 0 = columns [c0, c0 + 128) of op0, sub-tile 1 = columns
  // [c1, c1 + 128) of op1, K rows [k0, k0 + BKT). Waves 0-1 fill sub-tile 0,
  // waves 2-3 sub-tile 1. K rows past op.k fall outside the descriptor
  // (zeros); columns past the matrix only feed unstored outputs.
  __device__ __forceinline__ void issue_mc(const Operand& op0, int c0, const Operand& op1, int c1, int k0,
                                           char* tile, int wave, int j0 = 0, int j1 = G::PPW) {
    const bool second = wave >= 2;
    const char* base = second ? op1.base : op0.base;
    const int64_t ld = second ? op1.ld : op0.ld;
    const int kk = second ? op1.k : op0.k;
    const int cs = second ? c1 : c0;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(base + (int64_t)k0 * ld * 2 + (int64_t)cs * 2, ((int64_t)(kk - k0)) * ld * 2 - (int64_t)cs * 2);
#pragma unroll
    for (int j = 0; j < G::PPW; ++j) {
      if (j < j0 || j >= j1) continue;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + (wave * G::PPW + j) * 1024), 16, voff[j],
                                               0, 0, 0);
    }
  }
};

// Operand fragment of v_mfma_f32_16x16x32: 8 consecutive K of row (KC) or
// column (MC) ro + (lane & 15), K = ks * 32 + (lane >> 4) * 8 + 0..7, from a
// ring stage tile.
template <int LAYOUT, int BKT = BK>
__device__ __forceinline__ u32x4_t frag(const char* tile, int ro, int ks, int lane) {
  if constexpr (LAYOUT == KC) {
    return *(const u32x4_t*)(tile + kc_off<BKT>(ro + (lane & 15), ks * 4 + (lane >> 4)));
  } else {
    // ds_read_b64_tr_b16: lane i of each 16-lane block receives element j
    // from the address of lane 4j + i/4, column i % 4. Lane r of block b
    // points at K row ks*32 + 8b + r/4 (and + 4), columns ro + 4 (r % 4)
    // .. + 3, so after the transpose lane i of block b holds column ro + i,
    // K rows ks*32 + 8b .. + 7.
    const int krow = ks * 32 + (lane >> 4) * 8 + ((lane & 15) >> 2);
    const int col = ro + (lane & 3) * 4;
    s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + mc_off<BKT>(krow, col)));
    s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + mc_off<BKT>(krow + 4, col)));
    u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  }
}

// Half h of an M/N-major fragment (K rows + 4h of each lane's 8): one
// ds_read_b64_tr_b16 into registers 2h, 2h + 1 of d.
template <int BKT>
__device__ __forceinline__ void frag_half(u32x4_t& d, const char* tile, int ro, int ks, int lane, int h) {
  const int krow = ks * 32 + (lane >> 4) * 8 + ((lane & 15) >> 2) + 4 * h;
  const int col = ro + (lane & 3) * 4;
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + mc_off<BKT>(krow, col)));
  u32x2_t v2 = __builtin_bit_cast(u32x2_t, v);
  if (h == 0) { d[0] = v2[0]; d[1] = v2[1]; } else { d[2] = v2[0]; d[3] = v2[1]; }
}
// The LDS reads of a group after MFMA n of a quadrant: K-major, fragment
// n / 2 after each even n < 8; M/N-major, half n % 2 of fragment n / 2 after
// each n < 8 (one transposing read per MFMA).
template <int LAYOUT, int BKT>
__device__ __forceinline__ void read_piece(u32x4_t (&g)[4], const char* tile, const int (&rows)[8], int r0, int ks,
                                           int lane, int n) {
  if (n >= 8) return;
  if constexpr (LAYOUT == KC) {
    if (n % 2 == 0) g[n / 2] = frag<KC, BKT>(tile, rows[r0 + n / 2], ks, lane);
  } else {
    frag_half<BKT>(g[n / 2], tile, rows[r0 + n / 2], ks, lane, n % 2);
  }
}

// One wave's fragments for the 32-K steps of its 128 x 128 block, in four
// groups of four: A rows 0-63 and 64-127 (a[0], a[1]) and B columns 0-63 and
// 64-127 (b[0], b[1]), 64 registers. A step runs four quadrants of 16 MFMAs,
// one A half times one B half each, in an order that alternates with the
// step's parity P (f = P, s = 1 - P):
//   Q0 = a[0] x b[f], Q1 = a[0] x b[s], Q2 = a[1] x b[s], Q3 = a[1] x b[f].
// a[0] is last used in Q1, b[s] in Q2, a[1] and b[f] in Q3, and the next
// step (parity 1 - P) starts with a[0] x b[s]. So each quadrant reads one
// group into registers freed by the quadrant before and needed by the
// quadrant after: Q0 reads b[s] of this step, Q1 a[1] of this step, Q2 a[0]
// of the next, Q3 b[s] of the next (its b[f']). With the new group's
// fragments in the outer loop of the quadrant that uses it, every LDS read
// has at least 16 MFMAs to land, and no group is double-buffered.
//
// The MFMAs are volatile statements, and the compiler keeps loads and LDS
// reads in their source order around them, so the interleave written here
// is the one issued: the reads of a quadrant's group are spread over its
// first 8 MFMAs (read_piece; measured 1.5-2.5 % faster for the M/N-major
// weight gradients than all reads after MFMAs 0-3), and its NL global loads
// follow MFMAs 1,
// 1 + 16/NL, ... (all four waves leave a barrier together; loads issued back
// to back would queue at the texture unit at once and hold up the MFMA issue
// behind them).
template <class E, int AL, int BL, int BKT = BK>
struct RingFrags {
  u32x4_t a[2][4], b[2][4];

  template <int H>
  __device__ __forceinline__ void read_a(const char* at, const int (&ar)[8], int ks, int lane) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[H][k] = frag<AL, BKT>(at, ar[4 * H + k], ks, lane);
  }
  template <int H>
  __device__ __forceinline__ void read_b(const char* bt, const int (&br)[8], int ks, int lane) {
#pragma unroll
    for (int k = 0; k < 4; ++k) b[H][k] = frag<BL, BKT>(bt, br[4 * H + k], ks, lane);
  }
  // acc[4 HA + i][4 HB + j] += A x B (acc[i][j], lane l: output row
  // ar[i] + l % 16, columns br[j] + (l / 16) * 4 .. + 3); after(n) runs
  // after MFMA n (a constant once unrolled). BN: B fragments in the outer
  // loop (n = 4 j + i), for a quadrant whose B group was read in the
  // quadrant before: fragment k is then first used by MFMA 4 k, not k.
  template <int HA, int HB, bool BN, class After>
  __device__ __forceinline__ void quad(f32x4_t (&acc)[8][8], After&& after) {
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int i = BN ? p : o, j = BN ? o : p;
        E::mfma16(acc[4 * HA + i][4 * HB + j], b[HB][j], a[HA][i]);
        after(4 * o + p);
      }
  }

  // One step of parity P on the stage tile (at, bt) at K offset ks * 32.
  // mid() runs between Q1 and Q2 (the barrier that publishes the next
  // step's tile, if that is a new stage); the next step's fragments come
  // from (nat, nbt, nks) when NX. issue(q, k) issues load k (< NL) of
  // quadrant q.
  template <int P, int NL, bool NX, class Mid, class Issue>
  __device__ __forceinline__ void step(f32x4_t (&acc)[8][8], const char* at, const char* bt, int ks,
                                       const char* nat, const char* nbt, int nks, const int (&ar)[8],
                                       const int (&br)[8], int lane, Mid&& mid, Issue&& issue) {
    constexpr int F = P, S = 1 - P;
    static_assert(NL > 0 && NL <= 16 && 16 % NL == 0, "loads per quadrant");
    constexpr int EV = 16 / NL;
    auto load = [&](int q, int n) {
      if (n % EV == 1) issue(q, n / EV);
    };
    // Q0 and Q1 take the B group read in the quadrant before, Q2 the A
    // group; Q3 has none new
    quad<0, F, true>(acc, [&](int n) {
      read_piece<BL, BKT>(b[S], bt, br, 4 * S, ks, lane, n);
      load(0, n);
    });
    quad<0, S, true>(acc, [&](int n) {
      read_piece<AL, BKT>(a[1], at, ar, 4, ks, lane, n);
      load(1, n);
    });
    mid();
    quad<1, S, false>(acc, [&](int n) {
      if (NX) read_piece<AL, BKT>(a[0], nat, ar, 0, nks, lane, n);
      load(2, n);
    });
    quad<1, F, false>(acc, [&](int n) {
      if (NX) read_piece<BL, BKT>(b[S], nbt, br, 4 * S, nks, lane, n);
      load(3, n);
    });
  }
};

// The compiler does not see the MFMAs above as MFMAs, so it inserts none of
// the wait states that separate an MFMA from VALU work on its registers.
// acc_fence is a row of empty volatile statements, one per accumulator row,
// that each take the row as an in-out operand, so VALU accesses of a row
// stay on their side of its statement and the statements keep their order.
// START (after the zero fill): the last statement waits 5 states, which
// every fill precedes and every MFMA follows (a VALU result read by an
// MFMA). End (before the epilogue): the first one waits 24 states, which
// every MFMA precedes and every VALU read of an accumulator follows.
template <bool START>
__device__ __forceinline__ void acc_fence(f32x4_t (&acc)[8][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (START ? i == 7 : i == 0) {
      if constexpr (START)
        asm volatile("s_nop 4" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]),
                     "+a"(acc[i][4]), "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
      else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                       "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
    } else {
      asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                   "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
    }
  }
}

}  // namespace ring
}  // namespace swiglu
