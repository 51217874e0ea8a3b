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
//     c (0..15) of K row kr sits at c ^ ((kr & 3) << 2), so the 4 K rows x 4
//     chunks that 32 lanes of a ds_read_b64_tr_b16 read are distinct.
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

template <int BKT>
__device__ __forceinline__ int mc_off(int kr, int col) {
  const int sub = col >> 7, cc = col & 127;
  return sub * Geo<BKT>::SUB + kr * 256 + (((cc >> 3) ^ ((kr & 3) << 2)) << 4) + (cc & 7) * 2;
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
        const int c = (lane & 15) ^ ((kr & 3) << 2);
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
  // of op0, waves 2-3: from c1 of op1), built once per tile so that a stage
  // costs one multiply-add for its base and, only on the stage that reaches
  // the last K row, the exact size of the descriptor.
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
    const int rb = (int)m.rowb;
    int n = k0 + BKT < m.kk ? BKT * rb : (m.kk - k0) * rb - m.cs2;
    n = n < 0 ? 0 : n;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc32(m.base + (int64_t)k0 * m.rowb, n);
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

// Operand fragment (8 consecutive K of row ro + (lane & 31), K = ks*16 +
// (lane >> 5)*8 + 0..7) from a ring stage tile.
template <int LAYOUT, int BKT = BK>
__device__ __forceinline__ u32x4_t frag(const char* tile, int ro, int ks, int lane) {
  if constexpr (LAYOUT == KC) {
    return *(const u32x4_t*)(tile + kc_off<BKT>(ro + (lane & 31), ks * 2 + (lane >> 5)));
  } else {
    // ds_read_b64_tr_b16 (lane i of each 16-lane block receives element j
    // from the address of lane 4j + i/4, column i % 4)
    const int krow = ks * 16 + (lane >> 5) * 8 + ((lane & 15) >> 2);
    const int col = ro + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + mc_off<BKT>(krow, col)));
    s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + mc_off<BKT>(krow + 4, col)));
    u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  }
}

template <class E, int AL, int BL, int BKT = BK>
struct RFrags {
  u32x4_t a[4], b[4];
  // A tile at `at`, B tile at `bt`
  __device__ __forceinline__ void read(const char* at, const char* bt, const int (&ar)[4], const int (&br)[4],
                                       int ks, int lane) {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = frag<BL, BKT>(bt, br[j], ks, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = frag<AL, BKT>(at, ar[i], ks, lane);
  }
  __device__ __forceinline__ void read(const char* stage, const int (&ar)[4], const int (&br)[4], int ks,
                                       int lane) {
    read(stage, stage + Geo<BKT>::OPB, ar, br, ks, lane);
  }
  __device__ __forceinline__ void mma(f32x16_t (&acc)[4][4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = E::mfma(b[j], a[i], acc[i][j]);
  }
  static constexpr int kReads = 4 * (AL == MC ? 2 : 1) + 4 * (BL == MC ? 2 : 1);
};

// Scheduling hint for one sub-step of 16 MFMAs: each MFMA is followed by its
// share of the next sub-step's LDS reads, and the NVM loads are spaced evenly
// (one after every 16/NVM-th MFMA). All four waves reach this point together
// after a barrier; issuing a stage's loads back to back would queue 4 x 8
// loads at the texture unit at once and stall the MFMA issue behind them.
template <int NDS, int NVM>
__device__ __forceinline__ void interleave() {
  constexpr int pd = (NDS + 15) / 16;
  static_assert(NVM == 0 || (NVM <= 16 && 16 % NVM == 0), "loads per sub-step");
  constexpr int every = NVM > 0 ? 16 / NVM : 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, pd, 0);
    if constexpr (NVM > 0)
      if (i % every == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

}  // namespace ring
}  // namespace swiglu
