// gemm_tile.hpp -- LDS-staged MFMA tile engine for gfx950 (CDNA4).
//
// One engine serves the six contractions of the SwiGLU MLP ("[RFC] Full-
// pipeline SwiGLU MLP with forward/backward co-optimization", Liger-Kernel
// issue #1347, section "Summary"): every stage is a dense GEMM
//     C[m][n] = sum_k Aop[m][k] * Bop[k][n]
// whose operands arrive in one of two layouts:
//   K-contiguous  ("KC"): element (r, k) at base[r * ld + k]
//   MN-contiguous ("MC"): element (r, k) at base[k * ld + r]
// where r is the operand's row index (m for Aop, n for Bop).
//
// Work split. A workgroup is 256 threads = 4 waves in a 2 x 2 grid and owns a
// BM x BN tile of C; each wave owns (BM/2) x (BN/2) as 32 x 32 MFMA tiles.
// The MFMA computes D = P * Q with P rows = n and Q columns = m, so that each
// lane's accumulator holds 4 consecutive n for one m (an 8-byte row-major
// store in bf16). Accumulation is fp32 throughout.
//
// Data movement per K step (BK = 128 bytes of K per row):
//   global -> registers: raw buffer loads (16 B per lane) at per-lane offsets
//     fixed for the tile; K advances through the scalar offset or a rebased
//     descriptor. Out-of-range chunks get an offset past the descriptor's
//     size, so the hardware returns zeros: ragged M, N and K tails need no
//     separate loop.
//   registers -> LDS: KC tiles are stored [row][K] with the 16-byte chunk
//     index XOR-ed by (row >> 1) & 7; MC tiles are stored [K][row] with padding.
//   LDS -> MFMA operands: KC tiles with ds_read_b128 (8 consecutive K of one
//     row per lane); MC tiles with ds_read_b64_tr_b16, which transposes 16 x
//     4 blocks across each group of 16 lanes so that every lane again holds
//     consecutive K values of one row. fp32 tiles use ds_read_b128 / b32.
//   Two LDS stages: the global loads of step k+1 are in flight while step k
//   runs on the matrix cores; one barrier per step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swiglu {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

enum { KC = 0, MC = 1 };

// ---------------------------------------------------------------------------
// Element types
// ---------------------------------------------------------------------------
struct Bf16 {
  using elem = __bf16;
  using vec4 = bf16x4_t;
  static constexpr int kBytes = 2;
  static constexpr int kBK = 64;  // K per stage (128 bytes of each row)
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t p, u32x4_t q, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, p),
                                                   __builtin_bit_cast(bf16x8_t, q), c, 0, 0, 0);
  }
  // 16 x 16 x 32: lane l holds row l % 16 of p and column l % 16 of q, K
  // (l / 16) * 8 .. + 7; the result's lane l holds column l % 16, rows
  // (l / 16) * 4 .. + 3
  // c += p x q in place: the accumulator stays in its AGPRs (the builtin's
  // 4-register results are not kept tied to their inputs by the register
  // allocator, which then copies and spills them). A volatile statement also
  // keeps its place among the loads, so the source order is the issue order.
  // The compiler inserts no MFMA hazard waits around it: callers separate the
  // first and last MFMA of a tile from VALU accesses of the accumulators.
  static __device__ __forceinline__ void mfma16(f32x4_t& c, u32x4_t p, u32x4_t q) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(p), "v"(q));
  }
  static __device__ __forceinline__ elem from_f32(float x) { return (__bf16)x; }
  static __device__ __forceinline__ float to_f32(elem x) { return (float)x; }
};

struct Fp16 {
  using elem = _Float16;
  using vec4 = f16x4_t;
  static constexpr int kBytes = 2;
  static constexpr int kBK = 64;
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t p, u32x4_t q, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, p),
                                                  __builtin_bit_cast(f16x8_t, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void mfma16(f32x4_t& c, u32x4_t p, u32x4_t q) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(p), "v"(q));
  }
  static __device__ __forceinline__ elem from_f32(float x) { return (_Float16)x; }
  static __device__ __forceinline__ float to_f32(elem x) { return (float)x; }
};

struct Fp32 {
  using elem = float;
  using vec4 = f32x4_t;
  static constexpr int kBytes = 4;
  static constexpr int kBK = 32;
  static __device__ __forceinline__ elem from_f32(float x) { return x; }
  static __device__ __forceinline__ float to_f32(elem x) { return x; }
};

// ---------------------------------------------------------------------------
// Buffer resources
// ---------------------------------------------------------------------------
// Word 3 of a raw (unstructured) buffer descriptor on CDNA: 32-bit data
// format, no swizzle, offsets bounds-checked against num_records.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;  // offset that always fails the check

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  int32_t n = bytes > 0x7fffffffLL ? 0x7fffffff : (bytes < 0 ? 0 : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, kRsrcWord3);
}
// The same for a size already known to lie in [0, 2^31).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc32(const void* p, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, kRsrcWord3);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words (base, 16 address bits | stride 0, size, flags)
// for loads issued from inline assembly.
__device__ __forceinline__ i32x4_t rsrc_words(const void* p, int64_t bytes) {
  const uint64_t b = (uint64_t)p;
  const int n = bytes > 0x7fffffffLL ? 0x7fffffff : (bytes < 0 ? 0 : (int)bytes);
  return i32x4_t{(int)(uint32_t)b, (int)((b >> 32) & 0xffff), n, kRsrcWord3};
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const char*)p;
}

// Direct-to-LDS load of 16 bytes per lane from buffer offset voff + soff to
// LDS address lds + 16 * lane (lds is wave-uniform). Issued from inline
// assembly, the compiler neither sees the LDS write nor waits for it: the
// caller waits (s_waitcnt vmcnt counts this wave's loads in issue order) and
// publishes with a barrier. The memory clobber keeps other memory accesses
// on their side of it. The LDS address goes in through an {m0} operand, so
// the compiler itself writes M0 and knows that it changed; the s_nop is the
// wait state between that write and the load that reads it.
__device__ __forceinline__ void dma16(uint32_t lds, i32x4_t rs, uint32_t voff, uint32_t soff) {
  // wave-uniform by contract; readfirstlane keeps them in scalar registers
  // where the compiler could not prove it
  lds = __builtin_amdgcn_readfirstlane(lds);
  soff = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               ::"v"(voff), "s"(rs), "s"(soff), "{m0}"(lds)
               : "memory");
}

__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// An operand of the tile engine: where it is and how it is laid out.
// ---------------------------------------------------------------------------
struct Operand {
  const char* base;  // element (0, 0)
  int64_t ld;        // leading dimension in elements
  int rows;          // extent of the row index (m or n)
  int k;             // extent of K
};

// Tile geometry shared by kernels and host launchers.
template <class E, int BM, int BN, int AL, int BL>
struct Geometry {
  static constexpr int EB = E::kBytes;
  static constexpr int BK = E::kBK;
  static constexpr int CE = 16 / EB;  // elements per 16-byte chunk
  static constexpr int PAD = (EB == 2) ? 32 : 8;  // MC row padding (elements)
  static constexpr int A_BYTES = AL == KC ? BM * BK * EB : BK * (BM + PAD) * EB;
  static constexpr int B_BYTES = BL == KC ? BN * BK * EB : BK * (BN + PAD) * EB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int WTM = BM / 2, WTN = BN / 2;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold at least one 32x32 MFMA tile");
  static_assert(LDS <= 160 * 1024, "exceeds gfx950 LDS");
};

// XOR swizzle of the 16-byte chunk index of K-contiguous LDS rows (128 B per
// row). The LDS serves a 16-byte-per-lane read in groups of 16 lanes over 64
// banks (256 B); a group reads 16 consecutive rows at one logical chunk, and
// rows r and r+1 fall in different bank halves, so XOR-ing with (r >> 1) & 7
// spreads each group over all 16 bank quads.
__device__ __forceinline__ int kc_swz(int r) { return (r >> 1) & 7; }

// Loads of one operand tile (R rows x BK) into registers, and their LDS
// store. LR is the row count of the LDS tile the rows land in (a tile may be
// filled from two sources, each supplying R = LR/2 rows at a row offset).
template <class E, int R, int LAYOUT, int LR = R>
struct TileLoader {
  static constexpr int EB = E::kBytes;
  static constexpr int BK = E::kBK;
  static constexpr int CE = 16 / EB;
  static constexpr int PAD = (EB == 2) ? 32 : 8;
  static constexpr int CHUNKS = R * BK * EB / 16;  // 16-byte chunks per tile
  static constexpr int PER_THREAD = CHUNKS / 256;
  static_assert(CHUNKS % 256 == 0, "tile must split evenly over 256 threads");
  static constexpr int CPR = R * EB / 16;  // MC: chunks per K row

  u32x4_t v[PER_THREAD];
  uint32_t voff[PER_THREAD];  // per-lane byte offsets, fixed for the tile

  // Per-tile setup: the byte offset of each of this thread's chunks within a
  // K stage. KC: rows past the operand get an out-of-range offset (the
  // hardware returns zeros). MC: columns past the operand read whatever
  // follows in memory; they only feed output rows/columns that are never
  // stored, and K rows past the end fall outside the stage's descriptor.
  __device__ __forceinline__ void init(const Operand& op, int r0, int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = tid + 256 * i;
      if constexpr (LAYOUT == KC) {
        const int r = c >> 3, kc = c & 7;
        voff[i] = (r0 + r < op.rows) ? (uint32_t)(r * (int)op.ld * EB + kc * 16) : kOOB;
      } else {
        const int kr = c / CPR, mc = c % CPR;
        voff[i] = (uint32_t)(kr * (int)op.ld * EB + mc * 16);
      }
    }
  }

  // Global -> registers for K columns [k0, k0 + BK) and rows [r0, r0 + R).
  // Steady state: no per-lane address arithmetic (KC advances the scalar
  // offset, MC rebases the descriptor); only a ragged last K stage of a KC
  // operand masks its chunks.
  __device__ __forceinline__ void load(const Operand& op, int r0, int k0, int tid) {
    if constexpr (LAYOUT == KC) {
      const char* tb = op.base + (int64_t)r0 * op.ld * EB;
      const int64_t bytes = ((int64_t)(op.rows - r0)) * op.ld * EB;
      __amdgpu_buffer_rsrc_t rs = make_rsrc(tb, bytes);
      const int soff = k0 * EB;
      if (k0 + BK <= op.k) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], soff, 0);
      } else {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
          const int kc = (tid + 256 * i) & 7;
          const bool ok = k0 + kc * CE < op.k;
          v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? voff[i] : kOOB, soff, 0);
        }
      }
    } else {
      const char* tb = op.base + (int64_t)k0 * op.ld * EB + (int64_t)r0 * EB;
      const int64_t bytes = ((int64_t)(op.k - k0)) * op.ld * EB - (int64_t)r0 * EB;
      __amdgpu_buffer_rsrc_t rs = make_rsrc(tb, bytes);
#pragma unroll
      for (int i = 0; i < PER_THREAD; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i], 0, 0);
    }
  }

  // Registers -> LDS; the rows land at rows [row_off, row_off + R) of the
  // LDS tile.
  __device__ __forceinline__ void store(char* lds, int tid, int row_off = 0) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int c = tid + 256 * i;
      if constexpr (LAYOUT == KC) {
        int r = row_off + (c >> 3), kc = c & 7;
        *(u32x4_t*)(lds + r * 128 + ((kc ^ kc_swz(r)) << 4)) = v[i];
      } else {
        int kr = c / CPR, mc = c % CPR;
        *(u32x4_t*)(lds + kr * (LR + PAD) * EB + row_off * EB + mc * 16) = v[i];
      }
    }
  }
};

// MFMA operand fragment for rows [ro, ro + 32) of a tile with R rows and
// K sub-step ks. 16-bit types: one u32x4 = 8 consecutive K values of row
// ro + (lane & 31), K = ks*16 + (lane >> 5)*8 + 0..7.
template <class E, int R, int LAYOUT>
__device__ __forceinline__ u32x4_t frag16(const char* lds, int ro, int ks, int lane) {
  if constexpr (LAYOUT == KC) {
    int row = ro + (lane & 31);
    int chunk = ks * 2 + (lane >> 5);
    return *(const u32x4_t*)(lds + row * 128 + ((chunk ^ kc_swz(row)) << 4));
  } else {
    constexpr int PAD = 32;
    constexpr int STRIDE = (R + PAD) * 2;
    // ds_read_b64_tr_b16: in each 16-lane block, lane i receives element j
    // from the address given by lane 4j + i/4, at column i % 4. Lane r points
    // at K row (r / 4) and columns 4*(r % 4) .. +3 of its 16-column block.
    int krow = ks * 16 + (lane >> 5) * 8 + ((lane & 15) >> 2);
    int col = ro + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    const char* p = lds + krow * STRIDE + col * 2;
    s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
    s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * STRIDE));
    u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  }
}

// fp32: 4 K values of row ro + (lane & 31), K = ks*8 + (lane >> 5)*4 + 0..3.
// MFMA j of the sub-step takes value j; for both operands lane l < 32 then
// holds K = ks*8 + j and lane l >= 32 holds ks*8 + 4 + j, which is the same
// pairing on both sides, so the sum over K is unchanged.
template <int R, int LAYOUT>
__device__ __forceinline__ f32x4_t frag32(const char* lds, int ro, int ks, int lane) {
  if constexpr (LAYOUT == KC) {
    int row = ro + (lane & 31);
    int chunk = ks * 2 + (lane >> 5);
    return *(const f32x4_t*)(lds + row * 128 + ((chunk ^ kc_swz(row)) << 4));
  } else {
    constexpr int STRIDE = (R + 8) * 4;
    int k = ks * 8 + (lane >> 5) * 4;
    const char* p = lds + k * STRIDE + (ro + (lane & 31)) * 4;
    return f32x4_t{*(const float*)p, *(const float*)(p + STRIDE), *(const float*)(p + 2 * STRIDE),
                   *(const float*)(p + 3 * STRIDE)};
  }
}

// MFMA operands of one K sub-step for a wave: TM fragments of the A tile
// and TN of the B tile (4 dwords each). A K stage (BK) is NSUB = 4 sub-steps:
// 16 K per sub-step for 16-bit types (one MFMA), 8 K for fp32 (four MFMAs).
constexpr int NSUB = 4;

template <class E, int BM, int BN, int AL, int BL, int TM, int TN>
struct Frags {
  u32x4_t a[TM], b[TN];

  __device__ __forceinline__ void read(const char* lds_a, const char* lds_b, const int (&a_rows)[TM],
                                       const int (&b_rows)[TN], int ks, int lane) {
    if constexpr (E::kBytes == 2) {
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = frag16<E, BN, BL>(lds_b, b_rows[j], ks, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = frag16<E, BM, AL>(lds_a, a_rows[i], ks, lane);
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = __builtin_bit_cast(u32x4_t, frag32<BN, BL>(lds_b, b_rows[j], ks, lane));
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = __builtin_bit_cast(u32x4_t, frag32<BM, AL>(lds_a, a_rows[i], ks, lane));
    }
  }

  // acc[i][j] += P(b[j]) * Q(a[i]): rows of the MFMA result are n, columns m.
  __device__ __forceinline__ void mma(f32x16_t (&acc)[TM][TN]) const {
    if constexpr (E::kBytes == 2) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = E::mfma(b[j], a[i], acc[i][j]);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            // copy the element out first: bit-casting a vector-element
            // lvalue directly reads element 0
            const uint32_t bs = b[j][s], as = a[i][s];
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, bs),
                                                            __builtin_bit_cast(float, as), acc[i][j], 0, 0, 0);
          }
    }
  }

  static constexpr int kMfma = TM * TN * (E::kBytes == 2 ? 1 : 4);
  static constexpr int kReads = (E::kBytes == 2) ? (TM * (AL == MC ? 2 : 1) + TN * (BL == MC ? 2 : 1))
                                                 : (TM * (AL == MC ? 4 : 1) + TN * (BL == MC ? 4 : 1));
};

// Scheduling hint: alternate the sub-step's MFMAs with its LDS traffic so that
// the matrix pipe never waits behind a burst of DS instructions.
template <int NMFMA, int NDS>
__device__ __forceinline__ void interleave_mfma_ds() {
  constexpr int per = (NDS + NMFMA - 1) / NMFMA;
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x300, per, 0);  // then DS read/write
  }
}

// Map the workgroup id to a (tile_m, tile_n) pair. Consecutive workgroup ids
// are dealt round-robin to the 8 XCDs, each with its own L2; renumber so that
// each XCD receives a contiguous run of tiles, then walk tiles in groups of
// G M-tiles (M fastest) so that concurrently running tiles share operands:
// the 32 tiles an XCD runs at once cover G M-tiles x 32/G N-tiles.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int G, int& tm, int& tn) {
  int nb = tiles_m * tiles_n;
  int nb8 = nb & ~7;
  if (bid < nb8) bid = (bid & 7) * (nb8 >> 3) + (bid >> 3);
  int group = bid / (G * tiles_n);
  int first_m = group * G;
  int gm = tiles_m - first_m < G ? tiles_m - first_m : G;
  int in = bid - group * G * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

}  // namespace swiglu
