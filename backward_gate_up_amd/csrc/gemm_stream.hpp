// gemm_stream.hpp -- split-K weight streaming for the no-grad forward with
// few tokens (T <= 128), gfx950.
//
// With a handful of tokens the no-grad forward is a pass over the 3*D*H
// weights ("[RFC] Full-pipeline SwiGLU MLP with forward/backward
// co-optimization", sections "Summary" and "Inference results"). What limits
// such a pass on a CU is the number of requests it may have in flight to L2,
// so every request must carry a whole 128-byte line: a unit covers 64 output
// columns, whose weight rows are exactly one line (bf16/fp16). There are then
// only N/64 units (16 for the down projection at D = 1024), so K is split
// across workgroups as well: workgroup (unit, split) streams K steps
// [split * per, (split + 1) * per) of its 64 columns, its waves split that
// range again, add their sums through LDS and write one fp32 partial block
// to a workspace (the waves' sums are added one 16-column block at a time,
// so that they fit in LDS next to up to 8 token tiles). A second kernel adds
// the partials of each output in split order (deterministic) and applies the
// epilogue.
//
// Per wave and K step of 32: the 32 x 64 slab of each weight matrix (4 KiB:
// four direct-to-LDS loads of 8 rows x 128 bytes) and the activation tiles
// (16 tokens x 32 K each) land in a wave-private LDS slot, 2 to 4 slots deep,
// issued from inline assembly and waited for explicitly (dma16).
#pragma once
#include "gemm_skinny.hpp"

namespace swiglu {
namespace stream {

constexpr int KS = 32;        // K per step (one 16x16x32 MFMA)
constexpr int NC = 64;        // output columns per unit
constexpr int WSLAB = 4096;   // 32 K rows x 64 columns x 2 B

// Chunk swizzle of a 128-byte slab row: 16-byte chunk c of K row r sits at
// c ^ wswz(r). The transposed reads of one instruction touch rows
// {0..3, 8..11} (+16) of the slab at one 32-byte column block; with this
// swizzle the four even (odd) rows among them use four distinct chunk pairs,
// so the 32 lanes of a half-wave read 64 distinct banks.
__device__ __forceinline__ int wswz(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }

// Operand of the 16x16x32 MFMA: columns 16 cb .. 16 cb + 15 of the slab, as
// the 16 x 32 (column x K) matrix. ds_read_b64_tr_b16 gives lane i of each
// 16-lane block element j from the address of lane 4j + i/4, column i % 4, so
// lane r of block b points at K row 8b + r/4 (and + 4) and columns
// 16 cb + 4 (r % 4) .. + 3.
__device__ __forceinline__ u32x4_t wfrag(const char* slab, int cb, int lane) {
  const int b = lane >> 4, r = lane & 15;
  const int row = b * 8 + (r >> 2);
  const int byte = cb * 32 + (r & 3) * 8;  // within the logical row
  const char* p0 = slab + row * 128 + ((((byte >> 4) ^ wswz(row)) << 4) | (byte & 15));
  const char* p1 = slab + (row + 4) * 128 + ((((byte >> 4) ^ wswz(row + 4)) << 4) | (byte & 15));
  s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0);
  s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p1);
  u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
}

// Splits of K for `units` column units and `steps` K steps: about 512
// workgroups (two rounds over 256 CUs), each with at least two steps per wave.
__host__ __device__ inline int splits_for(int units, int steps, int waves) {
  int s = (512 + units - 1) / units;
  const int cap = steps / (2 * waves);
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

}  // namespace stream
}  // namespace swiglu
