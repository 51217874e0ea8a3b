// gemm_skinny.hpp -- weight-streaming kernels for few tokens (T <= 64), gfx950.
//
// With a handful of tokens the forward is a pass over the weights (the
// no-grad path of "[RFC] Full-pipeline SwiGLU MLP with forward/backward
// co-optimization", section "Summary"; its "Inference results" measure B=1,
// S up to 256): time is set by how fast 3*D*H weights stream from HBM. The
// output is cut into units of 16 weight columns; one workgroup per unit (688
// units for H = 11008), with consecutive units on one XCD so that the four
// units sharing a 128-byte line of a weight row share one L2. The waves of a
// workgroup (4 to 16, as many as LDS allows) split K and add their partial
// sums through LDS at the end; no global workspace, so the no-grad path
// still writes only A and Y.
//
// Per wave and K step of 32: the 32 x 16 weight slab (32-byte row segments)
// and the activation tiles (16 tokens x 32 K each) are copied straight into a
// wave-private LDS slot (buffer_load ... lds), 3 or 4 slots deep; the weights
// are read back transposed (ds_read_b64_tr_b16) as the 16 x 32 operand of
// v_mfma_f32_16x16x32, the activations with ds_read_b128. The waves never
// wait for one another inside the K loop. The loads are issued from inline
// assembly (dma16) and waited for explicitly: the compiler's own tracking of
// loads into LDS cannot tell the slots apart and would wait for the newest
// load before every read.
#pragma once
#include "gemm_tile.hpp"

namespace swiglu {
namespace skinny {

constexpr int KS = 32;     // K per step (one MFMA)
constexpr int SLAB = 1024; // 32 K rows x 16 columns x 2 B

template <class E>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t p, u32x4_t q, f32x4_t c) {
  if constexpr (sizeof(typename E::elem) == 2 && std::is_same<typename E::elem, __bf16>::value)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, p), __builtin_bit_cast(bf16x8_t, q),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, p), __builtin_bit_cast(f16x8_t, q), c,
                                                  0, 0, 0);
}

// Operand of the 16x16x32 MFMA from a 32 x 16 slab in LDS (row = K, 32 B):
// lane l gets column l % 16, K rows (l / 16) * 8 .. + 7. ds_read_b64_tr_b16
// gives lane i of a 16-lane block element j from the address of lane
// 4j + i/4 at column i % 4; lane r therefore points at K row 4h + r/4 of its
// block's 8 rows and at columns 4 (r % 4) .. + 3.
__device__ __forceinline__ u32x4_t slab_frag(const char* slab, int lane) {
  const int b = lane >> 4, r = lane & 15;
  const char* p = slab + (b * 8 + (r >> 2)) * 32 + (r & 3) * 8;
  s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
  s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * 32));
  u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
}

// Activation tile in LDS: 16 tokens x 32 K (64 B per token); the 16-byte
// chunk c of token row m sits at chunk c ^ ((m >> 2) & 3) so that the 16
// rows one 16-lane group reads fall on distinct bank quads.
__device__ __forceinline__ u32x4_t act_frag(const char* tile, int lane) {
  const int m = lane & 15, c = lane >> 4;
  return *(const u32x4_t*)(tile + m * 64 + ((c ^ ((m >> 2) & 3)) << 4));
}

}  // namespace skinny
}  // namespace swiglu
