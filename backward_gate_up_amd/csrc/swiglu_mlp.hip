// swiglu_mlp.hip -- the C ABI of include/swiglu_mlp.h: argument validation,
// size queries, dispatch to the per-dtype drivers (defined in
// instantiate.hip builds) and the stage timer.
#include <mutex>

#include "kernels.hpp"

namespace swiglu {

Timer g_timer;

// the drivers are compiled in their own translation units (instantiate.hip)
#define SWIGLU_DECLARE_DRIVERS(E, LIN)                                                                            \
  extern template int run_fwd<E, LIN>(const void*, const void*, const void*, const void*, void*, void*, int64_t,  \
                                      int64_t, int64_t, bool, hipStream_t);                                       \
  extern template int run_bwd<E, LIN>(const void*, const void*, const void*, const void*, const void*, void*,     \
                                      void*, void*, void*, void*, float*, int64_t, int64_t, int64_t, hipStream_t); \
  extern template int run_infer<E, LIN>(const void*, const void*, const void*, const void*, void*, void*,         \
                                        int64_t, int64_t, int64_t, bool, hipStream_t);
SWIGLU_DECLARE_DRIVERS(Bf16, false)
SWIGLU_DECLARE_DRIVERS(Fp16, false)
SWIGLU_DECLARE_DRIVERS(Fp32, false)
SWIGLU_DECLARE_DRIVERS(Bf16, true)
SWIGLU_DECLARE_DRIVERS(Fp16, true)
SWIGLU_DECLARE_DRIVERS(Fp32, true)
#undef SWIGLU_DECLARE_DRIVERS

// The driver for a dtype code and weight layout.
template <bool LIN>
static int fwd_for(int dtype, const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y, void* saved,
                   int64_t T, int64_t D, int64_t H, bool two_round, hipStream_t s) {
  switch (dtype) {
    case SWIGLU_BF16: return run_fwd<Bf16, LIN>(X, Wg, Wu, Wd, Y, saved, T, D, H, two_round, s);
    case SWIGLU_FP16: return run_fwd<Fp16, LIN>(X, Wg, Wu, Wd, Y, saved, T, D, H, two_round, s);
    default: return run_fwd<Fp32, LIN>(X, Wg, Wu, Wd, Y, saved, T, D, H, two_round, s);
  }
}
template <bool LIN>
static int bwd_for(int dtype, const void* dY, const void* X, const void* Wg, const void* Wu, const void* Wd,
                   void* saved, void* dX, void* dWg, void* dWu, void* dWd, float* P, int64_t T, int64_t D, int64_t H,
                   hipStream_t s) {
  switch (dtype) {
    case SWIGLU_BF16: return run_bwd<Bf16, LIN>(dY, X, Wg, Wu, Wd, saved, dX, dWg, dWu, dWd, P, T, D, H, s);
    case SWIGLU_FP16: return run_bwd<Fp16, LIN>(dY, X, Wg, Wu, Wd, saved, dX, dWg, dWu, dWd, P, T, D, H, s);
    default: return run_bwd<Fp32, LIN>(dY, X, Wg, Wu, Wd, saved, dX, dWg, dWu, dWd, nullptr, T, D, H, s);
  }
}
template <bool LIN>
static int infer_for(int dtype, const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y, void* ws,
                     int64_t T, int64_t D, int64_t H, bool two_round, hipStream_t s) {
  switch (dtype) {
    case SWIGLU_BF16: return run_infer<Bf16, LIN>(X, Wg, Wu, Wd, Y, ws, T, D, H, two_round, s);
    case SWIGLU_FP16: return run_infer<Fp16, LIN>(X, Wg, Wu, Wd, Y, ws, T, D, H, two_round, s);
    default: return run_infer<Fp32, LIN>(X, Wg, Wu, Wd, Y, ws, T, D, H, two_round, s);
  }
}

// Fill kernel (used to clear weight gradients when T = 0 would otherwise
// leave them unwritten; a kernel rather than a memset so that callers may
// capture the path in a graph).
__global__ void fill_zero(u32x4_t* p, int64_t n16) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n16; i += (int64_t)gridDim.x * blockDim.x) p[i] = u32x4_t{0, 0, 0, 0};
}

// ---- validation ----------------------------------------------------------

static size_t elt_bytes(int dt) { return dt == SWIGLU_FP32 ? 4 : (dt == SWIGLU_BF16 || dt == SWIGLU_FP16 ? 2 : 0); }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

struct Range {
  const void* p;
  size_t n;
};
static bool overlap(Range a, Range b) {
  if (a.n == 0 || b.n == 0) return false;
  uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Pointers to non-empty buffers must be non-NULL and 16-byte aligned;
// a buffer of zero bytes (T = 0) may be NULL.
static int check_ptrs(const Range* r, int n) {
  for (int i = 0; i < n; ++i)
    if (r[i].n > 0 && !r[i].p) return SWIGLU_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (r[i].p && !aligned16(r[i].p)) return SWIGLU_ERR_ALIGN;
  return SWIGLU_OK;
}

// Largest D or H (the leading dimensions of every operand) for which the
// kernels' 32-bit per-lane byte offsets stay in range: a tile spans 256 rows
// of an operand, at offsets up to 256 * ld * elt_bytes, and each buffer
// descriptor holds at most 2^31 - 1 bytes. 16-bit: 4194296; fp32: 2097144
// (multiples of 8).
static int64_t max_ld(size_t e) { return ((0x7fffffffLL / (256 * (int64_t)e)) / 8) * 8; }

static int check_shape(int64_t T, int64_t D, int64_t H, size_t e) {
  if (T < 0 || D <= 0 || H <= 0) return SWIGLU_ERR_SHAPE;
  if ((D & 7) || (H & 7)) return SWIGLU_ERR_SHAPE;
  if (D > max_ld(e) || H > max_ld(e)) return SWIGLU_ERR_SHAPE;
  // token rows are int32 inside the kernels, and so is every launch's tile
  // count (64-row tiles of T times 64-column tiles of the wider of D and H)
  if (T > 0x7fffffffLL) return SWIGLU_ERR_SHAPE;
  const int64_t w = (D > H ? D : H) / 64 + 1;
  if ((T / 64 + 1) > 0x3fffffffLL / w) return SWIGLU_ERR_SHAPE;
  return SWIGLU_OK;
}

static int check_device() {
  static int cached[64];  // 0 unknown, 1 ok, 2 bad
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SWIGLU_ERR_DEVICE;
  if (cached[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return SWIGLU_ERR_DEVICE;
    cached[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  return cached[dev] == 1 ? SWIGLU_OK : SWIGLU_ERR_DEVICE;
}

static int zero_fill(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return SWIGLU_OK;
  int64_t n16 = (int64_t)(bytes / 16);
  int blocks = (int)((n16 + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero, dim3(blocks), dim3(256), 0, s, (u32x4_t*)p, n16);
  return hipGetLastError() == hipSuccess ? SWIGLU_OK : SWIGLU_ERR_LAUNCH;
}

// ---- fixed scratch of the allocation-free no-grad entry point -------------
// The no-grad workspace of swiglu_mlp_infer_noalloc lives in this array,
// one copy per device, held until the process ends. In host code its name
// is only a host-side stand-in: the device address of this device's copy
// comes from hipGetSymbolAddress (once per device, with that device
// current), and only that address is ever handed to kernels.
static __device__ __attribute__((aligned(256))) unsigned char scratch[SWIGLU_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

static int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SWIGLU_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SWIGLU_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SWIGLU_OK;
}

}  // namespace swiglu

using namespace swiglu;

extern "C" {

size_t swiglu_mlp_saved_bytes(int64_t T, int64_t H, int dtype) {
  size_t e = elt_bytes(dtype);
  if (!e || T < 0 || H <= 0) return 0;
  return 3 * (size_t)T * (size_t)H * e;
}

size_t swiglu_mlp_infer_workspace_bytes(int64_t T, int64_t D, int64_t H, int dtype) {
  size_t e = elt_bytes(dtype);
  if (!e || T < 0 || D <= 0 || H <= 0) return 0;
  return infer_plan(T, D, H, e).total;
}

size_t swiglu_mlp_bwd_workspace_bytes(int64_t T, int64_t D, int64_t H, int dtype) {
  const size_t e = elt_bytes(dtype);
  if (e != 2 || T <= 0 || D <= 0 || H <= 0 || small_t(T)) return 0;
  return splitk_bytes(T, D, H);
}

int swiglu_mlp_fwd_ex(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y, void* saved, int64_t T,
                      int64_t D, int64_t H, int dtype, unsigned flags, hipStream_t stream) {
  size_t e = elt_bytes(dtype);
  if (!e) return SWIGLU_ERR_DTYPE;
  if (flags & ~SWIGLU_FLAGS_ALL) return SWIGLU_ERR_FLAGS;
  const bool two_round = (flags & SWIGLU_FLAG_TWO_ROUND) != 0;
  int rc = check_shape(T, D, H, e);
  if (rc) return rc;
  Range in[] = {{X, (size_t)T * D * e}, {Wg, (size_t)D * H * e}, {Wu, (size_t)D * H * e}, {Wd, (size_t)H * D * e}};
  Range out[] = {{Y, (size_t)T * D * e}, {saved, 3 * (size_t)T * H * e}};
  if ((rc = check_ptrs(in, 4)) || (rc = check_ptrs(out, 2))) return rc;
  for (auto& o : out)
    for (auto& i : in)
      if (overlap(o, i)) return SWIGLU_ERR_ALIAS;
  if (overlap(out[0], out[1])) return SWIGLU_ERR_ALIAS;
  if ((rc = check_device())) return rc;
  if (T == 0) return SWIGLU_OK;
  if (flags & SWIGLU_FLAG_LINEAR_WEIGHTS)
    return fwd_for<true>(dtype, X, Wg, Wu, Wd, Y, saved, T, D, H, two_round, stream);
  return fwd_for<false>(dtype, X, Wg, Wu, Wd, Y, saved, T, D, H, two_round, stream);
}

int swiglu_mlp_fwd(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y, void* saved, int64_t T,
                   int64_t D, int64_t H, int dtype, hipStream_t stream) {
  return swiglu_mlp_fwd_ex(X, Wg, Wu, Wd, Y, saved, T, D, H, dtype, 0u, stream);
}

int swiglu_mlp_bwd_ex(const void* dY, const void* X, const void* Wg, const void* Wu, const void* Wd, void* saved,
                      void* dX, void* dWg, void* dWu, void* dWd, void* workspace, size_t workspace_bytes, int64_t T,
                      int64_t D, int64_t H, int dtype, unsigned flags, hipStream_t stream) {
  size_t e = elt_bytes(dtype);
  if (!e) return SWIGLU_ERR_DTYPE;
  if (flags & ~SWIGLU_FLAGS_ALL) return SWIGLU_ERR_FLAGS;
  int rc = check_shape(T, D, H, e);
  if (rc) return rc;
  const size_t td = (size_t)T * D * e, dh = (size_t)D * H * e;
  const size_t need = swiglu_mlp_bwd_workspace_bytes(T, D, H, dtype);
  Range in[] = {{dY, td}, {X, td}, {Wg, dh}, {Wu, dh}, {Wd, dh}, {saved, 3 * (size_t)T * H * e}};
  Range out[] = {{dX, td}, {dWg, dh}, {dWu, dh}, {dWd, dh}, {workspace, need}};
  if ((rc = check_ptrs(in, 6)) || (rc = check_ptrs(out, 4))) return rc;
  if (need > 0 && (!workspace || workspace_bytes < need)) return SWIGLU_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return SWIGLU_ERR_ALIGN;
  for (int i = 0; i < 5; ++i) {
    for (auto& r : in)
      if (overlap(out[i], r)) return SWIGLU_ERR_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (overlap(out[i], out[j])) return SWIGLU_ERR_ALIAS;
  }
  if ((rc = check_device())) return rc;
  if (T == 0) {
    // Sums over zero tokens: the weight gradients are zero; dX is empty.
    if ((rc = zero_fill(dWg, dh, stream))) return rc;
    if ((rc = zero_fill(dWu, dh, stream))) return rc;
    return zero_fill(dWd, dh, stream);
  }
  if (flags & SWIGLU_FLAG_LINEAR_WEIGHTS)
    return bwd_for<true>(dtype, dY, X, Wg, Wu, Wd, saved, dX, dWg, dWu, dWd, (float*)workspace, T, D, H, stream);
  return bwd_for<false>(dtype, dY, X, Wg, Wu, Wd, saved, dX, dWg, dWu, dWd, (float*)workspace, T, D, H, stream);
}

int swiglu_mlp_bwd(const void* dY, const void* X, const void* Wg, const void* Wu, const void* Wd, void* saved,
                   void* dX, void* dWg, void* dWu, void* dWd, void* workspace, size_t workspace_bytes, int64_t T,
                   int64_t D, int64_t H, int dtype, hipStream_t stream) {
  return swiglu_mlp_bwd_ex(dY, X, Wg, Wu, Wd, saved, dX, dWg, dWu, dWd, workspace, workspace_bytes, T, D, H, dtype,
                           0u, stream);
}

int swiglu_mlp_infer_ex(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y, void* workspace,
                        size_t workspace_bytes, int64_t T, int64_t D, int64_t H, int dtype, unsigned flags,
                        hipStream_t stream) {
  size_t e = elt_bytes(dtype);
  if (!e) return SWIGLU_ERR_DTYPE;
  if (flags & ~SWIGLU_FLAGS_ALL) return SWIGLU_ERR_FLAGS;
  const bool two_round = (flags & SWIGLU_FLAG_TWO_ROUND) != 0;
  int rc = check_shape(T, D, H, e);
  if (rc) return rc;
  const size_t need = swiglu_mlp_infer_workspace_bytes(T, D, H, dtype);
  Range in[] = {{X, (size_t)T * D * e}, {Wg, (size_t)D * H * e}, {Wu, (size_t)D * H * e}, {Wd, (size_t)H * D * e}};
  Range yr[] = {{Y, (size_t)T * D * e}};
  if ((rc = check_ptrs(in, 4)) || (rc = check_ptrs(yr, 1))) return rc;
  if (need > 0 && (!workspace || workspace_bytes < need)) return SWIGLU_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return SWIGLU_ERR_ALIGN;
  Range out[] = {{Y, (size_t)T * D * e}, {workspace, need}};
  for (auto& o : out)
    for (auto& i : in)
      if (overlap(o, i)) return SWIGLU_ERR_ALIAS;
  if (overlap(out[0], out[1])) return SWIGLU_ERR_ALIAS;
  if ((rc = check_device())) return rc;
  if (T == 0) return SWIGLU_OK;
  if (flags & SWIGLU_FLAG_LINEAR_WEIGHTS)
    return infer_for<true>(dtype, X, Wg, Wu, Wd, Y, workspace, T, D, H, two_round, stream);
  return infer_for<false>(dtype, X, Wg, Wu, Wd, Y, workspace, T, D, H, two_round, stream);
}

int swiglu_mlp_infer(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y, void* workspace,
                     size_t workspace_bytes, int64_t T, int64_t D, int64_t H, int dtype, hipStream_t stream) {
  return swiglu_mlp_infer_ex(X, Wg, Wu, Wd, Y, workspace, workspace_bytes, T, D, H, dtype, 0u, stream);
}

int swiglu_mlp_infer_noalloc(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y, int64_t T,
                             int64_t D, int64_t H, int dtype, unsigned flags, hipStream_t stream) {
  size_t e = elt_bytes(dtype);
  if (!e) return SWIGLU_ERR_DTYPE;
  if (flags & ~SWIGLU_FLAGS_ALL) return SWIGLU_ERR_FLAGS;
  int rc = check_shape(T, D, H, e);
  if (rc) return rc;
  const size_t need = swiglu_mlp_infer_workspace_bytes(T, D, H, dtype);
  if (need > SWIGLU_NOALLOC_SCRATCH_BYTES) return SWIGLU_ERR_SCRATCH;
  Range in[] = {{X, (size_t)T * D * e}, {Wg, (size_t)D * H * e}, {Wu, (size_t)D * H * e}, {Wd, (size_t)H * D * e}};
  Range yr[] = {{Y, (size_t)T * D * e}};
  if ((rc = check_ptrs(in, 4)) || (rc = check_ptrs(yr, 1))) return rc;
  for (auto& i : in)
    if (overlap(yr[0], i)) return SWIGLU_ERR_ALIAS;
  if ((rc = check_device())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  // the scratch is not the caller's memory, but the inputs and Y must not
  // lie in it either
  Range sr{ws, need};
  if (overlap(yr[0], sr)) return SWIGLU_ERR_ALIAS;
  for (auto& i : in)
    if (overlap(i, sr)) return SWIGLU_ERR_ALIAS;
  return swiglu_mlp_infer_ex(X, Wg, Wu, Wd, Y, ws, SWIGLU_NOALLOC_SCRATCH_BYTES, T, D, H, dtype, flags, stream);
}

const char* swiglu_mlp_status_string(int status) {
  switch (status) {
    case SWIGLU_OK: return "ok";
    case SWIGLU_ERR_NULL: return "a required pointer is NULL";
    case SWIGLU_ERR_SHAPE:
      return "bad shape: need T >= 0 and D, H positive multiples of 8, at most 4194296 (bf16/fp16) or 2097144 (fp32)";
    case SWIGLU_ERR_DTYPE: return "unknown dtype";
    case SWIGLU_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SWIGLU_ERR_ALIAS: return "an output overlaps an input or another output";
    case SWIGLU_ERR_WORKSPACE: return "workspace missing or too small";
    case SWIGLU_ERR_DEVICE: return "current device is not gfx950 (or a HIP device query failed)";
    case SWIGLU_ERR_LAUNCH: return "kernel launch failed";
    case SWIGLU_ERR_FLAGS: return "unknown bits in flags";
    case SWIGLU_ERR_SCRATCH:
      return "the call needs more than the fixed scratch of the allocation-free entry point (see "
             "SWIGLU_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int swiglu_mlp_timer_start(int capacity) {
  if (capacity <= 0) return SWIGLU_ERR_SHAPE;
  for (int s = 0; s < SWIGLU_NUM_STAGES; ++s) {
    if (g_timer.ev[s]) {
      for (int i = 0; i < 2 * g_timer.cap; ++i) (void)hipEventDestroy(g_timer.ev[s][i]);
      delete[] g_timer.ev[s];
      g_timer.ev[s] = nullptr;
    }
  }
  g_timer.cap = capacity;
  for (int s = 0; s < SWIGLU_NUM_STAGES; ++s) {
    g_timer.count[s] = 0;
    g_timer.ev[s] = new hipEvent_t[2 * capacity];
    for (int i = 0; i < 2 * capacity; ++i)
      if (hipEventCreate(&g_timer.ev[s][i]) != hipSuccess) return SWIGLU_ERR_DEVICE;
  }
  g_timer.on = true;
  return SWIGLU_OK;
}

int swiglu_mlp_timer_stop(double* ms, int* count, int n) {
  g_timer.on = false;
  for (int s = 0; s < SWIGLU_NUM_STAGES && s < n; ++s) {
    double sum = 0.0;
    for (int i = 0; i < g_timer.count[s]; ++i) {
      float t = 0.f;
      if (hipEventSynchronize(g_timer.ev[s][2 * i + 1]) != hipSuccess) return SWIGLU_ERR_DEVICE;
      if (hipEventElapsedTime(&t, g_timer.ev[s][2 * i], g_timer.ev[s][2 * i + 1]) != hipSuccess)
        return SWIGLU_ERR_DEVICE;
      sum += t;
    }
    if (ms) ms[s] = sum;
    if (count) count[s] = g_timer.count[s];
  }
  return SWIGLU_OK;
}

}  // extern "C"
