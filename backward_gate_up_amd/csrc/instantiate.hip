// instantiate.hip -- defines one per-dtype driver of kernels.hpp (and so
// instantiates its kernels). Compiled once per combination with
// -DSWIGLU_INST_DTYPE=0|1|2 (bf16, fp16, fp32), -DSWIGLU_INST_OP=0|1|2
// (run_fwd, run_bwd, run_infer) and -DSWIGLU_INST_LIN=0|1 (kernel or linear
// weight layout); the build links all eighteen objects with the C ABI of
// swiglu_mlp.hip.
#include "kernels.hpp"

#if !defined(SWIGLU_INST_DTYPE) || !defined(SWIGLU_INST_OP) || !defined(SWIGLU_INST_LIN)
#error "compile with -DSWIGLU_INST_DTYPE=<0|1|2> -DSWIGLU_INST_OP=<0|1|2> -DSWIGLU_INST_LIN=<0|1>"
#endif

namespace swiglu {
#if SWIGLU_INST_DTYPE == 0
using InstE = Bf16;
#elif SWIGLU_INST_DTYPE == 1
using InstE = Fp16;
#else
using InstE = Fp32;
#endif

#if SWIGLU_INST_OP == 0
template int run_fwd<InstE, SWIGLU_INST_LIN>(const void*, const void*, const void*, const void*, void*, void*, int64_t, int64_t,
                            int64_t, bool, hipStream_t);
#elif SWIGLU_INST_OP == 1
template int run_bwd<InstE, SWIGLU_INST_LIN>(const void*, const void*, const void*, const void*, const void*, void*, void*, void*,
                            void*, void*, float*, int64_t, int64_t, int64_t, hipStream_t);
#else
template int run_infer<InstE, SWIGLU_INST_LIN>(const void*, const void*, const void*, const void*, void*, void*, int64_t, int64_t,
                              int64_t, bool, hipStream_t);
#endif
}  // namespace swiglu
