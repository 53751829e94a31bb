// Kernel instances of the forward for one (mask kind, causal) pair, chosen
// at compile time: the build compiles this file once per pair
// (-DJVPATTN_INST_MASK=<kind> -DJVPATTN_INST_CAUSAL=<0|1>) so the instances
// build in parallel; with -DJVPATTN_INST_FAMILY=1 it holds the 64-row split
// kernel's instances alone, with 2 the ping-pong kernel's, with 3 the 4-wave
// kernel's at width 128, with 4 the d = 256 kernel's (objects that can take
// compiler flags of their own).
#include "jvpattn_fwd_kernels.h"

#ifndef JVPATTN_INST_MASK
#error "JVPATTN_INST_MASK must be defined"
#endif
#ifndef JVPATTN_INST_CAUSAL
#error "JVPATTN_INST_CAUSAL must be defined"
#endif

namespace jvpattn {
#if defined(JVPATTN_INST_FAMILY) && JVPATTN_INST_FAMILY == 1
// the 64-row split kernel's instances only
template hipError_t launch_fwd_split64<JVPATTN_INST_MASK, (JVPATTN_INST_CAUSAL != 0)>(int, bool, const FwdArgs&,
                                                                                    dim3, hipStream_t);
#elif defined(JVPATTN_INST_FAMILY) && JVPATTN_INST_FAMILY == 2
// the ping-pong kernel's instances only
template hipError_t launch_fwd_pp<JVPATTN_INST_MASK, (JVPATTN_INST_CAUSAL != 0)>(int, bool, const FwdArgs&, dim3,
                                                                               hipStream_t);
#elif defined(JVPATTN_INST_FAMILY) && JVPATTN_INST_FAMILY == 3
// the 4-wave kernel's width-128 instances only
template hipError_t launch_fwd_d128<JVPATTN_INST_MASK, (JVPATTN_INST_CAUSAL != 0)>(int, bool, const FwdArgs&, dim3,
                                                                                 hipStream_t);
#elif defined(JVPATTN_INST_FAMILY) && JVPATTN_INST_FAMILY == 4
// the d = 256 kernel's instances only
template hipError_t launch_fwd_d256<JVPATTN_INST_MASK, (JVPATTN_INST_CAUSAL != 0)>(int, bool, const FwdArgs&, dim3,
                                                                                 hipStream_t);
#else
template hipError_t launch_fwd<JVPATTN_INST_MASK, (JVPATTN_INST_CAUSAL != 0)>(int, int, int, bool, const FwdArgs&,
                                                                            dim3, hipStream_t);
#endif
}  // namespace jvpattn
