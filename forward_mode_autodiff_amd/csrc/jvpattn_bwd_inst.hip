// One head dimension's and one side's instances of the reverse-pass kernels:
// JVPATTN_BWD_D = 64 or 128, JVPATTN_BWD_PART = kLaunchDkv (0; with the rows
// kernel) or kLaunchDq (1).
#include "jvpattn_bwd_kernels.h"

#if !defined(JVPATTN_BWD_D) || !defined(JVPATTN_BWD_PART)
#error "JVPATTN_BWD_D and JVPATTN_BWD_PART must be defined"
#endif

namespace jvpattn {
template hipError_t bwd_launch_part<JVPATTN_BWD_PART, JVPATTN_BWD_D>(const BwdArgs&, int64_t, jvpattn_dtype, int,
                                                                     bool, bool, hipStream_t);
#if JVPATTN_BWD_PART == 0
template hipError_t bwd_launch_part<kLaunchRows, JVPATTN_BWD_D>(const BwdArgs&, int64_t, jvpattn_dtype, int, bool,
                                                                bool, hipStream_t);
#endif
}  // namespace jvpattn
