// One (dtype, register rounds, LDS rounds) family of the persistent row kernel.
// The build compiles this file once per family with -DLCE_BF16=0/1,
// -DLCE_KR=<rounds in VGPRs> and -DLCE_KL=<rounds in LDS>, so the many
// instantiations compile in parallel.
#include "ce_rows.h"

#if !defined(LCE_BF16) || !defined(LCE_KR) || !defined(LCE_KL)
#error "compile with -DLCE_BF16=<0|1> -DLCE_KR=<n> -DLCE_KL=<n>"
#endif

#define LCE_JOIN4(a, b, c, d) a##_##b##_##c##_##d
#define LCE_FN(b, kr, kl) LCE_JOIN4(launch_rows, b, kr, kl)

namespace lce {
hipError_t LCE_FN(LCE_BF16, LCE_KR, LCE_KL)(const CEArgs &a, int max_groups, hipStream_t st) {
    return dev::launch_rows<LCE_BF16 != 0, LCE_KR, LCE_KL>(a, max_groups, st);
}
}  // namespace lce
