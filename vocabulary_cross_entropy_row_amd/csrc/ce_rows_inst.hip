// One (dtype, register rounds, LDS rounds, row alignment) family of the
// persistent row kernel.  The build compiles this file once per family with
// -DLCE_BF16=0/1, -DLCE_KR=<rounds in VGPRs>, -DLCE_KL=<rounds in LDS> and
// -DLCE_UA=0/1 (rows that need not start on a 16-byte boundary), so the many
// instantiations compile in parallel.
#include "ce_rows.h"

#if !defined(LCE_BF16) || !defined(LCE_KR) || !defined(LCE_KL) || !defined(LCE_UA)
#error "compile with -DLCE_BF16=<0|1> -DLCE_KR=<n> -DLCE_KL=<n> -DLCE_UA=<0|1>"
#endif

#define LCE_JOIN5(a, b, c, d, e) a##_##b##_##c##_##d##_##e
#define LCE_FN(ua, b, kr, kl) LCE_JOIN5(launch_rows, ua, b, kr, kl)

namespace lce {
hipError_t LCE_FN(LCE_UA, LCE_BF16, LCE_KR, LCE_KL)(const CEArgs &a, int max_groups, hipStream_t st) {
    return dev::launch_rows<LCE_BF16 != 0, LCE_KR, LCE_KL, LCE_UA != 0>(a, max_groups, st);
}
}  // namespace lce
