// One (dtype, rounds per half row) family of the half-row kernel.  The build
// compiles this file once per family with -DLCE_BF16=0/1 and -DLCE_KH=<rounds
// of 960 vectors per half row>.
#include <type_traits>

#include "ce_rows_half.h"

#if !defined(LCE_BF16) || !defined(LCE_KH)
#error "compile with -DLCE_BF16=<0|1> -DLCE_KH=<n>"
#endif

#define LCE_JOIN3(a, b, c) a##_##b##_##c
#define LCE_FN(b, kh) LCE_JOIN3(launch_rows_half, b, kh)

namespace lce {
hipError_t LCE_FN(LCE_BF16, LCE_KH)(const CEArgs &a, int groups, hipStream_t st) {
    return dev::launch_half_rows<LCE_BF16 != 0, LCE_KH>(a, groups, st);
}
}  // namespace lce
