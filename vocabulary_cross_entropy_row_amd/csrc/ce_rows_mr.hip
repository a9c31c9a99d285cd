// One (dtype, waves per row, vectors per lane) family of the short-row kernel.
// The build compiles this file once per family with -DLCE_BF16=0/1,
// -DLCE_P=<waves per row> and -DLCE_KV=<16-byte vectors per lane>.
#include "ce_rows_mr.h"

#if !defined(LCE_BF16) || !defined(LCE_P) || !defined(LCE_KV)
#error "compile with -DLCE_BF16=<0|1> -DLCE_P=<n> -DLCE_KV=<n>"
#endif

#define LCE_JOIN4(a, b, c, d) a##_##b##_##c##_##d
#define LCE_FN(b, p, kv) LCE_JOIN4(launch_rows_mr, b, p, kv)

namespace lce {
hipError_t LCE_FN(LCE_BF16, LCE_P, LCE_KV)(const CEArgs &a, int cus, hipStream_t st) {
    return dev::launch_rows_mr<LCE_BF16 != 0, LCE_P, LCE_KV>(a, cus, st);
}
}  // namespace lce
