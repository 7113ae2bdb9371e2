// fp32-io instances of the selective-scan kernel (see scan_kernel.h) with
// vector io; the element-by-element instances are in scan_f32_ew.hip.
#include "scan_kernel.h"

namespace ssm {
ScanFn pick_scan_f32(int nsw, int lpc, bool bv, bool cv, bool conv, int mode, bool vec) {
  return vec ? pick_scan<0, true>(nsw, lpc, bv, cv, conv, mode) : pick_scan_f32_ew(nsw, lpc, bv, cv, conv, mode);
}
ScanFn pick_mix_f32(bool bv, bool cv, bool conv, bool vec) {
  return vec ? pick_mix<0, true>(bv, cv, conv) : pick_mix_f32_ew(bv, cv, conv);
}
}  // namespace ssm
