// bf16-io instances of the selective-scan kernel (see scan_kernel.h) with
// vector io; the element-by-element instances are in scan_bf16_ew.hip.
#include "scan_kernel.h"

namespace ssm {
ScanFn pick_scan_bf16(int nsw, int lpc, bool bv, bool cv, bool conv, int mode, bool vec) {
  return vec ? pick_scan<1, true>(nsw, lpc, bv, cv, conv, mode) : pick_scan_bf16_ew(nsw, lpc, bv, cv, conv, mode);
}
ScanFn pick_mix_bf16(bool bv, bool cv, bool conv, bool vec) {
  return vec ? pick_mix<1, true>(bv, cv, conv) : pick_mix_bf16_ew(bv, cv, conv);
}
}  // namespace ssm
