// fp32-io instances of the selective-scan kernel (see scan_kernel.h) that
// move io element by element: misaligned pointers or seqlen % 8 != 0.
#include "scan_kernel.h"

namespace ssm {
ScanFn pick_scan_f32_ew(int nsw, int lpc, bool bv, bool cv, bool conv, int mode) {
  return pick_scan<0, false>(nsw, lpc, bv, cv, conv, mode);
}
ScanFn pick_mix_f32_ew(bool bv, bool cv, bool conv) {
  return pick_mix<0, false>(bv, cv, conv);
}
}  // namespace ssm
