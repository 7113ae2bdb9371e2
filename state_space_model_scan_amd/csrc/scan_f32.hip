// fp32-io instances of the selective-scan kernel (see scan_kernel.h).
#include "scan_kernel.h"

namespace ssm {
ScanFn pick_scan_f32(int nsw, int lpc, bool bv, bool cv, bool conv, int mode) {
  return pick_scan<0>(nsw, lpc, bv, cv, conv, mode);
}
}  // namespace ssm
