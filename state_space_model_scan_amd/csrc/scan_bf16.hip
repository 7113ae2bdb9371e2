// bf16-io instances of the selective-scan kernel (see scan_kernel.h).
#include "scan_kernel.h"

namespace ssm {
ScanFn pick_scan_bf16(int nsw, int lpc, bool bv, bool cv, bool conv, int mode) {
  return pick_scan<1>(nsw, lpc, bv, cv, conv, mode);
}
}  // namespace ssm
