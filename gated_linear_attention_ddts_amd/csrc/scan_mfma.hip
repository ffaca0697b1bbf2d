// scan_mfma.hip -- placeholder: the MFMA prefill kernel is not built yet.
#include "device_common.h"
#include "launch.h"

namespace rodimus {

ScanPlan plan_scan(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
    (void)B; (void)H; (void)T; (void)dk; (void)dv; (void)chunk; (void)dtype;
    return ScanPlan{false, 1, 0};
}

void launch_scan_mfma(const ScanArgs &a, const ScanPlan &p, hipStream_t st) {
    (void)p;
    launch_scan_generic(a, st);
}

}  // namespace rodimus
