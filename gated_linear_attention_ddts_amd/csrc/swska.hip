// swska.hip -- placeholder: the SW-SKA kernel is not built yet.
#include "device_common.h"
#include "launch.h"

namespace rodimus {

bool swska_supported(int dk, int dv, int dtype) { (void)dk; (void)dv; (void)dtype; return false; }
void launch_swska(const SkaArgs &a, hipStream_t st) { (void)a; (void)st; }

}  // namespace rodimus
