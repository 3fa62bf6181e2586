// Launch geometry of the persistent kernels: workgroups that fill the current
// device exactly once (resident workgroups per compute unit x compute units).
#include "launch.h"

namespace spdec {

hipError_t persistent_grid(const void* kernel, int block, size_t dyn_lds, int* grid) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, dyn_lds);
  if (e != hipSuccess) return e;
  *grid = cus * (per_cu > 0 ? per_cu : 1);
  return hipSuccess;
}

int device_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

}  // namespace spdec
