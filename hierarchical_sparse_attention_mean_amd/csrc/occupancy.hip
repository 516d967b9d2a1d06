// occupancy.hip -- grid sizing of the persistent kernels: how many workgroups of a kernel the current
// device holds at once (compute units x resident workgroups per unit), cached per device and kernel.
#include <mutex>
#include <utility>
#include <vector>

#include "launch.hpp"

namespace llsa {

int resident_workgroups(const void* kernel, int threads) {
  static std::mutex mu;
  static std::vector<std::pair<std::pair<int, const void*>, int>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : cache)
    if (e.first.first == dev && e.first.second == kernel) return e.second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0)
    return 0;
  const int n = cus * per_cu;
  cache.push_back({{dev, kernel}, n});
  return n;
}

int persistent_grid(const void* kernel, int threads, int64_t wanted) {
  int res = resident_workgroups(kernel, threads);
  if (res <= 0) res = 1024;  // occupancy query unavailable: a grid that still fills the chip
  int64_t g = wanted < res ? wanted : res;
  g = (g + 7) / 8 * 8;  // whole rounds over the 8 XCDs
  return (int)(g < 8 ? 8 : g);
}

}  // namespace llsa
