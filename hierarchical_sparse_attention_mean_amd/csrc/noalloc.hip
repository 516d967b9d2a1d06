// noalloc.hip -- llsa_index_transpose_noalloc: the CSR -> CSC transpose with its workspace in a static device
// array instead of a caller-provided buffer, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on holds its own copy until the
// process ends.  In host code its name is only a host-side stand-in, so the device address of each GPU's copy
// is looked up once per device with hipGetSymbolAddress (with that device current) and cached; only that
// address is ever passed to kernels.  Calls on one GPU share the array and keep the last call's contents: the
// transpose kernels clear what must start at zero themselves (the column counters, with a fill kernel), so a
// call never depends on an earlier one, but two calls that overlap in time on one GPU race on the array.
#include <atomic>
#include <mutex>

#include "launch.hpp"
#include "llsa.h"

namespace llsa {
int resolve_transpose(const llsa_problem* prob, Geom* g, CscGeom* cg, size_t* cnt_bytes, size_t* ws_bytes);
int check_device_gfx950();
}  // namespace llsa

namespace {

static __device__ __align__(256) unsigned char scratch[LLSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch` (looked up on the first call on that device).
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LLSA_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LLSA_ERR_LAUNCH;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LLSA_OK;
}

}  // namespace

extern "C" int llsa_index_transpose_noalloc(const llsa_problem* prob, const int32_t* idx, int32_t* col_ptr,
                                            int32_t* perm, hipStream_t stream) {
  llsa::Geom g;
  llsa::CscGeom cg;
  size_t cnt_bytes = 0, ws_bytes = 0;
  const int s = llsa::resolve_transpose(prob, &g, &cg, &cnt_bytes, &ws_bytes);
  if (s != LLSA_OK) return s;
  if (ws_bytes > (size_t)LLSA_NOALLOC_SCRATCH_BYTES) return LLSA_ERR_SCRATCH;
  if (g.bh == 0) return LLSA_OK;
  if (!idx || !col_ptr || !perm) return LLSA_ERR_NULL;
  if (((uintptr_t)idx | (uintptr_t)col_ptr | (uintptr_t)perm) & 15u) return LLSA_ERR_ALIGN;
  const int sd = llsa::check_device_gfx950();
  if (sd != LLSA_OK) return sd;
  void* base = nullptr;
  const int sp = scratch_ptr(&base);
  if (sp != LLSA_OK) return sp;
  int32_t* cnt = static_cast<int32_t*>(base);
  int32_t* tmp = reinterpret_cast<int32_t*>(static_cast<char*>(base) + cnt_bytes);
  return llsa::launch_index_transpose(g, cg, idx, col_ptr, perm, cnt, tmp, stream) == hipSuccess ? LLSA_OK
                                                                                                 : LLSA_ERR_LAUNCH;
}
