// coda_gemm_epi_noalloc: coda_gemm_epi with its cross-workgroup scratch
// (row / column reduction partials and counters, split partial tiles) in a
// fixed device array owned by the library, for callers that cannot allocate.
#include <mutex>

#include "coda_launch.h"

namespace coda {
namespace {

// The library's scratch on every GPU it runs on, held until the process ends.
// Host code never passes this name to a kernel: on the host it is only a
// stand-in for the symbol; each device's address comes from
// hipGetSymbolAddress below.
__device__ __attribute__((aligned(256))) unsigned char scratch[CODA_NOALLOC_SCRATCH_BYTES];

// The first kCounterBytes hold the cross-workgroup counters at fixed places
// (zero between calls, since every call leaves the counters it used at zero);
// the partial sums and partial tiles of a call follow.  A call's counters
// could otherwise land where an earlier, differently shaped call left partial
// sums.
constexpr size_t kCounterBytes = size_t(1) << 20;
constexpr size_t kCounterWords = kCounterBytes / 4;

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
bool g_cleared[kMaxDevices] = {};

__global__ void zero_kernel(uint4* p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += size_t(gridDim.x) * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

// The scratch address on the current device (looked up once per device, with
// that device current), or an error status.
int scratch_on_current_device(void** out, int* dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("no current HIP device (or more than %d devices)", kMaxDevices);
    return CODA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      set_error("hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return CODA_ERR_HIP;
    }
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  *dev_out = dev;
  return CODA_OK;
}

}  // namespace
}  // namespace coda

extern "C" int coda_gemm_epi_noalloc(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                                     const coda_epi_desc* desc, void* stream) {
  coda::clear_error();
  if (!desc) {
    coda::set_error("descriptor is NULL");
    return CODA_ERR_INVALID_ARG;
  }
  void* ptr = nullptr;
  int dev = -1;
  int st = coda::scratch_on_current_device(&ptr, &dev);
  if (st != CODA_OK) return st;
  coda_epi_desc d = *desc;
  d.workspace = static_cast<char*>(ptr) + coda::kCounterBytes;
  d.workspace_bytes = CODA_NOALLOC_SCRATCH_BYTES - coda::kCounterBytes;
  // the split of the last round takes partial tiles: fewer parts when they do
  // not fit, none at all if need be
  coda::Plan p;
  for (int s = coda::kMaxSplit; s >= 1; --s) {
    st = coda::build_plan_split(A, B, M, N, K, &d, 0, true, s, &p);
    if (st != CODA_ERR_WORKSPACE) break;
  }
  if (st == CODA_ERR_WORKSPACE) {
    coda::Plan q;
    coda::build_plan_split(A, B, M, N, K, &d, 0, false, 1, &q);
    coda::set_error("the call needs %zu bytes of scratch, above the fixed maximum of %zu bytes for partial sums",
                    coda::fused_workspace_bytes(q), size_t(CODA_NOALLOC_SCRATCH_BYTES) - coda::kCounterBytes);
    return st;
  }
  if (st != CODA_OK) return st;
  if (size_t(p.grid_m + p.grid_n + p.split_tiles) > coda::kCounterWords) {
    coda::set_error("the call needs %lld counters, above the fixed maximum of %zu",
                    (long long)(p.grid_m + p.grid_n + p.split_tiles), coda::kCounterWords);
    return CODA_ERR_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  {
    // counters in the scratch must start at zero (every call leaves them zero):
    // clear the whole array once per device, with a kernel rather than a
    // memset so that the call may be captured into a graph
    std::lock_guard<std::mutex> lock(coda::g_mu);
    if (!coda::g_cleared[dev]) {
      hipLaunchKernelGGL(coda::zero_kernel, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(ptr),
                         size_t(CODA_NOALLOC_SCRATCH_BYTES) / 16);
      if (hipGetLastError() != hipSuccess) {
        coda::set_error("clearing the scratch failed");
        return CODA_ERR_HIP;
      }
      coda::g_cleared[dev] = true;
    }
  }
  st = coda::launch_fused_with_counters(p, static_cast<unsigned*>(ptr), s);
  if (st == CODA_ERR_HIP) coda::set_error("HIP launch failed: %s", hipGetErrorString(hipGetLastError()));
  return st;
}
