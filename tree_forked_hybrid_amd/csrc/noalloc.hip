// Device scratch for callers that cannot allocate: the attention workspace (rotated keys and
// transposed values) and a rotary table, in one file-scope device array per GPU.
//
// The array lives in this library's code object: every GPU that runs the library holds its own copy
// until the process ends.  Host code never passes the array's name to a kernel (in host code that name
// is a stand-in, not a device address): the address comes from hipGetSymbolAddress, taken once per
// device with that device current, and every use goes through it.  All calls on one GPU share the
// array and it keeps the last call's contents; calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "flide_internal.hpp"

namespace flide {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocWorkspaceBytes + kNoAllocTableBytes];

__global__ void __launch_bounds__(256) scratch_clear_kernel(uint4* p, int64_t n16) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  void* base = nullptr;  // device address of `scratch` on this GPU
  // rotary table currently held in the table region (theta, d, positions)
  double theta = 0.0;
  int d = 0;
  int max_pos = 0;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

}  // namespace

int noalloc_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_dev[device].base) return int(hipSuccess);
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return int(e);
  // The workspace's value columns between segments are read under a zero mask and must hold finite
  // values: clear the whole array once (a fill kernel on a private stream, waited for here).
  hipStream_t s = nullptr;
  e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e != hipSuccess) return int(e);
  const int64_t n16 = (kNoAllocWorkspaceBytes + kNoAllocTableBytes) / 16;
  hipLaunchKernelGGL(scratch_clear_kernel, dim3(1024), dim3(256), 0, s, reinterpret_cast<uint4*>(ptr), n16);
  e = hipGetLastError();
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipStreamDestroy(s);
  if (e != hipSuccess) return int(e);
  g_dev[device].base = ptr;
  return int(hipSuccess);
}

void* noalloc_workspace(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_dev[device].base;
}

// The table region of the device's scratch and whether it already holds the table of (theta, d, at
// least max_pos positions).  `claim` records that the caller is about to write that table there.
float* noalloc_table(int device, double theta, int d, int max_pos, bool* holds, bool claim) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& ds = g_dev[device];
  if (!ds.base) return nullptr;
  *holds = ds.theta == theta && ds.d == d && ds.max_pos >= max_pos;
  if (claim && !*holds) {
    ds.theta = theta;
    ds.d = d;
    ds.max_pos = max_pos;
  }
  return reinterpret_cast<float*>(static_cast<unsigned char*>(ds.base) + kNoAllocWorkspaceBytes);
}

}  // namespace flide
