// The library's own device memory for fp8_block_gemm_backward_w_noalloc: a
// fixed-size array in the code object (every GPU the library runs on holds
// its own copy from module load until the process ends), used where the
// other entry points take a caller's workspace -- the fp32 partial tiles of
// output tiles whose reduction several workgroups share.
//
// Host code must not pass the array's name to a kernel: on the host it is
// only a stand-in symbol, not the device address.  The device address is
// looked up once per device, with that device current, and kept.
#include "../../include/fp8blk.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "fp8blk_launch.h"

namespace fp8blk {

namespace {

static_assert(FP8BLK_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte units");
static __device__ __align__(256) float scratch[FP8BLK_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

}  // namespace

hipError_t static_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // concurrent first calls on a device only repeat the same lookup
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  *bytes = FP8BLK_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace fp8blk
