// Scratch-free form of the split-K two-path GEMM (sharq_linear_scratchfree),
// for callers that cannot allocate device memory: code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc.
//
// The split-K GEMM keeps its fp32 partial tiles in scratch memory. Here that
// memory is a file-scope device array of a fixed size, which every GPU the
// library runs on holds from module load until the process ends. Host code
// never passes the array's name to a kernel (on the host it names a stand-in
// object, not device memory): the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and the kernels
// receive that address as their workspace argument.
//
// Every call on one GPU uses that GPU's one array, and the partials of a call
// are read back by its second kernel: calls that may overlap in time on one
// GPU (other streams, other host threads) race. Nothing in the array needs to
// start at zero: each split writes its whole partial tile before the second
// kernel reads it.

#include <mutex>

#include "../../include/sharq.h"
#include "sharq_internal.h"

namespace sharq {
namespace {

constexpr int64_t kScratchBytes = SHARQ_SCRATCHFREE_MAX_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte granules");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_addr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on that device).
hipError_t scratch_address(void** addr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_addr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *addr = g_addr[dev];
  return g_err[dev];
}

}  // namespace

bool linear_scratchfree_fits(int64_t T, int64_t O, int64_t K) {
  return linear_workspace_bytes(T, O, K) <= kScratchBytes;
}

hipError_t launch_linear_scratchfree(const uint8_t* bb_codes, const uint8_t* bb_scales, const uint8_t* res_codes,
                                     const uint8_t* res_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                                     int64_t T, int64_t O, int64_t K, float* y, int64_t ldy, hipStream_t stream) {
  if (linear_workspace_bytes(T, O, K) == 0)  // no split planned: no scratch needed
    return launch_linear(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, O, K, y, ldy, stream);
  void* addr = nullptr;
  const hipError_t e = scratch_address(&addr);
  if (e != hipSuccess) return e;
  return launch_linear_ws(bb_codes, bb_scales, res_codes, res_scales, w_codes, w_scales, T, O, K, y, ldy, addr,
                          kScratchBytes, stream);
}

}  // namespace sharq
