// lbq_linear_fwd_noalloc: the forward of lbq_linear_fwd for callers that
// cannot allocate device memory (code under stream capture, tight serving
// loops, harnesses that forbid hipMalloc).  The only scratch memory the
// forward uses -- the fp32 split-K partial sums of the small-batch kernel
// (2 <= m <= 64) and of GEMM launches that split K (m > 64) -- lives in a
// fixed array in the library's device image instead of a caller workspace;
// inputs and outputs are still the caller's.
//
// The array below is a device symbol.  Host code never passes its name to a
// kernel (on the host the name is only a stand-in, not a device address):
// the device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and that address is what the kernels receive.
//
// Every call on a device shares that device's array and leaves its contents
// behind.  Nothing in it needs to start at zero: every partial sum is written
// before it is read within the same call.  Calls that overlap on one device
// (two streams, or two host threads) race on the array.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "lbq_internal.h"

namespace {

constexpr size_t kScratchBytes = LBQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of this device's scratch array (looked up on first use).
lbq_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return lbq::set_error(LBQ_E_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return lbq::set_error(LBQ_E_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return lbq::set_error(LBQ_E_HIP, e != hipSuccess ? hipGetErrorString(e) : "scratch symbol has no address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LBQ_OK;
}

}  // namespace

extern "C" lbq_status lbq_linear_fwd_noalloc(const lbq_desc* desc, const lbq_qtensor* q, const uint16_t* X,
                                             int64_t m, uint16_t* Y, int64_t ldy, void* stream) {
  lbq_status st = lbq::check_fwd(desc, q, X, m, Y, ldy);
  if (st != LBQ_OK) return st;
  if (m == 0) return lbq::linear_fwd_body(desc, q, X, m, Y, ldy, nullptr, 0, stream, "lbq_linear_fwd_noalloc");
  // The small-batch kernel's partials are required; the GEMM's K-split
  // partials (m > kSkinnyMaxM) are used when they fit the array, and the
  // GEMM runs unsplit when they do not.
  const size_t need = lbq_linear_workspace_bytes(desc, m);
  if (m <= lbq::kSkinnyMaxM && need > kScratchBytes) {
    char buf[160];
    snprintf(buf, sizeof buf, "needs %zu bytes of scratch; the allocation-free forward holds %zu", need,
             kScratchBytes);
    return lbq::set_error(LBQ_E_WORKSPACE, buf);
  }
  void* p = nullptr;
  if (need > 0 && (st = scratch_of_current_device(&p)) != LBQ_OK) return st;
  return lbq::linear_fwd_body(desc, q, X, m, Y, ldy, p, need > 0 ? kScratchBytes : 0, stream,
                              "lbq_linear_fwd_noalloc");
}
