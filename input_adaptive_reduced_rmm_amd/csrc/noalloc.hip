// rmm_gemm_noalloc: the reduced product with its scratch memory in a fixed
// device array of the library instead of a caller's workspace, for callers
// that cannot allocate.
//
// `scratch` below is a file-scope device array: every GPU the library runs on
// holds its own copy (at its own address) until the process ends.  Host code
// never passes the array's name to a kernel (on the host that name is only a
// stand-in, not a device address): the first call on each device looks the
// device address up with hipGetSymbolAddress while that device is current,
// keeps it per device, and hands that pointer to rmm_gemm as the workspace.
//
// Every call on one device shares that device's array: calls that overlap on
// one GPU (two streams, two threads) race on it.  Nothing in it needs to start
// at zero: the pack writes every byte of A[:, I] and the index copy that the
// product reads, the transposed weight slice is written whole, and every
// split of the few-row kernel writes all of its partial sums.
#include <mutex>

#include "rmm_internal.h"

#define RMM_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = RMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up once per
// device, with that device current).
hipError_t scratch_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

RMM_API rmm_status_t rmm_gemm_noalloc(rmm_dtype_t dt, const void *A, int64_t lda, const void *B, int64_t ldb,
                                      const int32_t *idx, int64_t m, int64_t d, int64_t n, int64_t k, void *Y,
                                      int64_t ldy, rmm_stream_t stream) {
  // Argument errors first, as rmm_gemm reports them; then the scratch size.
  const rmm_status_t chk = rmm::gemm_args_check("gemm_noalloc", dt, A, lda, B, ldb, idx, m, d, n, k, Y, ldy, nullptr);
  if (chk != RMM_OK) return chk;
  const size_t need = rmm_gemm_workspace_bytes(dt, m, n, k);
  if (need > kScratchBytes)
    return rmm::set_error(RMM_ERR_UNSUPPORTED,
                          "gemm_noalloc: this product needs %zu bytes of scratch; the fixed array holds %zu "
                          "(use rmm_gemm with a workspace)", need, kScratchBytes);
  void *ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return rmm::set_error(RMM_ERR_HIP, "gemm_noalloc: scratch address: %s", hipGetErrorString(e));
  return rmm_gemm(dt, A, lda, B, ldb, idx, m, d, n, k, Y, ldy, ws, kScratchBytes, stream);
}
