// fa_bwd_noalloc (include/fa.h): the dense backward with its -D = -rowsum(dO*O)
// scratch in a static device array of the library instead of a caller
// buffer, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable; each GPU that loads the
// library's code holds its own copy at its own address. In host code its
// name is only a stand-in for that symbol, so the device address is looked
// up per device (hipGetSymbolAddress, with that device current) on the first
// call there and kept; kernels receive that address, never the name.
#include <mutex>

#include "fa.h"
#include "fa_common.h"

namespace {

static __device__ __align__(256) float scratch[fa::kBwdScratchRows];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
float* g_scratch[kMaxDevices] = {};  // per device: address of its copy of `scratch`

// Address of the current device's copy of the scratch array; looked up once
// per device. Returns an fa_status.
int scratch_of_current_device(void* stream, float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return FA_ERR_LAUNCH;
    if (sdev != dev) return FA_ERR_ARG;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_LAUNCH;
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* L, void* dQ, void* dK, void* dV,
                              int B, int H, int N, int d, float scale, int dtype, void* stream) {
  fa::BwdParams p{};
  int st = fa::prepare_bwd(Q, K, V, O, dO, L, dQ, dK, dV, nullptr, false, B, H, N, d, scale,
                           dtype, p);
  if (st != FA_OK) return st == fa::kEmptyProblem ? FA_OK : st;
  st = scratch_of_current_device(stream, &p.delta);
  if (st != FA_OK) return st;
  const hipError_t e =
      fa::launch_bwd(p, d, dtype == FA_BF16, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}
