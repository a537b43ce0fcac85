// The bf16 GEMM of mt_gemm_ws for callers that cannot allocate device
// memory: the stream-K partial tiles go to a static device array of the
// library instead of a caller workspace.
//
// The array is a device global, so each GPU the library runs on holds its
// own copy for the life of the process.  Host code must not pass the
// array's name to a kernel (on the host it names a host-side stand-in, not
// device memory): the device address is looked up once per device with
// hipGetSymbolAddress and only that address is used.
#include <mutex>

#include "kernels.h"
#include "mt_kernels.h"

// Largest stream-K workspace: 256 persistent workgroups x 2 segment slots x
// one 256 x 256 fp32 tile.  On 256 compute units every split the planner
// makes needs exactly this much (a tail of fewer tiles than workgroups is
// cut into ranges that touch at most two tiles each).
static constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace mt {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on the first
// call on the device, with the device current).
float* scratch_ptr() {
  int dev = 0;
  MT_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) throw ApiError{MT_E_INVALID, "device index beyond the scratch table"};
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    MT_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || ((uintptr_t)p & 255)) throw ApiError{MT_E_HIP, "scratch symbol address"};
    g_ptr[dev] = (float*)p;
  }
  return g_ptr[dev];
}

}  // namespace
}  // namespace mt

using namespace mt;

extern "C" size_t mt_gemm_noalloc_max_ws(void) { return kScratchBytes; }

extern "C" int mt_gemm_noalloc(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                               const float* R, int64_t ldr, int32_t M, int32_t N, int32_t K, int32_t epi,
                               int32_t layout, void* stream) {
  try {
    if (epi < 0 || epi > 2) throw ApiError{MT_E_INVALID, "epi"};
    if (layout < 0 || layout > 3) throw ApiError{MT_E_INVALID, "layout"};
    if (M < 0 || N < 0 || K < 0) throw ApiError{MT_E_INVALID, "negative size"};
    if (!((layout & MT_GEMM_A_KMAJOR ? lda >= M : lda >= K) && (layout & MT_GEMM_B_KMAJOR ? ldb >= N : ldb >= K) &&
          ldc >= N))
      throw ApiError{MT_E_INVALID, "leading dimensions"};
    if (epi == 2 && !(R && ldr >= N)) throw ApiError{MT_E_INVALID, "R"};
    const size_t need = (M > 0 && N > 0 && K > 0) ? gemm_ws_bytes(M, N, K) : 0;
    if (need > kScratchBytes)
      throw ApiError{MT_E_SIZE, "stream-K split needs " + std::to_string(need) + " bytes, more than the " +
                                    std::to_string(kScratchBytes) + "-byte static scratch"};
    float* ws = need ? scratch_ptr() : nullptr;
    gemm_bf16((const uint16_t*)A, lda, (const uint16_t*)B, ldb, layout, C, ldc, R, ldr, M, N, K, (Epi)epi,
              (hipStream_t)stream, ws, need ? kScratchBytes : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) throw HipError{e, "kernel launch"};
    return MT_OK;
  } catch (const ApiError& e) {
    set_error(e.msg);
    return e.code;
  } catch (const HipError& e) {
    set_error(std::string(hipGetErrorString(e.code)) + " in " + e.where);
    return MT_E_HIP;
  }
}
