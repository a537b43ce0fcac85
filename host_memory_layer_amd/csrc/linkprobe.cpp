// Host-link bandwidth measured with the copies the training step itself
// issues: hipMemcpyAsync on a prefetch and an offload stream, or the two
// SDMA engine queues of dma.h.  The pages size the host store so that one
// DMA burst per layer block fills the link (radar.chestersoft.de,
// "Methodik", layer-contiguous tiling); this probe measures what such
// bursts reach on this machine, per direction and with both at once.
#include <chrono>
#include <thread>

#include "common.h"
#include "dma.h"
#include "mt_kernels.h"

namespace mt {

namespace {

double seconds_since(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
}

// Wall time of `reps` copies per active direction, both directions issued
// at once when both are active.
double timed_streams(bool h2d, bool d2h, void* dev_in, const void* host_in, void* host_out, const void* dev_out,
                     size_t bytes, int reps, hipStream_t sp, hipStream_t so) {
  MT_HIP(hipStreamSynchronize(sp));
  MT_HIP(hipStreamSynchronize(so));
  auto t0 = std::chrono::steady_clock::now();
  for (int r = 0; r < reps; ++r) {
    if (h2d) MT_HIP(hipMemcpyAsync(dev_in, host_in, bytes, hipMemcpyHostToDevice, sp));
    if (d2h) MT_HIP(hipMemcpyAsync(host_out, dev_out, bytes, hipMemcpyDeviceToHost, so));
  }
  MT_HIP(hipStreamSynchronize(sp));
  MT_HIP(hipStreamSynchronize(so));
  return seconds_since(t0);
}

double timed_sdma(DmaEngines& dma, bool h2d, bool d2h, void* dev_in, const void* host_in, void* host_out,
                  const void* dev_out, size_t bytes, int reps) {
  auto t0 = std::chrono::steady_clock::now();
  std::thread out;
  if (d2h)
    out = std::thread([&] {
      for (int r = 0; r < reps; ++r) dma.copy(DMA_D2H, host_out, dev_out, bytes);
    });
  if (h2d)
    for (int r = 0; r < reps; ++r) dma.copy(DMA_H2D, dev_in, host_in, bytes);
  if (out.joinable()) out.join();
  return seconds_since(t0);
}

}  // namespace

}  // namespace mt

using namespace mt;

extern "C" int mt_link_probe(void* dev_a, void* dev_b, void* host_a, void* host_b, size_t bytes, int32_t reps,
                             int32_t flags, void* const streams[2], double out_gbs[3]) {
  try {
    if (!dev_a || !dev_b || !host_a || !host_b || !out_gbs || bytes == 0 || reps < 1)
      throw ApiError{MT_E_INVALID, "link probe: null buffer, zero size or reps < 1"};
    const bool sdma = flags & MT_FLAG_SDMA_QUEUES;
    if (!sdma && (!streams || !streams[0] || !streams[1] || streams[0] == streams[1]))
      throw ApiError{MT_E_INVALID, "link probe: two different streams needed"};
    unsigned int hf = 0;
    if (hipHostGetFlags(&hf, host_a) != hipSuccess || hipHostGetFlags(&hf, host_b) != hipSuccess) {
      (void)hipGetLastError();
      throw ApiError{MT_E_INVALID, "link probe: host buffers must be pinned"};
    }
    const double gb = (double)bytes * reps / 1e9;
    if (sdma) {
      DmaEngines dma(dev_a, host_a);
      timed_sdma(dma, true, false, dev_a, host_a, host_b, dev_b, bytes, 1);  // warm-up
      out_gbs[0] = gb / timed_sdma(dma, true, false, dev_a, host_a, host_b, dev_b, bytes, reps);
      out_gbs[1] = gb / timed_sdma(dma, false, true, dev_a, host_a, host_b, dev_b, bytes, reps);
      out_gbs[2] = 2 * gb / timed_sdma(dma, true, true, dev_a, host_a, host_b, dev_b, bytes, reps);
    } else {
      hipStream_t sp = (hipStream_t)streams[0], so = (hipStream_t)streams[1];
      timed_streams(true, false, dev_a, host_a, host_b, dev_b, bytes, 1, sp, so);  // warm-up
      out_gbs[0] = gb / timed_streams(true, false, dev_a, host_a, host_b, dev_b, bytes, reps, sp, so);
      out_gbs[1] = gb / timed_streams(false, true, dev_a, host_a, host_b, dev_b, bytes, reps, sp, so);
      out_gbs[2] = 2 * gb / timed_streams(true, true, dev_a, host_a, host_b, dev_b, bytes, reps, sp, so);
    }
    return MT_OK;
  } catch (const ApiError& e) {
    set_error(e.msg);
    return e.code;
  } catch (const HipError& e) {
    set_error(std::string(hipGetErrorString(e.code)) + " in " + e.where);
    return MT_E_HIP;
  }
}
