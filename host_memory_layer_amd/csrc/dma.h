// Host <-> device copies on the GPU's system DMA (SDMA) engines, issued
// through the HSA runtime, and the in-order transfer queues of the streamed
// step built on them.
//
// The weight prefetch and the gradient offload must not take compute units
// from the layer that computes beside them, and must not wait behind each
// other.  The HIP runtime may carry a hipMemcpyAsync between pinned host
// memory and the device out as a copy kernel on the shader cores (while
// such a kernel wrote host memory over PCIe, kernels of the compute stream
// were measured to progress at a small fraction of their usual rate), and
// it may queue copies of different streams on one SDMA engine, where a
// prefetch that waits for its weight slot holds back the offload queued
// behind it.  Here each direction owns one SDMA engine, picked once, and
// every copy runs there.
#pragma once

#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <condition_variable>
#include <cstddef>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

namespace mt {

enum DmaDir { DMA_H2D = 0, DMA_D2H = 1 };

class DmaEngines {
 public:
  // `dev` is any device allocation of the GPU, `host` any pinned host
  // allocation: the HSA agents that own them are the two ends of every copy.
  DmaEngines(const void* dev, const void* host);
  ~DmaEngines();
  DmaEngines(const DmaEngines&) = delete;
  DmaEngines& operator=(const DmaEngines&) = delete;

  // Copies `bytes` from `src` to `dst` in direction `dir` on that
  // direction's engine and returns once the data has arrived.  A device
  // source must have been written by work that has completed and released
  // its writes to system scope (a completed hipEvent does both).  Calls for
  // the two directions may run concurrently from two threads; calls for one
  // direction must not.  Throws ApiError on failure.
  void copy(DmaDir dir, void* dst, const void* src, size_t bytes);
  uint32_t engine_id(DmaDir dir) const { return eng_[dir]; }
  // Host-to-device jobs whose ready event has fired and whose copy has not
  // finished; device-to-host copies wait for none to be left (see
  // TransferQueue).
  void h2d_begin();
  void h2d_end();
  void wait_no_h2d();

 private:
  std::mutex link_mu_;
  std::condition_variable link_cv_;
  int h2d_active_ = 0;
  hsa_agent_t gpu_{}, cpu_{};
  hsa_signal_t sig_[2]{};
  uint32_t eng_[2]{};
  bool inited_ = false;
};

// One direction's copies, run in order by a worker thread.  A job first
// waits for its `ready` event (null: no wait), sleeps delay_us, then copies,
// then calls `on_done`.  The enqueueing thread waits for a job with wait(); after a
// failure every wait() throws.
class TransferQueue {
 public:
  struct Job {
    int u, j;
    hipEvent_t ready;
    void* dst;
    const void* src;
    size_t bytes;
    int delay_us = 0;  // the worker sleeps this long before the copy
  };
  // yield_link: a device-to-host copy starts only when no host-to-device
  // copy is ready or running, so offloads take the link between prefetches
  // instead of halving their rate (the two directions share one host link:
  // both at once move about as many bytes per second as one alone).
  // Prefetches never wait for offloads.
  TransferQueue(DmaEngines* dma, DmaDir dir, bool yield_link = true)
      : dma_(dma), dir_(dir), yield_(yield_link) {}
  ~TransferQueue() { stop(); }

  // Starts the worker for one step; job_ms(u) is filled with each job's
  // copy time (host clock).
  void start(std::vector<double>* job_ms, std::function<void(const Job&)> on_done);
  int push(const Job& job);
  void wait(int idx);
  // No more jobs this step: the worker finishes the queued ones and exits.
  void stop();

 private:
  void run();
  DmaEngines* dma_;
  DmaDir dir_;
  bool yield_;
  std::mutex mu_;
  std::condition_variable cv_;
  std::vector<Job> jobs_;
  size_t done_ = 0;
  bool closed_ = false;
  std::string error_;
  std::vector<double>* job_ms_ = nullptr;
  std::function<void(const Job&)> on_done_;
  std::thread worker_;
};

}  // namespace mt
