#include "dma.h"

#include <chrono>
#include <cstdint>

#include "common.h"

namespace mt {

namespace {

std::string hsa_msg(hsa_status_t s) {
  const char* t = nullptr;
  if (hsa_status_string(s, &t) != HSA_STATUS_SUCCESS || !t) return "HSA status " + std::to_string((int)s);
  return t;
}

#define MT_HSA(call)                                                                                \
  do {                                                                                              \
    hsa_status_t s_ = (call);                                                                       \
    if (s_ != HSA_STATUS_SUCCESS) throw ApiError{MT_E_HIP, std::string(#call) + ": " + hsa_msg(s_)}; \
  } while (0)

hsa_agent_t owner_of(const void* p, const char* what) {
  hsa_amd_pointer_info_t info{};
  info.size = sizeof(info);
  MT_HSA(hsa_amd_pointer_info(p, &info, nullptr, nullptr, nullptr));
  if (info.type == HSA_EXT_POINTER_TYPE_UNKNOWN || info.agentOwner.handle == 0)
    throw ApiError{MT_E_INVALID, std::string("DMA: ") + what + " is not an HSA allocation"};
  return info.agentOwner;
}

uint32_t lowest_bit(uint32_t m) { return m & (~m + 1u); }

}  // namespace

DmaEngines::DmaEngines(const void* dev, const void* host) {
  MT_HSA(hsa_init());
  inited_ = true;
  try {
    gpu_ = owner_of(dev, "device buffer");
    cpu_ = owner_of(host, "host buffer");
    hsa_device_type_t t;
    MT_HSA(hsa_agent_get_info(gpu_, HSA_AGENT_INFO_DEVICE, &t));
    if (t != HSA_DEVICE_TYPE_GPU) throw ApiError{MT_E_INVALID, "DMA: device buffer is not GPU memory"};
    MT_HSA(hsa_agent_get_info(cpu_, HSA_AGENT_INFO_DEVICE, &t));
    if (t != HSA_DEVICE_TYPE_CPU) throw ApiError{MT_E_INVALID, "DMA: host buffer is not host memory"};
    // Engines that can serve each direction, and those the runtime
    // recommends for bandwidth; the two directions get different engines.
    uint32_t avail[2] = {0, 0}, pref[2] = {0, 0};
    MT_HSA(hsa_amd_memory_copy_engine_status(gpu_, cpu_, &avail[DMA_H2D]));
    MT_HSA(hsa_amd_memory_copy_engine_status(cpu_, gpu_, &avail[DMA_D2H]));
    if (hsa_amd_memory_get_preferred_copy_engine(gpu_, cpu_, &pref[DMA_H2D]) != HSA_STATUS_SUCCESS) pref[DMA_H2D] = 0;
    if (hsa_amd_memory_get_preferred_copy_engine(cpu_, gpu_, &pref[DMA_D2H]) != HSA_STATUS_SUCCESS) pref[DMA_D2H] = 0;
    if (!avail[DMA_H2D] || !avail[DMA_D2H]) throw ApiError{MT_E_HIP, "DMA: no SDMA engine available"};
    eng_[DMA_H2D] = lowest_bit((avail[DMA_H2D] & pref[DMA_H2D]) ? (avail[DMA_H2D] & pref[DMA_H2D]) : avail[DMA_H2D]);
    const uint32_t rest = avail[DMA_D2H] & ~eng_[DMA_H2D];
    const uint32_t rest_pref = rest & pref[DMA_D2H];
    eng_[DMA_D2H] = lowest_bit(rest_pref ? rest_pref : (rest ? rest : avail[DMA_D2H]));
    MT_HSA(hsa_signal_create(1, 0, nullptr, &sig_[0]));
    MT_HSA(hsa_signal_create(1, 0, nullptr, &sig_[1]));
  } catch (...) {
    for (auto& s : sig_)
      if (s.handle) hsa_signal_destroy(s);
    hsa_shut_down();
    inited_ = false;
    throw;
  }
}

DmaEngines::~DmaEngines() {
  for (auto& s : sig_)
    if (s.handle) hsa_signal_destroy(s);
  if (inited_) hsa_shut_down();
}

void DmaEngines::copy(DmaDir dir, void* dst, const void* src, size_t bytes) {
  if (bytes == 0) return;
  hsa_signal_t sig = sig_[dir];
  hsa_signal_store_screlease(sig, 1);
  const hsa_agent_t dst_agent = dir == DMA_H2D ? gpu_ : cpu_;
  const hsa_agent_t src_agent = dir == DMA_H2D ? cpu_ : gpu_;
  MT_HSA(hsa_amd_memory_async_copy_on_engine(dst, dst_agent, src, src_agent, bytes, 0, nullptr, sig,
                                             (hsa_amd_sdma_engine_id_t)eng_[dir], true));
  // The runtime decrements the signal to 0 on completion and sets it
  // negative on a failed copy.
  const hsa_signal_value_t v =
      hsa_signal_wait_scacquire(sig, HSA_SIGNAL_CONDITION_LT, 1, UINT64_MAX, HSA_WAIT_STATE_BLOCKED);
  if (v != 0)
    throw ApiError{MT_E_HIP, std::string("DMA copy ") + (dir == DMA_H2D ? "host->device" : "device->host") +
                                 " failed (completion signal " + std::to_string(v) + ")"};
}

void DmaEngines::h2d_begin() {
  std::lock_guard<std::mutex> g(link_mu_);
  ++h2d_active_;
}

void DmaEngines::h2d_end() {
  {
    std::lock_guard<std::mutex> g(link_mu_);
    --h2d_active_;
  }
  link_cv_.notify_all();
}

void DmaEngines::wait_no_h2d() {
  std::unique_lock<std::mutex> lk(link_mu_);
  link_cv_.wait(lk, [&] { return h2d_active_ == 0; });
}

// ----------------------------------------------------------- queue --
void TransferQueue::start(std::vector<double>* job_ms, std::function<void(const Job&)> on_done) {
  stop();
  std::lock_guard<std::mutex> g(mu_);
  jobs_.clear();
  done_ = 0;
  closed_ = false;
  error_.clear();
  job_ms_ = job_ms;
  on_done_ = std::move(on_done);
  worker_ = std::thread([this] { run(); });
}

int TransferQueue::push(const Job& job) {
  int idx;
  {
    std::lock_guard<std::mutex> g(mu_);
    if (!error_.empty()) throw ApiError{MT_E_HIP, "transfer: " + error_};
    idx = (int)jobs_.size();
    jobs_.push_back(job);
  }
  cv_.notify_all();
  return idx;
}

void TransferQueue::wait(int idx) {
  std::unique_lock<std::mutex> lk(mu_);
  cv_.wait(lk, [&] { return done_ > (size_t)idx || !error_.empty(); });
  if (!error_.empty()) throw ApiError{MT_E_HIP, "transfer: " + error_};
}

void TransferQueue::stop() {
  {
    std::lock_guard<std::mutex> g(mu_);
    closed_ = true;
  }
  cv_.notify_all();
  if (worker_.joinable()) worker_.join();
}

void TransferQueue::run() {
  size_t next = 0;
  for (;;) {
    Job job;
    {
      std::unique_lock<std::mutex> lk(mu_);
      cv_.wait(lk, [&] { return next < jobs_.size() || closed_; });
      if (next >= jobs_.size()) return;
      job = jobs_[next];
    }
    std::string err;
    try {
      if (job.ready) MT_HIP(hipEventSynchronize(job.ready));
      if (job.delay_us > 0) std::this_thread::sleep_for(std::chrono::microseconds(job.delay_us));
      const bool h2d = dir_ == DMA_H2D;
      if (yield_) {
        if (h2d)
          dma_->h2d_begin();
        else
          dma_->wait_no_h2d();
      }
      auto t0 = std::chrono::steady_clock::now();
      try {
        dma_->copy(dir_, job.dst, job.src, job.bytes);
      } catch (...) {
        if (yield_ && h2d) dma_->h2d_end();
        throw;
      }
      if (job_ms_ && job.u >= 0 && (size_t)job.u < job_ms_->size())
        (*job_ms_)[job.u] = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
      if (yield_ && h2d) dma_->h2d_end();
      // Before the job counts as done: the enqueueing thread may close
      // what on_done feeds once the last job is done.
      if (on_done_) on_done_(job);
    } catch (const HipError& e) {
      err = std::string(hipGetErrorString(e.code)) + " in " + e.where;
    } catch (const ApiError& e) {
      err = e.msg;
    } catch (const std::exception& e) {
      err = e.what();
    }
    {
      std::lock_guard<std::mutex> g(mu_);
      if (!err.empty()) error_ = err;
      else done_ = ++next;
    }
    cv_.notify_all();
    if (!err.empty()) return;
  }
}

}  // namespace mt
