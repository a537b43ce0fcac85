// extern "C" entry points of include/mt.h: argument checks and translation
// of internal errors into MT_E_* codes; no exception crosses the ABI.
#include <cstdio>
#include <cstring>
#include <sched.h>
#include <sys/mman.h>

#include <algorithm>
#include <new>

#include "adam.h"
#include "engine.h"
#include "store.h"

namespace mt {

static thread_local std::string g_last_error;
void set_error(const std::string& msg) { g_last_error = msg; }
const char* last_error() { return g_last_error.c_str(); }

template <typename F>
static int guarded(F&& f) {
  try {
    return f();
  } catch (const ApiError& e) {
    set_error(e.msg);
    return e.code;
  } catch (const HipError& e) {
    set_error(std::string(hipGetErrorString(e.code)) + " in " + e.where);
    return MT_E_HIP;
  } catch (const std::bad_alloc&) {
    set_error("host allocation failed");
    return MT_E_OOM;
  } catch (const std::exception& e) {
    set_error(e.what());
    return MT_E_INVALID;
  }
}

}  // namespace mt

using namespace mt;

// The opaque handle of the C ABI is the engine's model object.
static Model* M_(mt_model* h) { return reinterpret_cast<Model*>(h); }
static const Model* M_(const mt_model* h) { return reinterpret_cast<const Model*>(h); }

extern "C" {

int mt_host_store_layout(const mt_config* cfg, mt_layout* out, mt_block_desc* blocks, int32_t capacity) {
  return guarded([&] {
    std::string why;
    if (!cfg || !out) throw ApiError{MT_E_INVALID, "null argument"};
    if (validate_config(*cfg, &why) != MT_OK) throw ApiError{MT_E_INVALID, why};
    uint64_t dma = 0, opt = 0;
    std::vector<mt_block_desc> b = store_layout(*cfg, &dma, &opt);
    *out = mt_layout{dma, opt, (int32_t)b.size(), 0};
    if (blocks)
      for (int32_t i = 0; i < std::min<int32_t>(capacity, (int32_t)b.size()); ++i) blocks[i] = b[i];
    return MT_OK;
  });
}

size_t mt_host_store_bytes(const mt_config* cfg) {
  std::string why;
  if (!cfg || validate_config(*cfg, &why) != MT_OK) {
    set_error(cfg ? why : "null config");
    return 0;
  }
  uint64_t total = 0;
  store_layout(*cfg, &total);
  return total;
}

size_t mt_host_opt_bytes(const mt_config* cfg) {
  std::string why;
  if (!cfg || validate_config(*cfg, &why) != MT_OK) {
    set_error(cfg ? why : "null config");
    return 0;
  }
  uint64_t total = 0, opt = 0;
  store_layout(*cfg, &total, &opt);
  return opt;
}

int mt_block_count(const mt_config* cfg) {
  std::string why;
  if (!cfg || validate_config(*cfg, &why) != MT_OK) {
    set_error(cfg ? why : "null config");
    return MT_E_INVALID;
  }
  return cfg->n_layers + 2;
}

int mt_block_info(const mt_config* cfg, int block, mt_block_desc* out) {
  return guarded([&] {
    std::string why;
    if (!cfg || !out) throw ApiError{MT_E_INVALID, "null argument"};
    if (validate_config(*cfg, &why) != MT_OK) throw ApiError{MT_E_INVALID, why};
    if (block < 0 || block >= cfg->n_layers + 2) throw ApiError{MT_E_INVALID, "block index"};
    uint64_t total = 0;
    *out = store_layout(*cfg, &total)[block];
    return MT_OK;
  });
}

size_t mt_device_bytes(const mt_config* cfg) {
  size_t r = 0;
  int rc = guarded([&] {
    if (!cfg) throw ApiError{MT_E_INVALID, "null config"};
    r = device_bytes_for(*cfg);
    return MT_OK;
  });
  return rc == MT_OK ? r : 0;
}

int mt_schedule(const mt_config* cfg, mt_sched_op* ops, int32_t capacity) {
  int32_t n = 0;
  int rc = guarded([&] {
    if (!cfg) throw ApiError{MT_E_INVALID, "null config"};
    if (capacity < 0 || (capacity > 0 && !ops)) throw ApiError{MT_E_INVALID, "null ops or negative capacity"};
    std::vector<mt_sched_op> v = schedule_for(*cfg);
    for (size_t i = 0; i < v.size() && (int64_t)i < capacity; ++i) ops[i] = v[i];
    n = (int32_t)v.size();
    return MT_OK;
  });
  return rc == MT_OK ? n : rc;
}

int mt_alloc_host_store(size_t bytes, void** out) {
  return guarded([&] {
    if (!out || bytes == 0) throw ApiError{MT_E_INVALID, "null out or zero size"};
    void* p = nullptr;
    const size_t n = round_up(bytes, kStoreAlign);
    hipError_t e = hipHostMalloc(&p, n, hipHostMallocDefault);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      throw ApiError{MT_E_OOM, std::string("hipHostMalloc: ") + hipGetErrorString(e)};
    }
    if ((uintptr_t)p % kStoreAlign) {
      (void)hipHostFree(p);
      throw ApiError{MT_E_ALIGN, "pinned allocation not 4 KiB aligned"};
    }
    *out = p;
    return MT_OK;
  });
}

void mt_free_host_store(void* p) {
  if (p) (void)hipHostFree(p);  // nothing to report from a void free
}

int mt_alloc_host_opt(size_t bytes, void** out) {
  return guarded([&] {
    if (!out || bytes == 0) throw ApiError{MT_E_INVALID, "null out or zero size"};
    const size_t n = round_up(bytes, kStoreAlign);
    void* p = mmap(nullptr, n, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
    if (p == MAP_FAILED) throw ApiError{MT_E_OOM, "mmap of the optimizer part failed"};
    madvise(p, n, MADV_HUGEPAGE);
    *out = p;
    return MT_OK;
  });
}

void mt_free_host_opt(void* p, size_t bytes) {
  if (p) munmap(p, round_up(bytes, kStoreAlign));
}

int mt_init_store_header(const mt_config* cfg, void* host_base, size_t bytes, void* opt_base, size_t opt_bytes) {
  return guarded([&] {
    std::string why;
    if (!cfg || !host_base || !opt_base) throw ApiError{MT_E_INVALID, "null argument"};
    if (validate_config(*cfg, &why) != MT_OK) throw ApiError{MT_E_INVALID, why};
    if ((uintptr_t)host_base % kStoreAlign || (uintptr_t)opt_base % kStoreAlign)
      throw ApiError{MT_E_ALIGN, "store parts not 4 KiB aligned"};
    uint64_t total = 0, opt = 0;
    store_layout(*cfg, &total, &opt);
    if (bytes < total) throw ApiError{MT_E_SIZE, "DMA part smaller than mt_host_store_bytes"};
    if (opt_bytes < opt) throw ApiError{MT_E_SIZE, "optimizer part smaller than mt_host_opt_bytes"};
    StoreHeader h{};
    h.magic = kStoreMagic;
    h.version = kStoreVersion;
    h.n_blocks = cfg->n_layers + 2;
    h.cfg = *cfg;
    h.step = 0;
    h.total_bytes = total;
    memset(host_base, 0, kHeaderBytes);
    memcpy(host_base, &h, sizeof(h));
    int threads = cfg->host_threads;
    if (threads <= 0) {
      cpu_set_t set;
      threads = sched_getaffinity(0, sizeof(set), &set) == 0 ? CPU_COUNT(&set) : 1;
    }
    ThreadPool pool(std::max(1, threads));
    const uint64_t chunk = 64ull << 20;
    const uint64_t body = total - kHeaderBytes;
    const int64_t n1 = (int64_t)((body + chunk - 1) / chunk), n2 = (int64_t)((opt + chunk - 1) / chunk);
    pool.run(n1 + n2, [&](int64_t i) {
      if (i < n1) {
        const uint64_t lo = kHeaderBytes + (uint64_t)i * chunk;
        memset((uint8_t*)host_base + lo, 0, std::min(chunk, total - lo));
      } else {
        const uint64_t lo = (uint64_t)(i - n1) * chunk;
        memset((uint8_t*)opt_base + lo, 0, std::min(chunk, opt - lo));
      }
    });
    return MT_OK;
  });
}

int mt_store_step(const void* host_base, int64_t* t) {
  return guarded([&] {
    if (!host_base || !t) throw ApiError{MT_E_INVALID, "null argument"};
    const StoreHeader* h = (const StoreHeader*)host_base;
    if (h->magic != kStoreMagic) throw ApiError{MT_E_INVALID, "bad store magic"};
    *t = h->step;
    return MT_OK;
  });
}

// Checkpoint file: an 8-byte tag, the store's header page, every block's W
// region in block order, then the optimizer part [m | v].  Gradients are
// overwritten by every step and are not part of the state.
static const char kCkptTag[8] = {'M', 'T', 'C', 'K', 'P', 'T', '0', '1'};

static const StoreHeader* checked_header(const void* dma_base, size_t dma_bytes, size_t opt_bytes,
                                         std::vector<mt_block_desc>* blocks, uint64_t* opt_total) {
  if (!dma_base) throw ApiError{MT_E_INVALID, "null argument"};
  const StoreHeader* h = (const StoreHeader*)dma_base;
  if (h->magic != kStoreMagic || h->version != kStoreVersion) throw ApiError{MT_E_INVALID, "bad store header"};
  uint64_t total = 0;
  *blocks = store_layout(h->cfg, &total, opt_total);
  if (dma_bytes < total || opt_bytes < *opt_total) throw ApiError{MT_E_SIZE, "store parts smaller than the layout"};
  return h;
}

static bool same_layout(const mt_config& a, const mt_config& b) {
  return a.n_layers == b.n_layers && a.d_model == b.d_model && a.n_heads == b.n_heads &&
         a.head_dim == b.head_dim && a.d_ff == b.d_ff && a.vocab == b.vocab && a.store_dtype == b.store_dtype &&
         (micro_count(a) > 1) == (micro_count(b) > 1);
}

int mt_store_init_master(const void* dma_base, size_t dma_bytes, void* opt_base, size_t opt_bytes) {
  return guarded([&] {
    if (!opt_base) throw ApiError{MT_E_INVALID, "null argument"};
    std::vector<mt_block_desc> blocks;
    uint64_t opt = 0;
    const StoreHeader* h = checked_header(dma_base, dma_bytes, opt_bytes, &blocks, &opt);
    if (!master_store(h->cfg)) throw ApiError{MT_E_STATE, "store has no fp32 master copy"};
    int threads = h->cfg.host_threads;
    if (threads <= 0) {
      cpu_set_t set;
      threads = sched_getaffinity(0, sizeof(set), &set) == 0 ? CPU_COUNT(&set) : 1;
    }
    ThreadPool pool(std::max(1, threads));
    const uint64_t chunk = 1ull << 22;
    for (const auto& b : blocks) {
      const uint16_t* w = (const uint16_t*)((const uint8_t*)dma_base + b.w_off);
      uint32_t* p = (uint32_t*)((uint8_t*)opt_base + b.p_off);
      const uint64_t n = b.region_elems;
      pool.run((int64_t)((n + chunk - 1) / chunk), [&](int64_t i) {
        const uint64_t lo = (uint64_t)i * chunk, hi = std::min(n, lo + chunk);
        for (uint64_t e = lo; e < hi; ++e) p[e] = (uint32_t)w[e] << 16;  // bf16 -> fp32 is exact
      });
    }
    return MT_OK;
  });
}

int mt_store_save(const void* dma_base, size_t dma_bytes, const void* opt_base, size_t opt_bytes, const char* path) {
  return guarded([&] {
    if (!opt_base || !path) throw ApiError{MT_E_INVALID, "null argument"};
    std::vector<mt_block_desc> blocks;
    uint64_t opt = 0;
    checked_header(dma_base, dma_bytes, opt_bytes, &blocks, &opt);
    FILE* f = fopen(path, "wb");
    if (!f) throw ApiError{MT_E_INVALID, std::string("cannot open ") + path};
    bool ok = fwrite(kCkptTag, 1, 8, f) == 8 && fwrite(dma_base, 1, kHeaderBytes, f) == kHeaderBytes;
    for (const auto& b : blocks)
      ok = ok && fwrite((const uint8_t*)dma_base + b.w_off, 1, b.w_bytes, f) == b.w_bytes;
    ok = ok && fwrite(opt_base, 1, opt, f) == opt;
    ok = (fclose(f) == 0) && ok;
    if (!ok) throw ApiError{MT_E_INVALID, std::string("short write to ") + path};
    return MT_OK;
  });
}

int mt_store_load(void* dma_base, size_t dma_bytes, void* opt_base, size_t opt_bytes, const char* path) {
  return guarded([&] {
    if (!opt_base || !path) throw ApiError{MT_E_INVALID, "null argument"};
    std::vector<mt_block_desc> blocks;
    uint64_t opt = 0;
    StoreHeader* h = (StoreHeader*)checked_header(dma_base, dma_bytes, opt_bytes, &blocks, &opt);
    FILE* f = fopen(path, "rb");
    if (!f) throw ApiError{MT_E_INVALID, std::string("cannot open ") + path};
    char tag[8];
    std::vector<uint8_t> page(kHeaderBytes);
    bool ok = fread(tag, 1, 8, f) == 8 && memcmp(tag, kCkptTag, 8) == 0 &&
              fread(page.data(), 1, kHeaderBytes, f) == kHeaderBytes;
    const StoreHeader* fh = (const StoreHeader*)page.data();
    if (!ok || fh->magic != kStoreMagic || fh->version != kStoreVersion || !same_layout(fh->cfg, h->cfg)) {
      fclose(f);
      throw ApiError{MT_E_INVALID, "checkpoint does not match the store's configuration"};
    }
    for (const auto& b : blocks) ok = ok && fread((uint8_t*)dma_base + b.w_off, 1, b.w_bytes, f) == b.w_bytes;
    ok = ok && fread(opt_base, 1, opt, f) == opt;
    fclose(f);
    if (!ok) throw ApiError{MT_E_INVALID, std::string("short checkpoint ") + path};
    h->step = fh->step;
    return MT_OK;
  });
}

int mt_create_model(const mt_config* cfg, void* dev_arena, size_t arena_bytes, void* const streams[3],
                    mt_model** out) {
  return guarded([&] {
    if (!cfg || !out) throw ApiError{MT_E_INVALID, "null argument"};
    *out = reinterpret_cast<mt_model*>(create_model(cfg, dev_arena, arena_bytes, streams));
    return MT_OK;
  });
}

int mt_bind_host_store(mt_model* model, void* host_base, size_t bytes, void* opt_base, size_t opt_bytes) {
  return guarded([&] {
    if (!model) throw ApiError{MT_E_INVALID, "null model"};
    return bind_store(M_(model), host_base, bytes, opt_base, opt_bytes);
  });
}

int mt_train_step(mt_model* model, const int32_t* tokens) {
  return guarded([&] {
    if (!model) throw ApiError{MT_E_INVALID, "null model"};
    return model_step(M_(model), tokens);
  });
}

int mt_get_loss(const mt_model* model, float* out) {
  return guarded([&] {
    if (!model || !out) throw ApiError{MT_E_INVALID, "null argument"};
    return model_loss(M_(model), out);
  });
}

int mt_get_stats(const mt_model* model, mt_stats* out) {
  return guarded([&] {
    if (!model || !out) throw ApiError{MT_E_INVALID, "null argument"};
    return model_stats(M_(model), out);
  });
}

int mt_get_kernel_times(const mt_model* model, mt_kernel_time* out, int32_t capacity) {
  return guarded([&] {
    if (!model) throw ApiError{MT_E_INVALID, "null model"};
    return model_kernel_times(M_(model), out, capacity);
  });
}

int mt_get_block_stats(const mt_model* model, int block, mt_block_stats* out) {
  return guarded([&] {
    if (!model || !out) throw ApiError{MT_E_INVALID, "null argument"};
    return model_block_stats(M_(model), block, out);
  });
}

int mt_debug_buffers(const mt_model* model, int layer, void** ckpt, void** row_loss) {
  return guarded([&] {
    if (!model) throw ApiError{MT_E_INVALID, "null model"};
    return model_debug(M_(model), layer, ckpt, row_loss);
  });
}

int mt_debug_grad(const mt_model* model, int layer, void** dx) {
  return guarded([&] {
    if (!model || !dx) throw ApiError{MT_E_INVALID, "null argument"};
    return model_debug_grad(M_(model), layer, dx);
  });
}

void mt_destroy_model(mt_model* model) { destroy_model(M_(model)); }

int mt_host_adam(int32_t store_dtype, void* w, const void* g, float* m, float* v, size_t n, int64_t t, double lr,
                 double beta1, double beta2, double eps, int32_t threads) {
  return guarded([&] {
    if ((!w || !g || !m || !v) && n) throw ApiError{MT_E_INVALID, "null buffer"};
    if (store_dtype != MT_F32 && store_dtype != MT_BF16) throw ApiError{MT_E_INVALID, "store_dtype"};
    if (t < 1) throw ApiError{MT_E_INVALID, "step t must be >= 1"};
    const AdamConsts k = adam_consts(t, lr, beta1, beta2, eps);
    ThreadPool pool(threads > 0 ? threads : 1);
    adam_parallel(pool, store_dtype, w, g, m, v, n, k);
    return MT_OK;
  });
}

int mt_host_adam_master(uint16_t* w, float* p, const uint16_t* g, float* m, float* v, size_t n, int64_t t, double lr,
                        double beta1, double beta2, double eps, int32_t threads) {
  return guarded([&] {
    if ((!w || !p || !g || !m || !v) && n) throw ApiError{MT_E_INVALID, "null buffer"};
    if (t < 1) throw ApiError{MT_E_INVALID, "step t must be >= 1"};
    const AdamConsts k = adam_consts(t, lr, beta1, beta2, eps);
    ThreadPool pool(threads > 0 ? threads : 1);
    adam_master_parallel(pool, w, p, g, m, v, n, k);
    return MT_OK;
  });
}

const char* mt_last_error(void) { return last_error(); }
const char* mt_version(void) { return "megatrain-mi355x 0.1 (gfx950)"; }

}  // extern "C"
