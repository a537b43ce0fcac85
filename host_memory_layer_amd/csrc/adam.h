// Host Adam (see adam.cpp).
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <cstring>

#include "mt.h"
#include "threadpool.h"

namespace mt {

struct AdamConsts {
  float b1, omb1, b2, omb2, c1, c2, lr, eps;
};

AdamConsts adam_consts(int64_t t, double lr, double b1, double b2, double eps);
void adam_range(int32_t dtype, void* w, const void* g, float* m, float* v, size_t n, const AdamConsts& k);
void adam_parallel(ThreadPool& pool, int32_t dtype, void* w, const void* g, float* m, float* v, size_t n,
                   const AdamConsts& k);
// fp32 master update: p' from p and the widened bf16 g; w = bf16 RNE of p'.
void adam_master_range(uint16_t* w, float* p, const uint16_t* g, float* m, float* v, size_t n, const AdamConsts& k);
void adam_master_parallel(ThreadPool& pool, uint16_t* w, float* p, const uint16_t* g, float* m, float* v, size_t n,
                          const AdamConsts& k);

// Gradient accumulation over micro-batches, gradients g in the store dtype:
// acc = widen(g) on the first micro-batch, acc = acc + widen(g) after it.
void grad_accumulate_parallel(ThreadPool& pool, int32_t store_dtype, float* acc, const void* g, size_t n, bool first);
// The last micro-batch: acc = acc + widen(g), then the Adam update of the
// store's weights (w, and the fp32 master p of an MT_BF16_MASTER store) with
// acc as the gradient.
void adam_accumulated_parallel(ThreadPool& pool, int32_t store_dtype, void* w, float* p, float* acc, const void* g,
                               float* m, float* v, size_t n, const AdamConsts& k);

}  // namespace mt
