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

}  // namespace mt
