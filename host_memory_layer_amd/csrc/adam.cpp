// Host Adam over a contiguous range of a store block.
//
// The pages put the optimizer step on the host CPU with AVX-512 (MegaTrain,
// radar.chestersoft.de "Methodik"), reading the layer's bf16 weights and
// gradients and fp32 moments from its contiguous block.  Per element, in
// float32 with this exact operation order (no fused multiply-add, so an
// all-fp32 store reproduces a plain float32 evaluation bit for bit):
//   m' = b1*m + (1-b1)*g
//   v' = b2*v + ((1-b2)*g)*g
//   w' = w - (lr * (m'/c1)) / (sqrt(v'/c2) + eps),  c1 = 1-b1^t, c2 = 1-b2^t
// with w, g widened from bf16 and w' rounded to nearest-even bf16.  With an
// fp32 master copy P of the weights (MT_BF16_MASTER) the update runs on P
// instead of the widened w, P keeps the fp32 result, and w receives its
// bf16 rounding.
// With micro-batches the gradient is first summed in an fp32 accumulator
// (acc + widen(g), one micro-batch after the other) and the update uses it.
// This file is compiled with -ffp-contract=off.
#include <immintrin.h>

#include <cmath>

#include "adam.h"

namespace mt {

static inline float widen1(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static inline uint16_t round1(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

AdamConsts adam_consts(int64_t t, double lr, double b1, double b2, double eps) {
  AdamConsts k;
  k.b1 = (float)b1;
  k.omb1 = (float)(1.0 - b1);
  k.b2 = (float)b2;
  k.omb2 = (float)(1.0 - b2);
  k.c1 = (float)(1.0 - std::pow(b1, (double)t));
  k.c2 = (float)(1.0 - std::pow(b2, (double)t));
  k.lr = (float)lr;
  k.eps = (float)eps;
  return k;
}

static inline float adam_one(float w, float g, float* m, float* v, const AdamConsts& k) {
  float m2 = k.b1 * *m + k.omb1 * g;
  float v2 = k.b2 * *v + (k.omb2 * g) * g;
  *m = m2;
  *v = v2;
  float mh = m2 / k.c1;
  float vh = v2 / k.c2;
  return w - (k.lr * mh) / (std::sqrt(vh) + k.eps);
}

static void adam_scalar_f32(float* w, const float* g, float* m, float* v, size_t n, const AdamConsts& k) {
  for (size_t i = 0; i < n; ++i) w[i] = adam_one(w[i], g[i], m + i, v + i, k);
}

static void adam_scalar_bf16(uint16_t* w, const uint16_t* g, float* m, float* v, size_t n,
                             const AdamConsts& k) {
  for (size_t i = 0; i < n; ++i)
    w[i] = round1(adam_one(widen1(w[i]), widen1(g[i]), m + i, v + i, k));
}

__attribute__((target("avx512f"))) static inline __m512 adam16(__m512 w, __m512 g, float* m, float* v,
                                                                const AdamConsts& k) {
  const __m512 b1 = _mm512_set1_ps(k.b1), omb1 = _mm512_set1_ps(k.omb1);
  const __m512 b2 = _mm512_set1_ps(k.b2), omb2 = _mm512_set1_ps(k.omb2);
  const __m512 c1 = _mm512_set1_ps(k.c1), c2 = _mm512_set1_ps(k.c2);
  const __m512 lr = _mm512_set1_ps(k.lr), eps = _mm512_set1_ps(k.eps);
  __m512 m0 = _mm512_loadu_ps(m), v0 = _mm512_loadu_ps(v);
  __m512 m2 = _mm512_add_ps(_mm512_mul_ps(b1, m0), _mm512_mul_ps(omb1, g));
  __m512 v2 = _mm512_add_ps(_mm512_mul_ps(b2, v0), _mm512_mul_ps(_mm512_mul_ps(omb2, g), g));
  _mm512_storeu_ps(m, m2);
  _mm512_storeu_ps(v, v2);
  __m512 mh = _mm512_div_ps(m2, c1);
  __m512 vh = _mm512_div_ps(v2, c2);
  __m512 den = _mm512_add_ps(_mm512_sqrt_ps(vh), eps);
  return _mm512_sub_ps(w, _mm512_div_ps(_mm512_mul_ps(lr, mh), den));
}

__attribute__((target("avx512f"))) static void adam_avx512_f32(float* w, const float* g, float* m, float* v,
                                                                size_t n, const AdamConsts& k) {
  size_t i = 0;
  for (; i + 16 <= n; i += 16) {
    __m512 r = adam16(_mm512_loadu_ps(w + i), _mm512_loadu_ps(g + i), m + i, v + i, k);
    _mm512_storeu_ps(w + i, r);
  }
  adam_scalar_f32(w + i, g + i, m + i, v + i, n - i, k);
}

// bf16 -> f32 widening is a 16-bit left shift of the bit pattern.
__attribute__((target("avx512f,avx512bw"))) static inline __m512 widen(const uint16_t* p) {
  __m256i h = _mm256_loadu_si256((const __m256i*)p);
  return _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(h), 16));
}

// f32 -> bf16 round to nearest even on the bit pattern, as round1 does: add
// 0x7FFF plus the lowest kept bit, keep the high half; NaN stays a quiet NaN.
// Subnormal results keep their bits (the hardware conversion instruction
// flushes them to zero, which would make the result depend on where a
// vector chunk starts).
__attribute__((target("avx512f,avx512bw"))) static inline void store_bf16x16(uint16_t* out, __m512 r) {
  const __m512i u = _mm512_castps_si512(r);
  const __m512i hi = _mm512_srli_epi32(u, 16);
  const __m512i lsb = _mm512_and_si512(hi, _mm512_set1_epi32(1));
  __m512i rn = _mm512_srli_epi32(_mm512_add_epi32(u, _mm512_add_epi32(lsb, _mm512_set1_epi32(0x7FFF))), 16);
  const __mmask16 nan =
      _mm512_cmpgt_epu32_mask(_mm512_and_si512(u, _mm512_set1_epi32(0x7FFFFFFF)), _mm512_set1_epi32(0x7F800000));
  rn = _mm512_mask_mov_epi32(rn, nan, _mm512_or_si512(hi, _mm512_set1_epi32(0x40)));
  _mm256_storeu_si256((__m256i*)out, _mm512_cvtepi32_epi16(rn));
}

__attribute__((target("avx512f,avx512bw"))) static void adam_avx512_bf16(
    uint16_t* w, const uint16_t* g, float* m, float* v, size_t n, const AdamConsts& k) {
  size_t i = 0;
  for (; i + 16 <= n; i += 16) {
    __m512 r = adam16(widen(w + i), widen(g + i), m + i, v + i, k);
    store_bf16x16(w + i, r);
  }
  adam_scalar_bf16(w + i, g + i, m + i, v + i, n - i, k);
}

static void adam_scalar_master(uint16_t* w, float* p, const uint16_t* g, float* m, float* v, size_t n,
                               const AdamConsts& k) {
  for (size_t i = 0; i < n; ++i) {
    p[i] = adam_one(p[i], widen1(g[i]), m + i, v + i, k);
    w[i] = round1(p[i]);
  }
}

__attribute__((target("avx512f,avx512bw"))) static void adam_avx512_master(
    uint16_t* w, float* p, const uint16_t* g, float* m, float* v, size_t n, const AdamConsts& k) {
  size_t i = 0;
  for (; i + 16 <= n; i += 16) {
    __m512 r = adam16(_mm512_loadu_ps(p + i), widen(g + i), m + i, v + i, k);
    _mm512_storeu_ps(p + i, r);
    store_bf16x16(w + i, r);
  }
  adam_scalar_master(w + i, p + i, g + i, m + i, v + i, n - i, k);
}

static bool cpu_has_avx512() {
  static int has = -1;
  if (has < 0) {
    __builtin_cpu_init();
    has = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw");
  }
  return has == 1;
}

void adam_range(int32_t dtype, void* w, const void* g, float* m, float* v, size_t n, const AdamConsts& k) {
  if (dtype == MT_BF16) {
    if (cpu_has_avx512())
      adam_avx512_bf16((uint16_t*)w, (const uint16_t*)g, m, v, n, k);
    else
      adam_scalar_bf16((uint16_t*)w, (const uint16_t*)g, m, v, n, k);
  } else {
    if (cpu_has_avx512())
      adam_avx512_f32((float*)w, (const float*)g, m, v, n, k);
    else
      adam_scalar_f32((float*)w, (const float*)g, m, v, n, k);
  }
}

void adam_parallel(ThreadPool& pool, int32_t dtype, void* w, const void* g, float* m, float* v, size_t n,
                   const AdamConsts& k) {
  const size_t chunk = size_t(1) << 18;  // 256 Ki elements: 5.5 MiB of traffic
  const size_t wb = dtype == MT_BF16 ? 2 : 4;
  int64_t tasks = (int64_t)((n + chunk - 1) / chunk);
  pool.run(tasks, [&](int64_t i) {
    size_t lo = (size_t)i * chunk, cnt = std::min(chunk, n - lo);
    adam_range(dtype, (char*)w + lo * wb, (const char*)g + lo * wb, m + lo, v + lo, cnt, k);
  });
}

// ---------------------------------------------------- accumulation --
static inline float gval(int32_t dtype, const void* g, size_t i) {
  return dtype == MT_F32 ? ((const float*)g)[i] : widen1(((const uint16_t*)g)[i]);
}

static void accumulate_scalar(int32_t dtype, float* acc, const void* g, size_t n, bool first) {
  for (size_t i = 0; i < n; ++i) acc[i] = first ? gval(dtype, g, i) : acc[i] + gval(dtype, g, i);
}

__attribute__((target("avx512f,avx512bw"))) static inline __m512 gvec(int32_t dtype, const void* g, size_t i) {
  return dtype == MT_F32 ? _mm512_loadu_ps((const float*)g + i) : widen((const uint16_t*)g + i);
}

__attribute__((target("avx512f,avx512bw"))) static void accumulate_avx512(int32_t dtype, float* acc, const void* g,
                                                                           size_t n, bool first) {
  size_t i = 0;
  for (; i + 16 <= n; i += 16) {
    __m512 x = gvec(dtype, g, i);
    _mm512_storeu_ps(acc + i, first ? x : _mm512_add_ps(_mm512_loadu_ps(acc + i), x));
  }
  accumulate_scalar(dtype, acc + i, (const char*)g + i * (dtype == MT_F32 ? 4 : 2), n - i, first);
}

static void adam_acc_scalar(int32_t dtype, void* w, float* p, float* acc, const void* g, float* m, float* v, size_t n,
                            const AdamConsts& k) {
  for (size_t i = 0; i < n; ++i) {
    const float gi = acc[i] + gval(dtype, g, i);
    acc[i] = gi;
    if (dtype == MT_F32) {
      ((float*)w)[i] = adam_one(((float*)w)[i], gi, m + i, v + i, k);
    } else if (dtype == MT_BF16) {
      ((uint16_t*)w)[i] = round1(adam_one(widen1(((uint16_t*)w)[i]), gi, m + i, v + i, k));
    } else {
      p[i] = adam_one(p[i], gi, m + i, v + i, k);
      ((uint16_t*)w)[i] = round1(p[i]);
    }
  }
}

__attribute__((target("avx512f,avx512bw"))) static void adam_acc_avx512(
    int32_t dtype, void* w, float* p, float* acc, const void* g, float* m, float* v, size_t n, const AdamConsts& k) {
  size_t i = 0;
  for (; i + 16 <= n; i += 16) {
    const __m512 gi = _mm512_add_ps(_mm512_loadu_ps(acc + i), gvec(dtype, g, i));
    _mm512_storeu_ps(acc + i, gi);
    if (dtype == MT_F32) {
      float* wf = (float*)w + i;
      _mm512_storeu_ps(wf, adam16(_mm512_loadu_ps(wf), gi, m + i, v + i, k));
    } else {
      uint16_t* wb = (uint16_t*)w + i;
      __m512 r;
      if (dtype == MT_BF16) {
        r = adam16(widen(wb), gi, m + i, v + i, k);
      } else {
        r = adam16(_mm512_loadu_ps(p + i), gi, m + i, v + i, k);
        _mm512_storeu_ps(p + i, r);
      }
      store_bf16x16(wb, r);
    }
  }
  const size_t wb = dtype == MT_F32 ? 4 : 2;
  adam_acc_scalar(dtype, (char*)w + i * wb, p ? p + i : nullptr, acc + i, (const char*)g + i * wb, m + i, v + i, n - i,
                  k);
}

void grad_accumulate_parallel(ThreadPool& pool, int32_t dtype, float* acc, const void* g, size_t n, bool first) {
  const size_t chunk = size_t(1) << 18;
  const size_t gb = dtype == MT_F32 ? 4 : 2;
  pool.run((int64_t)((n + chunk - 1) / chunk), [&](int64_t i) {
    size_t lo = (size_t)i * chunk, cnt = std::min(chunk, n - lo);
    if (cpu_has_avx512())
      accumulate_avx512(dtype, acc + lo, (const char*)g + lo * gb, cnt, first);
    else
      accumulate_scalar(dtype, acc + lo, (const char*)g + lo * gb, cnt, first);
  });
}

void adam_accumulated_parallel(ThreadPool& pool, int32_t dtype, void* w, float* p, float* acc, const void* g,
                               float* m, float* v, size_t n, const AdamConsts& k) {
  const size_t chunk = size_t(1) << 18;
  const size_t wb = dtype == MT_F32 ? 4 : 2;
  pool.run((int64_t)((n + chunk - 1) / chunk), [&](int64_t i) {
    size_t lo = (size_t)i * chunk, cnt = std::min(chunk, n - lo);
    float* pl = p ? p + lo : nullptr;
    if (cpu_has_avx512())
      adam_acc_avx512(dtype, (char*)w + lo * wb, pl, acc + lo, (const char*)g + lo * wb, m + lo, v + lo, cnt, k);
    else
      adam_acc_scalar(dtype, (char*)w + lo * wb, pl, acc + lo, (const char*)g + lo * wb, m + lo, v + lo, cnt, k);
  });
}

void adam_master_range(uint16_t* w, float* p, const uint16_t* g, float* m, float* v, size_t n, const AdamConsts& k) {
  if (cpu_has_avx512())
    adam_avx512_master(w, p, g, m, v, n, k);
  else
    adam_scalar_master(w, p, g, m, v, n, k);
}

void adam_master_parallel(ThreadPool& pool, uint16_t* w, float* p, const uint16_t* g, float* m, float* v, size_t n,
                          const AdamConsts& k) {
  const size_t chunk = size_t(1) << 18;
  int64_t tasks = (int64_t)((n + chunk - 1) / chunk);
  pool.run(tasks, [&](int64_t i) {
    size_t lo = (size_t)i * chunk, cnt = std::min(chunk, n - lo);
    adam_master_range(w + lo, p + lo, g + lo, m + lo, v + lo, cnt, k);
  });
}

}  // namespace mt
