// Shared internal definitions of the MI355X layer-streamed training library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstring>
#include <string>

#include "mt.h"

namespace mt {

// Thread-local error message behind mt_last_error().
void set_error(const std::string& msg);
const char* last_error();

struct HipError {
  hipError_t code;
  std::string where;
};

#define MT_HIP(call)                                                                 \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) throw ::mt::HipError{e_, std::string(#call) + " @" +       \
                                                       __FILE__ + ":" +              \
                                                       std::to_string(__LINE__)};    \
  } while (0)

struct ApiError {
  int code;
  std::string msg;
};

inline uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// bfloat16 storage type: raw bits, round-to-nearest-even from float.
struct bf16 {
  uint16_t bits;
};

__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

__host__ __device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);  // keep NaN a NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

}  // namespace mt
