// Memory-bound kernels of the decoder step: embedding, RMSNorm, RoPE,
// SwiGLU, cross-entropy, transposes and fixed-order reductions.
//
// The model they implement is the plain Llama-style reading of the
// MegaTrain pages (chatpaper.ai abstract: a decoder LLM trained one layer at
// a time, weights streamed in and gradients streamed out).  Every reduction
// runs in a fixed order that depends only on the shapes, so repeated runs
// and the streamed / resident schedules give identical bits.
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace mt {

template <typename T> __device__ inline float ldf(T x);
template <> __device__ inline float ldf<float>(float x) { return x; }
template <> __device__ inline float ldf<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <typename T> __device__ inline T stf(float x);
template <> __device__ inline float stf<float>(float x) { return x; }
template <> __device__ inline uint16_t stf<uint16_t>(float x) { return f32_to_bf16(x); }

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Four consecutive elements of type T as a float4 (16-byte loads for float,
// 8-byte for bf16); addresses must be aligned to 4 elements.
template <typename T> struct V4;
template <> struct V4<float> {
  static __device__ inline float4 ld(const float* p) { return *(const float4*)p; }
  static __device__ inline void st(float* p, float4 v) { *(float4*)p = v; }
};
template <> struct V4<uint16_t> {
  static __device__ inline float4 ld(const uint16_t* p) {
    const uint2 u = *(const uint2*)p;
    return make_float4(bf16_to_f32(u.x & 0xFFFF), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xFFFF),
                       bf16_to_f32(u.y >> 16));
  }
  static __device__ inline void st(uint16_t* p, float4 v) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    u.y = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
    *(uint2*)p = u;
  }
};

// Sum over a 256-thread block in a fixed tree order; every thread gets the result.
__device__ inline float block_sum256(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = (red[0] + red[1]) + (red[2] + red[3]);
  return r;
}

__device__ inline float block_max256(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ------------------------------------------------------------ embedding --
template <typename T>
__global__ void __launch_bounds__(256) k_embed_fwd(const int32_t* tok, const T* E, float* x, int d) {
  const int64_t m = blockIdx.x;
  const T* row = E + (int64_t)tok[m] * d;
  for (int i = threadIdx.x; i < d; i += 256) x[m * d + i] = ldf(row[i]);
}

template <typename T>
void embed_fwd(const int32_t* tok, const T* E, float* x, int M, int d, hipStream_t s) {
  if (M <= 0) return;
  hipLaunchKernelGGL(k_embed_fwd<T>, dim3(M), dim3(256), 0, s, tok, E, x, d);
}

template <typename T>
__global__ void __launch_bounds__(256) k_embed_bwd(const float* dx, const int32_t* order, const int32_t* seg, T* dE,
                                                   int d) {
  const int64_t v = blockIdx.x;
  const int lo = seg[v], hi = seg[v + 1];
  for (int i = threadIdx.x; i < d; i += 256) {
    float acc = 0.f;
    for (int s = lo; s < hi; ++s) acc += dx[(int64_t)order[s] * d + i];
    dE[v * d + i] = stf<T>(acc);
  }
}

template <typename T>
void embed_bwd(const float* dx, const int32_t* order, const int32_t* seg, T* dE, int V, int d, hipStream_t s) {
  hipLaunchKernelGGL(k_embed_bwd<T>, dim3(V), dim3(256), 0, s, dx, order, seg, dE, d);
}

// -------------------------------------------------------------- RMSNorm --
// A row of d floats lives in registers: thread t owns the 4-wide chunks
// t, t+256, ... (VPT of them); d must be a multiple of 4.
// ss + x^2 + y^2 + z^2 + w^2 as a fixed chain of fused multiply-adds: the
// forward norms (plain and with the residual add) round their statistics
// identically by construction, whatever contraction the compiler would
// choose for a written-out sum.
__device__ inline float sumsq4(float4 v, float ss) {
  ss = fmaf(v.x, v.x, ss);
  ss = fmaf(v.y, v.y, ss);
  ss = fmaf(v.z, v.z, ss);
  return fmaf(v.w, v.w, ss);
}

template <typename T, int VPT>
__global__ void __launch_bounds__(256) k_rmsnorm_fwd(const float* __restrict__ x, const T* __restrict__ g,
                                                     T* __restrict__ y, float* __restrict__ rstd, int d, float eps) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const float* xr = x + m * d;
  float4 v[VPT];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int c = (threadIdx.x + 256 * k) * 4;
    v[k] = c < d ? *(const float4*)(xr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    ss = sumsq4(v[k], ss);
  }
  ss = block_sum256(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  if (threadIdx.x == 0) rstd[m] = r;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int c = (threadIdx.x + 256 * k) * 4;
    if (c < d) {
      const float4 gg = V4<T>::ld(g + c);
      V4<T>::st(y + m * d + c, make_float4(v[k].x * r * gg.x, v[k].y * r * gg.y, v[k].z * r * gg.z, v[k].w * r * gg.w));
    }
  }
}

// The same norm of x = res + x (x updated in place): the residual add of a
// projection whose GEMM wrote only its product, done where the row is read
// anyway.  The add is the fp32 add the GEMM's residual epilogue would do.
template <typename T, int VPT>
__global__ void __launch_bounds__(256) k_rmsnorm_fwd_res(const float* __restrict__ res, float* __restrict__ x,
                                                         const T* __restrict__ g, T* __restrict__ y,
                                                         float* __restrict__ rstd, int d, float eps) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const float* rr = res + m * d;
  float* xr = x + m * d;
  float4 v[VPT];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int c = (threadIdx.x + 256 * k) * 4;
    if (c < d) {
      const float4 a = *(const float4*)(rr + c), p = *(const float4*)(xr + c);
      v[k] = make_float4(a.x + p.x, a.y + p.y, a.z + p.z, a.w + p.w);
      *(float4*)(xr + c) = v[k];
    } else {
      v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    ss = sumsq4(v[k], ss);
  }
  ss = block_sum256(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  if (threadIdx.x == 0) rstd[m] = r;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int c = (threadIdx.x + 256 * k) * 4;
    if (c < d) {
      const float4 gg = V4<T>::ld(g + c);
      V4<T>::st(y + m * d + c, make_float4(v[k].x * r * gg.x, v[k].y * r * gg.y, v[k].z * r * gg.z, v[k].w * r * gg.w));
    }
  }
}

static int rms_vpt(int d) {
  const int need = cdiv(d, 1024);
  const int opts[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16};
  for (int o : opts)
    if (o >= need) return o;
  throw ApiError{MT_E_INVALID, "RMSNorm supports d_model <= 16384"};
}

#define MT_RMS_DISPATCH(VPT_, LAUNCH) \
  switch (VPT_) {                     \
    case 1: LAUNCH(1); break;         \
    case 2: LAUNCH(2); break;         \
    case 3: LAUNCH(3); break;         \
    case 4: LAUNCH(4); break;         \
    case 5: LAUNCH(5); break;         \
    case 6: LAUNCH(6); break;         \
    case 8: LAUNCH(8); break;         \
    case 10: LAUNCH(10); break;       \
    case 12: LAUNCH(12); break;       \
    default: LAUNCH(16); break;       \
  }

template <typename T>
void rmsnorm_fwd(const float* x, const T* g, T* y, float* rstd, int M, int d, float eps, hipStream_t s) {
  if (M <= 0) return;
  if (d % 4) throw ApiError{MT_E_INVALID, "RMSNorm needs d_model % 4 == 0"};
#define L_(V) hipLaunchKernelGGL((k_rmsnorm_fwd<T, V>), dim3(M), dim3(256), 0, s, x, g, y, rstd, d, eps)
  MT_RMS_DISPATCH(rms_vpt(d), L_)
#undef L_
}

template <typename T>
void rmsnorm_fwd_res(const float* res, float* x, const T* g, T* y, float* rstd, int M, int d, float eps,
                     hipStream_t s) {
  if (M <= 0) return;
  if (d % 4) throw ApiError{MT_E_INVALID, "RMSNorm needs d_model % 4 == 0"};
#define L_(V) hipLaunchKernelGGL((k_rmsnorm_fwd_res<T, V>), dim3(M), dim3(256), 0, s, res, x, g, y, rstd, d, eps)
  MT_RMS_DISPATCH(rms_vpt(d), L_)
#undef L_
}

// Backward of RMSNorm over kRmsRows consecutive rows per block:
// dx = resid + r*(dy*g - xh*mean(dy*g*xh)) with xh = x*r, and the block's
// partial dgain sum_rows dy*xh written to part[block][d].  A second kernel
// adds the partials in block order.
constexpr int kRmsRows = 32;

size_t rmsnorm_dg_partial_elems(int M, int d) { return (size_t)std::max(1, cdiv(M, kRmsRows)) * d; }

template <typename T, int VPT>
__global__ void __launch_bounds__(256) k_rmsnorm_bwd(const float* __restrict__ dy, const float* __restrict__ x,
                                                     const T* __restrict__ g, const float* __restrict__ rstd,
                                                     const float* __restrict__ resid, float* __restrict__ dx,
                                                     T* __restrict__ dx_lp, float* __restrict__ part, int M, int d) {
  __shared__ float red[4];
  float4 gv[VPT], dg[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int c = (threadIdx.x + 256 * k) * 4;
    gv[k] = c < d ? V4<T>::ld(g + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    dg[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int m0 = blockIdx.x * kRmsRows, m1 = min(M, m0 + kRmsRows);
  for (int m = m0; m < m1; ++m) {
    const float r = rstd[m];
    const float* dyr = dy + (int64_t)m * d;
    const float* xr = x + (int64_t)m * d;
    float4 e[VPT], xh[VPT];
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int c = (threadIdx.x + 256 * k) * 4;
      if (c < d) {
        e[k] = *(const float4*)(dyr + c);
        const float4 xv = *(const float4*)(xr + c);
        xh[k] = make_float4(xv.x * r, xv.y * r, xv.z * r, xv.w * r);
      } else {
        e[k] = xh[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      dot += e[k].x * gv[k].x * xh[k].x + e[k].y * gv[k].y * xh[k].y + e[k].z * gv[k].z * xh[k].z +
             e[k].w * gv[k].w * xh[k].w;
    }
    dot = block_sum256(dot, red);
    const float mean = dot / (float)d;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int c = (threadIdx.x + 256 * k) * 4;
      if (c < d) {
        float4 o = make_float4(r * (e[k].x * gv[k].x - xh[k].x * mean), r * (e[k].y * gv[k].y - xh[k].y * mean),
                               r * (e[k].z * gv[k].z - xh[k].z * mean), r * (e[k].w * gv[k].w - xh[k].w * mean));
        if (resid) {
          const float4 rv = *(const float4*)(resid + (int64_t)m * d + c);
          o = make_float4(rv.x + o.x, rv.y + o.y, rv.z + o.z, rv.w + o.w);
        }
        *(float4*)(dx + (int64_t)m * d + c) = o;
        if (dx_lp) V4<T>::st(dx_lp + (int64_t)m * d + c, o);
        dg[k].x += e[k].x * xh[k].x;
        dg[k].y += e[k].y * xh[k].y;
        dg[k].z += e[k].z * xh[k].z;
        dg[k].w += e[k].w * xh[k].w;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int c = (threadIdx.x + 256 * k) * 4;
    if (c < d) *(float4*)(part + (int64_t)blockIdx.x * d + c) = dg[k];
  }
}

template <typename T>
__global__ void __launch_bounds__(256) k_dg_reduce(const float* __restrict__ part, T* __restrict__ dg, int chunks,
                                                   int d) {
  // One block: 32 columns (8 threads x float4) x 32 interleaved partial
  // sums; partial g adds chunks g, g+32, g+64, ... in order, then the 32
  // partials are added in order.  The order depends only on (chunks, d).
  __shared__ float4 red[32][8];
  const int c4 = threadIdx.x & 7, g = threadIdx.x >> 3;
  const int c = (blockIdx.x * 8 + c4) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < d) {
#pragma unroll 4
    for (int k = g; k < chunks; k += 32) {
      const float4 v = *(const float4*)(part + (int64_t)k * d + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
  }
  red[g][c4] = acc;
  __syncthreads();
  if (g == 0 && c < d) {
    float4 t = red[0][c4];
    for (int j = 1; j < 32; ++j) {
      const float4 v = red[j][c4];
      t.x += v.x;
      t.y += v.y;
      t.z += v.z;
      t.w += v.w;
    }
    V4<T>::st(dg + c, t);
  }
}

template <typename T>
void rmsnorm_bwd(const float* dy, const float* x, const T* g, const float* rstd, const float* resid, float* dx,
                 float* partial, T* dg, int M, int d, hipStream_t s, T* dx_lp) {
  if (d % 4) throw ApiError{MT_E_INVALID, "RMSNorm needs d_model % 4 == 0"};
  const int blocks = cdiv(M, kRmsRows);
  if (blocks > 0) {
#define L_(V)                                                                                                    \
  hipLaunchKernelGGL((k_rmsnorm_bwd<T, V>), dim3(blocks), dim3(256), 0, s, dy, x, g, rstd, resid, dx, dx_lp, partial, \
                     M, d)
    MT_RMS_DISPATCH(rms_vpt(d), L_)
#undef L_
  }
  if (dg) rmsnorm_dg_reduce<T>(partial, dg, blocks, d, s);
}

template <typename T>
void rmsnorm_dg_reduce(const float* partial, T* dg, int blocks, int d, hipStream_t s) {
  hipLaunchKernelGGL(k_dg_reduce<T>, dim3(cdiv(d, 32)), dim3(256), 0, s, partial, dg, blocks, d);
}

int rmsnorm_rows_per_block() { return kRmsRows; }

// ----------------------------------------------------------------- RoPE --
// Token-major transposed buffers [C x M] use a padded row stride (see
// kernels.h).
int64_t token_ld(int64_t M) {
  int64_t ld = (M + 127) / 128 * 128;
  if ((ld / 128) % 2 == 0) ld += 128;
  return ld;
}

// q and k rotate in place; one thread per (token, head of q or k, pair i):
// x_i, x_{i+hd/2} -> x_i cos - x_{i+hd/2} sin, x_i sin + x_{i+hd/2} cos.
template <typename T>
__global__ void __launch_bounds__(256) k_rope_qkv(T* qkv, const float* cosb, const float* sinb, int M, int T_, int d,
                                                  int hd, int64_t row0) {
  const int h2 = hd / 2;
  const int64_t per_tok = (int64_t)2 * (d / hd) * h2;  // q and k heads x pairs
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)M * per_tok) return;
  const int64_t m = id / per_tok;
  const int j = (int)(id % per_tok);
  const int hh = j / h2, i = j % h2;
  T* x = qkv + m * 3LL * d + (int64_t)hh * hd;
  const int t = (int)((m + row0) % T_);
  const float cs = cosb[(int64_t)t * h2 + i], sn = sinb[(int64_t)t * h2 + i];
  const float a = ldf(x[i]), b = ldf(x[i + h2]);
  x[i] = stf<T>(a * cs - b * sn);
  x[i + h2] = stf<T>(a * sn + b * cs);
}

// bf16, head_dim 128: one thread per (token, head of q or k, 8 adjacent
// pairs), 16-byte accesses.
__device__ inline void unpack8(const uint4 u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xFFFF);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}
__device__ inline uint4 pack8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ void __launch_bounds__(256) k_rope_qkv_bf16(uint16_t* __restrict__ qkv, const float* __restrict__ cosb,
                                                       const float* __restrict__ sinb, int M, int T_, int d,
                                                       int64_t row0) {
  const int per_tok = 2 * (d / 128) * 8;  // q and k heads x 8 groups of 8 pairs
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)M * per_tok) return;
  const int64_t m = id / per_tok;
  const int j = (int)(id % per_tok);
  const int hh = j >> 3, i0 = (j & 7) * 8;
  uint16_t* x = qkv + m * 3LL * d + (int64_t)hh * 128 + i0;
  const int t = (int)((m + row0) % T_);
  const float4* cp = (const float4*)(cosb + (int64_t)t * 64 + i0);
  const float4* sp = (const float4*)(sinb + (int64_t)t * 64 + i0);
  const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
  const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  float a[8], b[8], oa[8], ob[8];
  unpack8(*(const uint4*)x, a);
  unpack8(*(const uint4*)(x + 64), b);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    oa[e] = a[e] * cs[e] - b[e] * sn[e];
    ob[e] = a[e] * sn[e] + b[e] * cs[e];
  }
  *(uint4*)x = pack8(oa);
  *(uint4*)(x + 64) = pack8(ob);
}

template <typename T>
void rope_qkv_fwd(T* qkv, const float* cosb, const float* sinb, int M, int T_, int d, int hd, hipStream_t s,
                  int64_t row0) {
  if (M <= 0) return;
  if (std::is_same<T, uint16_t>::value && hd == 128 && d % 128 == 0 && ((uintptr_t)qkv & 15) == 0 &&
      ((uintptr_t)cosb & 15) == 0 && ((uintptr_t)sinb & 15) == 0) {
    const int64_t n = (int64_t)M * 2 * (d / 128) * 8;
    hipLaunchKernelGGL(k_rope_qkv_bf16, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, (uint16_t*)qkv, cosb, sinb,
                       M, T_, d, row0);
    return;
  }
  const int64_t n = (int64_t)M * 2 * (d / hd) * (hd / 2);
  hipLaunchKernelGGL(k_rope_qkv<T>, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, qkv, cosb, sinb, M, T_, d, hd, row0);
}

// Inverse rotation on the transposed layout: one thread per (pair, 8 tokens)
// when the token count is a multiple of 8, else per (pair, token).  The
// tables come transposed, [hd/2][T], so a thread's 8 positions are adjacent.
template <typename T>
__global__ void __launch_bounds__(256) k_rope_bwd_T(T* x, int64_t ldT, const float* cosT, const float* sinT, int M,
                                                    int T_, int d, int hd) {
  const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const int pr = blockIdx.y;  // pair index over q and k: [0, d)
  const int h2 = hd / 2;
  const int part = pr / (d / 2);
  const int rem = pr % (d / 2);
  const int head = rem / h2, i = rem % h2;
  const int64_t ra = (int64_t)part * d + (int64_t)head * hd + i, rb = ra + h2;
  const int t = (int)(m % T_);
  const float cs = cosT[(int64_t)i * T_ + t], sn = sinT[(int64_t)i * T_ + t];
  const float a = ldf(x[ra * ldT + m]), b = ldf(x[rb * ldT + m]);
  x[ra * ldT + m] = stf<T>(a * cs + b * sn);
  x[rb * ldT + m] = stf<T>(b * cs - a * sn);
}

__global__ void __launch_bounds__(256) k_rope_bwd_T8(uint16_t* x, int64_t ldT, const float* cosT, const float* sinT,
                                                     int M, int T_, int d, int hd) {
  const int64_t m = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (m >= M) return;
  const int pr = blockIdx.y;
  const int h2 = hd / 2;
  const int part = pr / (d / 2);
  const int rem = pr % (d / 2);
  const int head = rem / h2, i = rem % h2;
  const int64_t ra = (int64_t)part * d + (int64_t)head * hd + i, rb = ra + h2;
  float a[8], b[8], oa[8], ob[8];
  unpack8(*(const uint4*)(x + ra * ldT + m), a);
  unpack8(*(const uint4*)(x + rb * ldT + m), b);
  // T_ % 8 == 0, so the 8 positions t .. t+7 belong to one sequence
  const int t = (int)(m % T_);
  const float4* cp = (const float4*)(cosT + (int64_t)i * T_ + t);
  const float4* sp = (const float4*)(sinT + (int64_t)i * T_ + t);
  const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
  const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    oa[e] = a[e] * cs[e] + b[e] * sn[e];
    ob[e] = b[e] * cs[e] - a[e] * sn[e];
  }
  *(uint4*)(x + ra * ldT + m) = pack8(oa);
  *(uint4*)(x + rb * ldT + m) = pack8(ob);
}

template <typename T>
void rope_bwd_T(T* dqkvT, int64_t ldT, const float* cosT, const float* sinT, int M, int T_, int d, int hd,
                hipStream_t s) {
  if (M <= 0) return;
  if (std::is_same<T, uint16_t>::value && M % 8 == 0 && T_ % 8 == 0 && ldT % 8 == 0) {
    hipLaunchKernelGGL(k_rope_bwd_T8, dim3(cdiv(M / 8, 256), d), dim3(256), 0, s, (uint16_t*)dqkvT, ldT, cosT, sinT,
                       M, T_, d, hd);
    return;
  }
  hipLaunchKernelGGL(k_rope_bwd_T<T>, dim3(cdiv(M, 256), d), dim3(256), 0, s, dqkvT, ldT, cosT, sinT, M, T_, d, hd);
}

// --------------------------------------------------------------- SwiGLU --
__device__ inline float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }
__device__ inline float silu_(float g) { return g / (1.0f + expf(-g)); }

// Four outputs per thread (F % 4 == 0): gate g = gu[m][j], up u = gu[m][F+j].
template <typename T>
__global__ void __launch_bounds__(256) k_swiglu_fwd(const T* __restrict__ gu, T* __restrict__ y, int64_t n4, int F) {
  const int F4 = F / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / F4, j = (i % F4) * 4;
    const float4 g = V4<T>::ld(gu + m * 2 * F + j), u = V4<T>::ld(gu + m * 2 * F + F + j);
    V4<T>::st(y + m * F + j, make_float4(silu_(g.x) * u.x, silu_(g.y) * u.y, silu_(g.z) * u.z, silu_(g.w) * u.w));
  }
}

// bf16 with d_ff % 8 == 0: eight outputs per thread, 16-byte accesses; one
// grid row per token row (no index division).  Same arithmetic per element.

__global__ void __launch_bounds__(256) k_swiglu_fwd8(const uint16_t* __restrict__ gu, uint16_t* __restrict__ y, int F) {
  const int j = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (j >= F) return;
  const int64_t m = blockIdx.y;
  float g[8], u[8], o[8];
  unpack8(*(const uint4*)(gu + m * 2 * F + j), g);
  unpack8(*(const uint4*)(gu + m * 2 * F + F + j), u);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = silu_(g[i]) * u[i];
  *(uint4*)(y + m * F + j) = pack8(o);
}

template <typename T>
void swiglu_fwd(const T* gu, T* y, int M, int F, hipStream_t s) {
  if (F % 4) throw ApiError{MT_E_INVALID, "SwiGLU needs d_ff % 4 == 0"};
  const int64_t n4 = (int64_t)M * F / 4;
  if (n4 <= 0) return;
  if constexpr (std::is_same<T, uint16_t>::value) {
    if (F % 8 == 0) {
      // rows in chunks of at most 65535 grid rows
      for (int r0 = 0; r0 < M; r0 += 65535) {
        const int rows = std::min(65535, M - r0);
        hipLaunchKernelGGL(k_swiglu_fwd8, dim3(cdiv(F / 8, 256), rows), dim3(256), 0, s, gu + (int64_t)r0 * 2 * F,
                           y + (int64_t)r0 * F, F);
      }
      return;
    }
  }
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 65536);
  hipLaunchKernelGGL(k_swiglu_fwd<T>, dim3(blocks), dim3(256), 0, s, gu, y, n4, F);
}

__device__ inline void swiglu_grad1(float e, float g, float u, float* dg, float* du) {
  const float sg = sigmoidf_(g);
  *dg = e * u * (sg * (1.0f + g * (1.0f - sg)));
  *du = e * silu_(g);
}

template <typename T>
__global__ void __launch_bounds__(256) k_swiglu_bwd(const T* __restrict__ dy, const T* __restrict__ gu,
                                                    T* __restrict__ dgu, int64_t n4, int F) {
  const int F4 = F / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / F4, j = (i % F4) * 4;
    const float4 g = V4<T>::ld(gu + m * 2 * F + j), u = V4<T>::ld(gu + m * 2 * F + F + j);
    const float4 e = V4<T>::ld(dy + m * F + j);
    float4 a, b;
    swiglu_grad1(e.x, g.x, u.x, &a.x, &b.x);
    swiglu_grad1(e.y, g.y, u.y, &a.y, &b.y);
    swiglu_grad1(e.z, g.z, u.z, &a.z, &b.z);
    swiglu_grad1(e.w, g.w, u.w, &a.w, &b.w);
    V4<T>::st(dgu + m * 2 * F + j, a);
    V4<T>::st(dgu + m * 2 * F + F + j, b);
  }
}

__global__ void __launch_bounds__(256) k_swiglu_bwd8(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ gu,
                                                     uint16_t* __restrict__ dgu, int F) {
  const int j = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (j >= F) return;
  const int64_t m = blockIdx.y;
  float g[8], u[8], e[8], a[8], b[8];
  unpack8(*(const uint4*)(gu + m * 2 * F + j), g);
  unpack8(*(const uint4*)(gu + m * 2 * F + F + j), u);
  unpack8(*(const uint4*)(dy + m * F + j), e);
#pragma unroll
  for (int i = 0; i < 8; ++i) swiglu_grad1(e[i], g[i], u[i], &a[i], &b[i]);
  *(uint4*)(dgu + m * 2 * F + j) = pack8(a);
  *(uint4*)(dgu + m * 2 * F + F + j) = pack8(b);
}

template <typename T>
void swiglu_bwd(const T* dy, const T* gu, T* dgu, int M, int F, hipStream_t s) {
  if (F % 4) throw ApiError{MT_E_INVALID, "SwiGLU needs d_ff % 4 == 0"};
  const int64_t n4 = (int64_t)M * F / 4;
  if (n4 <= 0) return;
  if constexpr (std::is_same<T, uint16_t>::value) {
    if (F % 8 == 0) {
      for (int r0 = 0; r0 < M; r0 += 65535) {
        const int rows = std::min(65535, M - r0);
        hipLaunchKernelGGL(k_swiglu_bwd8, dim3(cdiv(F / 8, 256), rows), dim3(256), 0, s, dy + (int64_t)r0 * F,
                           gu + (int64_t)r0 * 2 * F, dgu + (int64_t)r0 * 2 * F, F);
      }
      return;
    }
  }
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 65536);
  hipLaunchKernelGGL(k_swiglu_bwd<T>, dim3(blocks), dim3(256), 0, s, dy, gu, dgu, n4, F);
}

// -------------------------------------------------------- cross-entropy --
template <typename T>
__global__ void __launch_bounds__(256) k_xent(const float* logits, const int32_t* tok, float* row_loss, T* dl, int T_,
                                              int V, float inv_n, int64_t row0) {
  __shared__ float red[4];
  // logits and dl hold the rows of one pass; m is the token's row in the batch
  const int64_t m = row0 + blockIdx.x;
  const float* z = logits + (int64_t)blockIdx.x * V;
  T* out = dl + (int64_t)blockIdx.x * V;
  if ((int)(m % T_) == T_ - 1) {
    for (int v = threadIdx.x; v < V; v += 256) out[v] = stf<T>(0.f);
    if (threadIdx.x == 0) row_loss[m] = 0.f;
    return;
  }
  const int label = tok[m + 1];
  float mx = -INFINITY;
  for (int v = threadIdx.x; v < V; v += 256) mx = fmaxf(mx, z[v]);
  mx = block_max256(mx, red);
  float se = 0.f;
  for (int v = threadIdx.x; v < V; v += 256) se += expf(z[v] - mx);
  se = block_sum256(se, red);
  const float inv_se = 1.0f / se;
  for (int v = threadIdx.x; v < V; v += 256) {
    float p = expf(z[v] - mx) * inv_se;
    if (v == label) p -= 1.0f;
    out[v] = stf<T>(p * inv_n);
  }
  if (threadIdx.x == 0) row_loss[m] = mx + logf(se) - z[label];
}

template <typename T>
void xent(const float* logits, const int32_t* tok, float* row_loss, T* dlogits, int rows, int64_t row0, int T_, int V,
          float inv_n, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_xent<T>, dim3(rows), dim3(256), 0, s, logits, tok, row_loss, dlogits, T_, V, inv_n, row0);
}

__global__ void __launch_bounds__(1024) k_sum_fixed(const float* x, float* out, int n, float scale) {
  __shared__ float red[1024];
  float acc = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) acc += x[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0] * scale;
}

void sum_fixed(const float* x, float* out, int n, float scale, hipStream_t s) {
  hipLaunchKernelGGL(k_sum_fixed, dim3(1), dim3(1024), 0, s, x, out, n, scale);
}

// ------------------------------------------------------------ transpose --
template <typename T>
__global__ void __launch_bounds__(256) k_transpose(const T* in, int64_t ld_in, T* out, int64_t ld_out, int R, int C) {
  __shared__ T tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    int r = idx / 64, c = idx % 64;
    if (r0 + r < R && c0 + c < C) tile[r][c] = in[(r0 + r) * ld_in + c0 + c];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    int c = idx / 64, r = idx % 64;
    if (r0 + r < R && c0 + c < C)
      out[(c0 + c) * ld_out + r0 + r] = tile[r][c];
  }
}

// bf16 64x64 tile with 16-byte global loads and stores (8 elements per
// access); rows and columns of the tile that fall outside R x C are skipped
// per 8-element group, so R, C, ld_in, ld_out must be multiples of 8.
//
// The tile sits in LDS row-major, 128 bytes per input row, 16-byte chunk j
// of row r at chunk j ^ ((r >> 3) & 7).  Each thread reads the 4-byte column
// pair (2p, 2p+1) of 8 consecutive rows and packs the two output runs with
// byte permutes; the 8 lanes of one output row cover 128 contiguous bytes.
__global__ void __launch_bounds__(256) k_transpose_bf16(const uint16_t* __restrict__ in, int64_t ld_in,
                                                        uint16_t* __restrict__ out, int64_t ld_out, int R, int C) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[64 * 128];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int id = threadIdx.x + 256 * k;
    const int r = id >> 3, c8 = id & 7;
    if (r0 + r < R && c0 + 8 * c8 < C)
      *(uint4*)(tile + r * 128 + ((c8 ^ ((r >> 3) & 7)) << 4)) =
          *(const uint4*)(in + (r0 + r) * ld_in + c0 + 8 * c8);
  }
  __syncthreads();
  const int p = threadIdx.x >> 3, r8 = (threadIdx.x & 7) * 8;
  if (c0 + 2 * p < C && r0 + r8 < R) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = r8 + i;
      w[i] = *(const uint32_t*)(tile + rr * 128 + (((p >> 2) ^ ((rr >> 3) & 7)) << 4) + ((p & 3) << 2));
    }
    uint4 lo, hi;  // output columns 2p and 2p+1: the low and high halves of w
    lo.x = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
    lo.y = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
    lo.z = __builtin_amdgcn_perm(w[5], w[4], 0x05040100u);
    lo.w = __builtin_amdgcn_perm(w[7], w[6], 0x05040100u);
    hi.x = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
    hi.y = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
    hi.z = __builtin_amdgcn_perm(w[5], w[4], 0x07060302u);
    hi.w = __builtin_amdgcn_perm(w[7], w[6], 0x07060302u);
    *(uint4*)(out + (c0 + 2 * p) * ld_out + r0 + r8) = lo;
    *(uint4*)(out + (c0 + 2 * p + 1) * ld_out + r0 + r8) = hi;
  }
}

template <typename T>
void transpose(const T* in, int64_t ld_in, T* out, int64_t ld_out, int R, int C, hipStream_t s) {
  if (R <= 0 || C <= 0) return;
  if (std::is_same<T, uint16_t>::value && R % 8 == 0 && C % 8 == 0 && ld_in % 8 == 0 && ld_out % 8 == 0 &&
      ((uintptr_t)in & 15) == 0 && ((uintptr_t)out & 15) == 0) {
    hipLaunchKernelGGL(k_transpose_bf16, dim3(cdiv(C, 64), cdiv(R, 64)), dim3(256), 0, s, (const uint16_t*)in, ld_in,
                       (uint16_t*)out, ld_out, R, C);
    return;
  }
  hipLaunchKernelGGL(k_transpose<T>, dim3(cdiv(C, 64), cdiv(R, 64)), dim3(256), 0, s, in, ld_in, out, ld_out, R, C);
}

template <typename T>
__global__ void __launch_bounds__(256) k_cast_transpose(const float* in, T* out, T* outT, int64_t ldT, int R, int C) {
  __shared__ T tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    int r = idx / 64, c = idx % 64;
    if (r0 + r < R && c0 + c < C) {
      T v = stf<T>(in[(r0 + r) * C + c0 + c]);
      out[(r0 + r) * C + c0 + c] = v;
      tile[r][c] = v;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    int c = idx / 64, r = idx % 64;
    if (r0 + r < R && c0 + c < C) outT[(c0 + c) * ldT + r0 + r] = tile[r][c];
  }
}

template <typename T>
void cast_transpose(const float* in, T* out, T* outT, int64_t ldT, int R, int C, hipStream_t s) {
  if (R <= 0 || C <= 0) return;
  hipLaunchKernelGGL(k_cast_transpose<T>, dim3(cdiv(C, 64), cdiv(R, 64)), dim3(256), 0, s, in, out, outT, ldT, R, C);
}

// out = T(in), 4 elements per thread (n % 4 == 0, 16-byte aligned), else 1.
template <typename T, bool V4_>
__global__ void __launch_bounds__(256) k_cast(const float* __restrict__ in, T* __restrict__ out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * (V4_ ? 4 : 1);
  if (i >= n) return;
  if (V4_)
    V4<T>::st(out + i, *(const float4*)(in + i));
  else
    out[i] = stf<T>(in[i]);
}

template <typename T>
void cast(const float* in, T* out, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  if (n % 4 == 0 && ((uintptr_t)in & 15) == 0 && ((uintptr_t)out & 7) == 0)
    hipLaunchKernelGGL((k_cast<T, true>), dim3((unsigned)cdiv(n / 4, 256)), dim3(256), 0, s, in, out, n);
  else
    hipLaunchKernelGGL((k_cast<T, false>), dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, in, out, n);
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = v;
}

void fill_u32(void* p, uint32_t value, size_t n_words, hipStream_t s) {
  if (!n_words) return;
  int blocks = (int)std::min<size_t>((n_words + 255) / 256, 65536);
  hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(256), 0, s, (uint32_t*)p, value, n_words);
}

// bf16 -> fp32, 8 values (16 bytes in, 32 out) per thread when n % 8 == 0
__global__ void __launch_bounds__(256) k_widen8(const uint16_t* __restrict__ in, float* __restrict__ out, int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float f[8];
    unpack8(*(const uint4*)(in + 8 * i), f);
    *(float4*)(out + 8 * i) = make_float4(f[0], f[1], f[2], f[3]);
    *(float4*)(out + 8 * i + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
}
__global__ void __launch_bounds__(256) k_widen1(const uint16_t* __restrict__ in, float* __restrict__ out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = bf16_to_f32(in[i]);
}

void widen_bf16(const uint16_t* in, float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  if (n % 8 == 0 && ((uintptr_t)in & 15) == 0 && ((uintptr_t)out & 15) == 0) {
    const int64_t n8 = n / 8;
    hipLaunchKernelGGL(k_widen8, dim3((unsigned)std::min<int64_t>(cdiv(n8, 256), 65536)), dim3(256), 0, s, in, out,
                       n8);
  } else {
    hipLaunchKernelGGL(k_widen1, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), dim3(256), 0, s, in, out, n);
  }
}

// ------------------------------------------------------ instantiations --
#define MT_INST(T)                                                                                              \
  template void embed_fwd<T>(const int32_t*, const T*, float*, int, int, hipStream_t);                          \
  template void embed_bwd<T>(const float*, const int32_t*, const int32_t*, T*, int, int, hipStream_t);          \
  template void rmsnorm_fwd<T>(const float*, const T*, T*, float*, int, int, float, hipStream_t);               \
  template void rmsnorm_fwd_res<T>(const float*, float*, const T*, T*, float*, int, int, float, hipStream_t);    \
  template void rmsnorm_bwd<T>(const float*, const float*, const T*, const float*, const float*, float*, float*, T*, \
                               int, int, hipStream_t, T*);                                                          \
  template void rope_qkv_fwd<T>(T*, const float*, const float*, int, int, int, int, hipStream_t, int64_t);       \
  template void rmsnorm_dg_reduce<T>(const float*, T*, int, int, hipStream_t);              \
  template void rope_bwd_T<T>(T*, int64_t, const float*, const float*, int, int, int, int, hipStream_t);        \
  template void swiglu_fwd<T>(const T*, T*, int, int, hipStream_t);                                             \
  template void swiglu_bwd<T>(const T*, const T*, T*, int, int, hipStream_t);                                   \
  template void xent<T>(const float*, const int32_t*, float*, T*, int, int64_t, int, int, float, hipStream_t);           \
  template void transpose<T>(const T*, int64_t, T*, int64_t, int, int, hipStream_t);                            \
  template void cast_transpose<T>(const float*, T*, T*, int64_t, int, int, hipStream_t);                       \
  template void cast<T>(const float*, T*, int64_t, hipStream_t);

MT_INST(float)
MT_INST(uint16_t)

}  // namespace mt
