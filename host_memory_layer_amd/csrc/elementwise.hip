// Memory-bound kernels of the decoder step: embedding, RMSNorm, RoPE,
// SwiGLU, cross-entropy, transposes and fixed-order reductions.
//
// The model they implement is the plain Llama-style reading of the
// MegaTrain pages (chatpaper.ai abstract: a decoder LLM trained one layer at
// a time, weights streamed in and gradients streamed out).  Every reduction
// runs in a fixed order that depends only on the shapes, so repeated runs
// and the streamed / resident schedules give identical bits.
#include "kernels.h"

namespace mt {

template <typename T> __device__ inline float ldf(T x);
template <> __device__ inline float ldf<float>(float x) { return x; }
template <> __device__ inline float ldf<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <typename T> __device__ inline T stf(float x);
template <> __device__ inline float stf<float>(float x) { return x; }
template <> __device__ inline uint16_t stf<uint16_t>(float x) { return f32_to_bf16(x); }

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

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
template <typename T>
__global__ void __launch_bounds__(256) k_rmsnorm_fwd(const float* x, const T* g, T* y, float* rstd, int d, float eps) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const float* xr = x + m * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) ss += xr[i] * xr[i];
  ss = block_sum256(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  if (threadIdx.x == 0) rstd[m] = r;
  for (int i = threadIdx.x; i < d; i += 256) y[m * d + i] = stf<T>(xr[i] * r * ldf(g[i]));
}

template <typename T>
void rmsnorm_fwd(const float* x, const T* g, T* y, float* rstd, int M, int d, float eps, hipStream_t s) {
  if (M <= 0) return;
  hipLaunchKernelGGL(k_rmsnorm_fwd<T>, dim3(M), dim3(256), 0, s, x, g, y, rstd, d, eps);
}

template <typename T>
__global__ void __launch_bounds__(256) k_rmsnorm_bwd(const float* dy, const float* x, const T* g, const float* rstd,
                                                     const float* resid, float* dx, int d) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const float r = rstd[m];
  const float* dyr = dy + m * d;
  const float* xr = x + m * d;
  float dot = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) dot += dyr[i] * ldf(g[i]) * (xr[i] * r);
  dot = block_sum256(dot, red);
  const float mean = dot / (float)d;
  for (int i = threadIdx.x; i < d; i += 256) {
    float xh = xr[i] * r;
    float v = r * (dyr[i] * ldf(g[i]) - xh * mean);
    if (resid) v = resid[m * d + i] + v;
    dx[m * d + i] = v;
  }
}

template <typename T>
void rmsnorm_bwd(const float* dy, const float* x, const T* g, const float* rstd, const float* resid, float* dx, int M,
                 int d, hipStream_t s) {
  if (M <= 0) return;
  hipLaunchKernelGGL(k_rmsnorm_bwd<T>, dim3(M), dim3(256), 0, s, dy, x, g, rstd, resid, dx, d);
}

constexpr int kDgRows = 128;

size_t rmsnorm_dg_partial_elems(int M, int d) { return (size_t)cdiv(M, kDgRows) * d; }

__global__ void __launch_bounds__(256) k_dg_partial(const float* dy, const float* x, const float* rstd, float* part,
                                                    int M, int d) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int chunk = blockIdx.y;
  if (c >= d) return;
  const int m0 = chunk * kDgRows, m1 = min(M, m0 + kDgRows);
  float acc = 0.f;
  for (int m = m0; m < m1; ++m) acc += dy[(int64_t)m * d + c] * (x[(int64_t)m * d + c] * rstd[m]);
  part[(int64_t)chunk * d + c] = acc;
}

template <typename T>
__global__ void __launch_bounds__(256) k_dg_reduce(const float* part, T* dg, int chunks, int d) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  float acc = 0.f;
  for (int k = 0; k < chunks; ++k) acc += part[(int64_t)k * d + c];
  dg[c] = stf<T>(acc);
}

template <typename T>
void rmsnorm_dg(const float* dy, const float* x, const float* rstd, float* partial, T* dg, int M, int d,
                hipStream_t s) {
  const int chunks = cdiv(M, kDgRows);
  if (chunks == 0) {
    hipLaunchKernelGGL(k_dg_reduce<T>, dim3(cdiv(d, 256)), dim3(256), 0, s, partial, dg, 0, d);
    return;
  }
  hipLaunchKernelGGL(k_dg_partial, dim3(cdiv(d, 256), chunks), dim3(256), 0, s, dy, x, rstd, partial, M, d);
  hipLaunchKernelGGL(k_dg_reduce<T>, dim3(cdiv(d, 256)), dim3(256), 0, s, partial, dg, chunks, d);
}

// ----------------------------------------------------------------- RoPE --
// One block: 64 tokens x one head of q, k or v.  q and k rotate in place;
// all three are also written transposed into qkvT [3d x M].
int64_t token_ld(int64_t M) {
  int64_t ld = (M + 127) / 128 * 128;
  if ((ld / 128) % 2 == 0) ld += 128;
  return ld;
}

template <typename T>
__global__ void __launch_bounds__(256) k_rope_qkv(T* qkv, T* qkvT, int64_t ldT, const float* cosb, const float* sinb,
                                                  int M, int T_, int d, int hd) {
  __shared__ float tile[64][129];
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int part = blockIdx.y / (d / hd);  // 0 q, 1 k, 2 v
  const int head = blockIdx.y % (d / hd);
  const int64_t col0 = (int64_t)part * d + (int64_t)head * hd;
  const int64_t ld = 3LL * d;
  for (int idx = threadIdx.x; idx < 64 * hd; idx += 256) {
    int r = idx / hd, c = idx % hd;
    int64_t m = m0 + r;
    tile[r][c] = m < M ? ldf(qkv[m * ld + col0 + c]) : 0.f;
  }
  __syncthreads();
  if (part < 2) {
    const int h2 = hd / 2;
    for (int idx = threadIdx.x; idx < 64 * h2; idx += 256) {
      int r = idx / h2, i = idx % h2;
      int64_t m = m0 + r;
      if (m >= M) continue;
      int t = (int)(m % T_);
      float cs = cosb[(int64_t)t * h2 + i], sn = sinb[(int64_t)t * h2 + i];
      float a = tile[r][i], b = tile[r][i + h2];
      tile[r][i] = a * cs - b * sn;
      tile[r][i + h2] = a * sn + b * cs;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * hd; idx += 256) {
      int r = idx / hd, c = idx % hd;
      int64_t m = m0 + r;
      if (m < M) qkv[m * ld + col0 + c] = stf<T>(tile[r][c]);
    }
  }
  for (int idx = threadIdx.x; idx < 64 * hd; idx += 256) {
    int c = idx / 64, r = idx % 64;
    int64_t m = m0 + r;
    if (m < M) qkvT[(col0 + c) * ldT + m] = stf<T>(tile[r][c]);
  }
}

template <typename T>
void rope_qkv_fwd(T* qkv, T* qkvT, int64_t ldT, const float* cosb, const float* sinb, int M, int T_, int d, int hd,
                  hipStream_t s) {
  if (M <= 0) return;
  hipLaunchKernelGGL(k_rope_qkv<T>, dim3(cdiv(M, 64), 3 * (d / hd)), dim3(256), 0, s, qkv, qkvT, ldT, cosb, sinb, M,
                     T_, d, hd);
}

template <typename T>
__global__ void __launch_bounds__(256) k_rope_bwd_T(T* x, int64_t ldT, const float* cosb, const float* sinb, int M,
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
  const float cs = cosb[(int64_t)t * h2 + i], sn = sinb[(int64_t)t * h2 + i];
  const float a = ldf(x[ra * ldT + m]), b = ldf(x[rb * ldT + m]);
  x[ra * ldT + m] = stf<T>(a * cs + b * sn);
  x[rb * ldT + m] = stf<T>(b * cs - a * sn);
}

template <typename T>
void rope_bwd_T(T* dqkvT, int64_t ldT, const float* cosb, const float* sinb, int M, int T_, int d, int hd,
                hipStream_t s) {
  if (M <= 0) return;
  hipLaunchKernelGGL(k_rope_bwd_T<T>, dim3(cdiv(M, 256), d), dim3(256), 0, s, dqkvT, ldT, cosb, sinb, M, T_, d, hd);
}

// --------------------------------------------------------------- SwiGLU --
__device__ inline float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

template <typename T>
__global__ void __launch_bounds__(256) k_swiglu_fwd(const T* gu, T* y, int64_t n, int F) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    int64_t m = i / F, j = i % F;
    float g = ldf(gu[m * 2 * F + j]), u = ldf(gu[m * 2 * F + F + j]);
    y[i] = stf<T>(g / (1.0f + expf(-g)) * u);
  }
}

template <typename T>
void swiglu_fwd(const T* gu, T* y, int M, int F, hipStream_t s) {
  int64_t n = (int64_t)M * F;
  if (n <= 0) return;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(k_swiglu_fwd<T>, dim3(blocks), dim3(256), 0, s, gu, y, n, F);
}

template <typename T>
__global__ void __launch_bounds__(256) k_swiglu_bwd(const T* dy, const T* gu, T* dgu, int64_t n, int F) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    int64_t m = i / F, j = i % F;
    float g = ldf(gu[m * 2 * F + j]), u = ldf(gu[m * 2 * F + F + j]);
    float e = ldf(dy[i]);
    float sg = sigmoidf_(g);
    float silu = g / (1.0f + expf(-g));
    dgu[m * 2 * F + j] = stf<T>(e * u * (sg * (1.0f + g * (1.0f - sg))));
    dgu[m * 2 * F + F + j] = stf<T>(e * silu);
  }
}

template <typename T>
void swiglu_bwd(const T* dy, const T* gu, T* dgu, int M, int F, hipStream_t s) {
  int64_t n = (int64_t)M * F;
  if (n <= 0) return;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(k_swiglu_bwd<T>, dim3(blocks), dim3(256), 0, s, dy, gu, dgu, n, F);
}

// -------------------------------------------------------- cross-entropy --
template <typename T>
__global__ void __launch_bounds__(256) k_xent(const float* logits, const int32_t* tok, float* row_loss, T* dl, int T_,
                                              int V, float inv_n) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const float* z = logits + m * V;
  T* out = dl + m * V;
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
void xent(const float* logits, const int32_t* tok, float* row_loss, T* dlogits, int M, int T_, int V, float inv_n,
          hipStream_t s) {
  if (M <= 0) return;
  hipLaunchKernelGGL(k_xent<T>, dim3(M), dim3(256), 0, s, logits, tok, row_loss, dlogits, T_, V, inv_n);
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
    if (r0 + r < R && c0 + c < C) out[(c0 + c) * ld_out + r0 + r] = tile[r][c];
  }
}

template <typename T>
void transpose(const T* in, int64_t ld_in, T* out, int64_t ld_out, int R, int C, hipStream_t s) {
  if (R <= 0 || C <= 0) return;
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

__global__ void k_fill_u32(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = v;
}

void fill_u32(void* p, uint32_t value, size_t n_words, hipStream_t s) {
  if (!n_words) return;
  int blocks = (int)std::min<size_t>((n_words + 255) / 256, 65536);
  hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(256), 0, s, (uint32_t*)p, value, n_words);
}

// ------------------------------------------------------ instantiations --
#define MT_INST(T)                                                                                              \
  template void embed_fwd<T>(const int32_t*, const T*, float*, int, int, hipStream_t);                          \
  template void embed_bwd<T>(const float*, const int32_t*, const int32_t*, T*, int, int, hipStream_t);          \
  template void rmsnorm_fwd<T>(const float*, const T*, T*, float*, int, int, float, hipStream_t);               \
  template void rmsnorm_bwd<T>(const float*, const float*, const T*, const float*, const float*, float*, int, int, \
                               hipStream_t);                                                                    \
  template void rmsnorm_dg<T>(const float*, const float*, const float*, float*, T*, int, int, hipStream_t);      \
  template void rope_qkv_fwd<T>(T*, T*, int64_t, const float*, const float*, int, int, int, int, hipStream_t);  \
  template void rope_bwd_T<T>(T*, int64_t, const float*, const float*, int, int, int, int, hipStream_t);        \
  template void swiglu_fwd<T>(const T*, T*, int, int, hipStream_t);                                             \
  template void swiglu_bwd<T>(const T*, const T*, T*, int, int, hipStream_t);                                   \
  template void xent<T>(const float*, const int32_t*, float*, T*, int, int, int, float, hipStream_t);           \
  template void transpose<T>(const T*, int64_t, T*, int64_t, int, int, hipStream_t);                            \
  template void cast_transpose<T>(const float*, T*, T*, int64_t, int, int, hipStream_t);

MT_INST(float)
MT_INST(uint16_t)

}  // namespace mt
