// Causal multi-head attention, forward and backward, flash-style: the
// T x T probability matrix is never stored; the forward keeps the base-2
// log-sum-exp per query and the backward recomputes the probabilities.
//
// The MegaTrain pages do not describe the attention kernels; the method
// only needs the layer's exact forward and backward.  CDNA4 design (bf16
// operands, fp32 accumulation, head_dim 128, v_mfma_f32_32x32x16_bf16):
//
//  * forward: one block = 128 queries of one (batch, head), 4 waves of 32
//    queries.  Each wave computes S^T = K . Q^T, so that a lane owns one
//    query column and the running max / sum stay in the lane (one exchange
//    with the partner half-wave).  O^T = V^T . P^T takes P^T straight from
//    the S^T accumulators as the B operand; V^T comes from the transposed
//    copy qkvT made by the RoPE kernel.  K and V^T tiles of 64 keys are
//    double-buffered in LDS.
//  * backward, two kernels and no atomics (deterministic):
//    dK/dV: one block = 128 keys, query tiles of 64 stream through LDS;
//    S = Q . K^T and dP = dO . V^T have a lane per key, so
//    dV^T += dO^T . P and dK^T += Q^T . dS take P and dS from registers.
//    dQ: one block = 128 queries; S^T = K . Q^T, dP^T = V . dO^T,
//    dQ^T += K^T . dS^T.
//    Gradients are written transposed into dqkvT [3d x M], coalesced.
//
// An MFMA contracts over 16 indices; the A and B operands pair their
// elements by (lane half, element), so any permutation of the contraction
// index that both operands share is exact.  When P (or dS) comes from an
// accumulator, element e of lane-half h holds key (or query) 8*(e/4)+4*h+(e%4)
// of a 16-wide slice; the LDS operand is read with the same mapping (two
// 8-byte reads per fragment).
#include "kernels.h"

namespace mt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Swizzled byte offsets: rows of 256 bytes (16 chunks) and of 128 bytes (8 chunks).
__device__ inline int sw256(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }
__device__ inline int sw128(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ inline f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Row index inside a 32x32 accumulator tile for register r of this lane.
__device__ inline int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// Fragment of a transposed tile (rows of 64 bf16, 128 bytes) for a
// contraction slice starting at column c0 (multiple of 16): two 8-byte reads
// at columns c0 + 4h and c0 + 8 + 4h.
__device__ inline bf16x8_t frag_T(const uint8_t* base, int row, int c0, int lane) {
  const int h = lane >> 5;
  const int ch = c0 >> 3;  // 16-byte chunk of column c0
  bf16x4_t lo = *(const bf16x4_t*)(base + sw128(row, ch) + 8 * h);
  bf16x4_t hi = *(const bf16x4_t*)(base + sw128(row, ch + 1) + 8 * h);
  bf16x8_t f;
  f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
  f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  return f;
}

// Registers 8*ks .. 8*ks+7 of an accumulator tile, as a bf16 B operand.
__device__ inline bf16x8_t acc_to_frag(const f32x16_t& a, int ks) {
  bf16x8_t f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (__bf16)a[8 * ks + e];
  return f;
}

// ------------------------------------------------------------ forward ----
__global__ void __launch_bounds__(256) k_attn_fwd_bf16(const uint16_t* __restrict__ qkv,
                                                     const uint16_t* __restrict__ qkvT, int64_t ldT,
                                                     uint16_t* __restrict__ o, float* __restrict__ lse, int T, int H) {
  constexpr int HD = 128;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 32768];
  const int nqb = (T + 127) / 128;
  const int qb = nqb - 1 - blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int d = H * HD;
  const int64_t ld = 3LL * d;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q0 = qb * 128 + wave * 32;
  const int64_t rowbase = (int64_t)b * T;
  const bool active = q0 < T;
  const float c = kLog2e / sqrtf((float)HD);

  bf16x8_t qf[8];
  if (active) {
    const uint16_t* qp = qkv + (rowbase + q0 + (lane & 31)) * ld + h * HD + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *(const bf16x8_t*)(qp + 16 * s);
  }

  const int nkb = min(T, (qb + 1) * 128) / 64;
  u32x4_t rk[4], rv[4];
  auto gload = [&](int kb) {
    const int key0 = kb * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int kr = id >> 4, kc = id & 15;
      rk[i] = *(const u32x4_t*)(qkv + (rowbase + key0 + kr) * ld + d + h * HD + 8 * kc);
      const int vr = id >> 3, vc = id & 7;
      rv[i] = *(const u32x4_t*)(qkvT + (int64_t)(2 * d + h * HD + vr) * ldT + rowbase + key0 + 8 * vc);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* Ks = smem + buf * 32768;
    uint8_t* Vs = Ks + 16384;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      *(u32x4_t*)(Ks + sw256(id >> 4, id & 15)) = rk[i];
      *(u32x4_t*)(Vs + sw128(id >> 3, id & 7)) = rv[i];
    }
  };

  float m_i = -INFINITY, l_i = 0.f;
  f32x16_t acc_o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc_o[t] = zero16();
  const int tq = q0 + (lane & 31);

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    const uint8_t* Ks = smem + buf * 32768;
    const uint8_t* Vs = Ks + 16384;
    if (active && kb * 64 <= q0 + 31) {
      f32x16_t s_acc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s_acc[kt] = zero16();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          bf16x8_t kf = *(const bf16x8_t*)(Ks + sw256(32 * kt + (lane & 31), 2 * s + (lane >> 5)));
          s_acc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s_acc[kt], 0, 0, 0);
        }
      }
      const bool need_mask = kb * 64 + 63 > q0;
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s_acc[kt][r] * c;
          if (need_mask && kb * 64 + 32 * kt + acc_row(r, lane) > tq) v = -INFINITY;
          s_acc[kt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_i, mx);
      const float alpha = exp2f(m_i - m_new);
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2f(s_acc[kt][r] - m_new);
          s_acc[kt][r] = p;
          rs += p;
        }
      rs += __shfl_xor(rs, 32);
      l_i = l_i * alpha + rs;
      m_i = m_new;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[t][r] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t pf = acc_to_frag(s_acc[ks >> 1], ks & 1);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          const bf16x8_t vf = frag_T(Vs, 32 * ht + (lane & 31), 16 * ks, lane);
          acc_o[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc_o[ht], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < nkb) sstore(buf ^ 1);
    __syncthreads();
  }

  // O^T accumulators -> LDS [query][hd] -> coalesced rows of o.
  uint16_t* Os = (uint16_t*)(smem + wave * 8192);
  if (active) {
    const float inv_l = 1.0f / l_i;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int r = 0; r < 16; ++r) Os[(lane & 31) * HD + 32 * ht + acc_row(r, lane)] = f32_to_bf16(acc_o[ht][r] * inv_l);
    if (lane < 32) lse[(int64_t)bh * T + tq] = m_i + log2f(l_i);
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = lane + 64 * i;
      const int r = id >> 4, ch = id & 15;
      *(u32x4_t*)(o + (rowbase + q0 + r) * d + h * HD + 8 * ch) = *(const u32x4_t*)(Os + r * HD + 8 * ch);
    }
  }
}

// ------------------------------------------------------------ D = dO.O --
template <typename T>
__device__ inline float ldf(T x);
template <>
__device__ inline float ldf<float>(float x) { return x; }
template <>
__device__ inline float ldf<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

template <typename T>
__global__ void __launch_bounds__(256) k_dsum(const T* dO, const T* O, float* Dsum, int T_, int H, int hd, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // row = m*H + h
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t m = row / H;
  const int h = (int)(row % H);
  const int64_t base = m * (int64_t)H * hd + (int64_t)h * hd;
  float acc = 0.f;
  for (int i = lane; i < hd; i += 64) acc += ldf(dO[base + i]) * ldf(O[base + i]);
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) {
    const int64_t b = m / T_, t = m % T_;
    Dsum[(b * H + h) * T_ + t] = acc;
  }
}

// ------------------------------------------------------- backward dK dV --
__global__ void __launch_bounds__(256) k_attn_dkdv_bf16(const uint16_t* __restrict__ qkv,
                                                      const uint16_t* __restrict__ qkvT,
                                                      const uint16_t* __restrict__ dO,
                                                      const uint16_t* __restrict__ dOT, const float* __restrict__ lse,
                                                      const float* __restrict__ Dsum, uint16_t* __restrict__ dqkvT,
                                                      int64_t ldT, int T, int H) {
  constexpr int HD = 128;
  // K, V: [128 keys][128 hd]; per query tile: Q, dO [64][128]; Q^T, dO^T [128][64]; lse, D [64].
  __shared__ __attribute__((aligned(16))) uint8_t smem[32768 * 2 + 16384 * 4 + 512];
  uint8_t* Ks = smem;
  uint8_t* Vs = smem + 32768;
  uint8_t* Qs = smem + 65536;
  uint8_t* dOs = Qs + 16384;
  uint8_t* QTs = dOs + 16384;
  uint8_t* dOTs = QTs + 16384;
  float* lse_s = (float*)(dOTs + 16384);
  float* D_s = lse_s + 64;

  const int kblk = blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int d = H * HD;
  const int64_t ld = 3LL * d;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t rowbase = (int64_t)b * T;
  const int kbase = kblk * 128;
  const int k0 = kbase + wave * 32;
  const bool active = k0 < T;
  const float c = kLog2e / sqrtf((float)HD);
  const float scale = 1.0f / sqrtf((float)HD);

  // K and V rows of the block's 128 keys (rows past T are never used).
  for (int i = 0; i < 8; ++i) {
    const int id = tid + 256 * i;
    const int r = id >> 4, ch = id & 15;
    u32x4_t kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (kbase + r < T) {
      kv = *(const u32x4_t*)(qkv + (rowbase + kbase + r) * ld + d + h * HD + 8 * ch);
      vv = *(const u32x4_t*)(qkv + (rowbase + kbase + r) * ld + 2 * d + h * HD + 8 * ch);
    }
    *(u32x4_t*)(Ks + sw256(r, ch)) = kv;
    *(u32x4_t*)(Vs + sw256(r, ch)) = vv;
  }

  f32x16_t acc_dk[4], acc_dv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc_dk[t] = zero16();
    acc_dv[t] = zero16();
  }
  const int key = k0 + (lane & 31);

  for (int qblk = kbase / 64; qblk < T / 64; ++qblk) {
    const int qs0 = qblk * 64;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int r = id >> 4, ch = id & 15;
      *(u32x4_t*)(Qs + sw256(r, ch)) = *(const u32x4_t*)(qkv + (rowbase + qs0 + r) * ld + h * HD + 8 * ch);
      *(u32x4_t*)(dOs + sw256(r, ch)) = *(const u32x4_t*)(dO + (rowbase + qs0 + r) * d + h * HD + 8 * ch);
      const int tr = id >> 3, tc = id & 7;
      *(u32x4_t*)(QTs + sw128(tr, tc)) =
          *(const u32x4_t*)(qkvT + (int64_t)(h * HD + tr) * ldT + rowbase + qs0 + 8 * tc);
      *(u32x4_t*)(dOTs + sw128(tr, tc)) =
          *(const u32x4_t*)(dOT + (int64_t)(h * HD + tr) * ldT + rowbase + qs0 + 8 * tc);
    }
    if (tid < 64) {
      lse_s[tid] = lse[(int64_t)bh * T + qs0 + tid];
      D_s[tid] = Dsum[(int64_t)bh * T + qs0 + tid];
    }
    __syncthreads();
    if (!active) continue;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int qbase = qs0 + 32 * qs;
      if (k0 > qbase + 31) continue;  // every key of the wave is after every query
      f32x16_t s_acc = zero16(), dp_acc = zero16();
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int ch = 2 * s + (lane >> 5);
        const bf16x8_t qf = *(const bf16x8_t*)(Qs + sw256(32 * qs + (lane & 31), ch));
        const bf16x8_t kf = *(const bf16x8_t*)(Ks + sw256(32 * wave + (lane & 31), ch));
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf, s_acc, 0, 0, 0);
        const bf16x8_t of = *(const bf16x8_t*)(dOs + sw256(32 * qs + (lane & 31), ch));
        const bf16x8_t vf = *(const bf16x8_t*)(Vs + sw256(32 * wave + (lane & 31), ch));
        dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(of, vf, dp_acc, 0, 0, 0);
      }
      // rows = queries, column = this lane's key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 32 * qs + acc_row(r, lane);
        const float p = (key <= qs0 + qi) ? exp2f(s_acc[r] * c - lse_s[qi]) : 0.f;
        s_acc[r] = p;
        dp_acc[r] = p * (dp_acc[r] - D_s[qi]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t pf = acc_to_frag(s_acc, ks);
        const bf16x8_t dsf = acc_to_frag(dp_acc, ks);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          const bf16x8_t oT = frag_T(dOTs, 32 * ht + (lane & 31), 32 * qs + 16 * ks, lane);
          acc_dv[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oT, pf, acc_dv[ht], 0, 0, 0);
          const bf16x8_t qT = frag_T(QTs, 32 * ht + (lane & 31), 32 * qs + 16 * ks, lane);
          acc_dk[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qT, dsf, acc_dk[ht], 0, 0, 0);
        }
      }
    }
  }
  if (!active) return;
  // dK^T, dV^T: lane = key column, registers = hd rows.
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hi = 32 * ht + acc_row(r, lane);
      dqkvT[(int64_t)(d + h * HD + hi) * ldT + rowbase + key] = f32_to_bf16(acc_dk[ht][r] * scale);
      dqkvT[(int64_t)(2 * d + h * HD + hi) * ldT + rowbase + key] = f32_to_bf16(acc_dv[ht][r]);
    }
}

// ----------------------------------------------------------- backward dQ --
__global__ void __launch_bounds__(256) k_attn_dq_bf16(const uint16_t* __restrict__ qkv,
                                                    const uint16_t* __restrict__ qkvT, const uint16_t* __restrict__ dO,
                                                    const float* __restrict__ lse, const float* __restrict__ Dsum,
                                                    uint16_t* __restrict__ dqkvT, int64_t ldT, int T, int H) {
  constexpr int HD = 128;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 49152];  // K, V [64][128], K^T [128][64]
  const int nqb = (T + 127) / 128;
  const int qb = nqb - 1 - blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int d = H * HD;
  const int64_t ld = 3LL * d;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q0 = qb * 128 + wave * 32;
  const int64_t rowbase = (int64_t)b * T;
  const bool active = q0 < T;
  const float c = kLog2e / sqrtf((float)HD);
  const float scale = 1.0f / sqrtf((float)HD);
  const int tq = q0 + (lane & 31);

  bf16x8_t qf[8], of[8];
  float lse_q = 0.f, D_q = 0.f;
  if (active) {
    const uint16_t* qp = qkv + (rowbase + tq) * ld + h * HD + 8 * (lane >> 5);
    const uint16_t* op = dO + (rowbase + tq) * d + h * HD + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[s] = *(const bf16x8_t*)(qp + 16 * s);
      of[s] = *(const bf16x8_t*)(op + 16 * s);
    }
    lse_q = lse[(int64_t)bh * T + tq];
    D_q = Dsum[(int64_t)bh * T + tq];
  }

  const int nkb = min(T, (qb + 1) * 128) / 64;
  u32x4_t rk[4], rv[4], rt[4];
  auto gload = [&](int kb) {
    const int key0 = kb * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int r = id >> 4, ch = id & 15;
      rk[i] = *(const u32x4_t*)(qkv + (rowbase + key0 + r) * ld + d + h * HD + 8 * ch);
      rv[i] = *(const u32x4_t*)(qkv + (rowbase + key0 + r) * ld + 2 * d + h * HD + 8 * ch);
      const int tr = id >> 3, tc = id & 7;
      rt[i] = *(const u32x4_t*)(qkvT + (int64_t)(d + h * HD + tr) * ldT + rowbase + key0 + 8 * tc);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* Ks = smem + buf * 49152;
    uint8_t* Vs = Ks + 16384;
    uint8_t* KTs = Vs + 16384;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      *(u32x4_t*)(Ks + sw256(id >> 4, id & 15)) = rk[i];
      *(u32x4_t*)(Vs + sw256(id >> 4, id & 15)) = rv[i];
      *(u32x4_t*)(KTs + sw128(id >> 3, id & 7)) = rt[i];
    }
  };

  f32x16_t acc_dq[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc_dq[t] = zero16();

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    const uint8_t* Ks = smem + buf * 49152;
    const uint8_t* Vs = Ks + 16384;
    const uint8_t* KTs = Vs + 16384;
    if (active) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int kstart = kb * 64 + 32 * kt;
        if (kstart > q0 + 31) continue;
        f32x16_t s_acc = zero16(), dp_acc = zero16();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int ch = 2 * s + (lane >> 5);
          const bf16x8_t kf = *(const bf16x8_t*)(Ks + sw256(32 * kt + (lane & 31), ch));
          s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s_acc, 0, 0, 0);
          const bf16x8_t vf = *(const bf16x8_t*)(Vs + sw256(32 * kt + (lane & 31), ch));
          dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, of[s], dp_acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kstart + acc_row(r, lane);
          const float p = (key <= tq) ? exp2f(s_acc[r] * c - lse_q) : 0.f;
          dp_acc[r] = p * (dp_acc[r] - D_q);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8_t dsf = acc_to_frag(dp_acc, ks);
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) {
            const bf16x8_t kT = frag_T(KTs, 32 * ht + (lane & 31), 32 * kt + 16 * ks, lane);
            acc_dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kT, dsf, acc_dq[ht], 0, 0, 0);
          }
        }
      }
    }
    if (kb + 1 < nkb) sstore(buf ^ 1);
    __syncthreads();
  }
  if (!active) return;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hi = 32 * ht + acc_row(r, lane);
      dqkvT[(int64_t)(h * HD + hi) * ldT + rowbase + tq] = f32_to_bf16(acc_dq[ht][r] * scale);
    }
}

// ----------------------------------------------------- fp32 SIMT kernels --
// One thread per query (forward, dQ) or per key (dK, dV); head_dim <= 64.
constexpr int kMaxHd = 64;

__global__ void __launch_bounds__(64) k_attn_fwd_f32(const float* qkv, float* o, float* lse, int T, int H, int hd) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  if (t >= T) return;
  const int d = H * hd;
  const int64_t ld = 3LL * d;
  const int64_t rowbase = (int64_t)b * T;
  const float c = kLog2e / sqrtf((float)hd);
  const float* q = qkv + (rowbase + t) * ld + h * hd;
  float acc[kMaxHd];
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int u = 0; u <= t; ++u) {
    const float* k = qkv + (rowbase + u) * ld + d + h * hd;
    const float* v = k + d;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxHd; ++i)
      if (i < hd) s += q[i] * k[i];
    s *= c;
    const float mn = fmaxf(m, s);
    const float alpha = exp2f(m - mn), p = exp2f(s - mn);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < kMaxHd; ++i)
      if (i < hd) acc[i] = acc[i] * alpha + p * v[i];
    m = mn;
  }
  float* op = o + (rowbase + t) * d + h * hd;
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i)
    if (i < hd) op[i] = acc[i] / l;
  lse[(int64_t)bh * T + t] = m + log2f(l);
}

__global__ void __launch_bounds__(64) k_attn_dq_f32(const float* qkv, const float* dO, const float* lse,
                                                   const float* Dsum, float* dqkvT, int64_t ldT, int T, int H, int hd) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  if (t >= T) return;
  const int d = H * hd;
  const int64_t ld = 3LL * d;
  const int64_t rowbase = (int64_t)b * T;
  const float c = kLog2e / sqrtf((float)hd), scale = 1.0f / sqrtf((float)hd);
  const float* q = qkv + (rowbase + t) * ld + h * hd;
  const float* go = dO + (rowbase + t) * d + h * hd;
  const float L = lse[(int64_t)bh * T + t], D = Dsum[(int64_t)bh * T + t];
  float acc[kMaxHd];
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) acc[i] = 0.f;
  for (int u = 0; u <= t; ++u) {
    const float* k = qkv + (rowbase + u) * ld + d + h * hd;
    const float* v = k + d;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxHd; ++i)
      if (i < hd) {
        s += q[i] * k[i];
        dp += go[i] * v[i];
      }
    const float p = exp2f(s * c - L);
    const float ds = p * (dp - D);
#pragma unroll
    for (int i = 0; i < kMaxHd; ++i)
      if (i < hd) acc[i] += ds * k[i];
  }
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i)
    if (i < hd) dqkvT[(int64_t)(h * hd + i) * ldT + rowbase + t] = acc[i] * scale;
}

__global__ void __launch_bounds__(64) k_attn_dkdv_f32(const float* qkv, const float* dO, const float* lse,
                                                     const float* Dsum, float* dqkvT, int64_t ldT, int T, int H,
                                                     int hd) {
  const int u = blockIdx.x * 64 + threadIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  if (u >= T) return;
  const int d = H * hd;
  const int64_t ld = 3LL * d;
  const int64_t rowbase = (int64_t)b * T;
  const float c = kLog2e / sqrtf((float)hd), scale = 1.0f / sqrtf((float)hd);
  const float* k = qkv + (rowbase + u) * ld + d + h * hd;
  const float* v = k + d;
  float dk[kMaxHd], dv[kMaxHd];
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) dk[i] = dv[i] = 0.f;
  for (int t = u; t < T; ++t) {
    const float* q = qkv + (rowbase + t) * ld + h * hd;
    const float* go = dO + (rowbase + t) * d + h * hd;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxHd; ++i)
      if (i < hd) {
        s += q[i] * k[i];
        dp += go[i] * v[i];
      }
    const float p = exp2f(s * c - lse[(int64_t)bh * T + t]);
    const float ds = p * (dp - Dsum[(int64_t)bh * T + t]);
#pragma unroll
    for (int i = 0; i < kMaxHd; ++i)
      if (i < hd) {
        dv[i] += p * go[i];
        dk[i] += ds * q[i];
      }
  }
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i)
    if (i < hd) {
      dqkvT[(int64_t)(d + h * hd + i) * ldT + rowbase + u] = dk[i] * scale;
      dqkvT[(int64_t)(2 * d + h * hd + i) * ldT + rowbase + u] = dv[i];
    }
}

}  // namespace

template <>
void attn_fwd<uint16_t>(const uint16_t* qkv, const uint16_t* qkvT, int64_t ldT, uint16_t* o, float* lse, int B,
                        int T_, int H, int hd, hipStream_t s) {
  if (hd != 128 || T_ % 64) throw ApiError{MT_E_INVALID, "bf16 attention needs head_dim 128, seq_len % 64 == 0"};
  if (ldT < (int64_t)B * T_ || ldT % 8) throw ApiError{MT_E_INVALID, "ldT must be >= batch*seq_len, multiple of 8"};
  hipLaunchKernelGGL(k_attn_fwd_bf16, dim3((T_ + 127) / 128, B * H), dim3(256), 0, s, qkv, qkvT, ldT, o, lse, T_, H);
}

template <>
void attn_fwd<float>(const float* qkv, const float*, int64_t, float* o, float* lse, int B, int T_, int H, int hd,
                     hipStream_t s) {
  if (hd > kMaxHd) throw ApiError{MT_E_INVALID, "fp32 attention needs head_dim <= 64"};
  hipLaunchKernelGGL(k_attn_fwd_f32, dim3((T_ + 63) / 64, B * H), dim3(64), 0, s, qkv, o, lse, T_, H, hd);
}

template <typename T>
void attn_bwd_dsum(const T* dO, const T* O, float* Dsum, int B, int T_, int H, int hd, hipStream_t s) {
  const int64_t rows = (int64_t)B * T_ * H;
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_dsum<T>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, dO, O, Dsum, T_, H, hd, rows);
}
template void attn_bwd_dsum<float>(const float*, const float*, float*, int, int, int, int, hipStream_t);
template void attn_bwd_dsum<uint16_t>(const uint16_t*, const uint16_t*, float*, int, int, int, int, hipStream_t);

template <>
void attn_bwd<uint16_t>(const uint16_t* qkv, const uint16_t* qkvT, const uint16_t* dO, const uint16_t* dOT,
                        int64_t ldT, const float* lse, const float* Dsum, uint16_t* dqkvT, int B, int T_, int H,
                        int hd, hipStream_t s) {
  if (hd != 128 || T_ % 64) throw ApiError{MT_E_INVALID, "bf16 attention needs head_dim 128, seq_len % 64 == 0"};
  if (ldT < (int64_t)B * T_ || ldT % 8) throw ApiError{MT_E_INVALID, "ldT must be >= batch*seq_len, multiple of 8"};
  hipLaunchKernelGGL(k_attn_dkdv_bf16, dim3((T_ + 127) / 128, B * H), dim3(256), 0, s, qkv, qkvT, dO, dOT, lse, Dsum,
                     dqkvT, ldT, T_, H);
  hipLaunchKernelGGL(k_attn_dq_bf16, dim3((T_ + 127) / 128, B * H), dim3(256), 0, s, qkv, qkvT, dO, lse, Dsum, dqkvT,
                     ldT, T_, H);
}

template <>
void attn_bwd<float>(const float* qkv, const float*, const float* dO, const float*, int64_t ldT, const float* lse,
                     const float* Dsum, float* dqkvT, int B, int T_, int H, int hd, hipStream_t s) {
  if (hd > kMaxHd) throw ApiError{MT_E_INVALID, "fp32 attention needs head_dim <= 64"};
  if (ldT < (int64_t)B * T_) throw ApiError{MT_E_INVALID, "ldT must be >= batch*seq_len"};
  hipLaunchKernelGGL(k_attn_dkdv_f32, dim3((T_ + 63) / 64, B * H), dim3(64), 0, s, qkv, dO, lse, Dsum, dqkvT, ldT, T_,
                     H, hd);
  hipLaunchKernelGGL(k_attn_dq_f32, dim3((T_ + 63) / 64, B * H), dim3(64), 0, s, qkv, dO, lse, Dsum, dqkvT, ldT, T_, H,
                     hd);
}

}  // namespace mt
