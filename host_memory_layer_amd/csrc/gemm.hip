// Dense contractions of the decoder layer: C = A . B^T with both operands
// contiguous along the contraction dimension.
//
// Every projection of the layer (QKV, O, gate/up, down, head) in forward,
// data-gradient and weight-gradient form reduces to this one shape once the
// operand that is not contraction-contiguous has been transposed.  The pages
// (MegaTrain) describe no compute kernel; this is the CDNA4 design:
//
//  * bf16: 256x256x64 macro tile, 8 waves (2 x 4), each wave owning a
//    128x64 sub-tile as 4x2 accumulators of v_mfma_f32_32x32x16_bf16;
//    operands staged through double-buffered LDS (128 KiB) with an XOR
//    swizzle of the 16-byte chunks so that fragment reads are conflict-free;
//    global loads for tile k+1 are issued before the MFMAs of tile k.
//  * fp32 (all-fp32 store): 64x64 SIMT tile with LDS staging.
//
// Accumulation is fp32 in a fixed order, so results depend only on shapes.
#include "kernels.h"

namespace mt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 512;
constexpr int TILE_BYTES = BM * BK * 2;  // one operand tile: 32 KiB

__device__ inline int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int EPI>
__global__ void __launch_bounds__(NTHREADS) k_gemm_bf16(const uint16_t* __restrict__ A, int64_t lda,
                                                      const uint16_t* __restrict__ B, int64_t ldb, void* C,
                                                      int64_t ldc, const float* R, int64_t ldr, int M, int N, int K,
                                                      int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * TILE_BYTES];

  // Grouped tile order: 8 tile-rows share their B tiles while they are hot in L2.
  const int pid = blockIdx.x;
  const int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int g = pid / group_size;
  const int first_m = g * GROUP;
  const int gm_cnt = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (pid % group_size) % gm_cnt;
  const int tn = (pid % group_size) / gm_cnt;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x;
  u32x4_t ra[4], rb[4];

  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + NTHREADS * i;
      const int row = id >> 3, c = id & 7;
      const int gk = k0 + c * 8;
      const int64_t gm = m0 + row, gn = n0 + row;
      u32x4_t z = {0u, 0u, 0u, 0u};
      ra[i] = (gm < M && gk < K) ? *(const u32x4_t*)(A + gm * lda + gk) : z;
      rb[i] = (gn < N && gk < K) ? *(const u32x4_t*)(B + gn * ldb + gk) : z;
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* As = smem + buf * 2 * TILE_BYTES;
    uint8_t* Bs = As + TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + NTHREADS * i;
      const int row = id >> 3, c = id & 7;
      *(u32x4_t*)(As + swz(row, c)) = ra[i];
      *(u32x4_t*)(Bs + swz(row, c)) = rb[i];
    }
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = (wave >> 2) * 128;
  const int wn = (wave & 3) * 64;
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* As = smem + buf * 2 * TILE_BYTES;
    const uint8_t* Bs = As + TILE_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      bf16x8_t a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm + 32 * i + (lane & 31);
        a[i] = *(const bf16x8_t*)(As + swz(row, c));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn + 32 * j + (lane & 31);
        b[j] = *(const bf16x8_t*)(Bs + swz(row, c));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Accumulator layout of a 32x32 MFMA tile: lane holds column (lane & 31);
  // register r holds row 8*(r/4) + 4*(lane/32) + (r%4).
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int64_t gm = m0 + wm + 32 * i + row;
        const int64_t gn = n0 + wn + 32 * j + (lane & 31);
        if (gm < M && gn < N) {
          const float v = acc[i][j][r];
          if (EPI == EPI_STORE)
            ((uint16_t*)C)[gm * ldc + gn] = f32_to_bf16(v);
          else if (EPI == EPI_F32)
            ((float*)C)[gm * ldc + gn] = v;
          else
            ((float*)C)[gm * ldc + gn] = R[gm * ldr + gn] + v;
        }
      }
}

// fp32 SIMT GEMM for the all-fp32 store: 64x64 tile, 4x4 per thread.
template <int EPI>
__global__ void __launch_bounds__(256) k_gemm_f32(const float* __restrict__ A, int64_t lda, const float* __restrict__ B,
                                                  int64_t ldb, void* C, int64_t ldc, const float* R, int64_t ldr, int M,
                                                  int N, int K) {
  __shared__ float As[16][68], Bs[16][68];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, row = id / 16, k = id % 16;
      As[k][row] = (m0 + row < M && k0 + k < K) ? A[(m0 + row) * lda + k0 + k] : 0.f;
      Bs[k][row] = (n0 + row < N && k0 + k < K) ? B[(n0 + row) * ldb + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += As[k][ty * 4 + a] * Bs[k][tx * 4 + b];
    __syncthreads();
  }
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b) {
      const int64_t gm = m0 + ty * 4 + a, gn = n0 + tx * 4 + b;
      if (gm < M && gn < N) {
        if (EPI == EPI_ADD_F32)
          ((float*)C)[gm * ldc + gn] = R[gm * ldr + gn] + acc[a][b];
        else
          ((float*)C)[gm * ldc + gn] = acc[a][b];
      }
    }
}

}  // namespace

template <>
void gemm_nt<uint16_t>(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, void* C, int64_t ldc,
                       const float* R, int64_t ldr, int M, int N, int K, Epi epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  if (K % 8 || lda % 8 || ldb % 8 || ((uintptr_t)A & 15) || ((uintptr_t)B & 15))
    throw ApiError{MT_E_INVALID, "bf16 GEMM needs K, lda, ldb multiples of 8 and 16-byte aligned operands"};
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n), block(NTHREADS);
  switch (epi) {
    case EPI_STORE:
      hipLaunchKernelGGL(k_gemm_bf16<EPI_STORE>, grid, block, 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, tiles_m,
                         tiles_n);
      break;
    case EPI_F32:
      hipLaunchKernelGGL(k_gemm_bf16<EPI_F32>, grid, block, 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, tiles_m,
                         tiles_n);
      break;
    case EPI_ADD_F32:
      hipLaunchKernelGGL(k_gemm_bf16<EPI_ADD_F32>, grid, block, 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K,
                         tiles_m, tiles_n);
      break;
  }
}

template <>
void gemm_nt<float>(const float* A, int64_t lda, const float* B, int64_t ldb, void* C, int64_t ldc, const float* R,
                    int64_t ldr, int M, int N, int K, Epi epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  const dim3 grid((N + 63) / 64, (M + 63) / 64), block(256);
  if (epi == EPI_ADD_F32)
    hipLaunchKernelGGL(k_gemm_f32<EPI_ADD_F32>, grid, block, 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K);
  else
    hipLaunchKernelGGL(k_gemm_f32<EPI_STORE>, grid, block, 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K);
}

}  // namespace mt
