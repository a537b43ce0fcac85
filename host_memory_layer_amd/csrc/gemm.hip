// Dense contractions of the decoder layer: C = A . B^T with both operands
// contiguous along the contraction dimension.
//
// Every projection of the layer (QKV, O, gate/up, down, head) in forward,
// data-gradient and weight-gradient form reduces to this one shape once the
// operand that is not contraction-contiguous has been transposed.  The pages
// (MegaTrain) describe no compute kernel; this is the CDNA4 design.
//
// bf16, K a multiple of 64 (every contraction of the step): k_gemm_bf16_nt.
//  * 256x256 macro tile, K steps of 64, 4 waves (2 x 2), one per SIMD; each
//    wave owns 128x128 as 4x4 accumulators of v_mfma_f32_32x32x16_bf16.
//  * Operands move global -> LDS with buffer loads that write LDS directly
//    (16 bytes per lane, no register staging); the buffer descriptors hold
//    the number of valid rows, so rows past M or N read as zero.
//  * A tile row is 64 bf16 = 128 bytes, so every global request covers
//    whole cache lines.  Chunk c of row r is stored at c ^ ((r >> 1) & 7):
//    the 16 lanes a 16-byte LDS read serves per cycle (16 consecutive rows,
//    one logical chunk) fall on 16 disjoint bank groups.
//  * Two LDS stages of 64 KiB.  A K step is four sub-steps of 16 MFMAs with
//    the next sub-step's fragment reads interleaved.  The A tile of step
//    k+2 is loaded during sub-step 3 of step k (its stage was freed by step
//    k's barrier), the B tile of step k+1 during sub-step 0 of step k.  One
//    barrier per step, after sub-step 2, once step k+1 has landed.
//  * The first and last two steps are peeled, so the steady-state step has
//    no branch; the wave index is made uniform so that every LDS
//    destination address is a scalar.
//  * Tile order: groups of 8 tile-rows for L2 reuse; consecutive workgroup
//    ids, which the dispatcher deals round-robin to the 8 XCDs, are remapped
//    so that each XCD works through a contiguous range of tiles.
// bf16 with other K (small test shapes): k_gemm_bf16_generic, register-staged.
// fp32 (all-fp32 store): 64x64 SIMT tile with LDS staging.
//
// Accumulation is fp32 in a fixed order, so results depend only on shapes.
#include <type_traits>

#include "kernels.h"

namespace mt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

namespace {

// ------------------------------------------------------------- generic --
// 256x256x64 macro tile, 8 waves (2 x 4), each 128x64 as 4x2 accumulators;
// operands staged through registers into double-buffered LDS.
constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 512;
constexpr int TILE_BYTES = BM * BK * 2;  // one operand tile: 32 KiB

__device__ inline int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int EPI>
__global__ void __launch_bounds__(NTHREADS) k_gemm_bf16_generic(const uint16_t* __restrict__ A, int64_t lda,
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

// ------------------------------------------------------------------ nt --
constexpr int STAGE = 2 * BM * BK * 2;  // A and B tiles of one K step: 64 KiB

__device__ inline int swz128(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

template <bool V>
using Flag = std::integral_constant<bool, V>;

template <int EPI>
__global__ void __launch_bounds__(256, 1) k_gemm_bf16_nt(const uint16_t* __restrict__ A, int64_t lda,
                                                       const uint16_t* __restrict__ B, int64_t ldb, void* C,
                                                       int64_t ldc, const float* R, int64_t ldr, int M, int N, int K,
                                                       int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  const int ntiles = tiles_m * tiles_n;
  int pid = blockIdx.x;
  const int per_xcd = ntiles / 8;
  if (pid < per_xcd * 8) pid = (pid % 8) * per_xcd + pid / 8;
  const int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int g = pid / group_size;
  const int first_m = g * GROUP;
  const int gm_cnt = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (pid % group_size) % gm_cnt;
  const int tn = (pid % group_size) / gm_cnt;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int arows = (int)min<int64_t>(BM, M - m0), brows = (int)min<int64_t>(BN, N - n0);
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * lda), 0, (int)(arows * lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t brsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(B + n0 * ldb), 0, (int)(brows * ldb * 2), 0x00020000);
  const int nk = K / BK;

  // Direct load i (0..7) of an operand tile: kilobyte j = wave*8 + i, rows
  // 8j .. 8j+7; lane l reads row 8j + l/8, logical chunk (l%8) ^ ((row>>1)&7),
  // which lands at physical chunk l%8 of that row.
  int aoff[8], boff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (wave * 8 + i) + (lane >> 3);
    const int lc = (lane & 7) ^ ((r >> 1) & 7);
    aoff[i] = (int)((r * lda + 8 * lc) * 2);
    boff[i] = (int)((r * ldb + 8 * lc) * 2);
  }
  auto load_a = [&](int kt, int i) {
    uint8_t* dst = smem + (kt & 1) * STAGE + (wave * 8 + i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_void_t*)dst, 16, aoff[i], kt * BK * 2, 0, 0);
  };
  auto load_b = [&](int kt, int i) {
    uint8_t* dst = smem + (kt & 1) * STAGE + STAGE / 2 + (wave * 8 + i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, (lds_void_t*)dst, 16, boff[i], kt * BK * 2, 0, 0);
  };

  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8_t a[2][4], b[2][4];
  // Fragment q (0..7) of a sub-step, in the order the next sub-step's MFMAs
  // first use them: a0, b0..b3, a1..a3.
  auto read_one = [&](int kt, int ks, int set, int q) {
    const uint8_t* As = smem + (kt & 1) * STAGE;
    const uint8_t* Bs = As + STAGE / 2;
    const int c = ks * 2 + (lane >> 5);
    if (q == 0 || q > 4) {
      const int i = q == 0 ? 0 : q - 4;
      a[set][i] = *(const bf16x8_t*)(As + swz128(wm + 32 * i + (lane & 31), c));
    } else {
      b[set][q - 1] = *(const bf16x8_t*)(Bs + swz128(wn + 32 * (q - 1) + (lane & 31), c));
    }
  };
  auto mfma16 = [&](int set, int p) {
    const int i = p >> 2, j = p & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[set][i], b[set][j], acc[i][j], 0, 0, 0);
  };

  // One K step.  LOAD_B: load B of step kt+1 during sub-step 0; LOAD_A2:
  // load A of step kt+2 during sub-step 3; NEXT: read step kt+1's first
  // fragments during sub-step 3.
  auto step = [&](int kt, auto load_b_next, auto load_a_next2, auto next) {
    constexpr bool LOAD_B = decltype(load_b_next)::value;
    constexpr bool LOAD_A2 = decltype(load_a_next2)::value;
    constexpr bool NEXT = decltype(next)::value;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      mfma16(0, p);
      if (p & 1)
        read_one(kt, 1, 1, p >> 1);
      else if (LOAD_B)
        load_b(kt + 1, p >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      mfma16(1, p);
      if (p & 1) read_one(kt, 2, 0, p >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      mfma16(0, p);
      if (p & 1) read_one(kt, 3, 1, p >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Every load in flight belongs to step kt+1, which sub-step 3 starts
    // reading; the barrier also frees step kt's stage for step kt+2.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      mfma16(1, p);
      if (NEXT && (p & 1)) read_one(kt + 1, 0, 0, p >> 1);
      if (LOAD_A2 && !(p & 1)) load_a(kt + 2, p >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: steps 0 and 1 in full.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    load_a(0, i);
    load_b(0, i);
  }
  if (nk > 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      load_a(1, i);
      load_b(1, i);
    }
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) read_one(0, 0, 0, i);

  if (nk == 1) {
    step(0, Flag<false>{}, Flag<false>{}, Flag<false>{});
  } else {
    // step 0: step 1 is already loaded
    if (nk == 2)
      step(0, Flag<false>{}, Flag<false>{}, Flag<true>{});
    else
      step(0, Flag<false>{}, Flag<true>{}, Flag<true>{});
    for (int kt = 1; kt + 2 < nk; ++kt) step(kt, Flag<true>{}, Flag<true>{}, Flag<true>{});
    if (nk >= 3) step(nk - 2, Flag<true>{}, Flag<false>{}, Flag<true>{});
    step(nk - 1, Flag<false>{}, Flag<false>{}, Flag<false>{});
  }

  // Accumulator layout of a 32x32 MFMA tile: lane holds column (lane & 31);
  // register r holds row 8*(r/4) + 4*(lane/32) + (r%4).
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
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
  const dim3 grid(tiles_m * tiles_n);
  if (K % BK == 0 && K > 0) {
    // buffer offsets are 32-bit: one operand panel of 256 rows must fit
    if ((int64_t)BM * lda * 2 >= (int64_t)1 << 31 || (int64_t)BN * ldb * 2 >= (int64_t)1 << 31)
      throw ApiError{MT_E_INVALID, "bf16 GEMM row stride too large"};
#define L_(E) \
  hipLaunchKernelGGL((k_gemm_bf16_nt<E>), grid, dim3(256), 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, tiles_m, tiles_n)
    switch (epi) {
      case EPI_STORE: L_(EPI_STORE); break;
      case EPI_F32: L_(EPI_F32); break;
      case EPI_ADD_F32: L_(EPI_ADD_F32); break;
    }
#undef L_
    return;
  }
#define L_(E)                                                                                                      \
  hipLaunchKernelGGL(k_gemm_bf16_generic<E>, grid, dim3(NTHREADS), 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, \
                     tiles_m, tiles_n)
  switch (epi) {
    case EPI_STORE: L_(EPI_STORE); break;
    case EPI_F32: L_(EPI_F32); break;
    case EPI_ADD_F32: L_(EPI_ADD_F32); break;
  }
#undef L_
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
