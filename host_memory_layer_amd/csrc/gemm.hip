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
#include <cstdlib>

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

// ------------------------------------------------------------------ v2 --
// 256x256x64 macro tile, 4 waves (2 x 2) each owning 128x128 as 4x4
// accumulators of v_mfma_f32_32x32x16_bf16 (256 fp32 per lane, held in
// AGPRs).  Operands move global -> LDS with global_load_lds_dwordx4 (no
// register staging): each lane's 16-byte source is chosen so that the
// contiguous kilobyte a wave writes lands in the XOR-swizzled layout the
// fragment reads expect.  Double-buffered LDS, one barrier per K step; the
// loads of step k+1 are issued right after the fragments of step k are read.
// Rows past M or N are clamped to the last valid row (their products only
// reach outputs that are never stored); K must be a multiple of 64.
typedef __attribute__((address_space(3))) void lds_void_t;

template <int EPI>
__global__ void __launch_bounds__(256, 1) k_gemm_bf16_v2(const uint16_t* __restrict__ A, int64_t lda,
                                                       const uint16_t* __restrict__ B, int64_t ldb, void* C,
                                                       int64_t ldc, const float* R, int64_t ldr, int M, int N, int K,
                                                       int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE_BYTES];
  const int ntiles = tiles_m * tiles_n;
  int pid = blockIdx.x;
  // Workgroup i runs on XCD i % 8: give each XCD a contiguous run of the
  // grouped tile order so that tiles sharing A rows or B rows share an L2.
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

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // Direct-load sources: kilobyte (wave*8 + i) of a tile holds rows
  // wave*64 + i*8 + lane/8, physical chunk lane%8 = logical chunk ^ (row & 7).
  const int lchunk = (lane & 7) ^ (lane >> 3);
  const int64_t ar0 = m0 + wave * 64 + (lane >> 3), br0 = n0 + wave * 64 + (lane >> 3);
  const uint16_t* abase = A + 8 * lchunk;
  const uint16_t* bbase = B + 8 * lchunk;
  auto issue = [&](int kt, int buf) {
    uint8_t* As = smem + buf * 2 * TILE_BYTES;
    uint8_t* Bs = As + TILE_BYTES;
    const int koff = kt * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t ra = min(ar0 + 8 * i, (int64_t)M - 1), rb = min(br0 + 8 * i, (int64_t)N - 1);
      __builtin_amdgcn_global_load_lds((const void*)(abase + ra * lda + koff),
                                       (lds_void_t*)(As + (wave * 8 + i) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(bbase + rb * ldb + koff),
                                       (lds_void_t*)(Bs + (wave * 8 + i) * 1024), 16, 0, 0);
    }
  };

  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const uint8_t* As = smem + buf * 2 * TILE_BYTES;
    const uint8_t* Bs = As + TILE_BYTES;
    // Pipeline phases separated by scheduling fences: fragments of
    // sub-step 0; direct loads of the next tile; then per sub-step, the
    // fragment reads of sub-step ks+1 are issued ahead of the 16 MFMAs of
    // sub-step ks so that LDS latency hides behind the matrix cores.
    bf16x8_t a[2][4], b[2][4];
    auto read = [&](int ks, int set) {
      const int c = ks * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[set][i] = *(const bf16x8_t*)(As + swz(wm + 32 * i + (lane & 31), c));
        b[set][i] = *(const bf16x8_t*)(Bs + swz(wn + 32 * i + (lane & 31), c));
      }
    };
    read(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // The last step reloads its own tile into the idle buffer (harmless),
    // keeping the loop body free of branches.
    issue(min(kt + 1, nk - 1), buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) read(ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks & 1][i], b[ks & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

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

// ------------------------------------------------------------------ v3 --
// 256x256 macro tile, K steps of 32, an LDS ring of STAGES stages (32 KiB
// each: A and B tiles of 256 rows x 64 bytes).  4 waves (2 x 2), each owning
// 128x128 as 4x4 accumulators of v_mfma_f32_32x32x16_bf16 (in AGPRs).
// Iteration k: wait for this wave's loads of stage k+1, barrier (so every
// wave's loads of stage k+1 have landed and every wave is done with stage
// k-1), issue the direct loads of stage k+STAGES-1 into the freed buffer,
// then run stage k's two MFMA sub-steps while the fragment reads of the next
// sub-step (the last one reads stage k+1) are in flight.  Row layout: 64 B
// per row, 16-byte chunk c stored at c ^ ((row >> 2) & 3).  The LDS serves a
// 16-byte read for 16 lanes per cycle across 64 banks; a fragment read has
// 16 lanes on 16 consecutive rows (aligned to 16) with one logical chunk,
// and this layout puts them on 16 disjoint 4-bank groups.
constexpr int BK3 = 32;
constexpr int STAGE_BYTES = 2 * BM * BK3 * 2;  // A + B: 32 KiB

__device__ inline int swz64(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

template <int EPI, int STAGES>
__global__ void __launch_bounds__(256, 1) k_gemm_bf16_v3(const uint16_t* __restrict__ A, int64_t lda,
                                                       const uint16_t* __restrict__ B, int64_t ldb, void* C,
                                                       int64_t ldc, const float* R, int64_t ldr, int M, int N, int K,
                                                       int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];
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

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // Kilobyte j = wave*4 + i of a tile holds rows 16*j + lane/4; the lane's
  // physical chunk lane%4 holds logical chunk (lane%4) ^ ((row >> 2) & 3).
  // Loads go through buffer resources covering this tile's rows only: rows
  // past M or N fall outside the range and read as zero.
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const int arows = (int)min<int64_t>(BM, M - m0), brows = (int)min<int64_t>(BN, N - n0);
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * lda), 0, (int)(arows * lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t brsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(B + n0 * ldb), 0, (int)(brows * ldb * 2), 0x00020000);
  const int arow = wave * 64 + (lane >> 2);
  const int nk = K / BK3;
  auto issue = [&](int kt) {
    const int st = kt % STAGES;
    uint8_t* As = smem + st * STAGE_BYTES;
    uint8_t* Bs = As + STAGE_BYTES / 2;
    const int kbytes = min(kt, nk - 1) * BK3 * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = arow + 16 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_void_t*)(As + (wave * 4 + i) * 1024), 16,
                                               (int)((r * lda + 8 * lchunk) * 2), kbytes, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, (lds_void_t*)(Bs + (wave * 4 + i) * 1024), 16,
                                               (int)((r * ldb + 8 * lchunk) * 2), kbytes, 0, 0);
    }
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
  auto read = [&](int kt, int ks, int set) {
    const uint8_t* As = smem + (kt % STAGES) * STAGE_BYTES;
    const uint8_t* Bs = As + STAGE_BYTES / 2;
    const int c = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[set][i] = *(const bf16x8_t*)(As + swz64(wm + 32 * i + (lane & 31), c));
      b[set][i] = *(const bf16x8_t*)(Bs + swz64(wn + 32 * i + (lane & 31), c));
    }
  };

  // One direct load (A or B kilobyte i of the stage) per call.
  auto issue_one = [&](int kt, int i) {
    const int st = kt % STAGES;
    uint8_t* As = smem + st * STAGE_BYTES;
    uint8_t* Bs = As + STAGE_BYTES / 2;
    const int kbytes = min(kt, nk - 1) * BK3 * 2;
    const int r = arow + 16 * (i & 3);
    if (i < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_void_t*)(As + (wave * 4 + (i & 3)) * 1024), 16,
                                               (int)((r * lda + 8 * lchunk) * 2), kbytes, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, (lds_void_t*)(Bs + (wave * 4 + (i & 3)) * 1024), 16,
                                               (int)((r * ldb + 8 * lchunk) * 2), kbytes, 0, 0);
  };
  // One fragment read (A or B tile i of a sub-step) per call.
  auto read_one = [&](int kt, int ks, int set, int i) {
    const uint8_t* As = smem + (kt % STAGES) * STAGE_BYTES;
    const uint8_t* Bs = As + STAGE_BYTES / 2;
    const int c = ks * 2 + (lane >> 5);
    if (i < 4)
      a[set][i] = *(const bf16x8_t*)(As + swz64(wm + 32 * i + (lane & 31), c));
    else
      b[set][i & 3] = *(const bf16x8_t*)(Bs + swz64(wn + 32 * (i & 3) + (lane & 31), c));
  };

  // Prologue: stages 0 .. STAGES-2 in flight; stage 0 landed everywhere.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue(s);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8 * (STAGES - 2)) : "memory");
  __syncthreads();
  read(0, 0, 0);
  // Each iteration is laid out by hand: after the barrier, the 16 MFMAs of
  // sub-step 0 each pair with one direct load of stage k+STAGES-1 or one
  // fragment read of sub-step 1; the 16 MFMAs of sub-step 1 pair with the
  // fragment reads of the next stage's sub-step 0.  Scheduling fences keep
  // this order, so a load that waits for the memory pipeline never holds
  // back more than two queued MFMAs.
  for (int kt = 0; kt < nk; ++kt) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8 * (STAGES - 3)) : "memory");
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int i = p >> 2, j = p & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][i], b[0][j], acc[i][j], 0, 0, 0);
      if (p & 1)
        read_one(kt, 1, 1, p >> 1);
      else
        issue_one(kt + STAGES - 1, p >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int kn = min(kt + 1, nk - 1);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int i = p >> 2, j = p & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][i], b[1][j], acc[i][j], 0, 0, 0);
      if (p & 1) read_one(kn, 0, 0, p >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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

// ------------------------------------------------------------------ v4 --
// 256x256x64 macro tile, two LDS stages of 64 KiB (A and B tiles of 256 rows
// x 128 B), 4 waves (2 x 2) each owning 128x128 as 4x4 accumulators of
// v_mfma_f32_32x32x16_bf16.  128-byte row segments make every global request
// a whole cache line.  Chunk c of row r sits at c ^ ((r >> 1) & 7), so the 16
// lanes a 16-byte LDS read serves per cycle (16 consecutive rows, one
// logical chunk) fall on 16 disjoint bank groups.  Per K step k:
//   sub-steps 0,1: MFMAs interleaved with the direct loads of step k+1 and
//                  the fragment reads of sub-steps 1,2;
//   sub-step 2:    MFMAs with the fragment reads of sub-step 3;
//   barrier:       step k+1 has landed and every wave has its step-k data;
//   sub-step 3:    MFMAs with the fragment reads of step k+1, sub-step 0.
constexpr int BK4 = 64;
constexpr int STAGE4 = 2 * BM * BK4 * 2;  // 64 KiB

__device__ inline int swz128(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

template <int EPI, int DMA>
__global__ void __launch_bounds__(256, 1) k_gemm_bf16_v4(const uint16_t* __restrict__ A, int64_t lda,
                                                       const uint16_t* __restrict__ B, int64_t ldb, void* C,
                                                       int64_t ldc, const float* R, int64_t ldr, int M, int N, int K,
                                                       int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE4];
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

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int arows = (int)min<int64_t>(BM, M - m0), brows = (int)min<int64_t>(BN, N - n0);
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * lda), 0, (int)(arows * lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t brsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(B + n0 * ldb), 0, (int)(brows * ldb * 2), 0x00020000);
  const int nk = K / BK4;
  // Direct load i (0..15) of a step: operand i/8, kilobyte j = wave*8 + i%8,
  // rows 8j .. 8j+7; lane l reads row 8j + l/8, logical chunk
  // (l%8) ^ ((row >> 1) & 7).
  auto issue_one = [&](int kt, int i) {
    uint8_t* base = smem + (kt & 1) * STAGE4 + (i >> 3) * (STAGE4 / 2);
    const int j = wave * 8 + (i & 7);
    const int r = 8 * j + (lane >> 3);
    const int lc = (lane & 7) ^ ((r >> 1) & 7);
    const int kbytes = kt * BK4 * 2;
    if (i < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_void_t*)(base + j * 1024), 16,
                                               (int)((r * lda + 8 * lc) * 2), kbytes, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, (lds_void_t*)(base + j * 1024), 16,
                                               (int)((r * ldb + 8 * lc) * 2), kbytes, 0, 0);
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
  auto read_one = [&](int kt, int ks, int set, int i) {
    const uint8_t* As = smem + (kt & 1) * STAGE4;
    const uint8_t* Bs = As + STAGE4 / 2;
    const int c = ks * 2 + (lane >> 5);
    if (i < 4)
      a[set][i] = *(const bf16x8_t*)(As + swz128(wm + 32 * i + (lane & 31), c));
    else
      b[set][i & 3] = *(const bf16x8_t*)(Bs + swz128(wn + 32 * (i & 3) + (lane & 31), c));
  };
  auto mfma16 = [&](int set, int p) {
    const int i = p >> 2, j = p & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[set][i], b[set][j], acc[i][j], 0, 0, 0);
  };

  // DMA == 0: step k+1's loads ride on sub-steps 0 and 1 of step k.
  // DMA == 1: step k+2's loads ride on sub-step 3 of step k (its buffer was
  //           freed by step k's barrier), doubling the prefetch distance.
  // DMA == 2: as 1, half of them on sub-step 3 of step k, half on
  //           sub-step 0 of step k+1.
#pragma unroll
  for (int i = 0; i < 16; ++i) issue_one(0, i);
  if (DMA != 0 && nk > 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) issue_one(1, i);
  }
  if (DMA != 0 && nk > 1)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) read_one(0, 0, 0, i);
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    const int kn = more ? kt + 1 : kt;
    const bool more2 = kt + 2 < nk;
    // sub-step 0 (set 0)
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      mfma16(0, p);
      if (p & 1)
        read_one(kt, 1, 1, p >> 1);
      else if (DMA == 0 && more)
        issue_one(kn, p >> 1);
      else if (DMA == 2 && more && kt >= 1)
        issue_one(kn, 8 + (p >> 1));  // second half of step k+1's loads (first half issued in step k-1)
      __builtin_amdgcn_sched_barrier(0);
    }
    // sub-step 1 (set 1)
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      mfma16(1, p);
      if (p & 1)
        read_one(kt, 2, 0, p >> 1);
      else if (DMA == 0 && more)
        issue_one(kn, 8 + (p >> 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    // sub-step 2 (set 0)
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      mfma16(0, p);
      if (p & 1) read_one(kt, 3, 1, p >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Every load still in flight here belongs to step k+1, which sub-step 3
    // starts reading: wait for all of them, then the barrier.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    // sub-step 3 (set 1)
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      mfma16(1, p);
      if ((p & 1) && more) read_one(kn, 0, 0, p >> 1);
      if (DMA == 1 && more2) issue_one(kt + 2, p);
      if (DMA == 2 && more2 && !(p & 1)) issue_one(kt + 2, p >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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

static int gemm_variant() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MT_GEMM_VARIANT");
    v = e ? atoi(e) : 4;
  }
  return v;
}

static int gemm_dma_mode() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MT_GEMM_DMA");
    v = e ? atoi(e) : 2;
  }
  return v;
}

template <>
void gemm_nt<uint16_t>(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, void* C, int64_t ldc,
                       const float* R, int64_t ldr, int M, int N, int K, Epi epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  if (K % 8 || lda % 8 || ldb % 8 || ((uintptr_t)A & 15) || ((uintptr_t)B & 15))
    throw ApiError{MT_E_INVALID, "bf16 GEMM needs K, lda, ldb multiples of 8 and 16-byte aligned operands"};
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n);
  const int variant = gemm_variant();
  if (K % BK4 == 0 && K >= BK4 && variant == 4) {
    const dim3 block(256);
#define MT_LAUNCH_V4(E, D) \
  hipLaunchKernelGGL((k_gemm_bf16_v4<E, D>), grid, block, 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, tiles_m, tiles_n)
    const int dm = gemm_dma_mode();
#define MT_V4_EPI(D)                                    \
  switch (epi) {                                        \
    case EPI_STORE: MT_LAUNCH_V4(EPI_STORE, D); break;   \
    case EPI_F32: MT_LAUNCH_V4(EPI_F32, D); break;       \
    case EPI_ADD_F32: MT_LAUNCH_V4(EPI_ADD_F32, D); break; \
  }
    if (dm == 1) {
      MT_V4_EPI(1)
    } else if (dm == 2) {
      MT_V4_EPI(2)
    } else {
      MT_V4_EPI(0)
    }
#undef MT_V4_EPI
#undef MT_LAUNCH_V4
    return;
  }
  if (K % BK3 == 0 && K >= 2 * BK3 && (variant >= 3 && variant <= 5)) {
    const dim3 block(256);
#define MT_LAUNCH_V3(E, S) \
  hipLaunchKernelGGL((k_gemm_bf16_v3<E, S>), grid, block, 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, tiles_m, tiles_n)
    if (variant == 5) {
      switch (epi) {
        case EPI_STORE: MT_LAUNCH_V3(EPI_STORE, 5); break;
        case EPI_F32: MT_LAUNCH_V3(EPI_F32, 5); break;
        case EPI_ADD_F32: MT_LAUNCH_V3(EPI_ADD_F32, 5); break;
      }
    } else {
      switch (epi) {
        case EPI_STORE: MT_LAUNCH_V3(EPI_STORE, 4); break;
        case EPI_F32: MT_LAUNCH_V3(EPI_F32, 4); break;
        case EPI_ADD_F32: MT_LAUNCH_V3(EPI_ADD_F32, 4); break;
      }
    }
#undef MT_LAUNCH_V3
    return;
  }
  if (K % BK == 0 && K > 0 && variant == 2) {
    const dim3 block(256);
#define MT_LAUNCH_V2(E) \
  hipLaunchKernelGGL(k_gemm_bf16_v2<E>, grid, block, 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, tiles_m, tiles_n)
    switch (epi) {
      case EPI_STORE: MT_LAUNCH_V2(EPI_STORE); break;
      case EPI_F32: MT_LAUNCH_V2(EPI_F32); break;
      case EPI_ADD_F32: MT_LAUNCH_V2(EPI_ADD_F32); break;
    }
#undef MT_LAUNCH_V2
    return;
  }
  const dim3 block(NTHREADS);
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
