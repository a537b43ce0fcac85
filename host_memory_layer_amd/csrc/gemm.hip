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
#include <algorithm>
#include <type_traits>

#include "kernels.h"
#include "lds_tr.h"

namespace mt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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
// K-major tiles [64 k x 256 columns] have 512-byte rows (two bank rows), so
// only the chunk index picks the bank: rows r..r+3 (r % 4 == 0) move their
// chunks to 4 different quarters of the bank row.
__device__ inline int kmkey(int row) { return (row & 3) << 2; }
__device__ inline int swz512(int row, int chunk) { return row * 512 + ((chunk ^ kmkey(row)) << 4); }


// MFMA fragment of a K-major tile: lane l gets column c0 + (l & 31) at the
// 8 contraction indices 16*ks + 8*(l/32) .. +7, by two transposing LDS
// reads.  A transposing read works on groups of 16 lanes: output lane i,
// element e is element i%4 of the 8 bytes addressed by lane 4e + i/4 of its
// group; so lane 4e + j of group g addresses row 16*ks + 8*(g/2) + e (+4 for
// the second read) at columns c0 + 16*(g%2) + 4j .. +3.
__device__ inline bf16x8_t frag_kmajor(const uint8_t* tile, int ks, int c0, int lane) {
  const int g = lane >> 4, e = (lane >> 2) & 3, j = lane & 3;
  const int col = c0 + 16 * (g & 1) + 4 * j;
  const int ra = 16 * ks + 8 * (g >> 1) + e, rb = ra + 4;
  const i16x4_t lo = lds_read_tr16(tile + swz512(ra, col >> 3) + (col & 7) * 2);
  const i16x4_t hi = lds_read_tr16(tile + swz512(rb, col >> 3) + (col & 7) * 2);
  const i16x8_t f = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, f);
}

template <bool V>
using Flag = std::integral_constant<bool, V>;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Grouped tile order: 8 tile-rows share their B panels while they are hot.
__device__ inline void tile_of(int lin, int tiles_m, int tiles_n, int64_t& m0, int64_t& n0) {
  const int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int g = lin / group_size;
  const int first_m = g * GROUP;
  const int gm_cnt = min(tiles_m - first_m, GROUP);
  m0 = (int64_t)(first_m + (lin % group_size) % gm_cnt) * BM;
  n0 = (int64_t)((lin % group_size) / gm_cnt) * BN;
}

// Stream-K tail.  The K steps of the tiles [t_dp, ntiles) that do not fill a
// whole round, taken in tile order, are cut into nwg contiguous ranges, one
// per workgroup (logical index v).  A cut that falls within 3 steps of a tile
// edge moves to that edge, so every segment of a tile has at least 3 K steps
// (the pipeline's minimum).  Both the GEMM and its fix-up derive the cuts
// from the shapes alone.
__host__ __device__ inline int64_t sk_cut(int v, int nwg, int64_t total, int nk) {
  int64_t x = total * v / nwg;
  const int64_t r = x % nk;
  if (r > 0 && r < 3)
    x -= r;
  else if (r > nk - 3)
    x += nk - r;
  return x;
}

// The problems one launch of k_gemm_bf16_tile computes: one, or a group
// that shares K and the operand layouts (a layer's weight gradients), whose
// tiles form one combined order, problem after problem, split over the
// persistent workgroups as a single tile space.
struct GemmProblem {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int64_t lda, ldb, ldc;
  int M, N, tiles_m, tiles_n;
  int t0;  // first tile of the problem in the combined order
};
struct GemmGroup {
  GemmProblem p[kGemmGroupMax];
  int n;
  int ntiles;  // tiles of all problems
};
// the problem holding combined tile t (problems are few: a linear scan)
__device__ inline int problem_of(const GemmGroup& G, int t) {
  int i = 0;
  while (i + 1 < G.n && t >= G.p[i + 1].t0) ++i;
  return i;
}

// VEC: N and ldc multiples of 4 and C 16-byte aligned, so every lane writes
// 4 consecutive outputs per store through a buffer descriptor that drops
// rows past M, while lanes past N aim beyond the descriptor.  Otherwise
// element stores.
// AKM / BKM: operand A (B) is K-major, [K x M] ([K x N]) with row stride
// lda (ldb), instead of K-contiguous [M x K] ([N x K]).
template <int EPI, bool VEC, bool AKM, bool BKM>
__global__ void __launch_bounds__(256, 1) k_gemm_bf16_tile(const GemmGroup G, const float* R, int64_t ldr, int K,
                                                       float* ws, int t_dp, int maxseg) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  const int ntiles = G.ntiles;
  // the current tile's problem (set by bind below)
  const uint16_t* A = nullptr;
  const uint16_t* B = nullptr;
  void* C = nullptr;
  int64_t lda = 0, ldb = 0, ldc = 0;
  int M = 0, N = 0;
  // Persistent schedule.  Workgroup w runs on XCD w % 8 (the dispatcher deals
  // workgroups round-robin over the XCDs); XCD x owns a contiguous range of
  // the grouped tile order, and its workgroups take turns through it.
  // Whole tiles [0, t_dp): workgroup w runs on XCD w % 8 (the dispatcher
  // deals workgroups round-robin over the XCDs); XCD x owns a contiguous
  // range of the grouped tile order, and its workgroups take turns through
  // it.  Tiles [t_dp, ntiles): the stream-K tail, whose segments are summed
  // by k_gemm_sk_fixup (t_dp == ntiles: none).
  const int nwg = gridDim.x, w = blockIdx.x;
  const int nk = K / BK;
  int t, hi, stride;
  if (nwg % 8 == 0 && nwg <= t_dp) {
    const int per = (t_dp + 7) / 8;
    const int lo = (w % 8) * per;
    hi = min(t_dp, lo + per);
    t = lo + w / 8;
    stride = nwg / 8;
  } else {
    t = w;
    hi = t_dp;
    stride = nwg;
  }
  // this workgroup's range of the tail's K steps, XCD-contiguous like the tiles
  const int u = nwg % 8 == 0 ? (w % 8) * (nwg / 8) + w / 8 : w;
  const int64_t sk_total = (int64_t)(ntiles - t_dp) * nk;
  int64_t sk_p = sk_total ? sk_cut(u, nwg, sk_total, nk) : 0;
  const int64_t sk_end = sk_total ? sk_cut(u + 1, nwg, sk_total, nk) : 0;
  const int64_t sk_tile0 = sk_p / nk;
  // Current work item: tile tc, K steps [kb, kb + n).  EPI_PARTIAL (the
  // tail launch): a segment of a tail tile, its partial sum written to ws
  // slot `slot`; otherwise a whole tile of [0, t_dp).
  int tc = 0, kb = 0, n = nk, slot = 0;
  auto take = [&]() -> bool {
    if (EPI != EPI_PARTIAL) {
      if (t >= hi) return false;
      tc = t;
      t += stride;
      return true;
    }
    if (sk_p >= sk_end) return false;
    const int64_t tile = sk_p / nk;
    const int64_t e = min(sk_end, (tile + 1) * nk);
    tc = t_dp + (int)tile;
    kb = (int)(sk_p - tile * nk);
    n = (int)(e - sk_p);
    slot = u * maxseg + (int)(tile - sk_tile0);
    sk_p = e;
    return true;
  };
  if (!take()) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto rsrc_of = [&](const void* base, int64_t row0, int64_t rows_total, int64_t ld, int esize) {
    const int rows = (int)min<int64_t>(BM, rows_total - row0);
    return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)base + row0 * ld * esize), 0,
                                             (int)(rows * ld * esize), 0x00020000);
  };
  // operand tiles: descriptors for the inline-assembly direct loads
  auto orsrc_of = [&](const uint16_t* base, int64_t row0, int64_t rows_total, int64_t ld) {
    const int64_t rows = min<int64_t>(BM, rows_total - row0);
    return make_rsrc(base + row0 * ld, (uint32_t)(rows * ld * 2));
  };
  // K-major operand: the descriptor starts at the tile's first column and
  // runs to the end of the matrix.  Columns past M (N) of a last tile read
  // neighbouring data, or zero past the end; they only reach outputs that
  // are never stored.
  auto rsrc_km = [&](const uint16_t* base, int64_t col0, int64_t ld) {
    return make_rsrc(base + col0, (uint32_t)(((int64_t)K * ld - col0) * 2));
  };

  // Direct load i (0..7) of an operand tile writes kilobyte j = wave*8 + i.
  // K-contiguous tile [256 rows x 64 k]: rows 8j .. 8j+7; lane l reads row
  // 8j + l/8, logical chunk (l%8) ^ ((row>>1)&7), which lands at physical
  // chunk l%8.  K-major tile [64 k x 256 columns]: rows 2j, 2j+1; lane l
  // reads row 2j + l/32, logical chunk (l%32) ^ kmkey(row).
  int aoff[8], boff[8];
  int astep = 0, bstep = 0;  // bytes per K step
  // byte offsets of the item's first K step (kt counts from it)
  int kofs_a = 0, kofs_b = 0;
  auto load_a = [&](i32x4_t rs, int kt, int i) {
    dma16(rs, smem + (kt & 1) * STAGE + (wave * 8 + i) * 1024, aoff[i], kofs_a + kt * astep);
  };
  auto load_b = [&](i32x4_t rs, int kt, int i) {
    dma16(rs, smem + (kt & 1) * STAGE + STAGE / 2 + (wave * 8 + i) * 1024, boff[i], kofs_b + kt * bstep);
  };

  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  f32x16_t acc[4][4];
  bf16x8_t a[2][4], b[2][4];
  // Fragment q (0..7) of a sub-step, in the order the next sub-step's MFMAs
  // first use them: a0, b0..b3, a1..a3.
  auto read_one = [&](int kt, int ks, int set, int q) {
    const uint8_t* As = smem + (kt & 1) * STAGE;
    const uint8_t* Bs = As + STAGE / 2;
    const int c = ks * 2 + (lane >> 5);
    auto rd128 = [&](const uint8_t* p) { return *(const bf16x8_t*)p; };
    if (q == 0 || q > 4) {
      const int i = q == 0 ? 0 : q - 4;
      a[set][i] = AKM ? frag_kmajor(As, ks, wm + 32 * i, lane) : rd128(As + swz128(wm + 32 * i + (lane & 31), c));
    } else {
      b[set][q - 1] = BKM ? frag_kmajor(Bs, ks, wn + 32 * (q - 1), lane)
                          : rd128(Bs + swz128(wn + 32 * (q - 1) + (lane & 31), c));
    }
  };
  // B fragments are the MFMA's first operand: the accumulator then holds
  // the tile transposed, so that a lane owns 4 consecutive output columns.
  auto mfma16 = [&](int set, int p) {
    const int i = p >> 2, j = p & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[set][j], a[set][i], acc[i][j], 0, 0, 0);
  };

  int64_t m0 = 0, n0 = 0;
  i32x4_t ar, br;
  // Bind the work item's tile: its problem's operands, strides and output,
  // the per-lane load offsets, the tile origin and the operand descriptors.
  auto bind = [&]() {
    const GemmProblem& P = G.p[problem_of(G, tc)];
    A = P.A;
    B = P.B;
    C = P.C;
    lda = P.lda;
    ldb = P.ldb;
    ldc = P.ldc;
    M = P.M;
    N = P.N;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = wave * 8 + i;
      const int r = 8 * j + (lane >> 3), lc = (lane & 7) ^ ((r >> 1) & 7);
      const int rk = 2 * j + (lane >> 5), lck = (lane & 31) ^ kmkey(rk);
      aoff[i] = AKM ? (int)((rk * lda + 8 * lck) * 2) : (int)((r * lda + 8 * lc) * 2);
      boff[i] = BKM ? (int)((rk * ldb + 8 * lck) * 2) : (int)((r * ldb + 8 * lc) * 2);
    }
    astep = AKM ? (int)(BK * lda * 2) : BK * 2;
    bstep = BKM ? (int)(BK * ldb * 2) : BK * 2;
    kofs_a = kb * astep;
    kofs_b = kb * bstep;
    tile_of(tc - P.t0, P.tiles_m, P.tiles_n, m0, n0);
    ar = AKM ? rsrc_km(A, m0, lda) : orsrc_of(A, m0, M, lda);
    br = BKM ? rsrc_km(B, n0, ldb) : orsrc_of(B, n0, N, ldb);
  };
  bind();

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
        load_b(br, kt + 1, p >> 1);
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
    // Step kt+1 must have landed before sub-step 3 reads it; the barrier
    // also frees step kt's stage for step kt+2.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      mfma16(1, p);
      if (NEXT && (p & 1)) read_one(kt + 1, 0, 0, p >> 1);
      if (LOAD_A2 && !(p & 1)) load_a(ar, kt + 2, p >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Steps 0 and 1 of a tile (nk >= 3); both stages are free.
  auto prologue = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      load_a(ar, 0, i);
      load_b(br, 0, i);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      load_a(ar, 1, i);
      load_b(br, 1, i);
    }
  };
  prologue();

  const Flag<true> T_;
  const Flag<false> F_;
  for (;;) {
    // Step 0 of this tile (and everything issued before it, the previous
    // tile's stores included) has landed; step 1 may still be in flight.
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    __syncthreads();
    read_one(0, 0, 0, 0);
    read_one(0, 0, 0, 1);
    read_one(0, 0, 0, 2);
    read_one(0, 0, 0, 3);
    read_one(0, 0, 0, 4);
    read_one(0, 0, 0, 5);
    read_one(0, 0, 0, 6);
    read_one(0, 0, 0, 7);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    step(0, F_, T_, T_);  // step 1 came with step 0
    for (int kt = 1; kt + 2 < n; ++kt) step(kt, T_, T_, T_);
    step(n - 2, T_, F_, T_);
    step(n - 1, F_, F_, F_);

    // Epilogue.  acc[i][j] register r holds row 32i + (lane & 31) and column
    // 32j + 8(r/4) + 4(lane/32) + r%4 of the wave's 128 x 128 sub-tile.
    if (EPI == EPI_PARTIAL) {
      // partial sum of a tail tile: the raw fp32 tile [256 x 256] into its slot
      const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(ws + (int64_t)slot * (BM * BN)), 0, BM * BN * 4, 0x00020000);
      const int c0 = 4 * (lane >> 5);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = q >> 2, j = q & 3;
        const int row = wm + 32 * i + (lane & 31);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = wn + 32 * j + 8 * g + c0;
          const f32x16_t& v = acc[i][j];
          u32x4_t pk = {__float_as_uint(v[4 * g]), __float_as_uint(v[4 * g + 1]), __float_as_uint(v[4 * g + 2]),
                        __float_as_uint(v[4 * g + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(pk, wrs, (row * BN + col) * 4, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (VEC) {
      const int esize = EPI == EPI_STORE ? 2 : 4;
      const __amdgpu_buffer_rsrc_t crs = rsrc_of(C, m0, M, ldc, esize);
      __amdgpu_buffer_rsrc_t rrs = crs;
      if (EPI == EPI_ADD_F32) rrs = rsrc_of(R, m0, M, ldr, 4);
      // column of this lane's first output relative to the sub-tile; lanes
      // whose 4 columns lie past N aim beyond the descriptor
      const int c0 = 4 * (lane >> 5);
      const int ncol = (int)min<int64_t>(BN, N - n0) - wn;  // valid columns of the sub-tile
      // EPI_ADD_F32: the residual of 32 x 32 block q = 4i + j is loaded
      // RLA = 3 blocks ahead, so a block's loads have three blocks of stores
      // to land.  Vector memory operations complete in issue order: block q
      // has landed once no more than the 4-instruction groups issued after
      // it are in flight, i.e. the loads of blocks q+1 .. min(q+3, 15) and
      // the stores of blocks max(0, q-3) .. q-1.
      constexpr int RLA = 3;
      u32x4_t rv[RLA + 1][4];
      auto load_res = [&](int q) {
        const int row = wm + 32 * (q >> 2) + (lane & 31);
        const int rbase = row * (int)ldr + (int)(n0 + wn) + c0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 32 * (q & 3) + 8 * g;
          const int off = col + c0 < ncol ? (rbase + col) * 4 : 0x7FFFFFF0;
          rv[q % (RLA + 1)][g] = __builtin_amdgcn_raw_buffer_load_b128(rrs, off, 0, 0);
        }
      };
      if (EPI == EPI_ADD_F32) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < RLA; ++q) load_res(q);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = q >> 2, j = q & 3;
        const int row = wm + 32 * i + (lane & 31);
        const int cbase = row * (int)ldc + (int)(n0 + wn) + c0;
        if (EPI == EPI_ADD_F32) {
          __builtin_amdgcn_sched_barrier(0);
          if (q + RLA < 16) load_res(q + RLA);
          // groups in flight after block q's loads (q is a constant once unrolled)
          const int after = (min(q + RLA, 15) - q) + min(q, RLA);
          switch (after) {
            case 3: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
            case 4: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
            case 5: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
            default: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 32 * j + 8 * g;
          const int off = col + c0 < ncol ? (cbase + col) * esize : 0x7FFFFFF0;
          const f32x16_t& v = acc[i][j];
          if (EPI == EPI_STORE) {
            u32x2_t pk;
            pk.x = (uint32_t)f32_to_bf16(v[4 * g]) | ((uint32_t)f32_to_bf16(v[4 * g + 1]) << 16);
            pk.y = (uint32_t)f32_to_bf16(v[4 * g + 2]) | ((uint32_t)f32_to_bf16(v[4 * g + 3]) << 16);
            __builtin_amdgcn_raw_buffer_store_b64(pk, crs, off, 0, 0);
          } else {
            float o0 = v[4 * g], o1 = v[4 * g + 1], o2 = v[4 * g + 2], o3 = v[4 * g + 3];
            if (EPI == EPI_ADD_F32) {
              const u32x4_t r = rv[q % (RLA + 1)][g];
              o0 = __uint_as_float(r.x) + o0;
              o1 = __uint_as_float(r.y) + o1;
              o2 = __uint_as_float(r.z) + o2;
              o3 = __uint_as_float(r.w) + o3;
            }
            u32x4_t pk = {__float_as_uint(o0), __float_as_uint(o1), __float_as_uint(o2), __float_as_uint(o3)};
            __builtin_amdgcn_raw_buffer_store_b128(pk, crs, off, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t gm = m0 + wm + 32 * i + (lane & 31);
            const int64_t gn = n0 + wn + 32 * j + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
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
    // Next tile: its loads go out right behind this tile's stores, so the
    // store drain, the load latency and the next tile's start overlap.
    if (!take()) break;
    bind();
    prologue();
  }
}

// Fix-up of the stream-K tail: tail tile blockIdx.y is the sum of the
// partial tiles of the workgroup ranges that cover its K steps, added in
// K order (so the result depends only on the shapes), then the epilogue.
// Each thread takes 4 consecutive columns of one row of the 256 x 256 tile.
template <int EPI>
__global__ void __launch_bounds__(256) k_gemm_sk_fixup(const float* __restrict__ ws, const GemmGroup G, const float* R,
                                                       int64_t ldr, int K, int t_dp, int nwg, int maxseg) {
  const int nk = K / BK;
  const int ntiles = G.ntiles;
  const int64_t total = (int64_t)(ntiles - t_dp) * nk;
  const int tt = blockIdx.y;
  const int64_t lo = (int64_t)tt * nk, hi = lo + nk;
  // the range holding step lo: the largest v with cut(v) <= lo
  int a = 0, b = nwg - 1;
  while (a < b) {
    const int mid = (a + b + 1) / 2;
    if (sk_cut(mid, nwg, total, nk) <= lo)
      a = mid;
    else
      b = mid - 1;
  }
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int row = e / BN, col = e % BN;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  for (int v = a; v < nwg; ++v) {
    const int64_t cv = sk_cut(v, nwg, total, nk);
    if (cv >= hi) break;
    if (sk_cut(v + 1, nwg, total, nk) == cv) continue;  // empty range
    const int slot = v * maxseg + (int)(tt - cv / nk);
    const float4 p = *(const float4*)(ws + (int64_t)slot * (BM * BN) + e);
    s0 += p.x;
    s1 += p.y;
    s2 += p.z;
    s3 += p.w;
  }
  const GemmProblem& P = G.p[problem_of(G, t_dp + tt)];
  void* C = P.C;
  const int64_t ldc = P.ldc;
  const int M = P.M, N = P.N;
  int64_t m0, n0;
  tile_of(t_dp + tt - P.t0, P.tiles_m, P.tiles_n, m0, n0);
  const int64_t gm = m0 + row;
  if (gm >= M) return;
  const float sv[4] = {s0, s1, s2, s3};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t gn = n0 + col + c;
    if (gn >= N) break;
    if (EPI == EPI_STORE)
      ((uint16_t*)C)[gm * ldc + gn] = f32_to_bf16(sv[c]);
    else if (EPI == EPI_F32)
      ((float*)C)[gm * ldc + gn] = sv[c];
    else
      ((float*)C)[gm * ldc + gn] = R[gm * ldr + gn] + sv[c];
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

// One workgroup per compute unit of the current device (LDS use allows one).
int persistent_workgroups() {
  static thread_local int dev = -1, cus = 0;
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) d = 0;
  if (d != dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess || n <= 0) n = 256;
    dev = d;
    cus = n;
  }
  return cus;
}

}  // namespace

bool gemm_layout_ok(int M, int N, int K, int64_t lda, int64_t ldb, int layout) {
  (void)M;
  (void)N;
  if (K % BK || K < 3 * BK || lda % 8 || ldb % 8) return false;
  const int64_t lim = (int64_t)1 << 31;
  // 32-bit buffer offsets: a K-major operand is addressed from its tile's
  // first column to the end of the matrix
  if ((layout & GEMM_A_KMAJOR) && (int64_t)K * lda * 2 >= lim) return false;
  if ((layout & GEMM_B_KMAJOR) && (int64_t)K * ldb * 2 >= lim) return false;
  return true;
}

// Stream-K plan for a bf16 GEMM on `nwg` persistent workgroups: the first
// t_dp tiles in whole rounds, the rest split along K.  Used when the last
// round would leave at least 5% of the launch idle, the tail holds at most
// 0.45 of a round and gives every workgroup at least 16 K steps; maxseg
// bounds the tail tiles one range touches.  Returns false (no split)
// otherwise.  The 0.45: measured at the 14B weight-gradient shapes, a
// split tail runs at about half the rate of whole tiles (its workgroups
// stand at different K offsets, so they share no operand panels in L2, and
// each segment pays a pipeline fill and a 256 KiB partial store): tails of
// 0.22 and 0.44 of a round gained 10.5% and 3.1%, tails of 0.56 and 0.69
// lost 7% and 1.5%.
static bool sk_plan(int ntiles, int nk, int nwg, int* t_dp, int* maxseg) {
  if (ntiles <= nwg || ntiles % nwg == 0 || nk < 8) return false;
  const int rounds = (ntiles + nwg - 1) / nwg;
  if ((int64_t)(rounds * nwg - ntiles) * 20 < (int64_t)rounds * nwg) return false;
  if ((int64_t)(ntiles % nwg) * 20 > (int64_t)nwg * 9) return false;
  const int64_t total = (int64_t)(ntiles % nwg) * nk;
  if (total / nwg < 16) return false;
  const int64_t longest = total / nwg + 1 + 4;  // a range, after its cuts moved by up to 2 each
  *t_dp = ntiles - ntiles % nwg;
  *maxseg = (int)((longest - 1) / nk) + 2;
  return true;
}

size_t gemm_ws_bytes(int M, int N, int K) {
  int t_dp = 0, maxseg = 0;
  const int ntiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (K % BK || !sk_plan(ntiles, K / BK, persistent_workgroups(), &t_dp, &maxseg)) return 0;
  return (size_t)persistent_workgroups() * maxseg * BM * BN * sizeof(float);
}

size_t gemm_group_ws_bytes(const int* M, const int* N, int n, int K) {
  int ntiles = 0;
  for (int i = 0; i < n; ++i) ntiles += ((M[i] + BM - 1) / BM) * ((N[i] + BN - 1) / BN);
  int t_dp = 0, maxseg = 0;
  if (K % BK || !sk_plan(ntiles, K / BK, persistent_workgroups(), &t_dp, &maxseg)) return 0;
  return (size_t)persistent_workgroups() * maxseg * BM * BN * sizeof(float);
}

// The persistent tile kernel over a group (one problem or several), then
// the stream-K tail's segments and their fix-up when a split is planned and
// the workspace holds it.
static void launch_tiles(const GemmGroup& G, const float* R, int64_t ldr, int K, int layout, Epi epi, bool vec,
                         hipStream_t s, float* ws, size_t ws_bytes) {
  const int ntiles = G.ntiles;
  const int nwg = std::min(ntiles, persistent_workgroups());
  const dim3 pgrid(nwg);
  int t_dp = ntiles, maxseg = 0;
  if (!ws || !sk_plan(ntiles, K / BK, nwg, &t_dp, &maxseg) ||
      (size_t)nwg * maxseg * BM * BN * sizeof(float) > ws_bytes) {
    t_dp = ntiles;  // whole tiles only
    maxseg = 0;
  }
#define L_(E, V, AK, BK_) \
  hipLaunchKernelGGL((k_gemm_bf16_tile<E, V, AK, BK_>), pgrid, dim3(256), 0, s, G, R, ldr, K, ws, t_dp, maxseg)
#define LL_(E, V)                  \
  switch (layout) {                \
    case 0: L_(E, V, false, false); break; \
    case 1: L_(E, V, true, false); break;  \
    case 2: L_(E, V, false, true); break;  \
    default: L_(E, V, true, true); break;  \
  }
#define LV_(E)     \
  if (vec) {       \
    LL_(E, true)   \
  } else {         \
    LL_(E, false)  \
  }
  switch (epi) {
    case EPI_STORE: LV_(EPI_STORE) break;
    case EPI_F32: LV_(EPI_F32) break;
    case EPI_ADD_F32: LV_(EPI_ADD_F32) break;
    default: throw ApiError{MT_E_INVALID, "GEMM epilogue"};
  }
#undef LV_
#undef LL_
  if (t_dp < ntiles) {
    // the tail's segments on every workgroup, then their sums
    switch (layout) {
      case 0: L_(EPI_PARTIAL, true, false, false); break;
      case 1: L_(EPI_PARTIAL, true, true, false); break;
      case 2: L_(EPI_PARTIAL, true, false, true); break;
      default: L_(EPI_PARTIAL, true, true, true); break;
    }
    const dim3 fgrid(BM * BN / (256 * 4), ntiles - t_dp);
#define F_(E) hipLaunchKernelGGL(k_gemm_sk_fixup<E>, fgrid, dim3(256), 0, s, ws, G, R, ldr, K, t_dp, nwg, maxseg)
    switch (epi) {
      case EPI_STORE: F_(EPI_STORE); break;
      case EPI_F32: F_(EPI_F32); break;
      default: F_(EPI_ADD_F32); break;
    }
#undef F_
  }
#undef L_
}

static void add_problem(GemmGroup& G, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, void* C,
                        int64_t ldc, int M, int N) {
  GemmProblem& P = G.p[G.n++];
  P.A = A;
  P.B = B;
  P.C = C;
  P.lda = lda;
  P.ldb = ldb;
  P.ldc = ldc;
  P.M = M;
  P.N = N;
  P.tiles_m = (M + BM - 1) / BM;
  P.tiles_n = (N + BN - 1) / BN;
  P.t0 = G.ntiles;
  G.ntiles += P.tiles_m * P.tiles_n;
}

// operand checks shared by the single and the grouped launch
static void check_tile_operands(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t ldc,
                                const float* R, int64_t ldr, int M, int N, int K, int layout) {
  if (K % 8 || lda % 8 || ldb % 8 || ((uintptr_t)A & 15) || ((uintptr_t)B & 15))
    throw ApiError{MT_E_INVALID, "bf16 GEMM needs K, lda, ldb multiples of 8 and 16-byte aligned operands"};
  if (layout != 0 && !gemm_layout_ok(M, N, K, lda, ldb, layout))
    throw ApiError{MT_E_INVALID, "K-major bf16 GEMM operands need K % 64 == 0, K >= 192, K*ld*2 < 2^31"};
  // buffer offsets are 32-bit: one 256-row panel of every operand must fit
  const int64_t lim = (int64_t)1 << 31;
  if ((!(layout & GEMM_A_KMAJOR) && (int64_t)BM * lda * 2 >= lim) ||
      (!(layout & GEMM_B_KMAJOR) && (int64_t)BN * ldb * 2 >= lim) || (int64_t)BM * ldc * 4 >= lim ||
      (R && (int64_t)BM * ldr * 4 >= lim))
    throw ApiError{MT_E_INVALID, "bf16 GEMM row stride too large"};
}

void gemm_bf16_group(const GemmDesc* d, int n, int K, int layout, Epi epi, hipStream_t s, float* ws,
                     size_t ws_bytes) {
  if (n < 1 || n > kGemmGroupMax) throw ApiError{MT_E_INVALID, "GEMM group size"};
  if (epi != EPI_STORE && epi != EPI_F32) throw ApiError{MT_E_INVALID, "grouped GEMM epilogue"};
  if (K % BK || K < 3 * BK) throw ApiError{MT_E_INVALID, "grouped GEMM needs K % 64 == 0 and K >= 192"};
  GemmGroup G{};
  bool vec = true;
  for (int i = 0; i < n; ++i) {
    if (d[i].M <= 0 || d[i].N <= 0) throw ApiError{MT_E_INVALID, "grouped GEMM problem size"};
    check_tile_operands(d[i].A, d[i].lda, d[i].B, d[i].ldb, d[i].ldc, nullptr, 0, d[i].M, d[i].N, K, layout);
    vec = vec && d[i].N % 4 == 0 && d[i].ldc % 4 == 0 && ((uintptr_t)d[i].C & 15) == 0;
    add_problem(G, d[i].A, d[i].lda, d[i].B, d[i].ldb, d[i].C, d[i].ldc, d[i].M, d[i].N);
  }
  launch_tiles(G, nullptr, 0, K, layout, epi, vec, s, ws, ws_bytes);
}

void gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int layout, void* C, int64_t ldc,
               const float* R, int64_t ldr, int M, int N, int K, Epi epi, hipStream_t s, float* ws,
               size_t ws_bytes) {
  if (M <= 0 || N <= 0) return;
  if (K % 8 || lda % 8 || ldb % 8 || ((uintptr_t)A & 15) || ((uintptr_t)B & 15))
    throw ApiError{MT_E_INVALID, "bf16 GEMM needs K, lda, ldb multiples of 8 and 16-byte aligned operands"};
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n);
  if (layout != 0 && !gemm_layout_ok(M, N, K, lda, ldb, layout))
    throw ApiError{MT_E_INVALID, "K-major bf16 GEMM operands need K % 64 == 0, K >= 192, K*ld*2 < 2^31"};
  if (K % BK == 0 && K >= 3 * BK) {
    check_tile_operands(A, lda, B, ldb, ldc, R, ldr, M, N, K, layout);
    const bool vec = N % 4 == 0 && ldc % 4 == 0 && ((uintptr_t)C & 15) == 0 &&
                     (epi != EPI_ADD_F32 || (ldr % 4 == 0 && ((uintptr_t)R & 15) == 0));
    GemmGroup G{};
    add_problem(G, A, lda, B, ldb, C, ldc, M, N);
    launch_tiles(G, R, ldr, K, layout, epi, vec, s, ws, ws_bytes);
    return;
  }
#define L_(E)                                                                                                      \
  hipLaunchKernelGGL(k_gemm_bf16_generic<E>, grid, dim3(NTHREADS), 0, s, A, lda, B, ldb, C, ldc, R, ldr, M, N, K, \
                     tiles_m, tiles_n)
  switch (epi) {
    case EPI_STORE: L_(EPI_STORE); break;
    case EPI_F32: L_(EPI_F32); break;
    case EPI_ADD_F32: L_(EPI_ADD_F32); break;
    default: throw ApiError{MT_E_INVALID, "GEMM epilogue"};
  }
#undef L_
}

template <>
void gemm_nt<uint16_t>(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, void* C, int64_t ldc,
                       const float* R, int64_t ldr, int M, int N, int K, Epi epi, hipStream_t s) {
  gemm_bf16(A, lda, B, ldb, 0, C, ldc, R, ldr, M, N, K, epi, s);
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
