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
//    the S^T accumulators as the B operand.  K and V tiles of 64 keys are
//    double-buffered in LDS.
//  * backward, two kernels and no atomics (deterministic):
//    dK/dV: one block = 128 keys (K, V held in LDS), query tiles of 32
//    stream through one LDS stage, two blocks per CU; S = Q . K^T and
//    dP = dO . V^T have a lane per key, so dV^T += dO^T . P and
//    dK^T += Q^T . dS take P and dS from registers.
//    dQ: one block = 128 queries, key tiles of 32 double-buffered, two
//    blocks per CU; S^T = K . Q^T, dP^T = V . dO^T, dQ^T += K^T . dS^T.
//    Gradients are written transposed into dqkvT [3d x M].
//
// Every LDS tile is row-major (a token per 256-byte row).  The transposed
// operands V^T, K^T, Q^T, dO^T are read from those tiles with transposing
// LDS reads (ds_read_b64_tr_b16), so no transposed copy of q, k, v or dO
// exists in memory.  An MFMA contracts over 16 indices; the A and B operands
// pair their elements by (lane half, element), so any permutation of the
// contraction index that both operands share is exact.  When P (or dS)
// comes from an accumulator, element e of lane-half h holds key (or query)
// 8*(e/4)+4*h+(e%4) of a 16-wide slice, and the transposing reads fetch the
// other operand in the same order.
#include <type_traits>

#include "kernels.h"
#include "lds_tr.h"

namespace mt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Swizzled byte offsets for rows of 256 bytes (16 chunks).  The key swaps the two bit pairs of row % 16: any 16 consecutive rows get 16
// different keys (row reads of one logical chunk), and the 4 rows r..r+3
// (r % 4 == 0) move a group of 4 adjacent chunks to 4 different quarters of
// the bank row (transposing reads).
__device__ inline int swkey(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ inline int sw256(int row, int chunk) { return row * 256 + ((chunk ^ swkey(row)) << 4); }

__device__ inline f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Workgroups are dealt round-robin to the 8 XCDs in dispatch order (x
// fastest), and each XCD has its own L2.  The grid's (x, y) is remapped so
// that XCD k runs a contiguous range of the row-major order (y outer): the
// blocks of one (batch, head), which read the same K, V (or Q, dO) tiles,
// share an L2.
struct BlockXY {
  int x, y;
};
__device__ inline BlockXY xcd_block() {
  const int n = gridDim.x * gridDim.y, gx = gridDim.x;
  const int i = blockIdx.y * gridDim.x + blockIdx.x;
  const int q = n / 8, r = n % 8, k = i % 8;
  const int l = k * q + min(k, r) + i / 8;
  // Inside each run of G = 2 (b, h) rows the blocks are taken column by
  // column: block x = 0 is the heaviest of a row under the causal mask (the
  // most key or query tiles), so the heavy blocks of both rows start first
  // and the blocks that finish the launch are light ones.  Taking each row
  // whole, heavy to light, left a tail of about 4% of the launch (a list
  // schedule of the 14B-shape grid over 64 block slots per XCD).  An
  // incomplete last run keeps the row order.
  constexpr int G = 2;
  const int S = G * gx, c = l / S;
  if ((c + 1) * S <= n) {
    const int w = l - c * S;
    return BlockXY{w / G, c * G + w % G};
  }
  return BlockXY{l % gx, l / gx};
}

// x of this lane combined with x of lane l ^ 32 (the partner half-wave) by
// one lane swap between the wave's halves (v_permlane32_swap), instead of a
// shuffle through LDS and its lane-index arithmetic.  The swap leaves lane l
// holding x[l] and x[l ^ 32] in the two halves of the result, lower lane's
// value first; max and + are commutative, so the result is that of
// op(x, shuffle_xor(x, 32)).
__device__ inline float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row index inside a 32x32 accumulator tile for register r of this lane.
__device__ inline int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// Transposed fragment from a row-major tile with 256-byte rows (128 bf16,
// sw256), by two transposing LDS reads (ds_read_b64_tr_b16).  For the MFMA
// A operand X^T (rows = tile columns c0 .. c0+31, contraction = tile rows
// r0 .. r0+15), lane l gets column c0 + (l & 31) at rows
// r0 + 8*(e/4) + 4*(l/32) + e%4 for element e: the pairing of a B operand
// taken from an accumulator.
//
// A transposing read works on groups of 16 lanes: output lane i, element e
// is element i%4 of the 8 bytes addressed by lane 4e + i/4 of its group.  So
// lane 4e + j of group g addresses row r0 + 4*(g/2) + e (+8 for the second
// read), columns c0 + 16*(g%2) + 4j .. +3, and output lane i receives
// column c0 + 16*(g%2) + i of rows e = 0..3.
__device__ inline bf16x8_t frag_tr(const uint8_t* tile, int r0, int c0, int lane) {
  const int g = lane >> 4, e = (lane >> 2) & 3, j = lane & 3;
  const int col = c0 + 16 * (g & 1) + 4 * j;
  const int ra = r0 + 4 * (g >> 1) + e, rb = ra + 8;
  const uint8_t* pa = tile + sw256(ra, col >> 3) + (col & 7) * 2;
  const uint8_t* pb = tile + sw256(rb, col >> 3) + (col & 7) * 2;
  const i16x4_t lo = lds_read_tr16(pa);
  const i16x4_t hi = lds_read_tr16(pb);
  const i16x8_t f = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, f);
}

// Registers 8*ks .. 8*ks+7 of an accumulator tile, as a bf16 B operand.
__device__ inline bf16x8_t acc_to_frag(const f32x16_t& a, int ks) {
  bf16x8_t f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (__bf16)a[8 * ks + e];
  return f;
}

// ------------------------------------------------------------ forward ----
__global__ void __launch_bounds__(256, 2) k_attn_fwd_bf16(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ o,
                                                          float* __restrict__ lse, int T, int H) {
  constexpr int HD = 128;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 32768];
  const int nqb = (T + 127) / 128;
  const BlockXY blk = xcd_block();
  const int qb = nqb - 1 - blk.x;
  const int bh = blk.y, b = bh / H, h = bh % H;
  const int d = H * HD;
  const int64_t ld = 3LL * d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  // K and V tiles [64 keys x 256 B] go global -> LDS with buffer_load ...
  // lds; kilobyte j = wave*4 + i of a tile is written by one instruction, so
  // each lane's source is chosen to land in the swizzled layout the fragment
  // reads expect.  V^T fragments come from the V tile by transposing reads.
  // Each tile's buffer descriptor starts at the tile's first key row, so the
  // 32-bit offsets stay within one tile for any sequence length.
  const uint16_t* kcol = qkv + rowbase * ld + d + h * HD;
  const uint16_t* vcol = kcol + d;
  const uint32_t tile_bytes = (uint32_t)(64 * ld * 2);
  auto issue = [&](int kb, int buf) {
    uint8_t* Ks = smem + buf * 32768;
    uint8_t* Vs = Ks + 16384;
    const int64_t key0 = (int64_t)kb * 64;
    const i32x4_t krs = make_rsrc(kcol + key0 * ld, tile_bytes);
    const i32x4_t vrs = make_rsrc(vcol + key0 * ld, tile_bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = wave * 4 + i;
      const int kr = 4 * j + (lane >> 4), kc = (lane & 15) ^ swkey(kr);
      const int off = (int)((kr * ld + 8 * kc) * 2);
      dma16(krs, Ks + j * 1024, off, 0);
      dma16(vrs, Vs + j * 1024, off, 0);
    }
  };

  float m_i = -INFINITY, l_i = 0.f;
  f32x16_t acc_o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc_o[t] = zero16();
  const int tq = q0 + (lane & 31);

  // One key block on LDS stage BUF.  The loop below runs the blocks in
  // pairs so that the stage is a constant: every LDS address is then a
  // loop-invariant register plus an immediate offset, with no per-block
  // address arithmetic on the vector ALU.
  auto key_block = [&](int kb, auto stage) {
    constexpr int buf = decltype(stage)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kb + 1 < nkb) issue(kb + 1, buf ^ 1);
    const uint8_t* Ks = smem + buf * 32768;
    const uint8_t* Vs = Ks + 16384;
    // Every wave runs every key block: a block wholly after the wave's
    // queries is fully masked (P = 0) and changes neither m nor l.
    {
      f32x16_t s_acc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s_acc[kt] = zero16();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          bf16x8_t kf = *(const bf16x8_t*)(Ks + sw256(32 * kt + (lane & 31), 2 * s + (lane >> 5)));
          s_acc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s_acc[kt], 0, 0, 0);
        }
        // Pacing: every other key block the wave waits here, after the
        // first score tile, for the next block's K and V it has just
        // requested.  A wave whose loads miss the caches is held back, so
        // the blocks of one (batch, head) sweep the keys together and share
        // their K and V tiles in L2: at 524288 tokens the forward takes
        // 10% less time with this wait, at 4096 about the same.
        if (buf == 0 && kt == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      // Only blocks that reach past the wave's first query need the causal
      // mask (wave-uniform branch).
      if (kb * 64 + 63 > q0) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s_acc[kt][r] = kb * 64 + 32 * kt + acc_row(r, lane) > tq ? -INFINITY : s_acc[kt][r];
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_acc[kt][r]);
      mx = max_halves(mx) * c;
      // Lazy rescaling: the reference max m_i moves only when the block max
      // exceeds it by more than 8 (in log2 units), so probabilities stay
      // below 2^8; the final O / l uses the same reference, so the result is
      // unchanged.  The branch is uniform across the wave.
      if (__any(mx > m_i + 8.0f)) {
        const float m_new = fmaxf(m_i, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_i - m_new);
        l_i *= alpha;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[t][r] *= alpha;
        m_i = m_new;
      }
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s_acc[kt][r], c, -m_i));
          s_acc[kt][r] = p;
          rs += p;
        }
      l_i += sum_halves(rs);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t pf = acc_to_frag(s_acc[ks >> 1], ks & 1);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          const bf16x8_t vf = frag_tr(Vs, 16 * ks, 32 * ht, lane);
          acc_o[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc_o[ht], 0, 0, 0);
        }
      }
    }
  };
  issue(0, 0);
  vm_wait_all();
  for (int kb = 0; kb < nkb; kb += 2) {
    key_block(kb, std::integral_constant<int, 0>{});
    if (kb + 1 < nkb) key_block(kb + 1, std::integral_constant<int, 1>{});
  }
  __syncthreads();

  // O^T accumulators -> LDS [query][hd] -> coalesced rows of o.  Registers
  // 4g..4g+3 hold 4 adjacent hd rows of the lane's query: one 8-byte write.
  // Rows are padded to 272 bytes, so the 32 queries of one write fall on 16
  // bank groups.
  constexpr int OLD = HD + 8;
  uint16_t* Os = (uint16_t*)(smem + wave * (32 * OLD * 2));
  if (active) {
    const float inv_l = 1.0f / l_i;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = (uint32_t)f32_to_bf16(acc_o[ht][4 * g] * inv_l) | ((uint32_t)f32_to_bf16(acc_o[ht][4 * g + 1] * inv_l) << 16);
        w.y = (uint32_t)f32_to_bf16(acc_o[ht][4 * g + 2] * inv_l) |
              ((uint32_t)f32_to_bf16(acc_o[ht][4 * g + 3] * inv_l) << 16);
        *(uint2*)(Os + (lane & 31) * OLD + 32 * ht + acc_row(4 * g, lane)) = w;
      }
    if (lane < 32) lse[(int64_t)bh * T + tq] = m_i + log2f(l_i);
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = lane + 64 * i;
      const int r = id >> 4, ch = id & 15;
      *(u32x4_t*)(o + (rowbase + q0 + r) * d + h * HD + 8 * ch) = *(const u32x4_t*)(Os + r * OLD + 8 * ch);
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
// One block = 128 keys of one (batch, head); query tiles of 32 stream
// through a double-buffered LDS ring filled by buffer_load ... lds.
__global__ void __launch_bounds__(256, 2) k_attn_dkdv_bf16(const uint16_t* __restrict__ qkv,
                                                           const uint16_t* __restrict__ dO,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ Dsum,
                                                           uint16_t* __restrict__ dqkvT, int64_t ldT, int T, int H) {
  constexpr int HD = 128;
  constexpr int QT = 32;                       // queries per tile
  constexpr int TILE = QT * HD * 2;            // 8 KiB per operand tile
  // K, V (64 KiB) and one stage of Q, dO (16 KiB): 80 KiB, so that two
  // blocks share a CU and each hides the other's tile loads.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 32768 + 2 * TILE];
  uint8_t* Ks = smem;
  uint8_t* Vs = smem + 32768;

  const BlockXY blk = xcd_block();
  const int kblk = blk.x;
  const int bh = blk.y, b = bh / H, h = bh % H;
  const int d = H * HD;
  const int64_t ld = 3LL * d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Each operand tile is 8 KiB = 8 direct-load kilobytes (4 rows of 256 B
  // each): wave w writes kilobytes 2w and 2w+1 of both tiles.  Q^T and dO^T
  // fragments come from the same tiles by transposing reads.  Descriptors
  // start at the tile's first query row (32-bit offsets for any length).
  const uint16_t* qcol = qkv + rowbase * ld + h * HD;
  const uint16_t* ocol = dO + rowbase * d + h * HD;
  auto issue = [&](int n) {
    uint8_t* st = smem + 65536;
    const int64_t q0 = (int64_t)n * QT;
    const i32x4_t qrs = make_rsrc(qcol + q0 * ld, (uint32_t)(QT * ld * 2));
    const i32x4_t ors = make_rsrc(ocol + q0 * d, (uint32_t)(QT * d * 2));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = wave * 2 + i;
      const int r = 4 * j + (lane >> 4), ch = (lane & 15) ^ swkey(r);
      dma16(qrs, st + j * 1024, (int)((r * ld + 8 * ch) * 2), 0);
      dma16(ors, st + TILE + j * 1024, (int)((r * d + 8 * ch) * 2), 0);
    }
  };
  // lse and D of the tile's queries in this lane's accumulator rows: rows
  // 4g .. 4g+3 are one 16-byte load.
  float4 ls[4], ds[4];
  auto load_stats = [&](int n) {
    const float* lp = lse + (int64_t)bh * T + n * QT;
    const float* dp = Dsum + (int64_t)bh * T + n * QT;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      ls[g] = *(const float4*)(lp + acc_row(4 * g, lane));
      ds[g] = *(const float4*)(dp + acc_row(4 * g, lane));
    }
  };

  f32x16_t acc_dk[4], acc_dv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc_dk[t] = zero16();
    acc_dv[t] = zero16();
  }
  const int key = k0 + (lane & 31);
  const int n0 = kbase / QT, n1 = T / QT;

  const uint8_t* Qs = smem + 65536;
  const uint8_t* dOs = Qs + TILE;
  for (int n = n0; n < n1; ++n) {
    if (n > n0) __syncthreads();  // every wave is done with tile n-1
    issue(n);
    load_stats(n);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int qbase = n * QT;
    // Every wave runs every tile: a tile wholly before the wave's keys gets
    // P = 0 from the causal mask, so the accumulators never leave the MFMA
    // register file inside the loop.
    {
      f32x16_t s_acc = zero16(), dp_acc = zero16();
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int ch = 2 * s + (lane >> 5);
        const bf16x8_t qf = *(const bf16x8_t*)(Qs + sw256(lane & 31, ch));
        const bf16x8_t kf = *(const bf16x8_t*)(Ks + sw256(32 * wave + (lane & 31), ch));
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf, s_acc, 0, 0, 0);
        const bf16x8_t of = *(const bf16x8_t*)(dOs + sw256(lane & 31, ch));
        const bf16x8_t vf = *(const bf16x8_t*)(Vs + sw256(32 * wave + (lane & 31), ch));
        dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(of, vf, dp_acc, 0, 0, 0);
      }
      // rows = queries of the tile, column = this lane's key
      const bool masked = k0 + 31 > qbase;  // wave-uniform
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = acc_row(r, lane);
        const float lq = ((const float*)&ls[r >> 2])[r & 3];
        const float dq = ((const float*)&ds[r >> 2])[r & 3];
        const float e = __builtin_amdgcn_exp2f(fmaf(s_acc[r], c, -lq));
        const float p = (!masked || key <= qbase + qi) ? e : 0.f;
        s_acc[r] = p;
        dp_acc[r] = p * (dp_acc[r] - dq);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t pf = acc_to_frag(s_acc, ks);
        const bf16x8_t dsf = acc_to_frag(dp_acc, ks);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          const bf16x8_t oT = frag_tr(dOs, 16 * ks, 32 * ht, lane);
          acc_dv[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oT, pf, acc_dv[ht], 0, 0, 0);
          const bf16x8_t qT = frag_tr(Qs, 16 * ks, 32 * ht, lane);
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
__global__ void __launch_bounds__(256, 2) k_attn_dq_bf16(const uint16_t* __restrict__ qkv,
                                                         const uint16_t* __restrict__ dO,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ Dsum,
                                                         uint16_t* __restrict__ dqkvT, int64_t ldT, int T, int H) {
  constexpr int HD = 128;
  // Two stages of 32 keys: K, V [32 keys x 256 B], 16 KiB each (K^T
  // fragments come from the K tile by transposing reads).
  constexpr int KB = 32, STAGE = 2 * 8192;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  const int nqb = (T + 127) / 128;
  const BlockXY blk = xcd_block();
  const int qb = nqb - 1 - blk.x;
  const int bh = blk.y, b = bh / H, h = bh % H;
  const int d = H * HD;
  const int64_t ld = 3LL * d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  const int nkb = min(T, (qb + 1) * 128) / KB;
  // 8 direct-load kilobytes per tile (4 rows of 256 B each); wave w writes
  // kilobytes 2w, 2w+1 of each.  Descriptors start at the tile's first key
  // row (32-bit offsets for any length).
  const uint16_t* kcol = qkv + rowbase * ld + d + h * HD;
  const uint16_t* vcol = kcol + d;
  auto issue = [&](int kb, int buf) {
    uint8_t* Ks = smem + buf * STAGE;
    uint8_t* Vs = Ks + 8192;
    const int64_t key0 = (int64_t)kb * KB;
    const i32x4_t krs = make_rsrc(kcol + key0 * ld, (uint32_t)(KB * ld * 2));
    const i32x4_t vrs = make_rsrc(vcol + key0 * ld, (uint32_t)(KB * ld * 2));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int j = wave * 2 + i;
      const int r = 4 * j + (lane >> 4), ch = (lane & 15) ^ swkey(r);
      const int voff = (int)((r * ld + 8 * ch) * 2);
      dma16(krs, Ks + j * 1024, voff, 0);
      dma16(vrs, Vs + j * 1024, voff, 0);
    }
  };

  f32x16_t acc_dq[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc_dq[t] = zero16();

  // One key tile on LDS stage BUF; tiles run in pairs so that the stage is
  // a constant (immediate LDS offsets, as in the forward).
  auto key_tile = [&](int kb, auto stage) {
    constexpr int buf = decltype(stage)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kb + 1 < nkb) issue(kb + 1, buf ^ 1);
    const uint8_t* Ks = smem + buf * STAGE;
    const uint8_t* Vs = Ks + 8192;
    // Every wave runs every key tile: one wholly after the wave's queries
    // gets P = 0 from the causal mask.
    {
      {
        const int kt = 0;
        const int kstart = kb * KB;
        f32x16_t s_acc = zero16(), dp_acc = zero16();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int ch = 2 * s + (lane >> 5);
          const bf16x8_t kf = *(const bf16x8_t*)(Ks + sw256(32 * kt + (lane & 31), ch));
          s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s_acc, 0, 0, 0);
          const bf16x8_t vf = *(const bf16x8_t*)(Vs + sw256(32 * kt + (lane & 31), ch));
          dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, of[s], dp_acc, 0, 0, 0);
        }
        if (kstart + 31 > q0) {  // sub-tile reaches past the wave's first query
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kstart + acc_row(r, lane);
            const float e = __builtin_amdgcn_exp2f(fmaf(s_acc[r], c, -lse_q));
            const float p = key <= tq ? e : 0.f;
            dp_acc[r] = p * (dp_acc[r] - D_q);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s_acc[r], c, -lse_q));
            dp_acc[r] = p * (dp_acc[r] - D_q);
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8_t dsf = acc_to_frag(dp_acc, ks);
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) {
            const bf16x8_t kT = frag_tr(Ks, 16 * ks, 32 * ht, lane);
            acc_dq[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kT, dsf, acc_dq[ht], 0, 0, 0);
          }
        }
      }
    }
  };
  issue(0, 0);
  vm_wait_all();
  for (int kb = 0; kb < nkb; kb += 2) {
    key_tile(kb, std::integral_constant<int, 0>{});
    if (kb + 1 < nkb) key_tile(kb + 1, std::integral_constant<int, 1>{});
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
void attn_fwd<uint16_t>(const uint16_t* qkv, uint16_t* o, float* lse, int B, int T_, int H, int hd, hipStream_t s) {
  if (hd != 128 || T_ % 64) throw ApiError{MT_E_INVALID, "bf16 attention needs head_dim 128, seq_len % 64 == 0"};
  hipLaunchKernelGGL(k_attn_fwd_bf16, dim3((T_ + 127) / 128, B * H), dim3(256), 0, s, qkv, o, lse, T_, H);
}

template <>
void attn_fwd<float>(const float* qkv, float* o, float* lse, int B, int T_, int H, int hd, hipStream_t s) {
  if (hd > kMaxHd) throw ApiError{MT_E_INVALID, "fp32 attention needs head_dim <= 64"};
  hipLaunchKernelGGL(k_attn_fwd_f32, dim3((T_ + 63) / 64, B * H), dim3(64), 0, s, qkv, o, lse, T_, H, hd);
}

// bf16, head_dim 128: 16 lanes per (token, head) row, 8 elements (16 bytes)
// each, summed in a fixed butterfly.
__global__ void __launch_bounds__(256) k_dsum_bf16(const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O,
                                                   float* __restrict__ Dsum, int T_, int H, int64_t rows) {
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;  // row = m*H + h
  const int sub = threadIdx.x & 15;
  if (row >= rows) return;  // whole 16-lane groups leave together
  const int64_t off = row * 128 + sub * 8;
  const u32x4_t a = *(const u32x4_t*)(dO + off);
  const u32x4_t b = *(const u32x4_t*)(O + off);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc += bf16_to_f32(a[i] & 0xFFFF) * bf16_to_f32(b[i] & 0xFFFF);
    acc += bf16_to_f32(a[i] >> 16) * bf16_to_f32(b[i] >> 16);
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (sub == 0) {
    const int64_t m = row / H, bb = m / T_, t = m % T_;
    Dsum[(bb * H + row % H) * T_ + t] = acc;
  }
}

template <typename T>
void attn_bwd_dsum(const T* dO, const T* O, float* Dsum, int B, int T_, int H, int hd, hipStream_t s) {
  const int64_t rows = (int64_t)B * T_ * H;
  if (rows <= 0) return;
  if (std::is_same<T, uint16_t>::value && hd == 128 && ((uintptr_t)dO & 15) == 0 && ((uintptr_t)O & 15) == 0) {
    hipLaunchKernelGGL(k_dsum_bf16, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, (const uint16_t*)dO,
                       (const uint16_t*)O, Dsum, T_, H, rows);
    return;
  }
  hipLaunchKernelGGL(k_dsum<T>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, dO, O, Dsum, T_, H, hd, rows);
}
template void attn_bwd_dsum<float>(const float*, const float*, float*, int, int, int, int, hipStream_t);
template void attn_bwd_dsum<uint16_t>(const uint16_t*, const uint16_t*, float*, int, int, int, int, hipStream_t);

template <>
void attn_bwd<uint16_t>(const uint16_t* qkv, const uint16_t* dO, const float* lse, const float* Dsum, uint16_t* dqkvT,
                        int64_t ldT, int B, int T_, int H, int hd, hipStream_t s) {
  if (hd != 128 || T_ % 64) throw ApiError{MT_E_INVALID, "bf16 attention needs head_dim 128, seq_len % 64 == 0"};
  if (ldT < (int64_t)B * T_) throw ApiError{MT_E_INVALID, "ldT must be >= batch*seq_len"};
  hipLaunchKernelGGL(k_attn_dkdv_bf16, dim3((T_ + 127) / 128, B * H), dim3(256), 0, s, qkv, dO, lse, Dsum, dqkvT, ldT,
                     T_, H);
  hipLaunchKernelGGL(k_attn_dq_bf16, dim3((T_ + 127) / 128, B * H), dim3(256), 0, s, qkv, dO, lse, Dsum, dqkvT, ldT,
                     T_, H);
}

template <>
void attn_bwd<float>(const float* qkv, const float* dO, const float* lse, const float* Dsum, float* dqkvT,
                     int64_t ldT, int B, int T_, int H, int hd, hipStream_t s) {
  if (hd > kMaxHd) throw ApiError{MT_E_INVALID, "fp32 attention needs head_dim <= 64"};
  if (ldT < (int64_t)B * T_) throw ApiError{MT_E_INVALID, "ldT must be >= batch*seq_len"};
  hipLaunchKernelGGL(k_attn_dkdv_f32, dim3((T_ + 63) / 64, B * H), dim3(64), 0, s, qkv, dO, lse, Dsum, dqkvT, ldT, T_,
                     H, hd);
  hipLaunchKernelGGL(k_attn_dq_f32, dim3((T_ + 63) / 64, B * H), dim3(64), 0, s, qkv, dO, lse, Dsum, dqkvT, ldT, T_, H,
                     hd);
}

}  // namespace mt
