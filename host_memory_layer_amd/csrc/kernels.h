// Launchers of the device kernels.  T is the storage type of weights and of
// GEMM operands: float (all-fp32 store) or uint16_t (bf16 bit patterns).
// Every launcher enqueues on `s` and returns without synchronising.
#pragma once

#include "common.h"

namespace mt {

// ---------------------------------------------------------------- GEMM --
// C[M x N] = A[M x K] . B[N x K]^T, both operands K-contiguous (row stride
// lda / ldb elements), fp32 accumulation.  Epilogues:
enum Epi {
  EPI_STORE = 0,   // C (type T) = acc, rounded to nearest-even for bf16
  EPI_F32 = 1,     // C (float) = acc
  EPI_ADD_F32 = 2,  // C (float) = R + acc, R float [M x N] with row stride ldr
  EPI_PARTIAL = 3   // internal to the bf16 GEMM: a stream-K partial tile into the workspace
};
template <typename T>
void gemm_nt(const T* A, int64_t lda, const T* B, int64_t ldb, void* C, int64_t ldc, const float* R,
             int64_t ldr, int M, int N, int K, Epi epi, hipStream_t s);
// bf16 with operand layouts: an operand is K-contiguous ([M x K] or [N x K],
// as in gemm_nt) or, with its bit in `layout`, K-major ([K x M] or [K x N],
// row stride lda / ldb), read through transposing LDS loads.  K-major
// operands need gemm_layout_ok().
enum GemmLayout { GEMM_A_KMAJOR = 1, GEMM_B_KMAJOR = 2 };
bool gemm_layout_ok(int M, int N, int K, int64_t lda, int64_t ldb, int layout);
// With a device workspace `ws` of at least gemm_ws_bytes(M, N, K) bytes,
// a GEMM whose last round of tiles would leave part of the GPU idle splits
// that round's tiles along K over every workgroup (stream-K) and adds the
// partial tiles in a fixed order in a second kernel: the results then
// differ from the unsplit GEMM by rounding in those tiles only, and still
// depend only on the shapes.  Without it (or with a smaller one) every tile
// is computed whole.
void gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int layout, void* C, int64_t ldc,
               const float* R, int64_t ldr, int M, int N, int K, Epi epi, hipStream_t s, float* ws = nullptr,
               size_t ws_bytes = 0);
// Workspace bytes the split needs for this shape (0: no split planned).
size_t gemm_ws_bytes(int M, int N, int K);
// Up to kGemmGroupMax bf16 products sharing K and the operand layout (store
// or fp32 epilogue, no residual) in one persistent launch: their tiles form
// one tile space, so one product's partial last round is filled with
// another's tiles, and a stream-K split covers the group's last round.
// Every tile is computed as by gemm_bf16; tiles in the group's split tail
// differ from an unsplit tile by rounding only.
constexpr int kGemmGroupMax = 3;
struct GemmDesc {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  void* C;
  int64_t ldc;
  int M, N;
};
void gemm_bf16_group(const GemmDesc* d, int n, int K, int layout, Epi epi, hipStream_t s, float* ws = nullptr,
                     size_t ws_bytes = 0);
size_t gemm_group_ws_bytes(const int* M, const int* N, int n, int K);

// ---------------------------------------------------------- elementwise --
template <typename T>
void embed_fwd(const int32_t* tok, const T* E, float* x, int M, int d, hipStream_t s);
// dE[v] = sum over positions m with tok[m] == v, in increasing m, of dx[m];
// order[] lists positions sorted by token (stable), seg[v]..seg[v+1] its range.
template <typename T>
void embed_bwd(const float* dx, const int32_t* order, const int32_t* seg, T* dE, int V, int d, hipStream_t s);
template <typename T>
void rmsnorm_fwd(const float* x, const T* g, T* y, float* rstd, int M, int d, float eps, hipStream_t s);
// x = res + x in place (fp32 add), then the same norm of x: the residual
// add of a projection whose GEMM wrote only its product.
template <typename T>
void rmsnorm_fwd_res(const float* res, float* x, const T* g, T* y, float* rstd, int M, int d, float eps,
                     hipStream_t s);
// dx = resid + r*(dy*g - xh*mean(dy*g*xh)), xh = x*r (resid may be null),
// (and, with dx_lp, dx rounded to T beside it: the operand of the next GEMM)
// and dg = sum_rows dy*xh written as T: per-block partial sums in `partial`
// (rmsnorm_dg_partial_elems(M, d) floats), then added in a fixed order that
// depends only on (M, d).
size_t rmsnorm_dg_partial_elems(int M, int d);
template <typename T>
void rmsnorm_bwd(const float* dy, const float* x, const T* g, const float* rstd, const float* resid, float* dx,
                 float* partial, T* dg, int M, int d, hipStream_t s, T* dx_lp = nullptr);
// With dg null, rmsnorm_bwd writes only the per-block partial sums (blocks
// of rmsnorm_rows_per_block() consecutive rows); rmsnorm_dg_reduce adds
// `blocks` of them in block order.  Rows processed in several calls, each
// starting at a multiple of the block rows with its partials at the matching
// block offset, reduce to the same dg as one call over all rows.
template <typename T>
void rmsnorm_dg_reduce(const float* partial, T* dg, int blocks, int d, hipStream_t s);
int rmsnorm_rows_per_block();
// Token-major transposed buffers [C x M] use a padded row stride
// (token_ld(M) >= M): a row stride that is a large power of two puts a
// tile's rows on the same memory channels.
int64_t token_ld(int64_t M);
// Rotate q and k of qkv [M x 3d] in place (pairs (i, i+hd/2), angle
// t*theta^(-2i/hd), t = (row0 + m) mod T: row0 is the batch row of qkv's
// first row when qkv points into a larger buffer).
template <typename T>
void rope_qkv_fwd(T* qkv, const float* cosb, const float* sinb, int M, int T_, int d, int hd, hipStream_t s,
                  int64_t row0 = 0);
// Inverse rotation of the dq, dk rows of dqkvT [3d x M] (row stride ldT), in
// place; cosT, sinT are the rotation tables transposed, [hd/2 x T].
template <typename T>
void rope_bwd_T(T* dqkvT, int64_t ldT, const float* cosT, const float* sinT, int M, int T_, int d, int hd,
                hipStream_t s);
template <typename T>
void swiglu_fwd(const T* gu, T* y, int M, int F, hipStream_t s);
template <typename T>
void swiglu_bwd(const T* dy, const T* gu, T* dgu, int M, int F, hipStream_t s);
// Row-wise loss and gradient of the mean next-token cross-entropy over the
// token rows m = row0 .. row0+rows-1 (logits and dlogits hold those rows):
// rows with t = m mod T < T-1 have label tok[m+1]; others get loss 0, grad 0.
// row_loss is indexed by m.
template <typename T>
void xent(const float* logits, const int32_t* tok, float* row_loss, T* dlogits, int rows, int64_t row0, int T_, int V,
          float inv_n, hipStream_t s);
// out[0] = (sum of x[0..n) in a fixed order) * scale.
void sum_fixed(const float* x, float* out, int n, float scale, hipStream_t s);
// out[C x R] = in[R x C]^T.
template <typename T>
void transpose(const T* in, int64_t ld_in, T* out, int64_t ld_out, int R, int C, hipStream_t s);
// out = T(in) for n floats.
template <typename T>
void cast(const float* in, T* out, int64_t n, hipStream_t s);
// out = float(in) for n bf16 values (exact).
void widen_bf16(const uint16_t* in, float* out, int64_t n, hipStream_t s);
// out = T(in) and outT = T(in)^T (row stride ldT) for in float [R x C].
template <typename T>
void cast_transpose(const float* in, T* out, T* outT, int64_t ldT, int R, int C, hipStream_t s);
void fill_u32(void* p, uint32_t value, size_t n_words, hipStream_t s);

// ------------------------------------------------------------ attention --
// qkv [M x 3d] (q, k rotated); o [M x d];
// lse [B*H x T] (base-2 log-sum-exp of the scaled scores).
template <typename T>
void attn_fwd(const T* qkv, T* o, float* lse, int B, int T_, int H, int hd, hipStream_t s);
// Dsum[b*H+h][t] = sum_i dO . O over the head.
template <typename T>
void attn_bwd_dsum(const T* dO, const T* O, float* Dsum, int B, int T_, int H, int hd, hipStream_t s);
// dqkvT [3d x M] (row stride ldT) receives dq, dk, dv transposed.
template <typename T>
void attn_bwd(const T* qkv, const T* dO, const float* lse, const float* Dsum, T* dqkvT, int64_t ldT, int B, int T_,
              int H, int hd, hipStream_t s);

}  // namespace mt
