/*
 * mt_kernels.h — C ABI of the individual device kernels that one training
 * step of the layer-streamed decoder is made of (the same code mt_train_step
 * launches), for testing and reuse.
 *
 * Pointers are device addresses unless said otherwise; `stream` is a
 * hipStream_t (null = the default stream).  Calls enqueue and return without
 * synchronising; they return 0 or a negative MT_E_* code (mt.h) and set
 * mt_last_error().  dtype is MT_BF16 (elements are bfloat16 bit patterns,
 * uint16) or MT_F32.
 */
#ifndef MT_KERNELS_H
#define MT_KERNELS_H

#include "mt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C[M x N] = sum_k A(m, k) B(n, k), fp32 accumulation.  Operand layouts
 * (bits of `layout`): A is [M x K] row-major (K-contiguous, row stride lda)
 * or, with MT_GEMM_A_KMAJOR, [K x M] (row stride lda); B likewise [N x K] or,
 * with MT_GEMM_B_KMAJOR, [K x N].  epi 0: C has dtype (bf16 rounded to
 * nearest-even); epi 1: C is float; epi 2: C (float) = R + A.B with R float
 * [M x N], row stride ldr.  bf16 needs K, lda, ldb multiples of 8 and
 * 16-byte aligned A, B; K-major operands also need K % 64 == 0, K >= 192 and
 * K * ld * 2 < 2^31 (else MT_E_INVALID); f32 supports layout 0 only.  Every
 * dense projection of the layer is one of these: forward Y = X W^T (layout
 * 0), data gradient dX = dY W (B K-major), weight gradient dW = dY^T X
 * (both K-major, K = tokens). */
#define MT_GEMM_A_KMAJOR 1
#define MT_GEMM_B_KMAJOR 2
int mt_gemm(int32_t dtype, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
            const float* R, int64_t ldr, int32_t M, int32_t N, int32_t K, int32_t epi, int32_t layout, void* stream);

/* mt_gemm for bf16 with a caller-owned device workspace `ws` (16-byte
 * aligned, ws_bytes long, not read before it is written).  When the last
 * round of 256 x 256 tiles would leave at least 5% of the persistent
 * workgroups idle, the tiles of that round are split along K over every
 * workgroup (stream-K) and a second kernel adds each tile's partial sums in
 * K order, then applies the epilogue.  Those tiles then differ from mt_gemm
 * by fp32 rounding; every other tile is bit-identical, and all results
 * depend only on the shapes.  With ws null or ws_bytes <
 * mt_gemm_ws_bytes(M, N, K) this is mt_gemm.  The training step uses the
 * same split for its weight gradients (the layer's d x d and d x F shapes
 * leave a partial last round on 256 compute units). */
int mt_gemm_ws(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, const float* R,
               int64_t ldr, int32_t M, int32_t N, int32_t K, int32_t epi, int32_t layout, void* ws, size_t ws_bytes,
               void* stream);

/* Workspace bytes mt_gemm_ws uses for a bf16 GEMM of this shape on the
 * current device; 0 when it would not split. */
size_t mt_gemm_ws_bytes(int32_t M, int32_t N, int32_t K);

/* Up to MT_GEMM_GROUP_MAX bf16 products C_i[M_i x N_i] = A_i . B_i^T that
 * share K and the operand layout, in one persistent launch: the layer's
 * weight gradients ([Abstract]: every layer's backward produces them on the
 * GPU) have one contraction length, the tokens, and together fill the
 * device where one alone leaves a partial last round.  Each product's tiles
 * are those of mt_gemm_ws; with a workspace of mt_gemm_group_ws_bytes, the
 * group's last partial round is split along K as in mt_gemm_ws.  epi 0
 * (bf16 C) or 1 (fp32 C), no residual.  K % 64 == 0, K >= 192.  Errors:
 * MT_E_INVALID (group size, shapes, strides, alignment), MT_E_HIP. */
#define MT_GEMM_GROUP_MAX 3
typedef struct mt_gemm_desc {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C;
  int64_t ldc;
  int32_t M, N;
} mt_gemm_desc;
int mt_gemm_group_ws(int32_t n, const mt_gemm_desc* d, int32_t K, int32_t epi, int32_t layout, void* ws,
                     size_t ws_bytes, void* stream);
size_t mt_gemm_group_ws_bytes(int32_t n, const mt_gemm_desc* d, int32_t K);

/* mt_gemm_ws for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * stream-K partial tiles go to a static device buffer of the library,
 * mt_gemm_noalloc_max_ws() = 128 MiB on each GPU it runs on, held until the
 * process ends; the call allocates nothing and its results are bit for bit
 * those of mt_gemm_ws with a large enough workspace.  The buffer is written
 * before it is read within each call, so no clearing is needed.  Shapes whose
 * split needs more than the buffer return MT_E_SIZE (on 256 compute units
 * every split needs exactly 128 MiB).  All calls on one GPU share that GPU's
 * buffer: calls that overlap in time on one GPU (on different streams or from
 * different threads) race on it and must be ordered by the caller, e.g. on
 * one stream. */
int mt_gemm_noalloc(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, const float* R,
                    int64_t ldr, int32_t M, int32_t N, int32_t K, int32_t epi, int32_t layout, void* stream);
size_t mt_gemm_noalloc_max_ws(void);

/* out[C x R] = in[R x C]^T (row strides ld_in, ld_out). */
int mt_transpose(int32_t dtype, const void* in, int64_t ld_in, void* out, int64_t ld_out, int32_t R, int32_t C,
                 void* stream);

/* Host: RoPE tables cos/sin [T x hd/2] of angle t * theta^(-2i/hd), computed
 * in double and rounded to float (host buffers of T*hd/2 floats). */
int mt_rope_tables(int32_t T, int32_t hd, double theta, float* cos_out, float* sin_out);

/* Row stride (elements) the library uses for token-major transposed
 * buffers [C x tokens]: tokens rounded up to a multiple of 128 so that the
 * stride in 256-byte units is odd (a large power-of-two stride puts a tile's
 * rows on the same memory channels). */
int64_t mt_token_ld(int64_t tokens);

/* qkv [B*T x 3d] (q | k | v columns, head-major inside each): rotate q and k
 * in place by +t*w_i on pairs (i, i+hd/2), t = position in the sequence.
 * cos/sin: device tables from mt_rope_tables. */
int mt_rope_qkv(int32_t dtype, void* qkv, const float* cos_t, const float* sin_t, int32_t B, int32_t T, int32_t H,
                int32_t hd, void* stream);

/* Causal softmax attention per (batch, head) with scale 1/sqrt(hd).
 * Input: qkv with q, k rotated (as left by mt_rope_qkv).
 * Outputs: o [B*T x d] (dtype) and lse [B*H x T] (float, base-2
 * log-sum-exp of the scaled scores times log2(e)).  bf16: hd = 128 and
 * T % 64 == 0; f32: hd <= 64. */
int mt_attention_fwd(int32_t dtype, const void* qkv, void* o, float* lse, int32_t B, int32_t T, int32_t H, int32_t hd,
                     void* stream);

/* Backward of mt_attention_fwd given dO [B*T x d]: writes Dsum [B*H x T]
 * (float scratch, rowsum(dO * O)) and dqkvT [3d x B*T] (row stride
 * ldT >= B*T) = (dq | dk | dv)^T with respect to the rotated q, k. */
int mt_attention_bwd(int32_t dtype, const void* qkv, const void* o, const void* dO, const float* lse, float* Dsum,
                     void* dqkvT, int64_t ldT, int32_t B, int32_t T, int32_t H, int32_t hd, void* stream);

/* ---- memory-bound kernels of the layer (the operations of the decoder the
 * pages train, a Llama-style model: RMSNorm, rotary positions, SwiGLU,
 * next-token cross-entropy; dtype as above, fp32 statistics) ---- */

/* RMSNorm forward: y[m] = x[m] * rstd[m] * g, rstd[m] = 1/sqrt(mean(x[m]^2) +
 * eps).  x float [M x d]; g, y dtype [d], [M x d]; rstd float [M].  d % 4 == 0. */
int mt_rmsnorm_fwd(int32_t dtype, const float* x, const void* g, void* y, float* rstd, int32_t M, int32_t d, float eps,
                   void* stream);
/* The same with the residual add in front: x = res + x (fp32, x updated in
 * place), then y, rstd of that x.  The layer's attention output projection
 * writes o.Wo^T and this adds the residual stream (the add the projection's
 * epilogue would otherwise do).  res float [M x d]. */
int mt_rmsnorm_fwd_res(int32_t dtype, const float* res, float* x, const void* g, void* y, float* rstd, int32_t M,
                       int32_t d, float eps, void* stream);
/* RMSNorm backward given dy float [M x d] and the forward's rstd:
 * dx = resid + rstd*(dy*g - xh*mean(dy*g*xh)), xh = x*rstd (resid float [M x
 * d] or null); dx_lp (dtype [M x d], or null) receives dx rounded; dg (dtype
 * [d]) = sum over rows of dy*xh, summed in a fixed order that depends only on
 * (M, d).  ws: float scratch of mt_rmsnorm_bwd_ws_bytes(M, d) bytes. */
size_t mt_rmsnorm_bwd_ws_bytes(int32_t M, int32_t d);
int mt_rmsnorm_bwd(int32_t dtype, const float* dy, const float* x, const void* g, const float* rstd,
                   const float* resid, float* dx, void* dx_lp, void* dg, float* ws, int32_t M, int32_t d,
                   void* stream);
/* SwiGLU: gu dtype [M x 2F] (gate columns then up columns); y [M x F] =
 * silu(gate) * up.  Backward: dgu [M x 2F] = (dy * up * silu'(gate),
 * dy * silu(gate)), silu'(z) = s(z)(1 + z(1 - s(z))).  F % 4 == 0. */
int mt_swiglu_fwd(int32_t dtype, const void* gu, void* y, int32_t M, int32_t F, void* stream);
int mt_swiglu_bwd(int32_t dtype, const void* dy, const void* gu, void* dgu, int32_t M, int32_t F, void* stream);
/* RoPE backward on dqkvT [3d x ldT] (the attention backward's output): the
 * dq and dk rows are rotated back by -t*w_i in place (the dv rows are left
 * as they are); cos_T, sin_T: the tables of mt_rope_tables transposed,
 * [hd/2 x T]. */
int mt_rope_bwd_t(int32_t dtype, void* dqkvT, int64_t ldT, const float* cos_T, const float* sin_T, int32_t B,
                  int32_t T, int32_t H, int32_t hd, void* stream);
/* Next-token cross-entropy rows m = row0 .. row0+rows-1 of a batch of
 * sequences of T tokens: logits float [rows x V] (row i is token row0+i);
 * for t = m mod T < T-1, row_loss[m] = logsumexp(z) - z[tok[m+1]] and
 * dlogits row = (softmax(z) - onehot(tok[m+1])) * inv_n; the last position of
 * a sequence gets 0 and a zero row.  tok: device int32 of the whole batch;
 * row_loss: float indexed by m. */
int mt_xent(int32_t dtype, const float* logits, const int32_t* tok, float* row_loss, void* dlogits, int32_t rows,
            int64_t row0, int32_t T, int32_t V, float inv_n, void* stream);
/* Embedding: x[m] = float(E[tok[m]]) (x float [M x d]).  Backward: dE[v] =
 * sum of dx[m] over the positions with tok[m] == v, in increasing m, fp32,
 * then rounded to dtype (rows of absent tokens are 0); order: the positions
 * stably sorted by token, seg [V+1]: the start of each token's run in it. */
int mt_embed_fwd(int32_t dtype, const int32_t* tok, const void* E, float* x, int32_t M, int32_t d, void* stream);
int mt_embed_bwd(int32_t dtype, const float* dx, const int32_t* order, const int32_t* seg, void* dE, int32_t V,
                 int32_t d, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MT_KERNELS_H */
