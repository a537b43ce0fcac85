// extern "C" entry points of include/mt_kernels.h.
#include <cmath>
#include <vector>

#include "kernels.h"
#include "mt_kernels.h"

namespace mt {
template <typename F>
static int kguard(F&& f) {
  try {
    f();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) throw HipError{e, "kernel launch"};
    return MT_OK;
  } catch (const ApiError& e) {
    set_error(e.msg);
    return e.code;
  } catch (const HipError& e) {
    set_error(std::string(hipGetErrorString(e.code)) + " in " + e.where);
    return MT_E_HIP;
  }
}
static void need(bool ok, const char* msg) {
  if (!ok) throw ApiError{MT_E_INVALID, msg};
}
}  // namespace mt

using namespace mt;

extern "C" {

int mt_gemm(int32_t dtype, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
            const float* R, int64_t ldr, int32_t M, int32_t N, int32_t K, int32_t epi, int32_t layout, void* stream) {
  return kguard([&] {
    need(epi >= 0 && epi <= 2, "epi");
    need(layout >= 0 && layout <= 3, "layout");
    need(M >= 0 && N >= 0 && K >= 0, "negative size");
    need((layout & MT_GEMM_A_KMAJOR ? lda >= M : lda >= K) && (layout & MT_GEMM_B_KMAJOR ? ldb >= N : ldb >= K) &&
             ldc >= N,
         "leading dimensions");
    need(epi != 2 || (R && ldr >= N), "R");
    if (dtype == MT_BF16)
      gemm_bf16((const uint16_t*)A, lda, (const uint16_t*)B, ldb, layout, C, ldc, R, ldr, M, N, K, (Epi)epi,
                (hipStream_t)stream);
    else if (dtype == MT_F32 && layout == 0)
      gemm_nt<float>((const float*)A, lda, (const float*)B, ldb, C, ldc, R, ldr, M, N, K, (Epi)epi,
                     (hipStream_t)stream);
    else
      need(false, "dtype / layout");
  });
}

int mt_gemm_ws(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, const float* R,
               int64_t ldr, int32_t M, int32_t N, int32_t K, int32_t epi, int32_t layout, void* ws, size_t ws_bytes,
               void* stream) {
  return kguard([&] {
    need(epi >= 0 && epi <= 2, "epi");
    need(layout >= 0 && layout <= 3, "layout");
    need(M >= 0 && N >= 0 && K >= 0, "negative size");
    need((layout & MT_GEMM_A_KMAJOR ? lda >= M : lda >= K) && (layout & MT_GEMM_B_KMAJOR ? ldb >= N : ldb >= K) &&
             ldc >= N,
         "leading dimensions");
    need(epi != 2 || (R && ldr >= N), "R");
    need(((uintptr_t)ws & 15) == 0, "workspace must be 16-byte aligned");
    gemm_bf16((const uint16_t*)A, lda, (const uint16_t*)B, ldb, layout, C, ldc, R, ldr, M, N, K, (Epi)epi,
              (hipStream_t)stream, (float*)ws, ws ? ws_bytes : 0);
  });
}

size_t mt_gemm_ws_bytes(int32_t M, int32_t N, int32_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return gemm_ws_bytes(M, N, K);
}

static_assert(MT_GEMM_GROUP_MAX == kGemmGroupMax, "group size");

int mt_gemm_group_ws(int32_t n, const mt_gemm_desc* d, int32_t K, int32_t epi, int32_t layout, void* ws,
                     size_t ws_bytes, void* stream) {
  return kguard([&] {
    need(n >= 1 && n <= MT_GEMM_GROUP_MAX && d, "group size");
    need(epi == 0 || epi == 1, "epi");
    need(layout >= 0 && layout <= 3, "layout");
    need(((uintptr_t)ws & 15) == 0, "workspace must be 16-byte aligned");
    GemmDesc g[kGemmGroupMax];
    for (int i = 0; i < n; ++i) {
      need(d[i].M > 0 && d[i].N > 0 && K > 0, "sizes");
      need((layout & MT_GEMM_A_KMAJOR ? d[i].lda >= d[i].M : d[i].lda >= K) &&
               (layout & MT_GEMM_B_KMAJOR ? d[i].ldb >= d[i].N : d[i].ldb >= K) && d[i].ldc >= d[i].N,
           "leading dimensions");
      g[i] = GemmDesc{(const uint16_t*)d[i].A, d[i].lda, (const uint16_t*)d[i].B, d[i].ldb, d[i].C, d[i].ldc,
                      d[i].M, d[i].N};
    }
    gemm_bf16_group(g, n, K, layout, (Epi)epi, (hipStream_t)stream, (float*)ws, ws ? ws_bytes : 0);
  });
}

size_t mt_gemm_group_ws_bytes(int32_t n, const mt_gemm_desc* d, int32_t K) {
  if (n < 1 || n > MT_GEMM_GROUP_MAX || !d || K <= 0) return 0;
  int M[kGemmGroupMax], N[kGemmGroupMax];
  for (int i = 0; i < n; ++i) {
    if (d[i].M <= 0 || d[i].N <= 0) return 0;
    M[i] = d[i].M;
    N[i] = d[i].N;
  }
  return gemm_group_ws_bytes(M, N, n, K);
}

int mt_transpose(int32_t dtype, const void* in, int64_t ld_in, void* out, int64_t ld_out, int32_t R, int32_t C,
                 void* stream) {
  return kguard([&] {
    need(ld_in >= C && ld_out >= R, "leading dimensions");
    if (dtype == MT_BF16)
      transpose<uint16_t>((const uint16_t*)in, ld_in, (uint16_t*)out, ld_out, R, C, (hipStream_t)stream);
    else if (dtype == MT_F32)
      transpose<float>((const float*)in, ld_in, (float*)out, ld_out, R, C, (hipStream_t)stream);
    else
      need(false, "dtype");
  });
}

int mt_rope_tables(int32_t T, int32_t hd, double theta, float* cos_out, float* sin_out) {
  return kguard([&] {
    need(T > 0 && hd > 0 && hd % 2 == 0 && cos_out && sin_out, "arguments");
    for (int t = 0; t < T; ++t)
      for (int i = 0; i < hd / 2; ++i) {
        const double a = (double)t * std::pow(theta, -2.0 * i / hd);
        cos_out[(size_t)t * (hd / 2) + i] = (float)std::cos(a);
        sin_out[(size_t)t * (hd / 2) + i] = (float)std::sin(a);
      }
  });
}

int64_t mt_token_ld(int64_t tokens) { return token_ld(tokens); }

int mt_rope_qkv(int32_t dtype, void* qkv, const float* cos_t, const float* sin_t, int32_t B, int32_t T, int32_t H,
                int32_t hd, void* stream) {
  return kguard([&] {
    need(B > 0 && T > 0 && H > 0 && hd > 0 && hd % 2 == 0 && hd <= 128, "shape");
    const int M = B * T, d = H * hd;
    if (dtype == MT_BF16)
      rope_qkv_fwd<uint16_t>((uint16_t*)qkv, cos_t, sin_t, M, T, d, hd, (hipStream_t)stream);
    else if (dtype == MT_F32)
      rope_qkv_fwd<float>((float*)qkv, cos_t, sin_t, M, T, d, hd, (hipStream_t)stream);
    else
      need(false, "dtype");
  });
}

int mt_attention_fwd(int32_t dtype, const void* qkv, void* o, float* lse, int32_t B, int32_t T, int32_t H, int32_t hd,
                     void* stream) {
  return kguard([&] {
    need(B > 0 && T > 0 && H > 0 && hd > 0, "shape");
    if (dtype == MT_BF16)
      attn_fwd<uint16_t>((const uint16_t*)qkv, (uint16_t*)o, lse, B, T, H, hd, (hipStream_t)stream);
    else if (dtype == MT_F32)
      attn_fwd<float>((const float*)qkv, (float*)o, lse, B, T, H, hd, (hipStream_t)stream);
    else
      need(false, "dtype");
  });
}

int mt_attention_bwd(int32_t dtype, const void* qkv, const void* o, const void* dO, const float* lse, float* Dsum,
                     void* dqkvT, int64_t ldT, int32_t B, int32_t T, int32_t H, int32_t hd, void* stream) {
  return kguard([&] {
    need(B > 0 && T > 0 && H > 0 && hd > 0, "shape");
    hipStream_t s = (hipStream_t)stream;
    if (dtype == MT_BF16) {
      attn_bwd_dsum<uint16_t>((const uint16_t*)dO, (const uint16_t*)o, Dsum, B, T, H, hd, s);
      attn_bwd<uint16_t>((const uint16_t*)qkv, (const uint16_t*)dO, lse, Dsum, (uint16_t*)dqkvT, ldT, B, T, H, hd, s);
    } else if (dtype == MT_F32) {
      attn_bwd_dsum<float>((const float*)dO, (const float*)o, Dsum, B, T, H, hd, s);
      attn_bwd<float>((const float*)qkv, (const float*)dO, lse, Dsum, (float*)dqkvT, ldT, B, T, H, hd, s);
    } else {
      need(false, "dtype");
    }
  });
}

#define MT_DT_DISPATCH(dtype, F_)       \
  if (dtype == MT_BF16) {               \
    F_(uint16_t)                        \
  } else if (dtype == MT_F32) {         \
    F_(float)                           \
  } else {                              \
    need(false, "dtype");               \
  }

int mt_rmsnorm_fwd(int32_t dtype, const float* x, const void* g, void* y, float* rstd, int32_t M, int32_t d, float eps,
                   void* stream) {
  return kguard([&] {
    need(M >= 0 && d > 0 && eps > 0, "shape");
#define F_(T) rmsnorm_fwd<T>(x, (const T*)g, (T*)y, rstd, M, d, eps, (hipStream_t)stream);
    MT_DT_DISPATCH(dtype, F_)
#undef F_
  });
}

int mt_rmsnorm_fwd_res(int32_t dtype, const float* res, float* x, const void* g, void* y, float* rstd, int32_t M,
                       int32_t d, float eps, void* stream) {
  return kguard([&] {
    need(M >= 0 && d > 0 && eps > 0, "shape");
#define F_(T) rmsnorm_fwd_res<T>(res, x, (const T*)g, (T*)y, rstd, M, d, eps, (hipStream_t)stream);
    MT_DT_DISPATCH(dtype, F_)
#undef F_
  });
}

size_t mt_rmsnorm_bwd_ws_bytes(int32_t M, int32_t d) {
  if (M < 0 || d <= 0) return 0;
  return rmsnorm_dg_partial_elems(M, d) * sizeof(float);
}

int mt_rmsnorm_bwd(int32_t dtype, const float* dy, const float* x, const void* g, const float* rstd,
                   const float* resid, float* dx, void* dx_lp, void* dg, float* ws, int32_t M, int32_t d,
                   void* stream) {
  return kguard([&] {
    need(M >= 0 && d > 0 && ws, "shape / workspace");
#define F_(T) rmsnorm_bwd<T>(dy, x, (const T*)g, rstd, resid, dx, ws, (T*)dg, M, d, (hipStream_t)stream, (T*)dx_lp);
    MT_DT_DISPATCH(dtype, F_)
#undef F_
  });
}

int mt_swiglu_fwd(int32_t dtype, const void* gu, void* y, int32_t M, int32_t F, void* stream) {
  return kguard([&] {
    need(M >= 0 && F > 0, "shape");
#define F_(T) swiglu_fwd<T>((const T*)gu, (T*)y, M, F, (hipStream_t)stream);
    MT_DT_DISPATCH(dtype, F_)
#undef F_
  });
}

int mt_swiglu_bwd(int32_t dtype, const void* dy, const void* gu, void* dgu, int32_t M, int32_t F, void* stream) {
  return kguard([&] {
    need(M >= 0 && F > 0, "shape");
#define F_(T) swiglu_bwd<T>((const T*)dy, (const T*)gu, (T*)dgu, M, F, (hipStream_t)stream);
    MT_DT_DISPATCH(dtype, F_)
#undef F_
  });
}

int mt_rope_bwd_t(int32_t dtype, void* dqkvT, int64_t ldT, const float* cos_T, const float* sin_T, int32_t B,
                  int32_t T, int32_t H, int32_t hd, void* stream) {
  return kguard([&] {
    need(B > 0 && T > 0 && H > 0 && hd > 0 && hd % 2 == 0 && hd <= 128 && ldT >= (int64_t)B * T, "shape");
    const int M = B * T, d = H * hd;
#define F_(T_) rope_bwd_T<T_>((T_*)dqkvT, ldT, cos_T, sin_T, M, T, d, hd, (hipStream_t)stream);
    MT_DT_DISPATCH(dtype, F_)
#undef F_
  });
}

int mt_xent(int32_t dtype, const float* logits, const int32_t* tok, float* row_loss, void* dlogits, int32_t rows,
            int64_t row0, int32_t T, int32_t V, float inv_n, void* stream) {
  return kguard([&] {
    need(rows >= 0 && row0 >= 0 && T > 1 && V > 1, "shape");
#define F_(T_) xent<T_>(logits, tok, row_loss, (T_*)dlogits, rows, row0, T, V, inv_n, (hipStream_t)stream);
    MT_DT_DISPATCH(dtype, F_)
#undef F_
  });
}

int mt_embed_fwd(int32_t dtype, const int32_t* tok, const void* E, float* x, int32_t M, int32_t d, void* stream) {
  return kguard([&] {
    need(M >= 0 && d > 0, "shape");
#define F_(T) embed_fwd<T>(tok, (const T*)E, x, M, d, (hipStream_t)stream);
    MT_DT_DISPATCH(dtype, F_)
#undef F_
  });
}

int mt_embed_bwd(int32_t dtype, const float* dx, const int32_t* order, const int32_t* seg, void* dE, int32_t V,
                 int32_t d, void* stream) {
  return kguard([&] {
    need(V > 0 && d > 0, "shape");
#define F_(T) embed_bwd<T>(dx, order, seg, (T*)dE, V, d, (hipStream_t)stream);
    MT_DT_DISPATCH(dtype, F_)
#undef F_
  });
}

}  // extern "C"
