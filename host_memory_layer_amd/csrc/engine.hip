// The layer-streamed training step: device arena, stateless layer
// templates, the three-stream prefetch / compute / offload schedule and the
// host Adam worker.
//
// MegaTrain (chatpaper.ai abstract; radar.chestersoft.de "Methodik"):
//  * parameters and optimizer state stay in host memory; the GPU is a
//    transient engine that receives one layer's weights, runs its forward or
//    backward, returns the gradients and drops the weights;
//  * a pipelined, double-buffered engine overlaps weight prefetch, compute
//    and gradient offload on three streams: while layer i computes, layer
//    i+1 loads into the second buffer (ping-pong);
//  * stateless layer templates bind the weights of whichever buffer holds
//    the layer (here: pointer arithmetic on the slot base, no graph state);
//  * the Adam step runs on the host CPU, block by block, as the gradients
//    of each block arrive, while the device continues its backward sweep.
// Only the layer-boundary activations x^l are kept (fp32, device-resident);
// each layer's forward is recomputed from x^l inside the backward sweep.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <memory>
#include <mutex>
#include <thread>
#include <type_traits>
#include <vector>

#include "adam.h"
#include "dma.h"
#include "engine.h"
#include "kernels.h"
#include "store.h"

namespace mt {

namespace {

struct Carver {
  uint8_t* base;
  uint64_t off = 0;
  template <typename P>
  P* take(uint64_t bytes) {
    off = round_up(off, 256);
    P* p = base ? (P*)(base + off) : nullptr;
    off += round_up(bytes, 256);
    return p;
  }
};

double ms_between(hipEvent_t a, hipEvent_t b) {
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return 0.0;
  return ms;
}

}  // namespace

// ------------------------------------------------------------ buffers --
template <typename T>
struct Acts {  // forward intermediates of one layer
  T *h, *qkv, *o, *h2, *gu, *y;
  float *r1, *lse, *x1, *r2;
};

template <typename T>
struct BwdWs {  // backward workspace (one set)
  T *dxb, *dxb1, *dxbT, *tmpT, *dy, *dgu, *dguT, *do_, *dqkvT, *dqkv;
  float *dh, *dx1, *Dsum, *part, *dxA, *dxB;
};

template <typename T>
struct HeadWs {
  T *z, *dlogits, *dlogitsT;       // dlogits, dlogitsT: one pass of HC tokens
  float *rz, *logits, *row_loss, *loss;
  float* gacc;                     // fp32 sum of the head weight gradient over passes (bf16, several passes)
};

template <typename T>
struct LayerW {  // a stateless layer template bound to a weight (or grad) region
  T *qkv, *o, *gu, *d, *anorm, *fnorm;
};

template <typename T>
struct LayerWT {  // transposed weights for the data-gradient contractions
  T *qkv, *o, *gu, *d;
};

template <typename T>
static LayerW<T> bind_layer(uint8_t* region, const mt_block_desc& b) {
  T* base = (T*)region;
  return LayerW<T>{base + b.tensors[T_QKV].offset, base + b.tensors[T_O].offset, base + b.tensors[T_GU].offset,
                   base + b.tensors[T_D].offset,   base + b.tensors[T_ANORM].offset, base + b.tensors[T_FNORM].offset};
}

// ---------------------------------------------------------------- model --
struct Model {
  mt_config cfg;
  std::vector<mt_block_desc> blocks;
  uint64_t store_bytes = 0, opt_bytes = 0, slot_bytes = 0;
  int L, d, H, hd, F, V, B, Tq, M;
  int64_t Mp;  // padded row stride of token-major transposed buffers
  // bf16 with supported shapes: the data- and weight-gradient GEMMs read
  // token-major activations and row-major weights as K-major operands, so
  // no activation or weight is transposed (kmajor: layers, kmajor_head: head)
  bool kmajor = false, kmajor_head = false;
  int E;  // bytes per weight element
  int HC, n_hc;  // output head: tokens per pass and passes
  int64_t HCp;   // padded row stride of one pass's transposed buffers
  // Layer token passes: a layer's per-token work (norms, projections,
  // SwiGLU) runs TC tokens at a time (n_tc passes; 1 = all tokens at once)
  int TC = 0, n_tc = 1;
  bool dqkv_kmajor = true;  // several passes: the q/k/v data gradient reads dqkvT as a K-major operand

  uint8_t* arena = nullptr;
  size_t arena_bytes = 0;
  hipStream_t sp, sc, so;  // prefetch, compute and offload streams (caller-owned)
  // Transfers: hipMemcpyAsync on the prefetch and offload streams, ordered
  // by events (hipq), or the two SDMA engine queues of dma.h
  bool hipq = true;
  bool yield_link = false;  // offloads give the host link to prefetches (see run_pass)
  uint8_t* host = nullptr;  // DMA part: header, [W | G] per block (pinned)
  uint8_t* hopt = nullptr;  // optimizer part: [m | v] per block

  // device
  uint8_t *wslot[2], *gslot[2], *wt;
  uint8_t *wres = nullptr, *gres = nullptr;  // resident mode: every block's W and G
  float* ckpt;            // fp32 layer-boundary checkpoints x^0..x^L
  // MT_FLAG_CKPT_BF16: the checkpoints are kept rounded to bf16 (ckpt16);
  // the forward carries the fp32 residual stream in two rotating buffers
  // (xrot), and the backward widens x^l into xrot[0]
  bool ckpt_lp = false;
  uint16_t* ckpt16 = nullptr;
  float* xrot[2] = {nullptr, nullptr};
  float *cosb, *sinb;  // RoPE tables [T x hd/2]
  float *cosT, *sinT;  // the same, transposed [hd/2 x T]
  int32_t *d_tok, *d_order, *d_seg;
  std::vector<uint8_t*> acts_mem;  // Acts storage per layer (1 in streamed modes)
  uint8_t* bwd_mem;
  uint8_t* head_mem;
  float* gemm_ws = nullptr;  // stream-K partial tiles of the bf16 GEMMs
  size_t gemm_ws_size = 0;
  float* dxkeep = nullptr;   // MT_FLAG_KEEP_DX: dl/dx^l of every layer boundary, l = 0..L
  float* wacc = nullptr;     // several token passes: fp32 sums of a layer's weight gradients (W region layout)
  // The bf16 copy ws.dxb mirrors one fp32 gradient at a time: the norm
  // backward that writes it records which, and the K-major backward that
  // reads it as the rounded dx2 checks that it is the dx2 it was given.
  const float* dxb_holds = nullptr;

  // host pinned
  int32_t *h_tok = nullptr, *h_order = nullptr, *h_seg = nullptr;
  float* h_loss = nullptr;

  // events per use: 0..L+1 forward (embed, layers, head), then backward L..1, 0
  int n_uses;
  std::vector<hipEvent_t> ev_c_s, ev_c_e;  // compute of each use: start, end
  std::vector<hipEvent_t> ev_slot_free;    // MT_FLAG_POISON: slot NaN-filled, ready for the prefetch of a use
  std::vector<hipEvent_t> ev_x_s, ev_x_e;  // prefetch stream: copy of each use's weights, start and end
  std::vector<hipEvent_t> ev_o_s, ev_o_e;  // offload stream: copy of each use's gradients, start and end
  std::vector<char> u_fetched, u_offloaded;  // which uses had a prefetch / an offload this pass
  hipEvent_t ev_h2d_s, ev_h2d_e, ev_d2h_s, ev_d2h_e;  // resident schedule: all uploads, all offloads
  hipEvent_t ev_loss, ev_start, ev_end;
  std::vector<hipEvent_t> kev;  // kernel timing pairs
  struct KernelMeta {
    double flops, bytes;  // algorithmic work of the launch
    int kind;             // 0 gemm, 1 attention
    int m, n, k, epi, layout;
  };
  std::vector<mt_kernel_time> ktimes;  // the last pass's timed launches
  std::vector<KernelMeta> kev_meta;
  size_t kev_used = 0;

  std::unique_ptr<ThreadPool> pool;
  mt_stats stats{};
  std::vector<mt_block_stats> bstats;
  float last_loss = NAN;
  bool have_loss = false;

  // ------------------------------------------------------------ layout --
  template <typename T>
  void carve_acts(Carver& c, Acts<T>& a) {
    // q/k/v, o and the statistics span every token (attention); the rest
    // one token pass (TC = M with a single pass)
    const uint64_t Md = (uint64_t)M * d, Cd = (uint64_t)TC * d;
    a.h = c.take<T>(Cd * E);
    a.qkv = c.take<T>(3 * Md * E);
    a.o = c.take<T>(Md * E);
    a.h2 = c.take<T>(Cd * E);
    a.gu = c.take<T>((uint64_t)TC * 2 * F * E);
    a.y = c.take<T>((uint64_t)TC * F * E);
    a.r1 = c.take<float>((uint64_t)M * 4);
    a.lse = c.take<float>((uint64_t)M * H * 4);
    a.x1 = c.take<float>(Cd * 4);
    a.r2 = c.take<float>((uint64_t)M * 4);
  }
  template <typename T>
  void carve_bwd(Carver& c, BwdWs<T>& w) {
    // several token passes: dy, dgu, dh and the transposed q/k/v gradient
    // hold one pass; dl/dx1 goes straight into the layer's output gradient
    const uint64_t Md = (uint64_t)M * d, CF = (uint64_t)TC * F, Cd = (uint64_t)TC * d;
    const bool tc = n_tc > 1;
    w.dxb = c.take<T>(Md * E);
    // bf16(dl/dx1) beside bf16(dl/dx2): the grouped weight gradients read both
    w.dxb1 = kmajor && !tc ? c.take<T>(Md * E) : nullptr;
    w.dxbT = kmajor ? nullptr : c.take<T>((uint64_t)d * Mp * E);
    w.tmpT = kmajor && kmajor_head ? nullptr : c.take<T>((uint64_t)std::max(d, F) * Mp * E);
    w.dy = c.take<T>(CF * E);
    w.dgu = c.take<T>(2 * CF * E);
    w.dguT = kmajor ? nullptr : c.take<T>(2 * (uint64_t)F * Mp * E);
    w.do_ = c.take<T>(Md * E);
    w.dqkvT = c.take<T>(3 * (uint64_t)d * Mp * E);
    w.dqkv = (kmajor && !tc) || (tc && dqkv_kmajor) ? nullptr : c.take<T>(3 * Cd * E);
    w.dh = c.take<float>(Cd * 4);
    w.dx1 = c.take<float>((tc ? Cd : Md) * 4);
    w.Dsum = c.take<float>((uint64_t)M * H * 4);
    w.part = c.take<float>(rmsnorm_dg_partial_elems(M, d) * 4);
    w.dxA = c.take<float>(Md * 4);
    w.dxB = c.take<float>(Md * 4);
  }
  template <typename T>
  void carve_head(Carver& c, HeadWs<T>& w) {
    const uint64_t CV = (uint64_t)HC * V;
    w.z = c.take<T>((uint64_t)M * d * E);
    w.dlogits = c.take<T>(CV * E);
    w.dlogitsT = kmajor_head ? nullptr : c.take<T>((uint64_t)V * HCp * E);
    w.rz = c.take<float>((uint64_t)M * 4);
    w.logits = c.take<float>(CV * 4);
    w.row_loss = c.take<float>((uint64_t)M * 4);
    w.loss = c.take<float>(256);
    w.gacc = n_hc > 1 && E == 2 ? c.take<float>((uint64_t)V * d * 4) : nullptr;
  }

  template <typename T>
  uint64_t carve_all(uint8_t* base) {
    Carver c{base};
    // MT_SINGLE_SLOT: one weight slot (the double-buffering ablation)
    wslot[1] = nullptr;
    for (int s = 0; s < (cfg.mode == MT_SINGLE_SLOT ? 1 : 2); ++s) wslot[s] = c.take<uint8_t>(slot_bytes);
    for (int s = 0; s < 2; ++s) gslot[s] = c.take<uint8_t>(slot_bytes);
    wt = kmajor && kmajor_head ? nullptr : c.take<uint8_t>(slot_bytes);
    if (cfg.mode == MT_RESIDENT) {
      uint64_t tot = 0;
      for (auto& b : blocks) tot += round_up(b.w_bytes, 256);
      wres = c.take<uint8_t>(tot);
      gres = c.take<uint8_t>(tot);
    }
    if (ckpt_lp) {
      ckpt = nullptr;
      ckpt16 = c.take<uint16_t>((uint64_t)(L + 1) * M * d * 2);
      for (int i = 0; i < 2; ++i) xrot[i] = c.take<float>((uint64_t)M * d * 4);
    } else {
      ckpt = c.take<float>((uint64_t)(L + 1) * M * d * 4);
    }
    cosb = c.take<float>((uint64_t)Tq * (hd / 2) * 4);
    sinb = c.take<float>((uint64_t)Tq * (hd / 2) * 4);
    cosT = c.take<float>((uint64_t)Tq * (hd / 2) * 4);
    sinT = c.take<float>((uint64_t)Tq * (hd / 2) * 4);
    d_tok = c.take<int32_t>((uint64_t)M * 4);
    d_order = c.take<int32_t>((uint64_t)M * 4);
    d_seg = c.take<int32_t>((uint64_t)(V + 1) * 4);
    // MT_RESIDENT: every layer's intermediates; otherwise one set per
    // retained layer plus the set the other layers share
    const int nacts = cfg.mode == MT_RESIDENT ? L : cfg.retain_layers + 1;
    acts_mem.assign(nacts, nullptr);
    for (int i = 0; i < nacts; ++i) {
      uint64_t start = round_up(c.off, 256);
      Acts<T> a;
      carve_acts(c, a);
      acts_mem[i] = base ? base + start : nullptr;
      (void)a;
    }
    {
      uint64_t start = round_up(c.off, 256);
      BwdWs<T> w;
      carve_bwd(c, w);
      bwd_mem = base ? base + start : nullptr;
    }
    {
      uint64_t start = round_up(c.off, 256);
      HeadWs<T> w;
      carve_head(c, w);
      head_mem = base ? base + start : nullptr;
    }
    if (bf16_store(cfg)) {
      // the largest split any GEMM of the step plans (the other GEMMs of the
      // step share the same M or N and K)
      gemm_ws_size = 0;
      const int shapes[][3] = {{M, 3 * d, d},     {M, d, d},     {M, 2 * F, d},    {M, d, F},  {d, F, M},
                               {M, F, d},         {2 * F, d, M}, {M, d, 2 * F},    {d, d, M},  {3 * d, d, M},
                               {M, d, 3 * d},     {V, d, HC},    {HC, V, d},       {HC, d, V}};
      for (const auto& sh : shapes) gemm_ws_size = std::max(gemm_ws_size, gemm_ws_bytes(sh[0], sh[1], sh[2]));
      if (kmajor && n_tc == 1) {
        const int gm[3] = {2 * F, d, d}, gn[3] = {d, F, d};
        gemm_ws_size = std::max(gemm_ws_size, gemm_group_ws_bytes(gm, gn, 3, M));
      }
      gemm_ws = gemm_ws_size ? c.take<float>(gemm_ws_size) : nullptr;
      if (!base) gemm_ws = nullptr;
    }
    dxkeep = cfg.flags & MT_FLAG_KEEP_DX ? c.take<float>((uint64_t)(L + 1) * M * d * 4) : nullptr;
    if (!base) dxkeep = nullptr;
    wacc = n_tc > 1 ? c.take<float>(blocks[1].region_elems * 4) : nullptr;
    if (!base) wacc = nullptr;
    return c.off;
  }
  // Layers whose forward intermediates stay on the device until their backward.
  bool retained(int layer) const { return cfg.mode != MT_RESIDENT && layer < cfg.retain_layers; }
  template <typename T>
  Acts<T> acts(int layer) {
    Carver c{acts_mem[cfg.mode == MT_RESIDENT || retained(layer) ? layer : cfg.retain_layers]};
    Acts<T> a;
    carve_acts(c, a);
    return a;
  }
  template <typename T>
  BwdWs<T> bwdws() {
    Carver c{bwd_mem};
    BwdWs<T> w;
    carve_bwd(c, w);
    return w;
  }
  template <typename T>
  HeadWs<T> headws() {
    Carver c{head_mem};
    HeadWs<T> w;
    carve_head(c, w);
    return w;
  }

  void init_dims(const mt_config& c) {
    cfg = c;
    blocks = store_layout(c, &store_bytes, &opt_bytes);
    slot_bytes = 0;
    for (auto& b : blocks) slot_bytes = std::max<uint64_t>(slot_bytes, b.w_bytes);
    L = c.n_layers;
    d = c.d_model;
    H = c.n_heads;
    hd = c.head_dim;
    F = c.d_ff;
    V = c.vocab;
    B = c.batch;
    Tq = c.seq_len;
    M = B * Tq;
    Mp = token_ld(M);
    E = wbytes(c);
    // Output head passes: all tokens at once unless their logits and logit
    // gradients would take more than 16 GiB; then passes of at most 4 GiB.
    const uint64_t head_row = (uint64_t)V * (4 + E);
    if (c.head_chunk_tokens > 0)
      HC = std::min(M, c.head_chunk_tokens);
    else if ((uint64_t)M * head_row <= (16ull << 30))
      HC = M;
    else
      HC = std::min<int64_t>(M, std::max<int64_t>(256, (int64_t)((4ull << 30) / head_row) / 256 * 256));
    n_hc = (M + HC - 1) / HC;
    HCp = token_ld(HC);
    TC = M;
    n_tc = 1;
    if (bf16_store(c)) {
      const int A_ = GEMM_A_KMAJOR, B_ = GEMM_B_KMAJOR;
      auto ok = [&](int m, int n, int k, int64_t lda, int64_t ldb, int lay) {
        return gemm_layout_ok(m, n, k, lda, ldb, lay);
      };
      // the layer's weight gradients contract over K = the tokens of a pass
      auto wgrads_ok = [&](int K) {
        return ok(d, F, K, d, F, A_ | B_) && ok(2 * F, d, K, 2 * F, d, A_ | B_) && ok(d, d, K, d, d, A_ | B_) &&
               ok(3 * d, d, K, Mp, d, B_);
      };
      const bool dgrads_ok = ok(M, F, d, d, F, B_) && ok(M, d, 2 * F, 2 * F, d, B_) && ok(M, d, d, d, d, B_);
      kmajor = wgrads_ok(M) && dgrads_ok && ok(M, d, 3 * d, Mp, d, A_ | B_);
      kmajor_head = ok(V, d, HC, V, d, A_ | B_) && ok(HC, d, V, V, d, B_);
      // token passes: asked for, or needed to keep the K-major weight
      // gradients within their operand addressing
      int want = 0;
      if (c.token_chunk > 0 && c.token_chunk < M)
        want = c.token_chunk;
      else if (c.token_chunk == 0 && !kmajor) {
        const int64_t ldmax = std::max<int64_t>({d, F, 2 * (int64_t)F});
        want = (int)std::min<int64_t>(32768, ((((int64_t)1 << 31) - 1) / (2 * ldmax)) / 256 * 256);
      }
      if (want > 0 && want < M) {
        const int n = (M + want - 1) / want;
        TC = (int)round_up((uint64_t)((M + n - 1) / n), 64);
        n_tc = (M + TC - 1) / TC;
        const int last = M - (n_tc - 1) * TC;
        if (n_tc > 1) {
          if (!(wgrads_ok(TC) && wgrads_ok(last) && dgrads_ok))
            throw ApiError{MT_E_INVALID, "token passes: each pass needs at least 192 tokens, a multiple of 64, "
                                         "within the matrix kernels' operand addressing"};
          kmajor = true;
          dqkv_kmajor = ok(TC, d, 3 * d, Mp, d, A_ | B_);
        } else {
          TC = M;
        }
      }
    } else if (c.token_chunk > 0 && c.token_chunk < M) {
      throw ApiError{MT_E_INVALID, "token passes need a bf16 store"};
    }
    ckpt_lp = c.flags & MT_FLAG_CKPT_BF16;
    if (ckpt_lp && (!bf16_store(c) || c.mode == MT_RESIDENT || c.retain_layers > 0))
      throw ApiError{MT_E_INVALID, "bf16 checkpoints need a bf16 store and a streamed, serialized or single-slot "
                                   "schedule without retained layers"};
    if (n_tc > 1 && (c.mode == MT_RESIDENT || c.retain_layers > 0))
      throw ApiError{MT_E_INVALID, "token passes need a streamed, serialized or single-slot schedule without "
                                   "retained layers"};
    n_uses = 2 * L + 3;
  }
  uint64_t device_bytes() { return bf16_store(cfg) ? carve_all<uint16_t>(nullptr) : carve_all<float>(nullptr); }

  float* x_ckpt(int l) { return ckpt + (uint64_t)l * M * d; }
  // x^l as the forward sweep reads and writes it (fp32)
  float* x_fwd(int l) { return ckpt_lp ? xrot[l & 1] : x_ckpt(l); }
  // after x^l is complete in the forward sweep: its bf16 checkpoint
  void store_ckpt(int l) {
    if (ckpt_lp) cast<uint16_t>(xrot[l & 1], ckpt16 + (uint64_t)l * M * d, (int64_t)M * d, sc);
  }
  // x^l for the backward sweep (widened from its bf16 checkpoint)
  const float* x_bwd(int l) {
    if (!ckpt_lp) return x_ckpt(l);
    widen_bf16(ckpt16 + (uint64_t)l * M * d, xrot[0], (int64_t)M * d, sc);
    return xrot[0];
  }
  // MT_FLAG_KEEP_DX: a copy of the gradient arriving at layer boundary l
  void keep_dx(int l, const float* dx) {
    if (dxkeep)
      MT_HIP(hipMemcpyAsync(dxkeep + (uint64_t)l * M * d, dx, (uint64_t)M * d * 4, hipMemcpyDeviceToDevice, sc));
  }

  // --------------------------------------------------------- kernels --
  template <typename T>
  void gemm(const T* A, int64_t lda, const T* Bm, int64_t ldb, void* C, int64_t ldc, const float* R, int64_t ldr,
            int m, int n, int k, Epi epi, int layout = 0) {
    const bool timed = cfg.flags & MT_FLAG_TIME_KERNELS;
    // operands read once, result written once (and the residual read once)
    const double out_b = epi == EPI_STORE ? sizeof(T) : 4.0;
    const double bytes = ((double)m * k + (double)n * k) * sizeof(T) + (double)m * n * (out_b + (epi == EPI_ADD_F32 ? 4 : 0));
    if (timed) record_kernel_start(2.0 * m * n * k, 0, bytes, m, n, k, (int)epi, layout);
    if constexpr (std::is_same<T, uint16_t>::value)
      gemm_bf16(A, lda, Bm, ldb, layout, C, ldc, R, ldr, m, n, k, epi, sc, gemm_ws, gemm_ws_size);
    else
      gemm_nt<T>(A, lda, Bm, ldb, C, ldc, R, ldr, m, n, k, epi, sc);
    if (timed) record_kernel_end();
  }
  // The layer's down, gate/up and output projection weight gradients in one
  // launch (K-major operands, contraction over the M tokens): their tiles
  // fill the device together where the output projection's 400 tiles alone
  // leave a half-empty last round.
  void wgrad_group(const uint16_t* dxb2, const uint16_t* y, uint16_t* gd, const uint16_t* dgu, const uint16_t* h2,
                   uint16_t* ggu, const uint16_t* dxb1, const uint16_t* o, uint16_t* go) {
    const GemmDesc g[3] = {{dgu, 2 * (int64_t)F, h2, d, ggu, d, 2 * F, d},
                           {dxb2, d, y, F, gd, F, d, F},
                           {dxb1, d, o, d, go, d, d, d}};
    const bool timed = cfg.flags & MT_FLAG_TIME_KERNELS;
    double flops = 0.0, bytes = 0.0;
    for (const auto& p : g) {
      flops += 2.0 * p.M * p.N * M;
      bytes += ((double)p.M + p.N) * M * 2 + (double)p.M * p.N * 2;
    }
    if (timed) record_kernel_start(flops, 2, bytes, 0, 0, M, (int)EPI_STORE, GEMM_A_KMAJOR | GEMM_B_KMAJOR);
    gemm_bf16_group(g, 3, M, GEMM_A_KMAJOR | GEMM_B_KMAJOR, EPI_STORE, sc, gemm_ws, gemm_ws_size);
    if (timed) record_kernel_end();
  }
  void record_kernel_start(double flops, int kind, double bytes = 0.0, int m = 0, int n = 0, int k = 0, int epi = 0,
                           int layout = 0) {
    if (kev_used + 2 > kev.size()) {
      hipEvent_t e0, e1;
      MT_HIP(hipEventCreate(&e0));
      MT_HIP(hipEventCreate(&e1));
      kev.push_back(e0);
      kev.push_back(e1);
      kev_meta.push_back(KernelMeta{0.0, 0.0, 0, 0, 0, 0, 0, 0});
    }
    kev_meta[kev_used / 2] = KernelMeta{flops, bytes, kind, m, n, k, epi, layout};
    MT_HIP(hipEventRecord(kev[kev_used], sc));
  }
  void record_kernel_end() {
    MT_HIP(hipEventRecord(kev[kev_used + 1], sc));
    kev_used += 2;
  }
  // Causal attention flops per layer: QK^T and PV over the lower triangle.
  double attn_fwd_flops() const { return 2.0 * 2.0 * B * H * ((double)Tq * (Tq + 1) / 2) * hd; }

  template <typename T>
  void layer_fwd(const LayerW<T>& w, const float* x, const Acts<T>& a, float* x_out, bool full) {
    const float eps = (float)cfg.rms_eps;
    rmsnorm_fwd<T>(x, w.anorm, a.h, a.r1, M, d, eps, sc);
    gemm<T>(a.h, d, w.qkv, d, a.qkv, 3 * d, nullptr, 0, M, 3 * d, d, EPI_STORE);
    rope_qkv_fwd<T>(a.qkv, cosb, sinb, M, Tq, d, hd, sc);
    const bool timed = cfg.flags & MT_FLAG_TIME_KERNELS;
    if (timed) record_kernel_start(attn_fwd_flops(), 1);
    attn_fwd<T>(a.qkv, a.o, a.lse, B, Tq, H, hd, sc);
    if (timed) record_kernel_end();
    // x1 = x + o.Wo^T: the GEMM writes the product, the norm that reads it adds x
    gemm<T>(a.o, d, w.o, d, a.x1, d, nullptr, 0, M, d, d, EPI_F32);
    rmsnorm_fwd_res<T>(x, a.x1, w.fnorm, a.h2, a.r2, M, d, eps, sc);
    gemm<T>(a.h2, d, w.gu, d, a.gu, 2 * F, nullptr, 0, M, 2 * F, d, EPI_STORE);
    swiglu_fwd<T>(a.gu, a.y, M, F, sc);
    if (full) gemm<T>(a.y, F, w.d, F, x_out, d, a.x1, d, M, d, F, EPI_ADD_F32);
  }

  template <typename T>
  void weight_transposes(const LayerW<T>& w, const LayerWT<T>& t) {
    transpose<T>(w.qkv, d, t.qkv, 3 * d, 3 * d, d, sc);
    transpose<T>(w.o, d, t.o, d, d, d, sc);
    transpose<T>(w.gu, d, t.gu, 2 * F, 2 * F, d, sc);
    transpose<T>(w.d, F, t.d, d, d, F, sc);
  }

  template <typename T>
  void layer_bwd(const LayerW<T>& w, const LayerWT<T>& wt_, const float* x, const Acts<T>& a, const float* dx2,
                 float* dx_out, const LayerW<T>& g) {
    BwdWs<T> ws = bwdws<T>();
    if (kmajor) {
      layer_bwd_kmajor<T>(w, x, a, dx2, dx_out, g, ws);
      return;
    }
    // down projection
    cast_transpose<T>(dx2, ws.dxb, ws.dxbT, Mp, M, d, sc);
    transpose<T>(a.y, F, ws.tmpT, Mp, M, F, sc);
    gemm<T>(ws.dxbT, Mp, ws.tmpT, Mp, g.d, F, nullptr, 0, d, F, M, EPI_STORE);
    gemm<T>(ws.dxb, d, wt_.d, d, ws.dy, F, nullptr, 0, M, F, d, EPI_STORE);
    // SwiGLU and gate/up projection
    swiglu_bwd<T>(ws.dy, a.gu, ws.dgu, M, F, sc);
    transpose<T>(ws.dgu, 2 * F, ws.dguT, Mp, M, 2 * F, sc);
    transpose<T>(a.h2, d, ws.tmpT, Mp, M, d, sc);
    gemm<T>(ws.dguT, Mp, ws.tmpT, Mp, g.gu, d, nullptr, 0, 2 * F, d, M, EPI_STORE);
    gemm<T>(ws.dgu, 2 * F, wt_.gu, 2 * F, ws.dh, d, nullptr, 0, M, d, 2 * F, EPI_F32);
    rmsnorm_bwd<T>(ws.dh, a.x1, w.fnorm, a.r2, dx2, ws.dx1, ws.part, g.fnorm, M, d, sc);
    // attention output projection
    cast_transpose<T>(ws.dx1, ws.dxb, ws.dxbT, Mp, M, d, sc);
    transpose<T>(a.o, d, ws.tmpT, Mp, M, d, sc);
    gemm<T>(ws.dxbT, Mp, ws.tmpT, Mp, g.o, d, nullptr, 0, d, d, M, EPI_STORE);
    gemm<T>(ws.dxb, d, wt_.o, d, ws.do_, d, nullptr, 0, M, d, d, EPI_STORE);
    // attention
    attn_bwd_dsum<T>(ws.do_, a.o, ws.Dsum, B, Tq, H, hd, sc);
    const bool timed = cfg.flags & MT_FLAG_TIME_KERNELS;
    if (timed) record_kernel_start(2.5 * attn_fwd_flops(), 1);
    attn_bwd<T>(a.qkv, ws.do_, a.lse, ws.Dsum, ws.dqkvT, Mp, B, Tq, H, hd, sc);
    if (timed) record_kernel_end();
    rope_bwd_T<T>(ws.dqkvT, Mp, cosT, sinT, M, Tq, d, hd, sc);
    // QKV projection
    transpose<T>(ws.dqkvT, Mp, ws.dqkv, 3 * d, 3 * d, M, sc);
    transpose<T>(a.h, d, ws.tmpT, Mp, M, d, sc);
    gemm<T>(ws.dqkvT, Mp, ws.tmpT, Mp, g.qkv, d, nullptr, 0, 3 * d, d, M, EPI_STORE);
    gemm<T>(ws.dqkv, 3 * d, wt_.qkv, 3 * d, ws.dh, d, nullptr, 0, M, d, 3 * d, EPI_F32);
    rmsnorm_bwd<T>(ws.dh, x, w.anorm, a.r1, ws.dx1, dx_out, ws.part, g.anorm, M, d, sc);
  }

  // The same backward with K-major operands (no transposes).  C = A.B with
  // A(i, k), B(j, k): a weight gradient dW[i][j] = sum over tokens m of
  // dY[m][i] X[m][j] reads both token-major matrices as K-major; a data
  // gradient dX[m][j] = sum_i dY[m][i] W[i][j] reads dY as is and the
  // weight [out x in] as K-major.
  template <typename T>
  void layer_bwd_kmajor(const LayerW<T>& w, const float* x, const Acts<T>& a, const float* dx2, float* dx_out,
                        const LayerW<T>& g, const BwdWs<T>& ws) {
    const int KA = GEMM_A_KMAJOR, KB = GEMM_B_KMAJOR;
    // down projection; ws.dxb = bf16(dx2) was written beside dx2 by the norm
    // backward that produced it (the layer above, or the head)
    if (dxb_holds != dx2) throw ApiError{MT_E_STATE, "K-major layer backward: bf16 copy does not mirror its dx"};
    gemm<T>(ws.dxb, d, w.d, F, ws.dy, F, nullptr, 0, M, F, d, EPI_STORE, KB);
    // SwiGLU and gate/up projection
    swiglu_bwd<T>(ws.dy, a.gu, ws.dgu, M, F, sc);
    gemm<T>(ws.dgu, 2 * F, w.gu, d, ws.dh, d, nullptr, 0, M, d, 2 * F, EPI_F32, KB);
    // dl/dx1, and bf16(dl/dx1) beside bf16(dl/dx2) (still in ws.dxb)
    rmsnorm_bwd<T>(ws.dh, a.x1, w.fnorm, a.r2, dx2, ws.dx1, ws.part, g.fnorm, M, d, sc, ws.dxb1);
    // attention output projection
    gemm<T>(ws.dxb1, d, w.o, d, ws.do_, d, nullptr, 0, M, d, d, EPI_STORE, KB);
    // weight gradients of the down, gate/up and output projections
    if constexpr (std::is_same<T, uint16_t>::value)
      wgrad_group(ws.dxb, a.y, g.d, ws.dgu, a.h2, g.gu, ws.dxb1, a.o, g.o);
    else
      throw ApiError{MT_E_STATE, "K-major layer backward needs a bf16 store"};
    // attention
    attn_bwd_dsum<T>(ws.do_, a.o, ws.Dsum, B, Tq, H, hd, sc);
    const bool timed = cfg.flags & MT_FLAG_TIME_KERNELS;
    if (timed) record_kernel_start(2.5 * attn_fwd_flops(), 1);
    attn_bwd<T>(a.qkv, ws.do_, a.lse, ws.Dsum, ws.dqkvT, Mp, B, Tq, H, hd, sc);
    if (timed) record_kernel_end();
    rope_bwd_T<T>(ws.dqkvT, Mp, cosT, sinT, M, Tq, d, hd, sc);
    // QKV projection: dqkvT [3d x M] is K-contiguous for the weight gradient
    // and K-major for the data gradient
    gemm<T>(ws.dqkvT, Mp, a.h, d, g.qkv, d, nullptr, 0, 3 * d, d, M, EPI_STORE, KB);
    gemm<T>(ws.dqkvT, Mp, w.qkv, d, ws.dh, d, nullptr, 0, M, d, 3 * d, EPI_F32, KA | KB);
    // dx_out, and bf16(dx_out) for the next layer's down projection
    rmsnorm_bwd<T>(ws.dh, x, w.anorm, a.r1, ws.dx1, dx_out, ws.part, g.anorm, M, d, sc, ws.dxb);
    dxb_holds = dx_out;
  }

  // ---- a layer in token passes (n_tc > 1) -------------------------------
  // The per-token work of a layer runs TC tokens at a time; the attention
  // runs over every token.  Rows [r0, r0 + rows) belong to pass p.
  void pass_rows(int p, int64_t* r0, int* rows) const {
    *r0 = (int64_t)p * TC;
    *rows = (int)std::min<int64_t>(TC, M - *r0);
  }
  // The attention's input for one pass: h, then q, k, v (q, k rotated)
  template <typename T>
  void qkv_pass(const LayerW<T>& w, const float* x, const Acts<T>& a, int64_t r0, int rows) {
    rmsnorm_fwd<T>(x + r0 * d, w.anorm, a.h, a.r1 + r0, rows, d, (float)cfg.rms_eps, sc);
    gemm<T>(a.h, d, w.qkv, d, a.qkv + r0 * 3 * d, 3 * d, nullptr, 0, rows, 3 * d, d, EPI_STORE);
    rope_qkv_fwd<T>(a.qkv + r0 * 3 * d, cosb, sinb, rows, Tq, d, hd, sc, r0);
  }
  // Output projection and FFN of one pass: x1, h2, gu, y (and x_out rows)
  template <typename T>
  void ffn_pass(const LayerW<T>& w, const float* x, const Acts<T>& a, int64_t r0, int rows, float* x_out) {
    gemm<T>(a.o + r0 * d, d, w.o, d, a.x1, d, nullptr, 0, rows, d, d, EPI_F32);
    rmsnorm_fwd_res<T>(x + r0 * d, a.x1, w.fnorm, a.h2, a.r2 + r0, rows, d, (float)cfg.rms_eps, sc);
    gemm<T>(a.h2, d, w.gu, d, a.gu, 2 * F, nullptr, 0, rows, 2 * F, d, EPI_STORE);
    swiglu_fwd<T>(a.gu, a.y, rows, F, sc);
    if (x_out) gemm<T>(a.y, F, w.d, F, x_out + r0 * d, d, a.x1, d, rows, d, F, EPI_ADD_F32);
  }
  // Forward of a layer in passes; without x_out (the recompute inside the
  // backward) it stops after the attention: the backward recomputes each
  // pass's FFN input just before it needs it.
  template <typename T>
  void layer_fwd_passes(const LayerW<T>& w, const float* x, const Acts<T>& a, float* x_out) {
    int64_t r0;
    int rows;
    for (int p = 0; p < n_tc; ++p) {
      pass_rows(p, &r0, &rows);
      qkv_pass<T>(w, x, a, r0, rows);
    }
    const bool timed = cfg.flags & MT_FLAG_TIME_KERNELS;
    if (timed) record_kernel_start(attn_fwd_flops(), 1);
    attn_fwd<T>(a.qkv, a.o, a.lse, B, Tq, H, hd, sc);
    if (timed) record_kernel_end();
    if (!x_out) return;
    for (int p = 0; p < n_tc; ++p) {
      pass_rows(p, &r0, &rows);
      ffn_pass<T>(w, x, a, r0, rows, x_out);
    }
  }
  // Backward of a layer in passes.  Weight gradients are summed over the
  // passes in fp32 (wacc, in the W region's layout) and rounded once; the
  // gain gradients' per-block partial sums cover all rows before their one
  // reduction, in the order of a single pass.
  template <typename T>
  void layer_bwd_passes(const LayerW<T>& w, const float* x, const Acts<T>& a, const float* dx2, float* dx_out,
                        const LayerW<T>& g, const mt_block_desc& b, const BwdWs<T>& ws) {
    const int KA = GEMM_A_KMAJOR, KB = GEMM_B_KMAJOR;
    if (dxb_holds != dx2) throw ApiError{MT_E_STATE, "layer backward in passes: bf16 copy does not mirror its dx"};
    const LayerW<float> acc = bind_layer<float>((uint8_t*)wacc, b);
    const int rpb = rmsnorm_rows_per_block();
    const int nblk = (M + rpb - 1) / rpb;
    int64_t r0;
    int rows;
    // FFN and output projection.  The pass's rows of dxb hold bf16(dx2),
    // then bf16(dl/dx1); dl/dx1 itself goes into dx_out.
    for (int p = 0; p < n_tc; ++p) {
      pass_rows(p, &r0, &rows);
      const Epi ep = p == 0 ? EPI_F32 : EPI_ADD_F32;
      ffn_pass<T>(w, x, a, r0, rows, nullptr);
      const T* dxb = ws.dxb + r0 * d;
      gemm<T>(dxb, d, a.y, F, acc.d, F, p ? acc.d : nullptr, F, d, F, rows, ep, KA | KB);
      gemm<T>(dxb, d, w.d, F, ws.dy, F, nullptr, 0, rows, F, d, EPI_STORE, KB);
      swiglu_bwd<T>(ws.dy, a.gu, ws.dgu, rows, F, sc);
      gemm<T>(ws.dgu, 2 * F, a.h2, d, acc.gu, d, p ? acc.gu : nullptr, d, 2 * F, d, rows, ep, KA | KB);
      gemm<T>(ws.dgu, 2 * F, w.gu, d, ws.dh, d, nullptr, 0, rows, d, 2 * F, EPI_F32, KB);
      rmsnorm_bwd<T>(ws.dh, a.x1, w.fnorm, a.r2 + r0, dx2 + r0 * d, dx_out + r0 * d, ws.part + (r0 / rpb) * d,
                     nullptr, rows, d, sc, ws.dxb + r0 * d);
      gemm<T>(dxb, d, a.o + r0 * d, d, acc.o, d, p ? acc.o : nullptr, d, d, d, rows, ep, KA | KB);
      gemm<T>(dxb, d, w.o, d, ws.do_ + r0 * d, d, nullptr, 0, rows, d, d, EPI_STORE, KB);
    }
    rmsnorm_dg_reduce<T>(ws.part, g.fnorm, nblk, d, sc);
    cast<T>(acc.d, g.d, (int64_t)d * F, sc);
    cast<T>(acc.gu, g.gu, 2 * (int64_t)F * d, sc);
    cast<T>(acc.o, g.o, (int64_t)d * d, sc);
    // attention over every token
    attn_bwd_dsum<T>(ws.do_, a.o, ws.Dsum, B, Tq, H, hd, sc);
    const bool timed = cfg.flags & MT_FLAG_TIME_KERNELS;
    if (timed) record_kernel_start(2.5 * attn_fwd_flops(), 1);
    attn_bwd<T>(a.qkv, ws.do_, a.lse, ws.Dsum, ws.dqkvT, Mp, B, Tq, H, hd, sc);
    if (timed) record_kernel_end();
    rope_bwd_T<T>(ws.dqkvT, Mp, cosT, sinT, M, Tq, d, hd, sc);
    // q/k/v projection (h of the pass recomputed); dx = dl/dx1 + the attention
    // norm's gradient, computed into a pass buffer and copied into dx_out
    for (int p = 0; p < n_tc; ++p) {
      pass_rows(p, &r0, &rows);
      const Epi ep = p == 0 ? EPI_F32 : EPI_ADD_F32;
      rmsnorm_fwd<T>(x + r0 * d, w.anorm, a.h, a.r1 + r0, rows, d, (float)cfg.rms_eps, sc);
      const T* dT = ws.dqkvT + r0;
      gemm<T>(dT, Mp, a.h, d, acc.qkv, d, p ? acc.qkv : nullptr, d, 3 * d, d, rows, ep, KB);
      if (dqkv_kmajor) {
        gemm<T>(dT, Mp, w.qkv, d, ws.dh, d, nullptr, 0, rows, d, 3 * d, EPI_F32, KA | KB);
      } else {
        transpose<T>(dT, Mp, ws.dqkv, 3 * d, 3 * d, rows, sc);
        gemm<T>(ws.dqkv, 3 * d, w.qkv, d, ws.dh, d, nullptr, 0, rows, d, 3 * d, EPI_F32, KB);
      }
      rmsnorm_bwd<T>(ws.dh, x + r0 * d, w.anorm, a.r1 + r0, dx_out + r0 * d, ws.dx1, ws.part + (r0 / rpb) * d,
                     nullptr, rows, d, sc, ws.dxb + r0 * d);
      MT_HIP(hipMemcpyAsync(dx_out + r0 * d, ws.dx1, (uint64_t)rows * d * 4, hipMemcpyDeviceToDevice, sc));
    }
    rmsnorm_dg_reduce<T>(ws.part, g.anorm, nblk, d, sc);
    cast<T>(acc.qkv, g.qkv, 3 * (int64_t)d * d, sc);
    dxb_holds = dx_out;
  }

  // Final norm, logits, loss, and the head's backward.  Returns dx^L in dx_out.
  // dl/dz for every token goes to the other dx buffer, free until the top
  // layer's backward (the layer workspace holds one token pass).
  template <typename T>
  void head_fwd_bwd(const mt_block_desc& b, uint8_t* wreg, uint8_t* greg, float* dx_out) {
    HeadWs<T> hw = headws<T>();
    BwdWs<T> ws = bwdws<T>();
    float* dz = dx_out == ws.dxA ? ws.dxB : ws.dxA;
    const T* wh = (const T*)wreg + b.tensors[T_WH].offset;
    const T* fin = (const T*)wreg + b.tensors[T_FINAL].offset;
    T* gwh = (T*)greg + b.tensors[T_WH].offset;
    T* gfin = (T*)greg + b.tensors[T_FINAL].offset;
    const float* xL = x_fwd(L);
    // mean over the labelled positions of every micro-batch of the step
    const float inv_n = 1.0f / (float)((int64_t)micro_count(cfg) * B * (Tq - 1));
    rmsnorm_fwd<T>(xL, fin, hw.z, hw.rz, M, d, (float)cfg.rms_eps, sc);
    T* whT = (T*)wt;
    if (!kmajor_head) transpose<T>(wh, d, whT, V, V, d, sc);
    // One pass per HC tokens: logits, loss rows and logit gradients of the
    // pass, its share of the head weight gradient, and its rows of dz.  With
    // several passes the weight gradient is summed in fp32 (in place for an
    // fp32 store) and rounded once at the end.
    float* gsum = n_hc == 1 ? nullptr : (E == 2 ? hw.gacc : (float*)gwh);
    for (int p = 0; p < n_hc; ++p) {
      const int64_t r0 = (int64_t)p * HC;
      const int rows = (int)std::min<int64_t>(HC, M - r0);
      const T* zc = hw.z + r0 * d;
      gemm<T>(zc, d, wh, d, hw.logits, V, nullptr, 0, rows, V, d, EPI_F32);
      xent<T>(hw.logits, d_tok, hw.row_loss, hw.dlogits, rows, r0, Tq, V, inv_n, sc);
      void* gout = gsum ? (void*)gsum : (void*)gwh;
      const float* R = gsum && p > 0 ? gsum : nullptr;
      const Epi epi = !gsum ? EPI_STORE : (p > 0 ? EPI_ADD_F32 : EPI_F32);
      if (kmajor_head) {
        gemm<T>(hw.dlogits, V, zc, d, gout, d, R, d, V, d, rows, epi, GEMM_A_KMAJOR | GEMM_B_KMAJOR);
        gemm<T>(hw.dlogits, V, wh, d, dz + r0 * d, d, nullptr, 0, rows, d, V, EPI_F32, GEMM_B_KMAJOR);
      } else {
        transpose<T>(hw.dlogits, V, hw.dlogitsT, HCp, rows, V, sc);
        transpose<T>(zc, d, ws.tmpT, HCp, rows, d, sc);
        gemm<T>(hw.dlogitsT, HCp, ws.tmpT, HCp, gout, d, R, d, V, d, rows, epi);
        gemm<T>(hw.dlogits, V, whT, V, dz + r0 * d, d, nullptr, 0, rows, d, V, EPI_F32);
      }
    }
    if (gsum && E == 2) cast<T>(gsum, gwh, (int64_t)V * d, sc);
    sum_fixed(hw.row_loss, hw.loss, M, inv_n, sc);
    MT_HIP(hipMemcpyAsync(h_loss, hw.loss, sizeof(float), hipMemcpyDeviceToHost, sc));
    MT_HIP(hipEventRecord(ev_loss, sc));
    // dx^L, and bf16(dx^L) for the top layer's down projection when it reads it
    rmsnorm_bwd<T>(dz, xL, fin, hw.rz, nullptr, dx_out, ws.part, gfin, M, d, sc, kmajor ? ws.dxb : nullptr);
    dxb_holds = kmajor ? dx_out : nullptr;
    keep_dx(L, dx_out);
  }

  // ------------------------------------------------------------ step --
  template <typename T>
  void compute_block_fwd(int j, uint8_t* wreg) {
    const mt_block_desc& b = blocks[j];
    if (b.kind == MT_BLOCK_EMBED) {
      embed_fwd<T>(d_tok, (const T*)wreg + b.tensors[0].offset, x_fwd(0), M, d, sc);
      store_ckpt(0);
    } else {
      const int l = b.layer;
      if (n_tc > 1)
        layer_fwd_passes<T>(bind_layer<T>(wreg, b), x_fwd(l), acts<T>(l), x_fwd(l + 1));
      else
        layer_fwd<T>(bind_layer<T>(wreg, b), x_fwd(l), acts<T>(l), x_fwd(l + 1), true);
      store_ckpt(l + 1);
    }
  }

  template <typename T>
  void compute_layer_bwd(int j, uint8_t* wreg, uint8_t* greg, const float* dx_in, float* dx_out) {
    const mt_block_desc& b = blocks[j];
    const int l = b.layer;
    LayerW<T> w = bind_layer<T>(wreg, b);
    LayerW<T> g = bind_layer<T>(greg, b);
    LayerWT<T> t{};
    if (!kmajor)
      t = LayerWT<T>{(T*)wt, (T*)wt + (uint64_t)3 * d * d, (T*)wt + (uint64_t)4 * d * d,
                     (T*)wt + (uint64_t)4 * d * d + (uint64_t)2 * F * d};
    Acts<T> a = acts<T>(l);
    const float* x = x_bwd(l);
    if (n_tc > 1) {
      layer_fwd_passes<T>(w, x, a, nullptr);  // recompute up to the attention
      layer_bwd_passes<T>(w, x, a, dx_in, dx_out, g, b, bwdws<T>());
      keep_dx(l, dx_out);
      return;
    }
    if (cfg.mode != MT_RESIDENT && !retained(l)) layer_fwd<T>(w, x, a, nullptr, false);  // recompute
    if (!kmajor) weight_transposes<T>(w, t);
    layer_bwd<T>(w, t, x, a, dx_in, dx_out, g);
    keep_dx(l, dx_out);
  }

  template <typename T>
  void step_streamed(bool serialize);
  template <typename T>
  void step_resident();
  int train_step(const int32_t* tokens);
  void run_pass(const int32_t* tokens, int64_t t, double* adam_total, double* adam_tail);
  void finish_stats(bool streamed, double wall_ms);
  int mb = 0;  // micro-batch of the running pass
  // MT_FLAG_DELAYS: the delay before operation (lane, use) of this step and
  // micro-batch, 0 to 1999 us (0 for about half), from a splitmix64 hash
  int64_t step_t = 0;
  int delay_us(int lane, int use) const {
    if (!(cfg.flags & MT_FLAG_DELAYS)) return 0;
    uint64_t z = (uint64_t)step_t * 0x9E3779B97F4A7C15ull ^ (uint64_t)(mb * 4 + lane) * 0xD1B54A32D192ED03ull ^
                 (uint64_t)(use + 1) * 0x8CB92BA72F3D8DD7ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (z & 1) ? 0 : (int)((z >> 1) % 2000);
  }
  static void sleep_host(void* us) { std::this_thread::sleep_for(std::chrono::microseconds((intptr_t)us)); }
  // MT_FLAG_PROGRESS: packed (use, block, uses per pass) of a finished use
  static void print_progress(void* packed) {
    const uint64_t v = (uint64_t)(uintptr_t)packed;
    fprintf(stderr, "mt: use %d of %d (block %d) done\n", (int)(v & 0xFFFFF) + 1, (int)((v >> 40) & 0xFFFFF),
            (int)((v >> 20) & 0xFFFFF));
    fflush(stderr);
  }
  // the stream's later work waits for a host function that sleeps
  void stream_delay(hipStream_t s, int lane, int use) {
    const int us = delay_us(lane, use);
    if (us > 0) MT_HIP(hipLaunchHostFunc(s, sleep_host, (void*)(intptr_t)us));
  }

  // Adam worker coordination
  std::mutex q_mu;
  std::condition_variable q_cv;
  std::vector<int> q_blocks;   // blocks whose D2H has been enqueued, in order
  std::vector<hipEvent_t> q_events;
  bool q_closed = false;
  std::atomic<bool> nonfinite{false};
  std::string adam_error;

  void push_adam(int block, hipEvent_t ev) {
    {
      std::lock_guard<std::mutex> g(q_mu);
      q_blocks.push_back(block);
      q_events.push_back(ev);
    }
    q_cv.notify_all();
  }
  void close_adam() {
    {
      std::lock_guard<std::mutex> g(q_mu);
      q_closed = true;
    }
    q_cv.notify_all();
  }
  void adam_worker(int64_t t, double* adam_total, double* adam_tail, std::atomic<bool>* device_done);

  // ---- the streamed schedule as data (mt_schedule) --------------------
  // A dry run of step_streamed records every operation it would issue and
  // the earlier operations each one waits for, and issues no device work.
  struct TraceOp {
    int lane, kind, use, block, wslot, gslot;
    std::vector<int> waits;  // data and ordering dependencies
    std::vector<int> link;   // orderings that only share out the host link
  };
  std::vector<TraceOp>* trace = nullptr;
  // Per ordered lane, the latest operation the enqueueing thread has waited
  // for: every operation issued after that wait follows it.
  int fence[3] = {-1, -1, -1};
  int tr_add(int lane, int kind, int use, int block, int ws, int gs, std::vector<int> waits, std::vector<int> link) {
    if (!trace) return -1;
    for (int f : fence) waits.push_back(f);
    waits.erase(std::remove(waits.begin(), waits.end(), -1), waits.end());
    std::sort(waits.begin(), waits.end());
    waits.erase(std::unique(waits.begin(), waits.end()), waits.end());
    link.erase(std::remove(link.begin(), link.end(), -1), link.end());
    trace->push_back(TraceOp{lane, kind, use, block, ws, gs, waits, link});
    return (int)trace->size() - 1;
  }
  void tr_fence(int op) {
    if (!trace || op < 0) return;
    const int lane = (*trace)[op].lane;
    fence[lane] = std::max(fence[lane], op);
  }
  // Offloads yield the host link to prefetches when a layer's backward is
  // compute-bound against the link (its flops per transferred weight and
  // gradient byte well above ~1 PFLOP/s over ~50 GB/s): the transfers are
  // hidden either way and each then runs at the full one-way rate.  When the
  // link is the bottleneck, both directions share it.
  bool link_yields() const {
    const double layer_bytes = 2.0 * (double)blocks[1].w_bytes;
    const double bwd_flops = 3.0 * (2.0 * M * (4.0 * d * d + 3.0 * d * F)) + 3.5 * attn_fwd_flops();
    return !(cfg.flags & MT_FLAG_DUPLEX_LINK) && bwd_flops / layer_bytes > 30000.0;
  }

  // Streamed schedules: weight prefetches and gradient offloads run on two
  // SDMA engines, each fed in order by a worker thread (dma.h).  The
  // enqueueing thread enqueues a block's compute once its weights have
  // arrived, and reuses a gradient slot once the offload that read it is done.
  std::unique_ptr<DmaEngines> dma;
  std::unique_ptr<TransferQueue> xq_in, xq_out;
  std::vector<double> h2d_host_ms, d2h_host_ms;  // per use: copy time (host clock)
};

// ---------------------------------------------------------------- Adam --
void Model::adam_worker(int64_t t, double* adam_total, double* adam_tail, std::atomic<bool>* device_done) {
  try {
    // The loss must be finite before any parameter changes.
    {
      std::unique_lock<std::mutex> lk(q_mu);
      q_cv.wait(lk, [&] { return !q_blocks.empty() || q_closed; });
    }
    MT_HIP(hipEventSynchronize(ev_loss));
    if (!std::isfinite(*h_loss)) nonfinite = true;
    const AdamConsts k = adam_consts(t, cfg.lr, cfg.beta1, cfg.beta2, cfg.adam_eps);
    const int K = micro_count(cfg);
    size_t next = 0;
    for (;;) {
      int blk;
      hipEvent_t ev;
      {
        std::unique_lock<std::mutex> lk(q_mu);
        q_cv.wait(lk, [&] { return next < q_blocks.size() || q_closed; });
        if (next >= q_blocks.size()) break;
        blk = q_blocks[next];
        ev = q_events[next];
        ++next;
      }
      if (ev) MT_HIP(hipEventSynchronize(ev));
      if (const int us = delay_us(MT_LANE_HOST, blk)) std::this_thread::sleep_for(std::chrono::microseconds(us));
      if (nonfinite) continue;
      auto t0 = std::chrono::steady_clock::now();
      const mt_block_desc& b = blocks[blk];
      float* acc = (float*)(hopt + b.a_off);
      float* pm = master_store(cfg) ? (float*)(hopt + b.p_off) : nullptr;
      if (K > 1 && mb < K - 1)
        grad_accumulate_parallel(*pool, cfg.store_dtype, acc, host + b.g_off, b.region_elems, mb == 0);
      else if (K > 1)
        adam_accumulated_parallel(*pool, cfg.store_dtype, host + b.w_off, pm, acc, host + b.g_off,
                                  (float*)(hopt + b.m_off), (float*)(hopt + b.v_off), b.region_elems, k);
      else if (master_store(cfg))
        adam_master_parallel(*pool, (uint16_t*)(host + b.w_off), (float*)(hopt + b.p_off),
                             (const uint16_t*)(host + b.g_off), (float*)(hopt + b.m_off), (float*)(hopt + b.v_off),
                             b.region_elems, k);
      else
        adam_parallel(*pool, cfg.store_dtype, host + b.w_off, host + b.g_off, (float*)(hopt + b.m_off),
                      (float*)(hopt + b.v_off), b.region_elems, k);
      double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
      *adam_total += ms;
      bstats[blk].adam_ms = ms;
      if (device_done->load()) *adam_tail += ms;
    }
  } catch (const HipError& e) {
    adam_error = std::string(hipGetErrorString(e.code)) + " in " + e.where;
  } catch (const std::exception& e) {
    adam_error = e.what();
  }
}

// Streamed (and serialized, single-slot) schedule.  Uses: u = j for the
// forward of block j (0 embed, 1..L layers, L+1 head, whose use also runs the
// head backward); u = L+2+i for the backward of block L-i (i = 0..L-1:
// layers), and u = 2L+2 for the embedding backward.  Block j uses weight
// slot j%2, and consecutive backward uses alternate between the two
// gradient slots.  A slot's next prefetch starts when the compute of its
// last use has ended; a block's compute starts once its prefetch is done;
// a gradient slot is written again once the offload that read it is done.
//
// With the three streams (the default) every one of these rules is an event
// wait on the GPU: the prefetch stream waits for the compute-end event of
// the slot's last use, the compute stream for the prefetch's copy-end event
// and for the offload that last read the gradient slot, the offload stream
// for the compute-end event of the use whose gradients it moves.  When the
// offloads give the host link to the prefetches (yield_link), the offload of
// a use is enqueued after the prefetch that becomes ready at the same moment
// (the next one issued) and also waits for that prefetch's copy to end.
// With MT_FLAG_SDMA_QUEUES the copies run on two SDMA engines fed by host
// worker threads, and the enqueueing thread applies the same rules by
// waiting on the host.
//
// The serialized schedule lets nothing overlap: every copy starts after all
// compute enqueued so far and ends before more work is enqueued.  The
// single-slot schedule keeps every block in slot 0, so each prefetch waits
// for the previous block's compute (weights are not double-buffered;
// gradient offloads still overlap), and block L is fetched again for its
// backward because the head has replaced it.
template <typename T>
void Model::step_streamed(bool serialize) {
  const bool dry = trace != nullptr;  // record the schedule, issue nothing
  const bool single = cfg.mode == MT_SINGLE_SLOT;
  auto slot_of = [&](int j) { return single ? 0 : j % 2; };
  const bool poison = cfg.flags & MT_FLAG_POISON;
  const uint32_t nan_word = E == 2 ? 0x7FC07FC0u : 0x7FC00000u;
  std::vector<int> slot_last_use(2, -1);   // use that last bound each weight slot
  std::vector<int> fetch_job(n_uses, -1);  // SDMA queues: prefetch job of each use
  std::vector<int> gslot_last(2, -1);      // the offload (job, or use on streams) that last read each grad slot
  int gcount = 0;
  int last_out = -1;
  u_fetched.assign(n_uses, 0);
  u_offloaded.assign(n_uses, 0);
  struct Pending {
    int u, j, g;
  } pending{-1, -1, -1};
  const bool defer = hipq && yield_link && !serialize;
  // dry run: the operation each event or job stands for
  std::vector<int> op_fetch(n_uses, -1), op_poison(n_uses, -1), op_comp(n_uses, -1), op_off(n_uses, -1);
  std::vector<int> op_gslot_last(2, -1);
  int op_last_comp = -1, op_last_out = -1;
  std::vector<int> comp_waits;  // dependencies gathered for the next compute operation
  for (int& f : fence) f = -1;

  auto fetch = [&](int u, int j) {
    const int s = slot_of(j);
    hipEvent_t ready = slot_last_use[s] >= 0 ? ev_c_e[slot_last_use[s]] : nullptr;
    int op_ready = slot_last_use[s] >= 0 ? op_comp[slot_last_use[s]] : -1;
    if (poison) {
      // NaN-fill the slot on the compute stream, after its last use.
      if (!dry) {
        fill_u32(wslot[s], nan_word, slot_bytes / 4, sc);
        MT_HIP(hipEventRecord(ev_slot_free[u], sc));
      }
      op_poison[u] = tr_add(MT_LANE_COMPUTE, MT_OP_POISON, u, j, s, -1, {op_last_comp}, {});
      op_last_comp = op_poison[u];
      ready = ev_slot_free[u];
      op_ready = op_poison[u];
    }
    if (serialize) {
      if (!dry) MT_HIP(hipStreamSynchronize(sc));
      tr_fence(op_last_comp);
      ready = nullptr;
      op_ready = -1;
    }
    u_fetched[u] = 1;
    op_fetch[u] = tr_add(MT_LANE_PREFETCH, MT_OP_FETCH, u, j, s, -1, {op_ready}, {});
    if (dry) {
      if (serialize) tr_fence(op_fetch[u]);
    } else if (hipq) {
      if (ready) MT_HIP(hipStreamWaitEvent(sp, ready, 0));
      stream_delay(sp, MT_LANE_PREFETCH, u);
      MT_HIP(hipEventRecord(ev_x_s[u], sp));
      MT_HIP(hipMemcpyAsync(wslot[s], host + blocks[j].w_off, blocks[j].w_bytes, hipMemcpyHostToDevice, sp));
      MT_HIP(hipEventRecord(ev_x_e[u], sp));
      if (serialize) MT_HIP(hipStreamSynchronize(sp));
    } else {
      fetch_job[u] = xq_in->push({u, j, ready, wslot[s], host + blocks[j].w_off, (size_t)blocks[j].w_bytes,
                                  delay_us(MT_LANE_PREFETCH, u)});
      if (serialize) xq_in->wait(fetch_job[u]);
    }
  };
  auto begin = [&](int u) {
    if (u_fetched[u]) {
      if (hipq) {
        if (!dry) MT_HIP(hipStreamWaitEvent(sc, ev_x_e[u], 0));
        comp_waits.push_back(op_fetch[u]);
      } else {
        if (!dry) xq_in->wait(fetch_job[u]);
        tr_fence(op_fetch[u]);
      }
    }
    if (!dry) {
      stream_delay(sc, MT_LANE_COMPUTE, u);
      MT_HIP(hipEventRecord(ev_c_s[u], sc));
    }
  };
  // the compute operation of use u: block j, weight slot ws (-1: none),
  // gradient slot gs (-1: none)
  auto end = [&](int u, int j, int ws, int gs) {
    if (!dry) MT_HIP(hipEventRecord(ev_c_e[u], sc));
    if (!dry && (cfg.flags & MT_FLAG_PROGRESS))
      MT_HIP(hipLaunchHostFunc(sc, print_progress,
                               (void*)(uintptr_t)((uint64_t)u | (uint64_t)j << 20 | (uint64_t)n_uses << 40)));
    comp_waits.push_back(op_last_comp);
    op_comp[u] = tr_add(MT_LANE_COMPUTE, MT_OP_COMPUTE, u, j, ws, gs, comp_waits, {});
    op_last_comp = op_comp[u];
    comp_waits.clear();
    if (ws >= 0) slot_last_use[ws] = u;
  };
  // Grad slot for a backward use: the offload that last read it has finished.
  auto grad_slot = [&]() -> int {
    const int g = gcount % 2;
    if (gslot_last[g] >= 0) {
      if (hipq) {
        if (!dry) MT_HIP(hipStreamWaitEvent(sc, ev_o_e[gslot_last[g]], 0));
        comp_waits.push_back(op_gslot_last[g]);
      } else {
        if (!dry) xq_out->wait(gslot_last[g]);
        tr_fence(op_gslot_last[g]);
      }
    }
    return g;
  };
  // after_fetch >= 0: the offload also waits for that use's prefetch copy
  auto issue_offload = [&](int u, int j, int g, int after_fetch) {
    hipEvent_t ready = ev_c_e[u];
    int op_ready = op_comp[u];
    if (serialize) {
      if (!dry) MT_HIP(hipStreamSynchronize(sc));
      tr_fence(op_last_comp);
      ready = nullptr;
      op_ready = -1;
    }
    u_offloaded[u] = 1;
    op_off[u] = tr_add(MT_LANE_OFFLOAD, MT_OP_OFFLOAD, u, j, -1, g, {op_ready},
                       {after_fetch >= 0 ? op_fetch[after_fetch] : -1});
    tr_add(MT_LANE_HOST, MT_OP_ADAM, u, j, -1, -1, {op_off[u]}, {});
    op_last_out = op_off[u];
    op_gslot_last[g] = op_off[u];
    if (dry) {
      last_out = u;
      if (serialize) tr_fence(op_off[u]);
    } else if (hipq) {
      if (ready) MT_HIP(hipStreamWaitEvent(so, ready, 0));
      if (after_fetch >= 0) MT_HIP(hipStreamWaitEvent(so, ev_x_e[after_fetch], 0));
      stream_delay(so, MT_LANE_OFFLOAD, u);
      MT_HIP(hipEventRecord(ev_o_s[u], so));
      MT_HIP(hipMemcpyAsync(host + blocks[j].g_off, gslot[g], blocks[j].w_bytes, hipMemcpyDeviceToHost, so));
      MT_HIP(hipEventRecord(ev_o_e[u], so));
      push_adam(j, ev_o_e[u]);
      last_out = u;
      if (serialize) MT_HIP(hipStreamSynchronize(so));
    } else {
      last_out = xq_out->push({u, j, ready, host + blocks[j].g_off, gslot[g], (size_t)blocks[j].w_bytes,
                               delay_us(MT_LANE_OFFLOAD, u)});
      if (serialize) xq_out->wait(last_out);
    }
    gslot_last[g] = last_out;
  };
  auto offload = [&](int u, int j, int g) {
    ++gcount;
    if (defer)
      pending = Pending{u, j, g};
    else
      issue_offload(u, j, g, -1);
  };
  // the held offload, ordered after prefetch `after_fetch` (-1: none left)
  auto flush = [&](int after_fetch) {
    if (pending.u >= 0) issue_offload(pending.u, pending.j, pending.g, after_fetch);
    pending = Pending{-1, -1, -1};
  };

  BwdWs<T> ws = bwdws<T>();
  // ---- forward sweep (blocks 0 .. L+1)
  fetch(0, 0);
  for (int j = 0; j <= L + 1; ++j) {
    if (j > 0 && single) fetch(j, j);
    if (j + 1 <= L + 1 && !single) fetch(j + 1, j + 1);
    if (j <= L) {
      begin(j);
      if (!dry) compute_block_fwd<T>(j, wslot[slot_of(j)]);
      end(j, j, slot_of(j), -1);
    } else {
      // head: forward, loss, backward; weights stay bound for both
      const int g = grad_slot();
      begin(j);
      if (!dry) head_fwd_bwd<T>(blocks[j], wslot[slot_of(j)], gslot[g], ws.dxA);
      end(j, j, slot_of(j), g);
      offload(j, j, g);
    }
  }
  // ---- backward sweep: layers L-1 .. 0 (blocks L .. 1), then the embedding
  float* dx_in = ws.dxA;
  float* dx_out = ws.dxB;
  for (int i = 0; i < L; ++i) {
    const int j = L - i;
    const int u = L + 2 + i;
    // block L is still in its slot from the forward; the others are fetched
    // again (the prefetch of use u+1 is issued before use u computes).  The
    // offload of use u-1 became ready when this prefetch did.
    int fu = -1;
    if (single) {
      fetch(u, j);
      fu = u;
    } else if (j - 1 >= 1) {
      fetch(u + 1, j - 1);
      fu = u + 1;
    }
    flush(fu);
    const int g = grad_slot();
    begin(u);
    if (!dry) compute_layer_bwd<T>(j, wslot[slot_of(j)], gslot[g], dx_in, dx_out);
    end(u, j, slot_of(j), g);
    offload(u, j, g);
    std::swap(dx_in, dx_out);
  }
  {
    const int u = 2 * L + 2;
    flush(-1);
    const int g = grad_slot();
    begin(u);
    const mt_block_desc& b = blocks[0];
    if (!dry) embed_bwd<T>(dx_in, d_order, d_seg, (T*)gslot[g] + b.tensors[0].offset, V, d, sc);
    end(u, 0, -1, g);
    offload(u, 0, g);
    flush(-1);
  }
  // The step's device timeline ends once the last offload has landed.
  if (hipq) {
    if (!dry) MT_HIP(hipStreamWaitEvent(sc, ev_o_e[last_out], 0));
    tr_add(MT_LANE_COMPUTE, MT_OP_END, -1, -1, -1, -1, {op_last_comp, op_last_out}, {});
  } else {
    if (!dry) xq_out->wait(last_out);
    tr_fence(op_last_out);
    tr_add(MT_LANE_COMPUTE, MT_OP_END, -1, -1, -1, -1, {op_last_comp}, {});
  }
  if (!dry) MT_HIP(hipEventRecord(ev_end, sc));
}

// Resident schedule: every block's weights are copied once into device
// memory, every layer keeps its forward intermediates (no recompute), and
// all gradients are offloaded at the end; the same kernels run in the same
// order on the same data as in the streamed schedule.
template <typename T>
void Model::step_resident() {
  std::vector<uint8_t*> wr(blocks.size()), gr(blocks.size());
  uint64_t off = 0;
  for (size_t j = 0; j < blocks.size(); ++j) {
    wr[j] = wres + off;
    gr[j] = gres + off;
    off += round_up(blocks[j].w_bytes, 256);
  }
  MT_HIP(hipEventRecord(ev_h2d_s, sc));
  for (size_t j = 0; j < blocks.size(); ++j)
    MT_HIP(hipMemcpyAsync(wr[j], host + blocks[j].w_off, blocks[j].w_bytes, hipMemcpyHostToDevice, sc));
  MT_HIP(hipEventRecord(ev_h2d_e, sc));
  MT_HIP(hipEventRecord(ev_c_s[0], sc));
  for (int j = 0; j <= L; ++j) compute_block_fwd<T>(j, wr[j]);
  BwdWs<T> ws = bwdws<T>();
  head_fwd_bwd<T>(blocks[L + 1], wr[L + 1], gr[L + 1], ws.dxA);
  float* dx_in = ws.dxA;
  float* dx_out = ws.dxB;
  for (int j = L; j >= 1; --j) {
    compute_layer_bwd<T>(j, wr[j], gr[j], dx_in, dx_out);
    std::swap(dx_in, dx_out);
  }
  embed_bwd<T>(dx_in, d_order, d_seg, (T*)gr[0] + blocks[0].tensors[0].offset, V, d, sc);
  MT_HIP(hipEventRecord(ev_c_e[0], sc));
  MT_HIP(hipEventRecord(ev_d2h_s, sc));
  for (size_t j = 0; j < blocks.size(); ++j)
    MT_HIP(hipMemcpyAsync(host + blocks[j].g_off, gr[j], blocks[j].w_bytes, hipMemcpyDeviceToHost, sc));
  MT_HIP(hipEventRecord(ev_d2h_e, sc));
  MT_HIP(hipEventRecord(ev_end, sc));
  for (size_t j = 0; j < blocks.size(); ++j) push_adam((int)j, ev_d2h_e);
}

int Model::train_step(const int32_t* tokens) {
  auto t0 = std::chrono::steady_clock::now();
  StoreHeader* hdr = (StoreHeader*)host;
  const int64_t t = hdr->step + 1;
  const int K = micro_count(cfg);
  for (int64_t m = 0; m < (int64_t)K * M; ++m)
    if (tokens[m] < 0 || tokens[m] >= V) throw ApiError{MT_E_INVALID, "token out of range [0, vocab)"};
  nonfinite = false;
  double adam_total = 0, adam_tail = 0, loss_sum = 0;
  for (mb = 0; mb < K; ++mb) {
    run_pass(tokens + (int64_t)mb * M, t, &adam_total, &adam_tail);
    loss_sum += (double)*h_loss;
  }
  last_loss = (float)loss_sum;
  have_loss = true;
  double wall = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
  stats.adam_ms = adam_total;
  stats.adam_tail_ms = adam_tail;
  finish_stats(cfg.mode != MT_RESIDENT, wall);
  if (nonfinite) throw ApiError{MT_E_NONFINITE, "loss is not finite; Adam skipped, W/m/v unchanged"};
  hdr->step = t;
  return MT_OK;
}

// One forward and backward sweep over a micro-batch of M tokens; the host
// worker accumulates or applies (last micro-batch) each block's gradients as
// they land.  With one micro-batch this is the whole step.
void Model::run_pass(const int32_t* tokens, int64_t t, double* adam_total, double* adam_tail) {
  step_t = t;
  // tokens and the stable token-sorted order for the embedding backward
  std::vector<int32_t> count(V + 1, 0);
  for (int m = 0; m < M; ++m) count[tokens[m] + 1]++;
  memcpy(h_tok, tokens, sizeof(int32_t) * M);
  h_seg[0] = 0;
  for (int v = 0; v < V; ++v) h_seg[v + 1] = h_seg[v] + count[v + 1];
  std::vector<int32_t> pos(h_seg, h_seg + V);
  for (int m = 0; m < M; ++m) h_order[pos[tokens[m]]++] = m;
  MT_HIP(hipEventRecord(ev_start, sc));
  MT_HIP(hipMemcpyAsync(d_tok, h_tok, sizeof(int32_t) * M, hipMemcpyHostToDevice, sc));
  MT_HIP(hipMemcpyAsync(d_order, h_order, sizeof(int32_t) * M, hipMemcpyHostToDevice, sc));
  MT_HIP(hipMemcpyAsync(d_seg, h_seg, sizeof(int32_t) * (V + 1), hipMemcpyHostToDevice, sc));

  {
    std::lock_guard<std::mutex> g(q_mu);
    q_blocks.clear();
    q_events.clear();
    q_closed = false;
  }
  adam_error.clear();
  kev_used = 0;
  for (auto& s : bstats) s = mt_block_stats{};
  std::atomic<bool> device_done{false};
  const bool streamed = cfg.mode != MT_RESIDENT;
  yield_link = link_yields();
  const bool queues = streamed && !hipq;
  if (queues && !dma) {
    dma.reset(new DmaEngines(gslot[0], host));
    xq_in.reset(new TransferQueue(dma.get(), DMA_H2D, yield_link));
    xq_out.reset(new TransferQueue(dma.get(), DMA_D2H, yield_link));
  }
  h2d_host_ms.assign(n_uses, 0.0);
  d2h_host_ms.assign(n_uses, 0.0);
  std::thread worker([&] { adam_worker(t, adam_total, adam_tail, &device_done); });
  if (queues) {
    xq_in->start(&h2d_host_ms, nullptr);
    xq_out->start(&d2h_host_ms, [this](const TransferQueue::Job& job) { push_adam(job.j, nullptr); });
  }

  std::string enqueue_error;
  int enqueue_code = MT_OK;
  try {
    const bool bf = bf16_store(cfg);
    if (!streamed) {
      bf ? step_resident<uint16_t>() : step_resident<float>();
    } else {
      const bool ser = cfg.mode == MT_SERIALIZED;  // MT_SINGLE_SLOT is read inside
      bf ? step_streamed<uint16_t>(ser) : step_streamed<float>(ser);
    }
  } catch (const HipError& e) {
    enqueue_code = MT_E_HIP;
    enqueue_error = std::string(hipGetErrorString(e.code)) + " in " + e.where;
  } catch (const ApiError& e) {
    enqueue_code = e.code;
    enqueue_error = e.msg;
  }
  // Every copy that was enqueued finishes (or fails) before the Adam queue
  // closes, so Adam sees every block whose gradients arrived.  On the
  // streams, each offload was handed to Adam with its completion event.
  if (queues) {
    xq_in->stop();
    xq_out->stop();
  }
  close_adam();
  hipError_t e1 = hipStreamSynchronize(sc);
  if (e1 == hipSuccess) e1 = hipStreamSynchronize(sp);
  if (e1 == hipSuccess) e1 = hipStreamSynchronize(so);
  device_done = true;
  worker.join();
  if (enqueue_code != MT_OK) throw ApiError{enqueue_code, enqueue_error};
  if (e1 != hipSuccess) throw ApiError{MT_E_HIP, std::string("stream synchronize: ") + hipGetErrorString(e1)};
  if (!adam_error.empty()) throw ApiError{MT_E_HIP, "host Adam: " + adam_error};
}

void Model::finish_stats(bool streamed, double wall_ms) {
  mt_stats& s = stats;
  double adam_ms = s.adam_ms, adam_tail = s.adam_tail_ms;
  s = mt_stats{};
  s.adam_ms = adam_ms;
  s.adam_tail_ms = adam_tail;
  s.step_ms = wall_ms;
  s.loss = last_loss;
  s.n_blocks = (int)blocks.size();
  s.device_ms = ms_between(ev_start, ev_end);
  if (streamed) {
    for (int u = 0; u < n_uses; ++u) {
      const bool has_h2d = u < (int)u_fetched.size() && u_fetched[u];
      const bool has_d2h = u < (int)u_offloaded.size() && u_offloaded[u];
      const int j = u <= L + 1 ? u : (u <= 2 * L + 1 ? L - (u - (L + 2)) : 0);
      if (hipq) {
        if (has_h2d) h2d_host_ms[u] = ms_between(ev_x_s[u], ev_x_e[u]);
        if (has_d2h) d2h_host_ms[u] = ms_between(ev_o_s[u], ev_o_e[u]);
      }
      const double c = ms_between(ev_c_s[u], ev_c_e[u]);
      // compute-stream idle time before this use: the enqueueing thread
      // held it back until the block's weights had arrived and its grad
      // slot was free
      const double st = ms_between(u == 0 ? ev_start : ev_c_e[u - 1], ev_c_s[u]);
      double h = 0, dd = 0;
      if (has_h2d) {
        h = h2d_host_ms[u];
        s.h2d_ms += h;
        s.h2d_bytes += (double)blocks[j].w_bytes;
      }
      if (has_d2h) {
        dd = d2h_host_ms[u];
        s.d2h_ms += dd;
        s.d2h_bytes += (double)blocks[j].w_bytes;
      }
      s.stall_ms += st;
      mt_block_stats& bs = bstats[j];
      if (u <= L + 1) {
        s.fwd_ms += c;
        bs.fwd_ms = c;
        bs.h2d_fwd_ms = h;
        bs.stall_fwd_ms = st;
        if (u == L + 1) bs.d2h_ms = dd;
      } else {
        s.bwd_ms += c;
        bs.bwd_ms = c;
        bs.h2d_bwd_ms = h;
        bs.stall_bwd_ms = st;
        bs.d2h_ms = dd;
      }
    }
  } else {
    s.h2d_ms = ms_between(ev_h2d_s, ev_h2d_e);
    s.d2h_ms = ms_between(ev_d2h_s, ev_d2h_e);
    for (auto& b : blocks) {
      s.h2d_bytes += (double)b.w_bytes;
      s.d2h_bytes += (double)b.w_bytes;
    }
    s.fwd_ms = ms_between(ev_c_s[0], ev_c_e[0]);
  }
  ktimes.clear();
  for (size_t i = 0; i + 1 < kev_used + 1 && i < kev_used; i += 2) {
    const double ms = ms_between(kev[i], kev[i + 1]);
    const auto& meta = kev_meta[i / 2];
    ktimes.push_back(mt_kernel_time{meta.kind, meta.m, meta.n, meta.k, meta.epi, meta.layout, meta.flops, meta.bytes, ms});
    if (meta.kind == 0 || meta.kind == 2) {
      s.gemm_ms += ms;
      s.gemm_flops += meta.flops;
      s.gemm_bytes += meta.bytes;
      s.gemm_launches++;
    } else {
      s.attn_ms += ms;
      s.attn_flops += meta.flops;
      s.attn_launches++;
    }
  }
}

// -------------------------------------------------------------- create --
static std::vector<float> rope_table(int T, int hd, double theta, bool sine) {
  std::vector<float> out((size_t)T * (hd / 2));
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < hd / 2; ++i) {
      const double w = std::pow(theta, -2.0 * i / hd);
      const double a = (double)t * w;
      out[(size_t)t * (hd / 2) + i] = (float)(sine ? std::sin(a) : std::cos(a));
    }
  return out;
}

Model* create_model(const mt_config* cfg, void* arena, size_t arena_bytes, void* const streams[3]) {
  std::string why;
  if (validate_config(*cfg, &why) != MT_OK) throw ApiError{MT_E_INVALID, why};
  if (!arena || !streams || !streams[0] || !streams[1] || !streams[2])
    throw ApiError{MT_E_INVALID, "null arena or stream"};
  if (streams[0] == streams[1] || streams[1] == streams[2] || streams[0] == streams[2])
    throw ApiError{MT_E_INVALID, "prefetch, compute and offload need three different streams"};
  if ((uintptr_t)arena & 255) throw ApiError{MT_E_ALIGN, "device arena must be 256-byte aligned"};
  std::unique_ptr<Model> m(new Model());
  m->init_dims(*cfg);
  const uint64_t need = m->device_bytes();
  if (arena_bytes < need) throw ApiError{MT_E_SIZE, "device arena smaller than mt_device_bytes"};
  m->arena = (uint8_t*)arena;
  m->arena_bytes = arena_bytes;
  m->sp = (hipStream_t)streams[0];
  m->sc = (hipStream_t)streams[1];
  m->so = (hipStream_t)streams[2];
  m->hipq = !(cfg->flags & MT_FLAG_SDMA_QUEUES);
  if (bf16_store(*cfg))
    m->carve_all<uint16_t>(m->arena);
  else
    m->carve_all<float>(m->arena);
  // RoPE tables (float64 angles rounded to float32) and zeroed grad slots:
  // tensor padding inside a grad slot is never written and must stay 0.
  auto c = rope_table(m->Tq, m->hd, cfg->rope_theta, false);
  auto s = rope_table(m->Tq, m->hd, cfg->rope_theta, true);
  MT_HIP(hipMemcpy(m->cosb, c.data(), c.size() * 4, hipMemcpyHostToDevice));
  MT_HIP(hipMemcpy(m->sinb, s.data(), s.size() * 4, hipMemcpyHostToDevice));
  {
    const int h2 = m->hd / 2;
    std::vector<float> ct(c.size()), st(s.size());
    for (int t = 0; t < m->Tq; ++t)
      for (int i = 0; i < h2; ++i) {
        ct[(size_t)i * m->Tq + t] = c[(size_t)t * h2 + i];
        st[(size_t)i * m->Tq + t] = s[(size_t)t * h2 + i];
      }
    MT_HIP(hipMemcpy(m->cosT, ct.data(), ct.size() * 4, hipMemcpyHostToDevice));
    MT_HIP(hipMemcpy(m->sinT, st.data(), st.size() * 4, hipMemcpyHostToDevice));
  }
  for (int g = 0; g < 2; ++g) MT_HIP(hipMemset(m->gslot[g], 0, m->slot_bytes));
  if (m->gres) {
    uint64_t tot = 0;
    for (auto& b : m->blocks) tot += round_up(b.w_bytes, 256);
    MT_HIP(hipMemset(m->gres, 0, tot));
  }
  MT_HIP(hipDeviceSynchronize());
  MT_HIP(hipHostMalloc((void**)&m->h_tok, sizeof(int32_t) * m->M, hipHostMallocDefault));
  MT_HIP(hipHostMalloc((void**)&m->h_order, sizeof(int32_t) * m->M, hipHostMallocDefault));
  MT_HIP(hipHostMalloc((void**)&m->h_seg, sizeof(int32_t) * (m->V + 1), hipHostMallocDefault));
  MT_HIP(hipHostMalloc((void**)&m->h_loss, 256, hipHostMallocDefault));
  *m->h_loss = NAN;
  auto mk = [&](std::vector<hipEvent_t>& v) {
    v.resize(m->n_uses);
    for (auto& e : v) MT_HIP(hipEventCreate(&e));
  };
  mk(m->ev_c_s);
  mk(m->ev_c_e);
  mk(m->ev_slot_free);
  mk(m->ev_x_s);
  mk(m->ev_x_e);
  mk(m->ev_o_s);
  mk(m->ev_o_e);
  for (hipEvent_t* e : {&m->ev_h2d_s, &m->ev_h2d_e, &m->ev_d2h_s, &m->ev_d2h_e}) MT_HIP(hipEventCreate(e));
  MT_HIP(hipEventCreate(&m->ev_loss));
  MT_HIP(hipEventCreate(&m->ev_start));
  MT_HIP(hipEventCreate(&m->ev_end));
  int threads = cfg->host_threads;
  if (threads <= 0) {
    cpu_set_t set;
    threads = sched_getaffinity(0, sizeof(set), &set) == 0 ? CPU_COUNT(&set) : (int)std::thread::hardware_concurrency();
    threads = std::max(1, threads);
  }
  m->pool.reset(new ThreadPool(threads));
  m->bstats.assign(m->blocks.size(), mt_block_stats{});
  return m.release();
}

void destroy_model(Model* m) {
  if (!m) return;
  hipStreamSynchronize(m->sc);
  hipStreamSynchronize(m->sp);
  hipStreamSynchronize(m->so);
  for (auto* v : {&m->ev_c_s, &m->ev_c_e, &m->ev_slot_free, &m->ev_x_s, &m->ev_x_e, &m->ev_o_s, &m->ev_o_e})
    for (auto e : *v) hipEventDestroy(e);
  for (hipEvent_t e : {m->ev_h2d_s, m->ev_h2d_e, m->ev_d2h_s, m->ev_d2h_e}) hipEventDestroy(e);
  for (auto e : m->kev) hipEventDestroy(e);
  hipEventDestroy(m->ev_loss);
  hipEventDestroy(m->ev_start);
  hipEventDestroy(m->ev_end);
  hipHostFree(m->h_tok);
  hipHostFree(m->h_order);
  hipHostFree(m->h_seg);
  hipHostFree(m->h_loss);
  delete m;
}

std::vector<mt_sched_op> schedule_for(const mt_config& cfg) {
  std::string why;
  if (validate_config(cfg, &why) != MT_OK) throw ApiError{MT_E_INVALID, why};
  if (cfg.mode == MT_RESIDENT) throw ApiError{MT_E_INVALID, "the resident schedule moves no weights"};
  Model m;
  m.init_dims(cfg);
  m.hipq = !(cfg.flags & MT_FLAG_SDMA_QUEUES);
  m.yield_link = m.link_yields();
  for (auto* v : {&m.ev_c_s, &m.ev_c_e, &m.ev_slot_free, &m.ev_x_s, &m.ev_x_e, &m.ev_o_s, &m.ev_o_e})
    v->assign(m.n_uses, nullptr);
  std::vector<Model::TraceOp> tr;
  m.trace = &tr;
  const bool ser = cfg.mode == MT_SERIALIZED;
  bf16_store(cfg) ? m.step_streamed<uint16_t>(ser) : m.step_streamed<float>(ser);
  std::vector<mt_sched_op> out(tr.size());
  for (size_t i = 0; i < tr.size(); ++i) {
    const auto& t = tr[i];
    if (t.waits.size() > MT_SCHED_MAX_WAITS || t.link.size() > 2) throw ApiError{MT_E_STATE, "schedule operation waits"};
    mt_sched_op& o = out[i];
    o = mt_sched_op{};
    o.lane = t.lane;
    o.kind = t.kind;
    o.use = t.use;
    o.block = t.block;
    o.wslot = t.wslot;
    o.gslot = t.gslot;
    o.n_waits = (int32_t)t.waits.size();
    o.n_link = (int32_t)t.link.size();
    for (size_t k = 0; k < t.waits.size(); ++k) o.waits[k] = t.waits[k];
    for (size_t k = 0; k < t.link.size(); ++k) o.link[k] = t.link[k];
  }
  return out;
}

uint64_t device_bytes_for(const mt_config& cfg) {
  std::string why;
  if (validate_config(cfg, &why) != MT_OK) throw ApiError{MT_E_INVALID, why};
  Model m;
  m.init_dims(cfg);
  return m.device_bytes();
}

int bind_store(Model* m, void* host, size_t bytes, void* opt, size_t opt_bytes) {
  if (!host || !opt) throw ApiError{MT_E_INVALID, "null store part"};
  if ((uintptr_t)host % kStoreAlign || (uintptr_t)opt % kStoreAlign)
    throw ApiError{MT_E_ALIGN, "host store parts must be 4 KiB aligned"};
  if (bytes < m->store_bytes) throw ApiError{MT_E_SIZE, "DMA part smaller than mt_host_store_bytes"};
  if (opt_bytes < m->opt_bytes) throw ApiError{MT_E_SIZE, "optimizer part smaller than mt_host_opt_bytes"};
  const StoreHeader* h = (const StoreHeader*)host;
  if (h->magic != kStoreMagic || h->version != kStoreVersion) throw ApiError{MT_E_INVALID, "store header magic/version"};
  const mt_config& a = h->cfg;
  const mt_config& c = m->cfg;
  if (a.n_layers != c.n_layers || a.d_model != c.d_model || a.n_heads != c.n_heads || a.head_dim != c.head_dim ||
      a.d_ff != c.d_ff || a.vocab != c.vocab || a.store_dtype != c.store_dtype)
    throw ApiError{MT_E_INVALID, "store header describes another model shape"};
  if ((micro_count(a) > 1) != (micro_count(c) > 1))
    throw ApiError{MT_E_INVALID, "micro-batches need a store with a gradient accumulator (and only then)"};
  unsigned int flags = 0;
  if (hipHostGetFlags(&flags, host) != hipSuccess) {
    (void)hipGetLastError();
    throw ApiError{MT_E_INVALID, "DMA part of the host store is not pinned (use mt_alloc_host_store)"};
  }
  // the DMA engines are picked for the agents that own this store
  m->xq_in.reset();
  m->xq_out.reset();
  m->dma.reset();
  m->host = (uint8_t*)host;
  m->hopt = (uint8_t*)opt;
  return MT_OK;
}

int model_step(Model* m, const int32_t* tokens) {
  if (!m->host) throw ApiError{MT_E_NOT_BOUND, "no host store bound"};
  if (!tokens) throw ApiError{MT_E_INVALID, "null tokens"};
  return m->train_step(tokens);
}

int model_loss(const Model* m, float* out) {
  if (!m->have_loss) throw ApiError{MT_E_STATE, "no completed step"};
  *out = m->last_loss;
  return MT_OK;
}

int model_kernel_times(const Model* m, mt_kernel_time* out, int32_t capacity) {
  if (!m->have_loss) throw ApiError{MT_E_STATE, "no step has run"};
  if (!(m->cfg.flags & MT_FLAG_TIME_KERNELS)) throw ApiError{MT_E_STATE, "kernel times need MT_FLAG_TIME_KERNELS"};
  if (capacity < 0 || (capacity > 0 && !out)) throw ApiError{MT_E_INVALID, "null out or negative capacity"};
  for (size_t i = 0; i < m->ktimes.size() && (int64_t)i < capacity; ++i) out[i] = m->ktimes[i];
  return (int)m->ktimes.size();
}

int model_stats(const Model* m, mt_stats* out) {
  *out = m->stats;
  return MT_OK;
}

int model_block_stats(const Model* m, int block, mt_block_stats* out) {
  if (block < 0 || block >= (int)m->bstats.size()) throw ApiError{MT_E_INVALID, "block index"};
  *out = m->bstats[block];
  return MT_OK;
}

int model_debug_grad(const Model* m, int layer, void** dx) {
  if (!m->dxkeep) throw ApiError{MT_E_STATE, "gradients are kept only with MT_FLAG_KEEP_DX"};
  if (layer < 0 || layer > m->L) throw ApiError{MT_E_INVALID, "layer index"};
  *dx = m->dxkeep + (uint64_t)layer * m->M * m->d;
  return MT_OK;
}

int model_debug(const Model* m, int layer, void** ckpt, void** row_loss) {
  if (layer < 0 || layer > m->L) throw ApiError{MT_E_INVALID, "layer index"};
  if (ckpt)
    *ckpt = m->ckpt_lp ? (void*)(m->ckpt16 + (uint64_t)layer * m->M * m->d)
                       : (void*)(m->ckpt + (uint64_t)layer * m->M * m->d);
  if (row_loss) {
    if (bf16_store(m->cfg)) {
      HeadWs<uint16_t> h = const_cast<Model*>(m)->headws<uint16_t>();
      *row_loss = h.row_loss;
    } else {
      HeadWs<float> h = const_cast<Model*>(m)->headws<float>();
      *row_loss = h.row_loss;
    }
  }
  return MT_OK;
}

}  // namespace mt
