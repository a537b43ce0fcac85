/*
 * mt.h — C ABI of the MI355X layer-streamed training library.
 *
 * The method (MegaTrain, arXiv 2026; chatpaper.ai abstract and
 * radar.chestersoft.de "Methodik"): parameters and optimizer state live in
 * host memory; for each layer the weights stream in to the GPU and the
 * gradients stream out; a double-buffered engine overlaps prefetch, compute
 * and gradient offload on three streams; stateless layer templates bind the
 * incoming weights; every state of a layer (bf16 weights, bf16 gradients,
 * fp32 Adam moments) sits in one contiguous 4 KiB-aligned block; the Adam
 * step runs on the host CPU.
 *
 * Conventions of every call:
 *   - return 0 (MT_OK) on success or a negative MT_E_* code; no exception or
 *     abort crosses the ABI; mt_last_error() gives a message (thread-local);
 *   - pointers are plain host or device addresses as stated per argument;
 *   - the caller owns the device arena, the three streams, the host store and
 *     the token buffer; all of them must outlive the model handle;
 *   - calls on one model handle are not thread-safe; use one thread per model.
 */
#ifndef MT_H
#define MT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- errors -- */
#define MT_OK 0
#define MT_E_INVALID (-1)    /* bad configuration or argument */
#define MT_E_SIZE (-2)       /* buffer too small */
#define MT_E_ALIGN (-3)      /* buffer not 4 KiB (store) or 256 B (arena) aligned */
#define MT_E_NOT_BOUND (-4)  /* mt_train_step before mt_bind_host_store */
#define MT_E_HIP (-5)        /* a HIP runtime call failed; see mt_last_error() */
#define MT_E_NONFINITE (-6)  /* loss not finite: no Adam ran, the store's W/m/v are untouched */
#define MT_E_OOM (-7)        /* host allocation failed */
#define MT_E_STATE (-8)      /* wrong call order or unsupported mode for this call */

/* ------------------------------------------------------------- constants -- */
#define MT_F32 0             /* all-fp32 store: W, G, m, v in float32 */
#define MT_BF16 1            /* bf16 W and G, fp32 m and v */
#define MT_BF16_MASTER 2     /* bf16 W and G streamed as with MT_BF16, plus an fp32 master copy of W
                                beside m and v on the host: Adam updates the master in fp32 and W is
                                its bf16 rounding, so updates below bf16 resolution accumulate */

#define MT_STREAMED 0        /* two weight slots; prefetch, compute and offload overlap (the method) */
#define MT_SERIALIZED 1      /* the streamed schedule on the compute stream only */
#define MT_RESIDENT 2        /* every block's W on the device, no recompute */
#define MT_SINGLE_SLOT 3     /* one weight slot: each prefetch waits for the previous block's compute
                                (the method without double buffering; offloads still overlap) */

#define MT_BLOCK_EMBED 0
#define MT_BLOCK_LAYER 1
#define MT_BLOCK_HEAD 2

#define MT_STORE_ALIGN 4096
#define MT_MAX_TENSORS 8

/* Model and step configuration.  The architecture is a pre-norm decoder:
 * RMSNorm, causal multi-head attention with rotary positions (half-split
 * pairs), SwiGLU feed-forward, untied output head, mean next-token
 * cross-entropy over batch*(seq_len-1) positions; Adam without weight decay. */
typedef struct mt_config {
  int32_t n_layers, d_model, n_heads, head_dim, d_ff, vocab, batch, seq_len;
  int32_t store_dtype;   /* MT_F32, MT_BF16 or MT_BF16_MASTER */
  double rms_eps;        /* added inside the square root (used as float32 on the device) */
  double rope_theta;     /* rotation frequency base */
  double lr, beta1, beta2, adam_eps;  /* Adam: rounded to float32 as the host update uses them */
  int32_t mode;          /* MT_STREAMED, MT_SERIALIZED, MT_RESIDENT or MT_SINGLE_SLOT */
  int32_t host_threads;  /* Adam worker threads; 0 = every core in the affinity mask */
  int32_t flags;         /* MT_FLAG_* bits */
  int32_t micro_batches; /* gradient accumulation: mt_train_step takes micro_batches * batch * seq_len
                            tokens, runs one forward and backward sweep per micro-batch of `batch`
                            sequences, sums the gradients in an fp32 accumulator on the host and
                            applies one Adam step to the mean over all micro-batches.  0 or 1: none */
  int32_t head_chunk_tokens; /* tokens per pass of the output head (logits, loss, head backward): the
                                logits of that many tokens are held at once and the head's weight
                                gradient is summed over the passes in fp32.  0: automatic (one pass
                                while batch*seq_len*vocab*(4 + weight bytes) <= 16 GiB, else passes of
                                at most 4 GiB) */
  int32_t retain_layers; /* layers 0 .. retain_layers-1 keep their forward intermediates on the
                            device until their backward, which then skips the recompute: every
                            result is bit for bit that of the full recompute, the device arena
                            grows by one layer's intermediates per retained layer (about 5.4 GB at
                            d 5120, F 13824, 32768 tokens).  0: recompute every layer (the default:
                            layer-boundary checkpoints only).  Ignored by MT_RESIDENT, which keeps
                            every layer's */
} mt_config;

#define MT_FLAG_TIME_KERNELS 1  /* bracket every GEMM and attention launch with events */
#define MT_FLAG_POISON 2        /* fill a weight slot with NaN before each prefetch */
#define MT_FLAG_DUPLEX_LINK 4   /* let an offload start while a prefetch is ready or running.  Default:
                                   offloads wait for prefetches (which never wait for offloads) when a
                                   layer's backward does more than 30k flops per transferred byte, and
                                   share the link otherwise */

/* One tensor inside a block region: element offset from the region start,
 * row-major [rows x cols]. */
typedef struct mt_tensor_desc {
  uint64_t offset;
  int32_t rows, cols;
} mt_tensor_desc;

/* One block of the host store.  The store has two parts:
 *   - the DMA part (pinned, hipHostMalloc): a 4 KiB header page, then per
 *     block [W | G] — the only state that crosses the host link, one burst
 *     per region;
 *   - the optimizer part (pageable host memory): per block [m | v], then
 *     P (the fp32 master weights) with MT_BF16_MASTER, then A (the fp32
 *     gradient accumulator) with micro_batches > 1; read and written only by
 *     the host.
 * Every region and tensor start is 4 KiB-aligned and each block's regions
 * are contiguous inside their part.  base, w_off, g_off are byte offsets in
 * the DMA part; m_off, v_off, p_off, a_off byte offsets in the optimizer
 * part (p_off, a_off are 0 when the region does not exist).  Region element
 * counts are equal for all regions; W and G hold wb-byte elements (2 for
 * bf16, 4 for f32), m, v, P and A hold float32.  After a step with
 * micro-batches, A holds the summed gradient that Adam used and G the last
 * micro-batch's gradient.
 * Tensor order — embed: E [V x d]; layer: Wqkv [3d x d] (q, k, v rows),
 * Wo [d x d], Wgu [2F x d] (gate rows then up rows), Wd [d x F],
 * attn_norm [1 x d], ffn_norm [1 x d]; head: Wh [V x d], final_norm [1 x d]. */
typedef struct mt_block_desc {
  int32_t kind, layer, n_tensors, pad_;
  uint64_t base, w_off, g_off, m_off, v_off;
  uint64_t region_elems;
  uint64_t w_bytes, mv_bytes;
  mt_tensor_desc tensors[MT_MAX_TENSORS];
  uint64_t p_off, a_off;
} mt_block_desc;

/* Step statistics (milliseconds unless named otherwise); filled by
 * mt_train_step, read by mt_get_stats.  With micro-batches, step_ms,
 * adam_ms, adam_tail_ms and loss cover the whole step and the other fields
 * (and mt_block_stats) the last micro-batch's sweep. */
typedef struct mt_stats {
  double step_ms;            /* wall time of the last mt_train_step */
  double device_ms;          /* compute-stream events: step start to the end of the last offload */
  double fwd_ms, bwd_ms;     /* compute stream: forward sweep, head, backward sweep */
  double h2d_ms, d2h_ms;     /* summed copy durations (offloads: host clock, issue to completion) */
  double h2d_bytes, d2h_bytes;
  double stall_ms;           /* compute stream idle between blocks: weights not yet arrived, or a
                                gradient slot not yet offloaded */
  double adam_ms;            /* summed host Adam time */
  double adam_tail_ms;       /* host Adam time after the device finished */
  double gemm_ms, gemm_flops;/* MT_FLAG_TIME_KERNELS: summed GEMM launch time and flops */
  double attn_ms, attn_flops;
  int64_t gemm_launches, attn_launches;
  double loss;
  int32_t n_blocks, pad_;
  double gemm_bytes;         /* MT_FLAG_TIME_KERNELS: summed algorithmic bytes of the GEMM launches
                                (operands and residual read once, result written once) */
} mt_stats;

/* Per-block timing of the last step: forward and backward compute time on
 * the compute stream, prefetch and offload copy time, and the idle time of
 * the compute stream before the block's compute began. */
typedef struct mt_block_stats {
  double fwd_ms, bwd_ms, h2d_fwd_ms, h2d_bwd_ms, d2h_ms, stall_fwd_ms, stall_bwd_ms, adam_ms;
} mt_block_stats;

/* ------------------------------------------------------------ layout ----- */
/* Bytes of the DMA part of the host store (header page + [W | G] of every block). */
size_t mt_host_store_bytes(const mt_config* cfg);
/* Bytes of the optimizer part of the host store ([m | v] of every block). */
size_t mt_host_opt_bytes(const mt_config* cfg);
/* Number of blocks: embed, n_layers layers, head. */
int mt_block_count(const mt_config* cfg);
/* Layout of block i (0 = embed, 1..L = layers, L+1 = head). */
int mt_block_info(const mt_config* cfg, int block, mt_block_desc* out);
/* Bytes of the device arena the caller must allocate for cfg. */
size_t mt_device_bytes(const mt_config* cfg);

/* DMA part: pinned host memory (hipHostMalloc) of `bytes` rounded up to
 * 4 KiB; *out receives the host address.  Free with mt_free_host_store. */
int mt_alloc_host_store(size_t bytes, void** out);
void mt_free_host_store(void* p);
/* Optimizer part: anonymous pageable memory (4 KiB-aligned, transparent huge
 * pages requested).  Free with mt_free_host_opt and the same byte count. */
int mt_alloc_host_opt(size_t bytes, void** out);
void mt_free_host_opt(void* p, size_t bytes);
/* Write the 4 KiB header page (magic, version, config, Adam step 0) at the
 * start of the DMA part and zero both parts (W, G, m, v and the padding
 * between tensors), using the host threads of cfg (host_threads, 0 = all
 * allowed cores). */
int mt_init_store_header(const mt_config* cfg, void* dma_base, size_t dma_bytes, void* opt_base, size_t opt_bytes);
/* MT_BF16_MASTER stores: set every block's fp32 master P to the exact
 * widening of its bf16 W (call once, after writing the initial weights).
 * MT_E_STATE for stores of another dtype. */
int mt_store_init_master(const void* dma_base, size_t dma_bytes, void* opt_base, size_t opt_bytes);
/* Adam step counter t stored in the header (number of completed steps). */
int mt_store_step(const void* dma_base, int64_t* t);

/* Checkpoint and resume (steps 1..k, save, resume: the resumed run continues
 * bit for bit).  mt_store_save writes the resumable state of a host store to
 * the file `path`: the header page (configuration, completed Adam steps),
 * every block's W region and the whole optimizer part ([m | v], with P for
 * MT_BF16_MASTER); gradients are
 * rewritten by every step and are not saved.  mt_store_load reads such a
 * file into a store initialised by mt_init_store_header with the same layout
 * (layers, widths, vocabulary, store dtype): W, m, v and the step count.
 * The caller owns the buffers; no model may be running a step on the store.
 * Errors: MT_E_INVALID (bad header, layout mismatch, I/O failure or short
 * file), MT_E_SIZE (parts smaller than the layout). */
int mt_store_save(const void* dma_base, size_t dma_bytes, const void* opt_base, size_t opt_bytes, const char* path);
int mt_store_load(void* dma_base, size_t dma_bytes, void* opt_base, size_t opt_bytes, const char* path);

/* ------------------------------------------------------------- model ----- */
/* Create a model.  dev_arena: device memory of at least mt_device_bytes(cfg),
 * 256-byte aligned, caller-owned.  stream: the compute hipStream_t (default
 * priority), caller-owned; every kernel of the step runs on it.  The other
 * two streams of the method, weight prefetch and gradient offload, are
 * queues on two of the GPU's SDMA engines, each fed in order by a host
 * worker thread of the model.  No device work except uploading the RoPE
 * table; *out receives the handle. */
int mt_create_model(const mt_config* cfg, void* dev_arena, size_t arena_bytes, void* stream, void** out);
/* Bind a host store (DMA part from mt_alloc_host_store, optimizer part from
 * mt_alloc_host_opt or any 4 KiB-aligned host memory; header written,
 * weights initialised).  Checked: sizes >= mt_host_store_bytes and
 * mt_host_opt_bytes, 4 KiB alignment, header magic and shape; the DMA part
 * must be pinned. */
int mt_bind_host_store(void* model, void* dma_base, size_t dma_bytes, void* opt_base, size_t opt_bytes);
/* One training step on tokens (host int32 [micro_batches*batch*seq_len], or
 * [batch*seq_len] without micro-batches, values in [0, vocab)).  The loss is
 * the mean next-token loss over all micro-batches.  Synchronous: on return 0 the store holds the post-Adam W, m,
 * v, this step's G, and t+1 in the header.  On MT_E_NONFINITE no Adam ran. */
int mt_train_step(void* model, const int32_t* tokens);
/* Loss of the last completed step. */
int mt_get_loss(const void* model, float* out);
int mt_get_stats(const void* model, mt_stats* out);
int mt_get_block_stats(const void* model, int block, mt_block_stats* out);
/* Device addresses inside the arena for inspection by tests: the fp32
 * layer-boundary checkpoint x^l [batch*seq_len x d_model] (l = 0..n_layers)
 * and the fp32 per-position loss [batch*seq_len] (0 on the last position of
 * each sequence).  Valid until the next step. */
int mt_debug_buffers(const void* model, int layer, void** ckpt, void** row_loss);
void mt_destroy_model(void* model);

/* ------------------------------------------------------------ host Adam -- */
/* One Adam step over n elements on the host (the routine mt_train_step
 * uses per block): w, g of store dtype (bf16 as uint16 bits, or f32), m, v
 * float32; updated in place; step number t >= 1; threads as in mt_config. */
int mt_host_adam(int32_t store_dtype, void* w, const void* g, float* m, float* v, size_t n,
                 int64_t t, double lr, double beta1, double beta2, double eps, int32_t threads);
/* The MT_BF16_MASTER update: the same fp32 arithmetic on the master p
 * (float32, updated in place) with g widened from bf16; w (bf16 bits) receives
 * p' rounded to nearest even. */
int mt_host_adam_master(uint16_t* w, float* p, const uint16_t* g, float* m, float* v, size_t n,
                        int64_t t, double lr, double beta1, double beta2, double eps, int32_t threads);

const char* mt_last_error(void);
const char* mt_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MT_H */
