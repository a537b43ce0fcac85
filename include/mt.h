/*
 * mt.h — C ABI of the MI355X layer-streamed training library.
 *
 * The method (MegaTrain; pages cited as [Abstract] = chatpaper.ai,
 * "MegaTrain: Full Precision Training of 100B+ Parameter Large Language
 * Models on a Single GPU", Abstract; [Methodik], [Kernaussagen] =
 * radar.chestersoft.de summary of the paper, those sections;
 * [Innovaciones] = ecosistemastartup.com, "MegaTrain: entrena LLMs de 100B+
 * en una sola GPU", section on the key technical innovations):
 *   - parameters and optimizer state live in host memory and the GPU is a
 *     transient engine: per layer, weights stream in and gradients stream
 *     out [Abstract], [Kernaussagen], [Innovaciones] 1;
 *   - a double-buffered engine overlaps weight prefetch, compute and
 *     gradient offload on three streams in a ping-pong over two weight
 *     buffers [Methodik] (execution engine), [Abstract] 1);
 *   - stateless layer templates bind the incoming weights instead of an
 *     autograd graph [Methodik], [Abstract] 2), [Innovaciones] 3;
 *   - each layer's states (bf16 weights and gradients, fp32 Adam moments)
 *     are packed into contiguous 4 KiB-aligned blocks, and the Adam step
 *     runs on the host CPU with AVX-512 [Methodik] (layer-contiguous tiling).
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

/* Opaque model handle (mt_create_model .. mt_destroy_model). */
typedef struct mt_model mt_model;

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
  int32_t token_chunk;   /* tokens per pass of a layer's per-token work (the two norms, the q/k/v, output,
                            gate/up and down projections, SwiGLU): a layer runs its attention over all
                            tokens and the rest pass by pass, and its weight gradients are summed over
                            the passes in fp32 (gain gradients reduce in the same order as in one pass).
                            Passes are evened out to multiples of 64 tokens, each at least 192.  0:
                            automatic, one pass unless a weight gradient contracting over all tokens
                            would exceed the 2^31-byte operand addressing of the matrix kernels, then
                            passes of at most 32768 tokens.  Several passes need a bf16 store and a
                            streamed, serialized or single-slot schedule without retained layers */
} mt_config;

#define MT_FLAG_TIME_KERNELS 1  /* bracket every GEMM and attention launch with events */
#define MT_FLAG_POISON 2        /* fill a weight slot with NaN before each prefetch */
#define MT_FLAG_DUPLEX_LINK 4   /* let an offload start while a prefetch is ready or running.  Default:
                                   offloads wait for prefetches (which never wait for offloads) when a
                                   layer's backward does more than 30k flops per transferred byte, and
                                   share the link otherwise */
#define MT_FLAG_KEEP_DX 8       /* keep the gradient of the loss at every layer boundary, dl/dx^l for
                                   l = 0..n_layers (fp32, batch*seq_len x d_model each), in the device
                                   arena until the next step, for inspection (mt_debug_grad); adds
                                   (n_layers+1)*batch*seq_len*d_model*4 bytes to mt_device_bytes */
#define MT_FLAG_CKPT_BF16 32    /* keep the layer-boundary checkpoints x^0..x^n_layers rounded to bf16 (nearest
                                   even) instead of fp32, halving their device memory (long contexts): the
                                   forward still carries the fp32 residual stream from layer to layer, and
                                   the backward recomputes each layer from its rounded checkpoint.  Needs a
                                   bf16 store and a streamed, serialized or single-slot schedule without
                                   retained layers; mt_debug_buffers then returns bf16 checkpoints */
#define MT_FLAG_DELAYS 64       /* a test aid for ordering bugs: seeded host-side delays of 0 to 2 ms (about
                                   half of them 0), drawn per step, micro-batch, lane and use, before each
                                   prefetch copy, each compute use and each offload copy (a sleeping host
                                   function on the stream, or a sleep in the SDMA queue's worker) and before
                                   each host Adam update.  The results are bit for bit those without */
#define MT_FLAG_PROGRESS 128    /* print one line to stderr as each block use of a streamed step finishes
                                   on the device (a host function on the compute stream): progress for
                                   steps that run for minutes (very long contexts) */
#define MT_FLAG_SDMA_QUEUES 16  /* run the weight prefetches and gradient offloads on two of the GPU's
                                   SDMA engines (one per direction), each fed in order by a host worker
                                   thread that waits for the events the copy depends on, instead of
                                   hipMemcpyAsync on the prefetch and offload streams; the schedule and
                                   the results are the same.  The prefetch and offload streams then
                                   carry no work */

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

/* Sizes of the whole host store (mt_host_store_layout). */
typedef struct mt_layout {
  uint64_t dma_bytes;  /* pinned part: header page + [W | G] per block */
  uint64_t opt_bytes;  /* pageable part: [m | v] (+ P, A) per block */
  int32_t n_blocks;    /* embed, n_layers layers, head */
  int32_t pad_;
} mt_layout;

/* ------------------------------------------------------------ layout ----- */
/* Layout of the host store of cfg ([Methodik], layer-contiguous tiling: one
 * contiguous 4 KiB-aligned block of states per layer).  Fills *out; when
 * `blocks` is not null, also blocks[i] for every block i < min(n_blocks,
 * capacity) (same contents as mt_block_info).  Returns MT_OK, or
 * MT_E_INVALID for a bad configuration or a null `out`. */
int mt_host_store_layout(const mt_config* cfg, mt_layout* out, mt_block_desc* blocks, int32_t capacity);
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
/* Create a model: the engine that streams each layer through the GPU
 * ([Abstract]: the GPU as a transient compute engine; [Methodik]: the
 * pipelined double-buffered engine on three streams).
 *   dev_arena: device memory of at least mt_device_bytes(cfg) bytes,
 *     256-byte aligned, caller-owned (e.g. a torch uint8 tensor); it holds
 *     the two weight slots, two gradient slots, the fp32 layer-boundary
 *     checkpoints and one layer's workspace;
 *   streams[3]: hipStream_t values, caller-owned, three different streams,
 *     default priority: [0] weight prefetch (host -> device copies into the
 *     ping-pong slots), [1] compute (every kernel of the step), [2] gradient
 *     offload (device -> host copies); the library orders them with its own
 *     hipEvents;
 *   *out receives the handle.
 * The arena and the streams must outlive the handle.  No device work except
 * uploading the RoPE tables and zeroing the gradient slots.  Errors:
 * MT_E_INVALID (configuration, null or repeated stream), MT_E_ALIGN, MT_E_SIZE
 * (arena too small), MT_E_HIP. */
int mt_create_model(const mt_config* cfg, void* dev_arena, size_t arena_bytes, void* const streams[3],
                    mt_model** out);
/* Bind a host store ([Kernaussagen], [Innovaciones] 1: parameters and
 * optimizer state live in host memory).  DMA part from mt_alloc_host_store,
 * optimizer part from mt_alloc_host_opt or any 4 KiB-aligned host memory;
 * header written, weights initialised; both caller-owned and must outlive
 * the handle.  Checked: sizes >= mt_host_store_bytes and mt_host_opt_bytes,
 * 4 KiB alignment (MT_E_ALIGN), header magic and shape (MT_E_INVALID); the
 * DMA part must be pinned (MT_E_INVALID). */
int mt_bind_host_store(mt_model* model, void* dma_base, size_t dma_bytes, void* opt_base, size_t opt_bytes);
/* One training step ([Abstract]: for each layer, parameters stream in and
 * gradients stream out; the Adam step on the host CPU, [Methodik]) on tokens:
 * host int32 [micro_batches*batch*seq_len] (or [batch*seq_len] without
 * micro-batches), values in [0, vocab), copied before the call returns.
 * The loss is the mean next-token loss over all micro-batches.  Synchronous:
 * on return 0 the store holds the post-Adam W, m, v, this step's G, and t+1
 * in the header.  Errors: MT_E_NOT_BOUND, MT_E_INVALID (token out of range),
 * MT_E_NONFINITE (no Adam ran: W, m, v untouched), MT_E_HIP. */
int mt_train_step(mt_model* model, const int32_t* tokens);
/* Loss of the last completed step (MT_E_STATE before the first). */
int mt_get_loss(const mt_model* model, float* out);
/* Timings of the last step: per-block compute against transfer time and the
 * compute stream's idle time, the quantities the pages' overlap claim is
 * about ([Methodik]: the ping-pong keeps the GPU busy). */
int mt_get_stats(const mt_model* model, mt_stats* out);
int mt_get_block_stats(const mt_model* model, int block, mt_block_stats* out);
/* With MT_FLAG_TIME_KERNELS: every timed launch of the last step (the last
 * micro-batch's pass), in launch order, split by kernel so that the step
 * time [Rendimiento] reports can be traced to each kernel's rate.  Writes up
 * to `capacity` records and returns how many there are, or a negative error
 * (MT_E_STATE before the first step or without the flag). */
typedef struct mt_kernel_time {
  int32_t kind;          /* 0: GEMM, 1: attention, 2: the layer's grouped weight-gradient GEMM (down,
                            gate/up and output projections in one launch; m, n 0, k the tokens) */
  int32_t m, n, k;       /* GEMM: C [m x n] contracted over k (0 for attention) */
  int32_t epi, layout;   /* GEMM epilogue (0 bf16/store type, 1 fp32, 2 fp32 + residual) and K-major bits */
  double flops, bytes;   /* algorithmic work: 2mnk (attention: the causal forward's or 2.5x it), and
                            operands read once plus the result written once */
  double ms;             /* duration between HIP events around the launch on the compute stream */
} mt_kernel_time;
int mt_get_kernel_times(const mt_model* model, mt_kernel_time* out, int32_t capacity);
/* Device addresses inside the arena for inspection by tests: the fp32 (bf16
 * with MT_FLAG_CKPT_BF16) layer-boundary checkpoint x^l [batch*seq_len x
 * d_model] (l = 0..n_layers)
 * and the fp32 per-position loss [batch*seq_len] (0 on the last position of
 * each sequence).  Either output may be null.  Valid until the next step. */
int mt_debug_buffers(const mt_model* model, int layer, void** ckpt, void** row_loss);
/* With MT_FLAG_KEEP_DX: device address of dl/dx^l, the gradient arriving at
 * layer boundary l (l = n_layers: from the head; l = 0: the input of the
 * embedding backward), fp32 [batch*seq_len x d_model], of the last
 * micro-batch of the last step.  MT_E_STATE without the flag, MT_E_INVALID
 * for l outside 0..n_layers. */
int mt_debug_grad(const mt_model* model, int layer, void** dx);
void mt_destroy_model(mt_model* model);

/* ------------------------------------------------------------ host Adam -- */
/* One Adam step over n elements on the host ([Methodik]: the optimizer step
 * runs on the CPU with AVX-512; the routine mt_train_step uses per block):
 * w, g of store dtype (bf16 as uint16 bits, or f32), m, v float32; updated
 * in place; step number t >= 1; threads as in mt_config.  bf16 results are
 * rounded to nearest even (subnormals kept). */
int mt_host_adam(int32_t store_dtype, void* w, const void* g, float* m, float* v, size_t n,
                 int64_t t, double lr, double beta1, double beta2, double eps, int32_t threads);
/* The MT_BF16_MASTER update: the same fp32 arithmetic on the master p
 * (float32, updated in place) with g widened from bf16; w (bf16 bits) receives
 * p' rounded to nearest even. */
int mt_host_adam_master(uint16_t* w, float* p, const uint16_t* g, float* m, float* v, size_t n,
                        int64_t t, double lr, double beta1, double beta2, double eps, int32_t threads);

/* ------------------------------------------------------- measurement -- */
/* Host-link bandwidth with the copies mt_train_step issues ([Methodik]:
 * single DMA bursts of layer blocks are meant to fill the host link): `reps`
 * copies of `bytes` host_a -> dev_a (host to device), dev_b -> host_b (device
 * to host), and both directions at once.  Copies run as hipMemcpyAsync on
 * streams[0] (host to device) and streams[1] (device to host), or, with
 * MT_FLAG_SDMA_QUEUES in `flags`, on the SDMA engine queues (streams unused,
 * may be null).  host_a, host_b: pinned (mt_alloc_host_store), dev_a, dev_b:
 * device memory, each at least `bytes`; all caller-owned.  out_gbs[0..2]
 * receive host->device, device->host and the two together in GB/s (1e9
 * bytes; wall clock of the copies after one warm-up copy).  Synchronous.
 * Errors: MT_E_INVALID (null or unpinned buffer, zero size, reps < 1,
 * missing or equal streams), MT_E_HIP. */
int mt_link_probe(void* dev_a, void* dev_b, void* host_a, void* host_b, size_t bytes, int32_t reps, int32_t flags,
                  void* const streams[2], double out_gbs[3]);

/* ------------------------------------------------------------ schedule -- */
/* The operations one streamed step issues, in issue order, as data: the
 * double-buffered pipeline of [Methodik] (weights of the next block stream in
 * while the current one computes; gradients stream out behind it) for the
 * schedule `cfg` selects.  Nothing is allocated on or sent to the device; the
 * result depends only on `cfg` and lets a checker prove from the waits alone
 * that no operation can read a weight slot, gradient slot or host region
 * before the write it needs, or while another write to it is in flight.
 *
 * Lanes: operations of one lane 0..2 run in issue order (a HIP stream or an
 * SDMA queue's worker); MT_LANE_HOST operations (per-block Adam updates) are
 * not ordered among themselves.  An operation starts after every operation in
 * `waits` has finished; `link` lists orderings that only share out the host
 * link (an offload held back behind a prefetch) and carry no data.  The host
 * thread's own waits (serialized schedule, SDMA queues) appear as waits of
 * every later operation. */
#define MT_LANE_PREFETCH 0
#define MT_LANE_COMPUTE 1
#define MT_LANE_OFFLOAD 2
#define MT_LANE_HOST 3
#define MT_OP_FETCH 0    /* host W of `block` -> weight slot `wslot` */
#define MT_OP_POISON 1   /* NaN fill of weight slot `wslot` (MT_FLAG_POISON) */
#define MT_OP_COMPUTE 2  /* use `use` of `block`: reads weight slot `wslot` (-1: none), writes gradient
                            slot `gslot` (-1: none) */
#define MT_OP_OFFLOAD 3  /* gradient slot `gslot` -> host G of `block` */
#define MT_OP_ADAM 4     /* host Adam of `block`: reads its G, writes its W, m, v */
#define MT_OP_END 5      /* the step's device timeline ends (its completion event) */
#define MT_SCHED_MAX_WAITS 8
typedef struct mt_sched_op {
  int32_t lane, kind, use, block, wslot, gslot;
  int32_t n_waits, n_link;
  int32_t waits[MT_SCHED_MAX_WAITS];  /* indices of earlier operations */
  int32_t link[2];
} mt_sched_op;
/* Writes up to `capacity` operations to `ops` (may be null with capacity 0)
 * and returns how many the step has (call again with that capacity), or a
 * negative error: MT_E_INVALID (bad config, or MT_RESIDENT, whose step moves
 * no weights). */
int mt_schedule(const mt_config* cfg, mt_sched_op* ops, int32_t capacity);

const char* mt_last_error(void);
const char* mt_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MT_H */
