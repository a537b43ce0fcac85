// Host store layout (see store.h).
#include "store.h"

#include <algorithm>

namespace mt {

int validate_config(const mt_config& c, std::string* why) {
  auto bad = [&](const char* m) { *why = m; return MT_E_INVALID; };
  if (c.n_layers < 1) return bad("n_layers must be >= 1");
  if (c.d_model < 8 || c.n_heads < 1 || c.head_dim < 2) return bad("bad width");
  if (c.n_heads * c.head_dim != c.d_model) return bad("n_heads * head_dim must equal d_model");
  if (c.head_dim % 2) return bad("head_dim must be even");
  if (c.d_ff < 1 || c.vocab < 2 || c.batch < 1 || c.seq_len < 2) return bad("bad sizes");
  if (c.d_model % 4 || c.d_ff % 4) return bad("d_model and d_ff must be multiples of 4");
  if (c.d_model > 16384) return bad("d_model > 16384");
  if (c.store_dtype != MT_F32 && c.store_dtype != MT_BF16 && c.store_dtype != MT_BF16_MASTER)
    return bad("store_dtype");
  if (c.mode < MT_STREAMED || c.mode > MT_SINGLE_SLOT) return bad("mode");
  if (bf16_store(c)) {
    // MFMA tiles move 8 bf16 (16 bytes) per lane along every contraction dim.
    if (c.d_model % 64 || c.d_ff % 64 || c.head_dim != 128)
      return bad("bf16 store needs d_model, d_ff multiples of 64 and head_dim 128");
    if (c.seq_len % 64) return bad("bf16 store needs seq_len multiple of 64");
  } else {
    if (c.head_dim > 64) return bad("f32 store supports head_dim <= 64");
    if (c.seq_len > 4096) return bad("f32 store supports seq_len <= 4096");
  }
  if ((int64_t)c.batch * c.seq_len > (int64_t)1 << 30) return bad("too many tokens");
  if (c.micro_batches < 0 || c.micro_batches > 4096) return bad("micro_batches must be in [0, 4096]");
  if (c.head_chunk_tokens < 0) return bad("head_chunk_tokens must be >= 0");
  if (c.retain_layers < 0 || c.retain_layers > c.n_layers) return bad("retain_layers must be in [0, n_layers]");
  if (c.token_chunk < 0) return bad("token_chunk must be >= 0");
  if (c.flags & ~(MT_FLAG_TIME_KERNELS | MT_FLAG_POISON | MT_FLAG_DUPLEX_LINK | MT_FLAG_KEEP_DX | MT_FLAG_SDMA_QUEUES |
                  MT_FLAG_CKPT_BF16 | MT_FLAG_DELAYS | MT_FLAG_PROGRESS))
    return bad("unknown flag bits");
  if ((int64_t)micro_count(c) * c.batch * c.seq_len > ((int64_t)1 << 31) - 1) return bad("too many tokens per step");
  if (!(c.rms_eps > 0) || !(c.rope_theta > 1) || !(c.lr >= 0) || !(c.beta1 >= 0 && c.beta1 < 1) ||
      !(c.beta2 >= 0 && c.beta2 < 1) || !(c.adam_eps > 0))
    return bad("bad hyper-parameters");
  return MT_OK;
}

static void add_tensor(mt_block_desc& b, uint64_t& cursor, int rows, int cols) {
  mt_tensor_desc& t = b.tensors[b.n_tensors++];
  t.offset = cursor;
  t.rows = rows;
  t.cols = cols;
  cursor = round_up(cursor + (uint64_t)rows * cols, kTensorAlignElems);
}

std::vector<mt_block_desc> store_layout(const mt_config& c, uint64_t* dma_bytes, uint64_t* opt_bytes) {
  const uint64_t d = c.d_model, F = c.d_ff, V = c.vocab;
  const uint64_t wb = wbytes(c);
  std::vector<mt_block_desc> blocks(c.n_layers + 2);
  uint64_t pos = kHeaderBytes, opos = 0;
  for (int i = 0; i < c.n_layers + 2; ++i) {
    mt_block_desc& b = blocks[i];
    memset(&b, 0, sizeof(b));
    uint64_t cur = 0;
    if (i == 0) {
      b.kind = MT_BLOCK_EMBED;
      b.layer = -1;
      add_tensor(b, cur, V, d);
    } else if (i == c.n_layers + 1) {
      b.kind = MT_BLOCK_HEAD;
      b.layer = -1;
      add_tensor(b, cur, V, d);
      add_tensor(b, cur, 1, d);
    } else {
      b.kind = MT_BLOCK_LAYER;
      b.layer = i - 1;
      add_tensor(b, cur, 3 * d, d);
      add_tensor(b, cur, d, d);
      add_tensor(b, cur, 2 * F, d);
      add_tensor(b, cur, d, F);
      add_tensor(b, cur, 1, d);
      add_tensor(b, cur, 1, d);
    }
    b.region_elems = cur;
    b.w_bytes = cur * wb;
    b.mv_bytes = cur * 4;
    b.base = pos;
    b.w_off = pos;
    b.g_off = b.w_off + b.w_bytes;
    pos = b.g_off + b.w_bytes;
    b.m_off = opos;
    b.v_off = b.m_off + b.mv_bytes;
    opos = b.v_off + b.mv_bytes;
    if (master_store(c)) {
      b.p_off = opos;
      opos += b.mv_bytes;
    }
    if (micro_count(c) > 1) {
      b.a_off = opos;
      opos += b.mv_bytes;
    }
  }
  *dma_bytes = pos;
  if (opt_bytes) *opt_bytes = opos;
  return blocks;
}

}  // namespace mt
