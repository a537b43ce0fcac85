// Layout of the host layer store and of the device arena.
//
// Host store (MegaTrain, radar.chestersoft.de "Methodik", layer-contiguous
// tiling): one block per embed / layer / head holding the block's weights,
// gradients and both Adam moments, every region and tensor start 4 KiB-aligned
// so one DMA burst moves a block's weights or gradients.  The weights and
// gradients of all blocks sit in the pinned DMA part (after a 4 KiB header
// page); the moments, and the fp32 master weights of an MT_BF16_MASTER store,
// never leave the host and sit in a pageable optimizer part with the same
// per-block order.
#pragma once

#include <vector>

#include "common.h"

namespace mt {

constexpr uint64_t kStoreAlign = MT_STORE_ALIGN;
constexpr uint64_t kTensorAlignElems = 2048;  // 4 KiB of bf16, 8 KiB of f32
constexpr uint64_t kHeaderBytes = 4096;
constexpr uint64_t kStoreMagic = 0x3145524f5453544dull;  // "MTSTORE1"
constexpr int32_t kStoreVersion = 2;

struct StoreHeader {
  uint64_t magic;
  int32_t version, n_blocks;
  mt_config cfg;
  int64_t step;  // completed Adam steps
  uint64_t total_bytes;
};

// Layer-block tensor indices.
enum { T_QKV = 0, T_O = 1, T_GU = 2, T_D = 3, T_ANORM = 4, T_FNORM = 5 };
// Head-block tensor indices.
enum { T_WH = 0, T_FINAL = 1 };

int validate_config(const mt_config& c, std::string* why);
// bf16 W and G on the link and the device (MT_BF16 and MT_BF16_MASTER)
inline bool bf16_store(const mt_config& c) { return c.store_dtype != MT_F32; }
inline bool master_store(const mt_config& c) { return c.store_dtype == MT_BF16_MASTER; }
inline int wbytes(const mt_config& c) { return bf16_store(c) ? 2 : 4; }
// micro-batches per step (gradient accumulation); 1 = none
inline int micro_count(const mt_config& c) { return c.micro_batches > 1 ? c.micro_batches : 1; }
std::vector<mt_block_desc> store_layout(const mt_config& c, uint64_t* dma_bytes, uint64_t* opt_bytes = nullptr);

}  // namespace mt
