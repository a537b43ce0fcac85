// Model handle of the layer-streamed training step (see engine.hip).
#pragma once

#include <vector>

#include "common.h"

namespace mt {

struct Model;
Model* create_model(const mt_config* cfg, void* arena, size_t arena_bytes, void* const streams[3]);
void destroy_model(Model* m);
uint64_t device_bytes_for(const mt_config& cfg);
// The operations of one streamed step as data (no device work).
std::vector<mt_sched_op> schedule_for(const mt_config& cfg);
int bind_store(Model* m, void* host, size_t bytes, void* opt, size_t opt_bytes);
int model_step(Model* m, const int32_t* tokens);
int model_loss(const Model* m, float* out);
int model_stats(const Model* m, mt_stats* out);
int model_kernel_times(const Model* m, mt_kernel_time* out, int32_t capacity);
int model_block_stats(const Model* m, int block, mt_block_stats* out);
int model_debug(const Model* m, int layer, void** ckpt, void** row_loss);
int model_debug_grad(const Model* m, int layer, void** dx);

}  // namespace mt
