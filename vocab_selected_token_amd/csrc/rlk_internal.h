// rlk_internal.h -- launch arguments shared by the boundary and the kernels.
// Internal to librlk_logp.so; every field has been validated by the boundary
// before a launcher sees it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

struct Stage1Args {
  const void* logits;  // bf16 [num_rows, ld]
  int64_t ld;          // elements, multiple of 8
  int32_t num_rows;
  int32_t real_vocab;
  int32_t padded_vocab;
  int32_t num_tiles;
  int32_t tile_width;  // V_pad / T if exact, else 0
  int32_t tile_begin;  // this virtual shard's tiles
  int32_t tile_count;
  float* pmax;  // [num_rows][num_tiles]
  float* psum;
};

struct Stage2Args {
  const void* logits;
  int64_t ld;
  int32_t num_rows;
  int32_t real_vocab;
  int32_t num_tiles;
  const float* pmax;
  const float* psum;
  const int32_t* targets;
  const uint8_t* mask;  // may be null
  int32_t ignore_index;
  float* logp;
  float* lse;
  uint32_t* status;
};

struct BwdArgs {
  const void* logits;
  int64_t ld;
  int32_t num_rows;
  int32_t real_vocab;
  int32_t padded_vocab;
  const int32_t* targets;
  const uint8_t* mask;  // may be null
  int32_t ignore_index;
  const float* lse;
  const float* grad;
  void* dlogits;
  int64_t ld_d;
  bool out_bf16;
  uint32_t* status;
};

int64_t stage1_blocks(int64_t items);
int64_t bwd_col_blocks(int32_t padded_vocab);
hipError_t launch_stage1(const Stage1Args& a, hipStream_t stream);
hipError_t launch_stage2(const Stage2Args& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_clear_status(uint32_t* status, hipStream_t stream);

}  // namespace rlk
