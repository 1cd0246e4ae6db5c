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
  float* pent;  // entropy statistic [num_rows][num_tiles], or null
};

struct Stage2Args {
  const void* logits;           // bf16 logits for the target gather, or
  const float* target_logit;    // if non-null: the fp32 target logit of each row
  int64_t ld;
  int32_t num_rows;
  int32_t real_vocab;
  int32_t num_tiles;
  const float* pmax;
  const float* psum;
  const float* pent;  // with entropy: the stage-1 entropy statistic
  const int32_t* targets;
  const uint8_t* mask;  // may be null
  int32_t ignore_index;
  float* logp;
  float* lse;
  float* entropy;  // per-row entropy out, or null
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
  const float* grad;      // may be null with grad_lse or grad_ent given
  const float* grad_lse;  // null = zero
  const float* grad_ent;  // null = zero
  const float* entropy;   // read where grad_ent is nonzero
  void* dlogits;
  int64_t ld_d;
  bool out_bf16;
  uint32_t* status;
};

// Forward and backward in one launch (g known before the forward): one block
// per row keeps the row's tile partials in LDS, so T is bounded.
constexpr int32_t kFbMaxTiles = 1024;

struct FwdBwdArgs {
  const void* logits;
  int64_t ld;
  int32_t num_rows;
  int32_t real_vocab;
  int32_t padded_vocab;
  int32_t num_tiles;
  int32_t tile_width;  // V_pad / T if exact, else 0
  const int32_t* targets;
  const uint8_t* mask;  // may be null
  int32_t ignore_index;
  const float* grad;
  float* logp;
  float* lse;
  void* dlogits;
  int64_t ld_d;
  bool out_bf16;
  uint32_t* status;
  // Unit schedule: [num_rows][num_tiles] 64-bit partial slots (two such arrays
  // with the entropy), or null for the one-block-per-row schedule (the same
  // bits either way).
  uint64_t* slots;
  // The extended form (unit schedule only): entropy out [num_rows] (non-null:
  // the forward of rlk_logp_fwd_ex); grad_lse / grad_ent (either non-null: the
  // gradient of rlk_logp_bwd_ex, with grad, grad_lse and grad_ent each null =
  // zero).
  float* entropy = nullptr;
  const float* grad_lse = nullptr;
  const float* grad_ent = nullptr;
};

// Whether the unit schedule of the one-launch forward+backward takes this
// geometry: T <= 64, tiles of at least 8 columns, and every tile's full
// chunks within the passes a lane group keeps in registers.
bool fwd_bwd_units_fit(int32_t real_vocab, int32_t padded_vocab, int32_t num_tiles);
// Polls of a row's partial slots before a block computes them itself (read
// once per process: RLK_FB_SPIN_LIMIT, default 16384; 0 makes every block
// compute its row's partials itself -- a hook for tests).
int32_t fwd_bwd_spin_limit();

// Fused LM-head variant: vocabulary rows per GEMM block (tiles must be at
// least this wide, so a block holds at most one tile bound).
constexpr int32_t kLmheadBlockVocab = 256;
constexpr int32_t kLmheadSlabK = 64;  // hidden_dim must be a multiple of this
// and at most this: a block's 256 rows of one operand then span under 2^31
// bytes, the range of the buffer resource its loads go through
constexpr int64_t kLmheadMaxHidden = int64_t{1} << 21;

struct LmheadArgs {
  const void* hidden;  // bf16 [num_tokens, hidden_dim]
  const void* weight;  // bf16 [>= real_vocab, hidden_dim]
  int32_t hidden_dim;
  int32_t num_tokens;
  int32_t real_vocab;
  int32_t padded_vocab;
  int32_t num_tiles;
  int32_t num_shards;  // virtual shards: launched one after another
  const int32_t* targets;
  const uint8_t* mask;  // may be null
  int32_t ignore_index;
  float* seg_m;  // [num_tokens][2 * ceil(real_vocab / 256)]
  float* seg_s;
  float* target_logit;  // [num_tokens]
  float* pmax;          // [num_tokens][num_tiles]
  float* psum;
};

// Most threads one launch may have.  A dispatch holds its grid size in 32 bits
// of threads: at 2^32 the launch fails, and above it the size wraps around and
// the kernel silently runs on a fraction of the grid.  Every launcher splits
// its work into launches of at most this many threads (2^31, or less when the
// RLK_MAX_LAUNCH_THREADS environment variable says so at the process's first
// launch -- a hook for tests, which check that any split gives the same bits).
int64_t launch_thread_limit();

// The allocation-free forward's workspace: a device array of the library's own,
// one per GPU, of this many bytes (status words plus 2 * N * T fp32 partials:
// N * T <= 4,194,304, e.g. 65,536 rows of 64 tiles).
constexpr size_t kNoAllocScratchBytes = (size_t{32} << 20) + 256;
// Its device address on the current device (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

int64_t stage1_blocks(int64_t items);
int64_t lmhead_grid_blocks(int32_t num_tokens, int32_t real_vocab);
hipError_t launch_lmhead(const LmheadArgs& a, hipStream_t stream);
int64_t bwd_col_blocks(int32_t padded_vocab);
hipError_t launch_stage1(const Stage1Args& a, hipStream_t stream);
hipError_t launch_stage2(const Stage2Args& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_bwd(const FwdBwdArgs& a, hipStream_t stream);
hipError_t launch_clear_status(uint32_t* status, hipStream_t stream);

}  // namespace rlk
