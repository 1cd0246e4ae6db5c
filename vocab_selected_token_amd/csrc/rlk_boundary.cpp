// rlk_boundary.cpp -- the C ABI of librlk_logp.so (declared in include/rlk_logp.h).
//
// Validates every descriptor field, pointer and size on the host before
// anything is enqueued, derives the tile / virtual-shard geometry, and
// launches the kernels of rlk_kernels.hip on the caller's stream.  The
// library allocates nothing; its only state is the per-thread detail string.
//
// Error semantics follow PR #289 "[WS2][PR4][Logp] feat: add distributed TP/CP
// logprob drift report": dispatch is fail-closed (PR1 commit messages: a backend
// that cannot run is an error, never replaced by another), and the op refuses
// an active target beyond the real vocabulary and an active row whose LSE is
// not finite (review excerpt of the op's apply()).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <stdlib.h>
#include <string>

#include "rlk_internal.h"
#include "rlk_logp.h"

namespace {

thread_local std::string g_detail;

rlk_status fail(rlk_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return st;
}

rlk_status ok() { return RLK_OK; }

constexpr size_t kStatusBytes = 256;
constexpr int64_t kI32Max = 2147483647;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Validates the descriptor's sizes, tiling and flags.
rlk_status check_desc(const rlk_logp_desc* d) {
  if (!d) return fail(RLK_ERR_NULL_POINTER, "desc is NULL");
  if (d->num_tokens < 0 || d->num_tokens > kI32Max)
    return fail(RLK_ERR_BAD_SHAPE, "num_tokens=%lld outside [0, 2^31-1]",
                (long long)d->num_tokens);
  if (d->real_vocab < 1)
    return fail(RLK_ERR_BAD_SHAPE, "real_vocab=%lld must be >= 1", (long long)d->real_vocab);
  if (d->padded_vocab < d->real_vocab)
    return fail(RLK_ERR_BAD_SHAPE, "padded_vocab=%lld < real_vocab=%lld",
                (long long)d->padded_vocab, (long long)d->real_vocab);
  if (d->padded_vocab > kI32Max)
    return fail(RLK_ERR_BAD_SHAPE, "padded_vocab=%lld exceeds 2^31-1",
                (long long)d->padded_vocab);
  if (d->ld_logits < d->padded_vocab)
    return fail(RLK_ERR_BAD_SHAPE, "ld_logits=%lld < padded_vocab=%lld",
                (long long)d->ld_logits, (long long)d->padded_vocab);
  if (d->ld_logits % 8 != 0)
    return fail(RLK_ERR_ALIGNMENT, "ld_logits=%lld is not a multiple of 8 elements",
                (long long)d->ld_logits);
  if (d->num_vocab_tiles < 1 || (int64_t)d->num_vocab_tiles > d->padded_vocab)
    return fail(RLK_ERR_BAD_TILING, "num_vocab_tiles=%d outside [1, padded_vocab=%lld]",
                d->num_vocab_tiles, (long long)d->padded_vocab);
  if (d->num_virtual_shards < 1 || d->num_virtual_shards > d->num_vocab_tiles)
    return fail(RLK_ERR_BAD_TILING, "num_virtual_shards=%d outside [1, num_vocab_tiles=%d]",
                d->num_virtual_shards, d->num_vocab_tiles);
  if (d->flags & ~RLK_FLAG_VALIDATE)
    return fail(RLK_ERR_BAD_SHAPE, "unknown flag bits 0x%x", d->flags & ~RLK_FLAG_VALIDATE);
  // the partials must be addressable: N * T * 4 bytes, twice
  if ((double)d->num_tokens * (double)d->num_vocab_tiles * 8.0 > 9.0e18)
    return fail(RLK_ERR_BAD_SHAPE, "num_tokens * num_vocab_tiles too large");
  return RLK_OK;
}

size_t partial_bytes(const rlk_logp_desc* d) {
  return round256((size_t)d->num_tokens * (size_t)d->num_vocab_tiles * sizeof(float));
}

size_t needed_workspace(const rlk_logp_desc* d) { return kStatusBytes + 2 * partial_bytes(d); }

// The extended forward adds a third [N][T] array (the entropy statistic).
size_t needed_workspace_ex(const rlk_logp_desc* d) { return kStatusBytes + 3 * partial_bytes(d); }

rlk_status hip_fail(hipError_t e, const char* what) {
  return fail(RLK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// With RLK_FLAG_VALIDATE: wait for the stream, then read the status words.
rlk_status finish_validate(uint32_t* status, hipStream_t stream, bool check_nonfinite) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t host[2] = {0, 0};
  e = hipMemcpy(host, status, sizeof host, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(status)");
  if (host[0])
    return fail(RLK_ERR_TARGET_RANGE,
                "an effective-active target is outside [0, real_vocab); its outputs are NaN");
  if (check_nonfinite && host[1])
    return fail(RLK_ERR_NONFINITE_LSE,
                "an effective-active row has a non-finite LSE (its real logits are all "
                "-inf, or one of them is NaN or +inf)");
  return ok();
}

}  // namespace

extern "C" {

size_t rlk_logp_workspace_bytes(const rlk_logp_desc* desc) {
  if (check_desc(desc) != RLK_OK) return 0;
  return needed_workspace(desc);
}

rlk_status rlk_logp_tile_geometry(int64_t padded_vocab, int32_t num_vocab_tiles,
                                  int32_t num_virtual_shards, int64_t* bounds,
                                  int32_t* shard_first_tile) {
  if (padded_vocab < 1 || padded_vocab > kI32Max)
    return fail(RLK_ERR_BAD_SHAPE, "padded_vocab=%lld outside [1, 2^31-1]",
                (long long)padded_vocab);
  if (num_vocab_tiles < 1 || (int64_t)num_vocab_tiles > padded_vocab)
    return fail(RLK_ERR_BAD_TILING, "num_vocab_tiles=%d outside [1, padded_vocab]",
                num_vocab_tiles);
  if (num_virtual_shards < 1 || num_virtual_shards > num_vocab_tiles)
    return fail(RLK_ERR_BAD_TILING, "num_virtual_shards=%d outside [1, num_vocab_tiles]",
                num_virtual_shards);
  if (bounds)
    for (int32_t t = 0; t <= num_vocab_tiles; ++t)
      bounds[t] = ((int64_t)t * padded_vocab) / num_vocab_tiles;
  if (shard_first_tile)
    for (int32_t s = 0; s <= num_virtual_shards; ++s)
      shard_first_tile[s] = (int32_t)(((int64_t)s * num_vocab_tiles) / num_virtual_shards);
  return ok();
}

}  // extern "C"

namespace {

// The forward of rlk_logp_fwd and rlk_logp_fwd_ex (entropy != null: the
// entropy statistic rides along in stage 1 and stage 2 merges it).
rlk_status run_forward(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                       const uint8_t* active_mask, float* logp, float* lse, float* entropy,
                       void* workspace, size_t workspace_bytes, void* stream_ptr) {
  rlk_status st = check_desc(desc);
  if (st != RLK_OK) return st;
  const int64_t n = desc->num_tokens;
  if (n == 0) return ok();
  if (!logits || !targets || !logp || !lse)
    return fail(RLK_ERR_NULL_POINTER, "logits, targets, logp and lse must be non-NULL");
  const size_t need = entropy ? needed_workspace_ex(desc) : needed_workspace(desc);
  if (!workspace) return fail(RLK_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(RLK_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, need);
  if (!aligned(logits, 16)) return fail(RLK_ERR_ALIGNMENT, "logits not 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(RLK_ERR_ALIGNMENT, "workspace not 256-byte aligned");
  if (!aligned(targets, 4) || !aligned(logp, 4) || !aligned(lse, 4) || !aligned(entropy, 4))
    return fail(RLK_ERR_ALIGNMENT, "targets, logp, lse and entropy must be 4-byte aligned");

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  const int32_t T = desc->num_vocab_tiles, S = desc->num_virtual_shards;
  char* ws = static_cast<char*>(workspace);
  uint32_t* status = reinterpret_cast<uint32_t*>(ws);
  float* pmax = reinterpret_cast<float*>(ws + kStatusBytes);
  float* psum = reinterpret_cast<float*>(ws + kStatusBytes + partial_bytes(desc));
  float* pent =
      entropy ? reinterpret_cast<float*>(ws + kStatusBytes + 2 * partial_bytes(desc)) : nullptr;
  const bool validate = (desc->flags & RLK_FLAG_VALIDATE) != 0;

  hipError_t e;
  if (validate) {
    e = rlk::launch_clear_status(status, stream);
    if (e != hipSuccess) return hip_fail(e, "clear_status launch");
  }
  rlk::Stage1Args a1;
  a1.logits = logits;
  a1.ld = desc->ld_logits;
  a1.num_rows = (int32_t)n;
  a1.real_vocab = (int32_t)desc->real_vocab;
  a1.padded_vocab = (int32_t)desc->padded_vocab;
  a1.num_tiles = T;
  a1.tile_width = (desc->padded_vocab % T == 0) ? (int32_t)(desc->padded_vocab / T) : 0;
  a1.pmax = pmax;
  a1.psum = psum;
  a1.pent = pent;
  for (int32_t s = 0; s < S; ++s) {  // one launch per virtual shard
    const int32_t t0 = (int32_t)(((int64_t)s * T) / S);
    const int32_t t1 = (int32_t)(((int64_t)(s + 1) * T) / S);
    a1.tile_begin = t0;
    a1.tile_count = t1 - t0;
    if (rlk::stage1_blocks((int64_t)n * a1.tile_count) > kI32Max)
      return fail(RLK_ERR_BAD_SHAPE, "num_tokens * tiles per shard too large for one launch");
    e = rlk::launch_stage1(a1, stream);
    if (e != hipSuccess) return hip_fail(e, "stage1_partials launch");
  }
  rlk::Stage2Args a2;
  a2.logits = logits;
  a2.target_logit = nullptr;
  a2.ld = desc->ld_logits;
  a2.num_rows = (int32_t)n;
  a2.real_vocab = (int32_t)desc->real_vocab;
  a2.num_tiles = T;
  a2.pmax = pmax;
  a2.psum = psum;
  a2.pent = pent;
  a2.targets = targets;
  a2.mask = active_mask;
  a2.ignore_index = desc->ignore_index;
  a2.logp = logp;
  a2.lse = lse;
  a2.entropy = entropy;
  a2.status = status;
  e = rlk::launch_stage2(a2, stream);
  if (e != hipSuccess) return hip_fail(e, "stage2_merge launch");
  if (validate) return finish_validate(status, stream, true);
  return ok();
}

}  // namespace

extern "C" {

rlk_status rlk_logp_fwd(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                        const uint8_t* active_mask, float* logp, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream_ptr) {
  return run_forward(desc, logits, targets, active_mask, logp, lse, nullptr, workspace,
                     workspace_bytes, stream_ptr);
}

rlk_status rlk_logp_fwd_noalloc(const rlk_logp_desc* desc, const void* logits,
                                const int32_t* targets, const uint8_t* active_mask, float* logp,
                                float* lse, void* stream_ptr) {
  rlk_status st = check_desc(desc);
  if (st != RLK_OK) return st;
  if (desc->num_tokens == 0) return ok();
  const size_t need = needed_workspace(desc);
  if (need > rlk::kNoAllocScratchBytes)
    return fail(RLK_ERR_WORKSPACE,
                "rlk_logp_fwd_noalloc needs %zu bytes of scratch for num_tokens=%lld x "
                "num_vocab_tiles=%d; its fixed scratch holds %zu (use rlk_logp_fwd with a "
                "caller-allocated workspace)",
                need, (long long)desc->num_tokens, desc->num_vocab_tiles,
                rlk::kNoAllocScratchBytes);
  void* ws = nullptr;
  const hipError_t e = rlk::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  return run_forward(desc, logits, targets, active_mask, logp, lse, nullptr, ws,
                     rlk::kNoAllocScratchBytes, stream_ptr);
}

size_t rlk_logp_ex_workspace_bytes(const rlk_logp_desc* desc) {
  if (check_desc(desc) != RLK_OK) return 0;
  return needed_workspace_ex(desc);
}

rlk_status rlk_logp_fwd_ex(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                           const uint8_t* active_mask, float* logp, float* lse, float* entropy,
                           void* workspace, size_t workspace_bytes, void* stream_ptr) {
  rlk_status st = check_desc(desc);
  if (st != RLK_OK) return st;
  if (desc->num_tokens > 0 && !entropy)
    return fail(RLK_ERR_NULL_POINTER, "entropy must be non-NULL (rlk_logp_fwd has no entropy)");
  return run_forward(desc, logits, targets, active_mask, logp, lse, entropy, workspace,
                     workspace_bytes, stream_ptr);
}

}  // extern "C"

namespace {

// The backward of rlk_logp_bwd and rlk_logp_bwd_ex.  With grad_lse and
// grad_ent both null the plain kernel runs, so rlk_logp_bwd_ex without the
// extra gradients gives rlk_logp_bwd's bits.
rlk_status run_backward(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                        const uint8_t* active_mask, const float* lse, const float* entropy,
                        const float* grad_logp, const float* grad_lse, const float* grad_ent,
                        void* dlogits, int64_t ld_dlogits, rlk_dtype dlogits_dtype,
                        void* workspace, size_t workspace_bytes, void* stream_ptr, bool ex) {
  rlk_status st = check_desc(desc);
  if (st != RLK_OK) return st;
  if (dlogits_dtype != RLK_DTYPE_F32 && dlogits_dtype != RLK_DTYPE_BF16)
    return fail(RLK_ERR_DTYPE, "dlogits_dtype=%d is neither RLK_DTYPE_F32 nor RLK_DTYPE_BF16",
                (int)dlogits_dtype);
  if (ld_dlogits < desc->padded_vocab)
    return fail(RLK_ERR_BAD_SHAPE, "ld_dlogits=%lld < padded_vocab=%lld", (long long)ld_dlogits,
                (long long)desc->padded_vocab);
  if (ld_dlogits % 8 != 0)
    return fail(RLK_ERR_ALIGNMENT, "ld_dlogits=%lld is not a multiple of 8 elements",
                (long long)ld_dlogits);
  const int64_t n = desc->num_tokens;
  if (n == 0) return ok();
  if (!ex) {
    if (!logits || !targets || !lse || !grad_logp || !dlogits)
      return fail(RLK_ERR_NULL_POINTER, "logits, targets, lse, grad_logp and dlogits must be "
                                        "non-NULL");
  } else {
    if (!logits || !targets || !lse || !dlogits)
      return fail(RLK_ERR_NULL_POINTER, "logits, targets, lse and dlogits must be non-NULL");
    if (!grad_logp && !grad_lse && !grad_ent)
      return fail(RLK_ERR_NULL_POINTER, "at least one of grad_logp, grad_lse and grad_ent must "
                                        "be non-NULL");
    if (grad_ent && !entropy)
      return fail(RLK_ERR_NULL_POINTER, "grad_ent needs the forward's entropy");
  }
  if (!workspace) return fail(RLK_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < kStatusBytes)
    return fail(RLK_ERR_WORKSPACE, "workspace_bytes=%zu < %zu", workspace_bytes, kStatusBytes);
  if (!aligned(logits, 16) || !aligned(dlogits, 16))
    return fail(RLK_ERR_ALIGNMENT, "logits and dlogits must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(RLK_ERR_ALIGNMENT, "workspace not 256-byte aligned");
  if (!aligned(targets, 4) || !aligned(lse, 4) || !aligned(grad_logp, 4) ||
      !aligned(grad_lse, 4) || !aligned(grad_ent, 4) || !aligned(entropy, 4))
    return fail(RLK_ERR_ALIGNMENT, "targets, lse, entropy and the gradients must be 4-byte "
                                   "aligned");
  if (n * rlk::bwd_col_blocks((int32_t)desc->padded_vocab) > kI32Max)
    return fail(RLK_ERR_BAD_SHAPE, "num_tokens * column blocks too large for one launch");

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  uint32_t* status = reinterpret_cast<uint32_t*>(workspace);
  const bool validate = (desc->flags & RLK_FLAG_VALIDATE) != 0;
  hipError_t e;
  if (validate) {
    e = rlk::launch_clear_status(status, stream);
    if (e != hipSuccess) return hip_fail(e, "clear_status launch");
  }
  rlk::BwdArgs a;
  a.logits = logits;
  a.ld = desc->ld_logits;
  a.num_rows = (int32_t)n;
  a.real_vocab = (int32_t)desc->real_vocab;
  a.padded_vocab = (int32_t)desc->padded_vocab;
  a.targets = targets;
  a.mask = active_mask;
  a.ignore_index = desc->ignore_index;
  a.lse = lse;
  a.grad = grad_logp;
  a.grad_lse = grad_lse;
  a.grad_ent = grad_ent;
  a.entropy = entropy;
  a.dlogits = dlogits;
  a.ld_d = ld_dlogits;
  a.out_bf16 = dlogits_dtype == RLK_DTYPE_BF16;
  a.status = status;
  e = rlk::launch_bwd(a, stream);  // the plain kernel unless grad_lse or grad_ent is given
  if (e != hipSuccess) return hip_fail(e, "bwd_dlogits launch");
  if (validate) return finish_validate(status, stream, false);
  return ok();
}

}  // namespace

extern "C" {

rlk_status rlk_logp_bwd(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                        const uint8_t* active_mask, const float* lse, const float* grad_logp,
                        void* dlogits, int64_t ld_dlogits, rlk_dtype dlogits_dtype,
                        void* workspace, size_t workspace_bytes, void* stream_ptr) {
  return run_backward(desc, logits, targets, active_mask, lse, nullptr, grad_logp, nullptr,
                      nullptr, dlogits, ld_dlogits, dlogits_dtype, workspace, workspace_bytes,
                      stream_ptr, false);
}

rlk_status rlk_logp_bwd_ex(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                           const uint8_t* active_mask, const float* lse, const float* entropy,
                           const float* grad_logp, const float* grad_lse, const float* grad_ent,
                           void* dlogits, int64_t ld_dlogits, rlk_dtype dlogits_dtype,
                           void* workspace, size_t workspace_bytes, void* stream_ptr) {
  return run_backward(desc, logits, targets, active_mask, lse, entropy, grad_logp, grad_lse,
                      grad_ent, dlogits, ld_dlogits, dlogits_dtype, workspace, workspace_bytes,
                      stream_ptr, true);
}

// ---------------------------------------------------------------------------
// Forward and backward in one launch.
// ---------------------------------------------------------------------------
namespace {

rlk_status check_fwd_bwd_desc(const rlk_logp_desc* d) {
  rlk_status st = check_desc(d);
  if (st != RLK_OK) return st;
  if (d->num_vocab_tiles > rlk::kFbMaxTiles)
    return fail(RLK_ERR_BAD_TILING, "fused forward+backward takes num_vocab_tiles <= %d (got %d)",
                rlk::kFbMaxTiles, d->num_vocab_tiles);
  return RLK_OK;
}

}  // namespace

namespace {

// Bytes of partial slots the unit schedule needs for desc (0 where it does not
// apply: the one-block-per-row schedule runs with the status words alone).
size_t fwd_bwd_slot_bytes(const rlk_logp_desc* d) {
  if (!rlk::fwd_bwd_units_fit((int32_t)d->real_vocab, (int32_t)d->padded_vocab,
                              d->num_vocab_tiles))
    return 0;
  return (size_t)d->num_tokens * (size_t)d->num_vocab_tiles * sizeof(uint64_t);
}

}  // namespace

size_t rlk_logp_fwd_bwd_workspace_bytes(const rlk_logp_desc* desc) {
  if (check_fwd_bwd_desc(desc) != RLK_OK) return 0;
  return kStatusBytes + fwd_bwd_slot_bytes(desc);
}

rlk_status rlk_logp_fwd_bwd(const rlk_logp_desc* desc, const void* logits,
                            const int32_t* targets, const uint8_t* active_mask,
                            const float* grad_logp, float* logp, float* lse, void* dlogits,
                            int64_t ld_dlogits, rlk_dtype dlogits_dtype, void* workspace,
                            size_t workspace_bytes, void* stream_ptr) {
  rlk_status st = check_fwd_bwd_desc(desc);
  if (st != RLK_OK) return st;
  if (dlogits_dtype != RLK_DTYPE_F32 && dlogits_dtype != RLK_DTYPE_BF16)
    return fail(RLK_ERR_DTYPE, "dlogits_dtype=%d is neither RLK_DTYPE_F32 nor RLK_DTYPE_BF16",
                (int)dlogits_dtype);
  if (ld_dlogits < desc->padded_vocab)
    return fail(RLK_ERR_BAD_SHAPE, "ld_dlogits=%lld < padded_vocab=%lld", (long long)ld_dlogits,
                (long long)desc->padded_vocab);
  if (ld_dlogits % 8 != 0)
    return fail(RLK_ERR_ALIGNMENT, "ld_dlogits=%lld is not a multiple of 8 elements",
                (long long)ld_dlogits);
  const int64_t n = desc->num_tokens;
  if (n == 0) return ok();
  if (!logits || !targets || !grad_logp || !logp || !lse || !dlogits)
    return fail(RLK_ERR_NULL_POINTER, "logits, targets, grad_logp, logp, lse and dlogits must "
                                      "be non-NULL");
  if (!workspace) return fail(RLK_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < kStatusBytes)
    return fail(RLK_ERR_WORKSPACE, "workspace_bytes=%zu < %zu", workspace_bytes, kStatusBytes);
  if (!aligned(logits, 16) || !aligned(dlogits, 16))
    return fail(RLK_ERR_ALIGNMENT, "logits and dlogits must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(RLK_ERR_ALIGNMENT, "workspace not 256-byte aligned");
  if (!aligned(targets, 4) || !aligned(grad_logp, 4) || !aligned(logp, 4) || !aligned(lse, 4))
    return fail(RLK_ERR_ALIGNMENT, "targets, grad_logp, logp and lse must be 4-byte aligned");

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  uint32_t* status = reinterpret_cast<uint32_t*>(workspace);
  const bool validate = (desc->flags & RLK_FLAG_VALIDATE) != 0;
  hipError_t e;
  if (validate) {
    e = rlk::launch_clear_status(status, stream);
    if (e != hipSuccess) return hip_fail(e, "clear_status launch");
  }
  const int32_t T = desc->num_vocab_tiles;
  rlk::FwdBwdArgs a;
  a.logits = logits;
  a.ld = desc->ld_logits;
  a.num_rows = (int32_t)n;
  a.real_vocab = (int32_t)desc->real_vocab;
  a.padded_vocab = (int32_t)desc->padded_vocab;
  a.num_tiles = T;
  a.tile_width = (desc->padded_vocab % T == 0) ? (int32_t)(desc->padded_vocab / T) : 0;
  a.targets = targets;
  a.mask = active_mask;
  a.ignore_index = desc->ignore_index;
  a.grad = grad_logp;
  a.logp = logp;
  a.lse = lse;
  a.dlogits = dlogits;
  a.ld_d = ld_dlogits;
  a.out_bf16 = dlogits_dtype == RLK_DTYPE_BF16;
  a.status = status;
  // the unit schedule where the geometry fits and the workspace holds its slots
  const size_t slot_bytes = fwd_bwd_slot_bytes(desc);
  a.slots = (slot_bytes > 0 && workspace_bytes >= kStatusBytes + slot_bytes)
                ? reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kStatusBytes)
                : nullptr;
  e = rlk::launch_fwd_bwd(a, stream);
  if (e != hipSuccess) return hip_fail(e, "fwd_bwd launch");
  if (validate) return finish_validate(status, stream, true);
  return ok();
}

// ---------------------------------------------------------------------------
// The extended forward and backward in one launch.
// ---------------------------------------------------------------------------
namespace {

// Bytes of the two partial-slot arrays of the extended unit schedule (0 where
// the geometry does not take it).
size_t fwd_bwd_ex_slot_bytes(const rlk_logp_desc* d) { return 2 * fwd_bwd_slot_bytes(d); }

}  // namespace

size_t rlk_logp_fwd_bwd_ex_workspace_bytes(const rlk_logp_desc* desc) {
  if (check_desc(desc) != RLK_OK) return 0;
  const size_t units = kStatusBytes + fwd_bwd_ex_slot_bytes(desc);
  const size_t calls = needed_workspace_ex(desc);
  return fwd_bwd_ex_slot_bytes(desc) > 0 && units > calls ? units : calls;
}

rlk_status rlk_logp_fwd_bwd_ex(const rlk_logp_desc* desc, const void* logits,
                               const int32_t* targets, const uint8_t* active_mask,
                               const float* grad_logp, const float* grad_lse,
                               const float* grad_ent, float* logp, float* lse, float* entropy,
                               void* dlogits, int64_t ld_dlogits, rlk_dtype dlogits_dtype,
                               void* workspace, size_t workspace_bytes, void* stream_ptr) {
  rlk_status st = check_desc(desc);
  if (st != RLK_OK) return st;
  if (dlogits_dtype != RLK_DTYPE_F32 && dlogits_dtype != RLK_DTYPE_BF16)
    return fail(RLK_ERR_DTYPE, "dlogits_dtype=%d is neither RLK_DTYPE_F32 nor RLK_DTYPE_BF16",
                (int)dlogits_dtype);
  if (ld_dlogits < desc->padded_vocab)
    return fail(RLK_ERR_BAD_SHAPE, "ld_dlogits=%lld < padded_vocab=%lld", (long long)ld_dlogits,
                (long long)desc->padded_vocab);
  if (ld_dlogits % 8 != 0)
    return fail(RLK_ERR_ALIGNMENT, "ld_dlogits=%lld is not a multiple of 8 elements",
                (long long)ld_dlogits);
  const int64_t n = desc->num_tokens;
  if (n == 0) return ok();
  if (!logits || !targets || !logp || !lse || !entropy || !dlogits)
    return fail(RLK_ERR_NULL_POINTER, "logits, targets, logp, lse, entropy and dlogits must be "
                                      "non-NULL");
  if (!grad_logp && !grad_lse && !grad_ent)
    return fail(RLK_ERR_NULL_POINTER, "at least one of grad_logp, grad_lse and grad_ent must be "
                                      "non-NULL");
  if (!workspace) return fail(RLK_ERR_WORKSPACE, "workspace is NULL");
  const size_t slot_bytes = fwd_bwd_ex_slot_bytes(desc);
  const bool units = slot_bytes > 0 && workspace_bytes >= kStatusBytes + slot_bytes;
  if (!units && workspace_bytes < needed_workspace_ex(desc))
    return fail(RLK_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes,
                rlk_logp_fwd_bwd_ex_workspace_bytes(desc));
  if (!aligned(logits, 16) || !aligned(dlogits, 16))
    return fail(RLK_ERR_ALIGNMENT, "logits and dlogits must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(RLK_ERR_ALIGNMENT, "workspace not 256-byte aligned");
  if (!aligned(targets, 4) || !aligned(logp, 4) || !aligned(lse, 4) || !aligned(entropy, 4) ||
      !aligned(grad_logp, 4) || !aligned(grad_lse, 4) || !aligned(grad_ent, 4))
    return fail(RLK_ERR_ALIGNMENT, "targets, logp, lse, entropy and the gradients must be 4-byte "
                                   "aligned");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  uint32_t* status = reinterpret_cast<uint32_t*>(workspace);
  const bool validate = (desc->flags & RLK_FLAG_VALIDATE) != 0;
  hipError_t e;
  if (!units) {
    // the geometry (or the workspace) does not take the unit schedule: the two
    // extended calls, which give the same bits, with the status words cleared
    // once before them and checked once after
    if (n * rlk::bwd_col_blocks((int32_t)desc->padded_vocab) > kI32Max)
      return fail(RLK_ERR_BAD_SHAPE, "num_tokens * column blocks too large for one launch");
    rlk_logp_desc d1 = *desc;
    d1.flags &= ~RLK_FLAG_VALIDATE;
    if (validate) {
      e = rlk::launch_clear_status(status, stream);
      if (e != hipSuccess) return hip_fail(e, "clear_status launch");
    }
    st = run_forward(&d1, logits, targets, active_mask, logp, lse, entropy, workspace,
                     workspace_bytes, stream_ptr);
    if (st != RLK_OK) return st;
    st = run_backward(&d1, logits, targets, active_mask, lse, entropy, grad_logp, grad_lse,
                      grad_ent, dlogits, ld_dlogits, dlogits_dtype, workspace, workspace_bytes,
                      stream_ptr, true);
    if (st != RLK_OK) return st;
    if (validate) return finish_validate(status, stream, true);
    return ok();
  }

  if (validate) {
    e = rlk::launch_clear_status(status, stream);
    if (e != hipSuccess) return hip_fail(e, "clear_status launch");
  }
  const int32_t T = desc->num_vocab_tiles;
  rlk::FwdBwdArgs a;
  a.logits = logits;
  a.ld = desc->ld_logits;
  a.num_rows = (int32_t)n;
  a.real_vocab = (int32_t)desc->real_vocab;
  a.padded_vocab = (int32_t)desc->padded_vocab;
  a.num_tiles = T;
  a.tile_width = (desc->padded_vocab % T == 0) ? (int32_t)(desc->padded_vocab / T) : 0;
  a.targets = targets;
  a.mask = active_mask;
  a.ignore_index = desc->ignore_index;
  a.grad = grad_logp;
  a.logp = logp;
  a.lse = lse;
  a.dlogits = dlogits;
  a.ld_d = ld_dlogits;
  a.out_bf16 = dlogits_dtype == RLK_DTYPE_BF16;
  a.status = status;
  a.slots = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kStatusBytes);
  a.entropy = entropy;
  a.grad_lse = grad_lse;
  a.grad_ent = grad_ent;
  e = rlk::launch_fwd_bwd(a, stream);
  if (e != hipSuccess) return hip_fail(e, "fwd_bwd_units launch");
  if (validate) return finish_validate(status, stream, true);
  return ok();
}

// ---------------------------------------------------------------------------
// Fused LM-head variant.
// ---------------------------------------------------------------------------
namespace {

rlk_status check_fused_desc(const rlk_logp_desc* d) {
  if (!d) return fail(RLK_ERR_NULL_POINTER, "desc is NULL");
  if (d->num_tokens < 0 || d->num_tokens > kI32Max)
    return fail(RLK_ERR_BAD_SHAPE, "num_tokens=%lld outside [0, 2^31-1]",
                (long long)d->num_tokens);
  if (d->real_vocab < 1 || d->padded_vocab < d->real_vocab || d->padded_vocab > kI32Max)
    return fail(RLK_ERR_BAD_SHAPE, "need 1 <= real_vocab=%lld <= padded_vocab=%lld <= 2^31-1",
                (long long)d->real_vocab, (long long)d->padded_vocab);
  if (d->num_vocab_tiles < 1 || (int64_t)d->num_vocab_tiles > d->padded_vocab)
    return fail(RLK_ERR_BAD_TILING, "num_vocab_tiles=%d outside [1, padded_vocab]",
                d->num_vocab_tiles);
  if (d->padded_vocab / d->num_vocab_tiles < rlk::kLmheadBlockVocab)
    return fail(RLK_ERR_BAD_TILING,
                "fused LM-head needs tiles of at least %d columns (padded_vocab / "
                "num_vocab_tiles = %lld)",
                rlk::kLmheadBlockVocab, (long long)(d->padded_vocab / d->num_vocab_tiles));
  if (d->num_virtual_shards < 1 || d->num_virtual_shards > d->num_vocab_tiles)
    return fail(RLK_ERR_BAD_TILING, "num_virtual_shards=%d outside [1, num_vocab_tiles=%d]",
                d->num_virtual_shards, d->num_vocab_tiles);
  if (d->flags & ~RLK_FLAG_VALIDATE)
    return fail(RLK_ERR_BAD_SHAPE, "unknown flag bits 0x%x", d->flags & ~RLK_FLAG_VALIDATE);
  return RLK_OK;
}

struct FusedLayout {
  size_t pmax, psum, tlogit, seg_m, seg_s, total;
};

FusedLayout fused_layout(const rlk_logp_desc* d) {
  const size_t n = (size_t)d->num_tokens;
  const size_t n_vb = ((size_t)d->real_vocab + rlk::kLmheadBlockVocab - 1) /
                      rlk::kLmheadBlockVocab;
  const size_t part = round256(n * (size_t)d->num_vocab_tiles * sizeof(float));
  const size_t seg = round256(n * 2 * n_vb * sizeof(float));
  FusedLayout l;
  l.pmax = kStatusBytes;
  l.psum = l.pmax + part;
  l.tlogit = l.psum + part;
  l.seg_m = l.tlogit + round256(n * sizeof(float));
  l.seg_s = l.seg_m + seg;
  l.total = l.seg_s + seg;
  return l;
}

}  // namespace

size_t rlk_logp_fused_lmhead_workspace_bytes(const rlk_logp_desc* desc) {
  if (check_fused_desc(desc) != RLK_OK) return 0;
  return fused_layout(desc).total;
}

rlk_status rlk_logp_fused_lmhead(const rlk_logp_desc* desc, const void* hidden,
                                 const void* weight, int64_t hidden_dim, const int32_t* targets,
                                 const uint8_t* active_mask, float* logp, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream_ptr) {
  rlk_status st = check_fused_desc(desc);
  if (st != RLK_OK) return st;
  if (hidden_dim < rlk::kLmheadSlabK || hidden_dim % rlk::kLmheadSlabK != 0 ||
      hidden_dim > rlk::kLmheadMaxHidden)
    return fail(RLK_ERR_BAD_SHAPE, "hidden_dim=%lld must be a positive multiple of %d, at most %lld",
                (long long)hidden_dim, rlk::kLmheadSlabK, (long long)rlk::kLmheadMaxHidden);
  const int64_t n = desc->num_tokens;
  if (n == 0) return ok();
  if (!hidden || !weight || !targets || !logp || !lse)
    return fail(RLK_ERR_NULL_POINTER, "hidden, weight, targets, logp and lse must be non-NULL");
  const FusedLayout lay = fused_layout(desc);
  if (!workspace) return fail(RLK_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < lay.total)
    return fail(RLK_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes,
                lay.total);
  if (!aligned(hidden, 16) || !aligned(weight, 16))
    return fail(RLK_ERR_ALIGNMENT, "hidden and weight must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(RLK_ERR_ALIGNMENT, "workspace not 256-byte aligned");
  if (!aligned(targets, 4) || !aligned(logp, 4) || !aligned(lse, 4))
    return fail(RLK_ERR_ALIGNMENT, "targets, logp and lse must be 4-byte aligned");
  // the kernel addresses both operands with 32-bit offsets in 16-byte chunks
  if ((int64_t)desc->real_vocab * (hidden_dim / 8) > kI32Max || n * (hidden_dim / 8) > kI32Max)
    return fail(RLK_ERR_BAD_SHAPE, "hidden or weight holds 2^31 or more 16-byte chunks");
  if (rlk::lmhead_grid_blocks((int32_t)n, (int32_t)desc->real_vocab) > kI32Max)
    return fail(RLK_ERR_BAD_SHAPE, "num_tokens x vocabulary blocks too large for one launch");

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  char* ws = static_cast<char*>(workspace);
  uint32_t* status = reinterpret_cast<uint32_t*>(ws);
  const bool validate = (desc->flags & RLK_FLAG_VALIDATE) != 0;
  hipError_t e;
  if (validate) {
    e = rlk::launch_clear_status(status, stream);
    if (e != hipSuccess) return hip_fail(e, "clear_status launch");
  }
  rlk::LmheadArgs a;
  a.hidden = hidden;
  a.weight = weight;
  a.hidden_dim = (int32_t)hidden_dim;
  a.num_tokens = (int32_t)n;
  a.real_vocab = (int32_t)desc->real_vocab;
  a.padded_vocab = (int32_t)desc->padded_vocab;
  a.num_tiles = desc->num_vocab_tiles;
  a.num_shards = desc->num_virtual_shards;
  a.targets = targets;
  a.mask = active_mask;
  a.ignore_index = desc->ignore_index;
  a.seg_m = reinterpret_cast<float*>(ws + lay.seg_m);
  a.seg_s = reinterpret_cast<float*>(ws + lay.seg_s);
  a.target_logit = reinterpret_cast<float*>(ws + lay.tlogit);
  a.pmax = reinterpret_cast<float*>(ws + lay.pmax);
  a.psum = reinterpret_cast<float*>(ws + lay.psum);
  e = rlk::launch_lmhead(a, stream);
  if (e != hipSuccess) return hip_fail(e, "lmhead launch");
  rlk::Stage2Args a2;
  a2.logits = nullptr;
  a2.target_logit = a.target_logit;
  a2.ld = 0;
  a2.num_rows = (int32_t)n;
  a2.real_vocab = (int32_t)desc->real_vocab;
  a2.num_tiles = desc->num_vocab_tiles;
  a2.pmax = a.pmax;
  a2.psum = a.psum;
  a2.pent = nullptr;
  a2.targets = targets;
  a2.mask = active_mask;
  a2.ignore_index = desc->ignore_index;
  a2.logp = logp;
  a2.lse = lse;
  a2.entropy = nullptr;
  a2.status = status;
  e = rlk::launch_stage2(a2, stream);
  if (e != hipSuccess) return hip_fail(e, "stage2_merge launch");
  if (validate) return finish_validate(status, stream, true);
  return ok();
}

const char* rlk_status_string(rlk_status s) {
  switch (s) {
    case RLK_OK: return "RLK_OK";
    case RLK_ERR_NULL_POINTER: return "RLK_ERR_NULL_POINTER";
    case RLK_ERR_BAD_SHAPE: return "RLK_ERR_BAD_SHAPE";
    case RLK_ERR_BAD_TILING: return "RLK_ERR_BAD_TILING";
    case RLK_ERR_ALIGNMENT: return "RLK_ERR_ALIGNMENT";
    case RLK_ERR_WORKSPACE: return "RLK_ERR_WORKSPACE";
    case RLK_ERR_DTYPE: return "RLK_ERR_DTYPE";
    case RLK_ERR_TARGET_RANGE: return "RLK_ERR_TARGET_RANGE";
    case RLK_ERR_NONFINITE_LSE: return "RLK_ERR_NONFINITE_LSE";
    case RLK_ERR_HIP: return "RLK_ERR_HIP";
  }
  return "RLK_ERR_UNKNOWN";
}

const char* rlk_last_error_detail(void) { return g_detail.c_str(); }

}  // extern "C"

namespace rlk {

namespace {

int64_t read_thread_limit() {
  constexpr int64_t kLimit = int64_t{1} << 31;
  const char* v = getenv("RLK_MAX_LAUNCH_THREADS");
  if (!v || !*v) return kLimit;
  char* end = nullptr;
  const long long n = strtoll(v, &end, 10);
  if (end == v) return kLimit;  // not a number: the default
  if (n < 1024) return 1024;    // at least two blocks of every kernel
  return n < kLimit ? (int64_t)n : kLimit;
}

int32_t read_spin_limit() {
  constexpr int32_t kDefault = 1 << 14;
  const char* v = getenv("RLK_FB_SPIN_LIMIT");
  if (!v || !*v) return kDefault;
  char* end = nullptr;
  const long long n = strtoll(v, &end, 10);
  if (end == v) return kDefault;
  if (n < 0) return 0;
  return n < (1 << 30) ? (int32_t)n : (1 << 30);
}

}  // namespace

// The environment is read once, at the first launch of the process (a
// function-local static: initialised once, safely under concurrent first calls).
int64_t launch_thread_limit() {
  static const int64_t limit = read_thread_limit();
  return limit;
}

int32_t fwd_bwd_spin_limit() {
  static const int32_t limit = read_spin_limit();
  return limit;
}

}  // namespace rlk
