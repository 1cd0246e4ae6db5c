/*
 * rlk_logp.h -- deterministic selected-token log-probability over a
 * tile-decomposed vocabulary, for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources are web pages, cited by title and section):
 *
 *   [PR289] PR #289 "[WS2][PR4][Logp] feat: add distributed TP/CP logprob drift
 *           report": the stacked PR1 commit messages define the contract --
 *           padded vs real vocabulary, an explicit active mask plus
 *           ignore_index, padding columns excluded from the per-tile fp32
 *           (max, sumexp) partials, the (-inf, 0) partial of a tile that has
 *           no finite real logit, a merge in fixed global tile order,
 *           and fp32 selected-logprob and fp32 LSE outputs.  The review excerpt
 *           of the op's apply() shows the target-range check on active tokens
 *           and the refusal of an active row whose LSE is not finite.
 *   [H100V] "H100 canonical TP/CP validation" (docs/usage/h100-matrix-validation.md):
 *           the RL runs whose log metrics include the mean entropy.
 *   [I323]  Issue #323 "[WS2][Logprob] H100 validation and reproduction guide
 *           for Issue #241 PR1-PR5", "Test Order / 2. Six-Case TP/CP Matrix":
 *           64 vocabulary tiles over a real = padded vocabulary of 151936;
 *           "4. Cross-Topology Bitwise Check": regrouping the tiles across
 *           1/2/4 vocabulary shards leaves the fp32 outputs bitwise identical.
 *
 * For row r of the logits X (bf16, [N, ld]) with real vocabulary V_real:
 *
 *   LSE_r  = log sum_{j < V_real} exp(X[r, j])
 *   a_r    = (mask == NULL || mask[r] != 0) && target[r] != ignore_index
 *   logp_r = a_r ? float(X[r, target[r]]) - LSE_r : +0.0f
 *   dX[r, j] = a_r ? g_r * ([j == target[r]] - exp(X[r, j] - LSE_r)) : +0   (j < V_real)
 *   dX[r, j] = +0                                                   (V_real <= j < V_pad)
 *
 * The forward computes it as the pages do: tile t covers the columns
 * [floor(t*V_pad/T), floor((t+1)*V_pad/T)); each tile yields an fp32
 * (max, sumexp) over its real columns (columns >= V_real never contribute and
 * are never read for arithmetic, so any bit pattern may sit there); the T
 * partials are merged in ascending tile order into LSE.  Tiles may be grouped
 * into S contiguous "virtual shards" (shard s = tiles [floor(s*T/S),
 * floor((s+1)*T/S)), one launch each, standing in for the pages' tensor-
 * parallel ranks); every tile's arithmetic is independent of the launch that
 * computes it, so logp and LSE are bitwise identical for every S, across
 * repeated calls, and for a row whatever other rows share the call.
 *
 * Conventions shared by every call:
 *   - Ownership: the caller allocates and owns every buffer, device and host,
 *     including the workspace.  The library never allocates, frees or keeps a
 *     pointer after a call returns.  Its global state is the per-thread
 *     error-detail string, two settings read once per process from the
 *     environment (RLK_MAX_LAUNCH_THREADS below, RLK_FB_SPIN_LIMIT at
 *     rlk_logp_fwd_bwd), and, for rlk_logp_fwd_noalloc only, a device array of
 *     its own on each GPU it runs on.
 *   - Pointers marked (device) must be device-accessible memory of the device
 *     that is current on the calling thread; `desc` is a host pointer.
 *   - Streams: every call enqueues its kernels on `stream` (0 = the null
 *     stream) and returns without waiting, unless RLK_FLAG_VALIDATE is set.
 *   - Host errors (null pointer, shape, tiling, alignment, workspace, dtype)
 *     are detected before anything is enqueued; nothing is written then.
 *   - Data errors (an effective-active target outside [0, V_real); a
 *     non-finite LSE on an effective-active row) are found on the device.  The
 *     outputs are always safe: a bad target yields NaN and no out-of-bounds
 *     read.  With RLK_FLAG_VALIDATE the call synchronises the stream and
 *     reports them as RLK_ERR_TARGET_RANGE / RLK_ERR_NONFINITE_LSE.
 *   - There is one computation and no fallback to another: if the GPU path
 *     cannot run, the call fails.  Where a call has more than one schedule
 *     (rlk_logp_fwd_bwd, rlk_logp_fwd_bwd_ex), every schedule computes each
 *     value with the same code in the same order and gives the same bits; the
 *     geometry and the workspace passed decide which runs.
 *   - Graph capture: without RLK_FLAG_VALIDATE a call enqueues kernel launches
 *     only -- no allocation, memset, copy or synchronisation -- so it may be
 *     captured into a HIP graph and replayed; the replays read whatever the
 *     captured buffers hold at the time.  With the flag the call synchronises
 *     and copies the status words to the host, so it cannot be captured.
 *   - Batch size: a dispatch holds its grid size in 32 bits of threads, so a
 *     large batch is split into several launches of at most 2^31 threads each
 *     (the backward of 152576-column rows, at 75 blocks of 128 threads per
 *     row, splits from 223K rows on).  The split never changes a result bit.
 *     The environment variable RLK_MAX_LAUNCH_THREADS (read once per process,
 *     at its first launch; values below 1024 count as 1024) lowers the limit,
 *     so that tests can check this on small inputs.
 */
#ifndef RLK_LOGP_H_
#define RLK_LOGP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rlk_status {
  RLK_OK = 0,
  RLK_ERR_NULL_POINTER = 1,  /* a required pointer is NULL                        */
  RLK_ERR_BAD_SHAPE = 2,     /* sizes violate the limits stated on rlk_logp_desc  */
  RLK_ERR_BAD_TILING = 3,    /* T or S outside their ranges                        */
  RLK_ERR_ALIGNMENT = 4,     /* a pointer or leading dimension is misaligned       */
  RLK_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than required            */
  RLK_ERR_DTYPE = 6,         /* unknown rlk_dtype                                  */
  RLK_ERR_TARGET_RANGE = 7,  /* (VALIDATE) an effective-active target not in [0, V_real) */
  RLK_ERR_NONFINITE_LSE = 8, /* (VALIDATE) non-finite LSE on an effective-active row */
  RLK_ERR_HIP = 9            /* the HIP runtime reported an error                   */
} rlk_status;

typedef enum rlk_dtype { RLK_DTYPE_F32 = 0, RLK_DTYPE_BF16 = 1 } rlk_dtype;

/* Synchronise `stream` after the launches and turn the device status words
 * into RLK_ERR_TARGET_RANGE (checked first) or RLK_ERR_NONFINITE_LSE. */
#define RLK_FLAG_VALIDATE 1u

/* Problem description (host struct, read during the call only).
 * Limits (else RLK_ERR_BAD_SHAPE / RLK_ERR_BAD_TILING):
 *   num_tokens N        >= 0 (N == 0 enqueues nothing and returns RLK_OK)
 *   real_vocab V_real   >= 1 and <= padded_vocab
 *   padded_vocab V_pad  <= 2^31 - 1 (targets are int32 column indices)
 *   ld_logits           >= V_pad, a multiple of 8 elements (16-byte rows)
 *   num_vocab_tiles T   in [1, V_pad]; the pages fix T = 64
 *   num_virtual_shards S in [1, T]; it must not and does not change results
 *   ignore_index        any int32; the usual value is -100
 *   flags               0 or RLK_FLAG_VALIDATE                                  */
typedef struct rlk_logp_desc {
  int64_t num_tokens;
  int64_t real_vocab;
  int64_t padded_vocab;
  int64_t ld_logits;
  int32_t num_vocab_tiles;
  int32_t num_virtual_shards;
  int32_t ignore_index;
  uint32_t flags;
} rlk_logp_desc;

/* Bytes of device workspace that rlk_logp_fwd and rlk_logp_bwd need for
 * `desc` (0 if `desc` is NULL or invalid).  Layout, from the workspace base
 * (which must be 256-byte aligned):
 *   [0, 256)                     uint32 status words: [0] target-range flag,
 *                                [1] non-finite-LSE flag (nonzero = seen),
 *                                [2] after the unit schedule of
 *                                rlk_logp_fwd_bwd or rlk_logp_fwd_bwd_ex: the
 *                                blocks that computed their row's partials
 *                                themselves (0 when every exchange completed)
 *   [256, 256 + P)               float pmax[N][T]  per-tile maxima
 *   [256 + P, 256 + 2P)          float psum[N][T]  per-tile sums of exp(x - pmax)
 * where P = N*T*4 rounded up to a multiple of 256.  After rlk_logp_fwd the
 * partials hold the per-tile statistics of [PR289]'s contract (the identity
 * partial is (-inf, 0)); they stay valid until the workspace is reused. */
size_t rlk_logp_workspace_bytes(const rlk_logp_desc* desc);

/* Forward: per-tile partials, fixed-order merge, target gather.
 *   logits      (device) bf16 [N, ld_logits], 16-byte aligned; columns
 *               [V_real, ld_logits) are never used in arithmetic.
 *   targets     (device) int32 [N]; read only where the mask is set.
 *   active_mask (device) uint8 [N], nonzero = active; NULL = all active.
 *   logp        (device) float [N] out: selected log-probability; +0.0 on
 *               rows that are not effective-active; NaN for a bad target.
 *   lse         (device) float [N] out: LSE over the real vocabulary for every
 *               row (-inf for a row whose real logits are all -inf; NaN if one
 *               is NaN or +inf).
 *   workspace   (device) >= rlk_logp_workspace_bytes(desc) bytes, 256-byte
 *               aligned.
 * Rows are independent; outputs for row r depend only on row r's inputs. */
rlk_status rlk_logp_fwd(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                        const uint8_t* active_mask, float* logp, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Backward: dX = g * (onehot(target) - softmax(X)) on effective-active rows,
 * using the forward's LSE ([PR289]: the op is an autograd function whose
 * gradient flows to the logits; the formula is the derivative of logp_r).
 *   logits, targets, active_mask  as for rlk_logp_fwd (inactive rows' logits
 *               are not read).
 *   lse         (device) float [N]: the forward's LSE output.
 *   grad_logp   (device) float [N]: upstream gradient g; read on
 *               effective-active rows only.
 *   dlogits     (device) [N, ld_dlogits] of `dlogits_dtype`, 16-byte aligned,
 *               out.  Every element of columns [0, V_pad) is written: +0 on
 *               inactive rows and padded columns; on a row with a bad target
 *               the real columns are NaN.  Columns [V_pad, ld_dlogits) are not
 *               touched.  bf16 results are rounded to nearest even.
 *   ld_dlogits  >= V_pad, a multiple of 8 elements.
 *   workspace   as for rlk_logp_fwd (only the status words are used).
 * With RLK_FLAG_VALIDATE a bad effective-active target reports
 * RLK_ERR_TARGET_RANGE. */
rlk_status rlk_logp_bwd(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                        const uint8_t* active_mask, const float* lse, const float* grad_logp,
                        void* dlogits, int64_t ld_dlogits, rlk_dtype dlogits_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* rlk_logp_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a device array of the library's
 * own, one per GPU, of 32 MiB + 256 bytes, held until the process ends; the
 * call allocates nothing and frees nothing.  Outputs are bitwise those of
 * rlk_logp_fwd on the same arguments.
 *   desc, logits, targets, active_mask, logp, lse   as for rlk_logp_fwd.
 * Limit: rlk_logp_workspace_bytes(desc) <= 32 MiB + 256, i.e.
 * num_tokens * num_vocab_tiles <= 4,194,304 (65,536 rows of 64 tiles); a larger
 * problem returns RLK_ERR_WORKSPACE before anything is enqueued.  Every call on
 * one GPU uses the same array: calls that overlap on one GPU (from two host
 * threads, or on two streams without ordering between them) race and must not
 * be made.  Its first call on a device looks up the array's address there (no
 * allocation); other errors as for rlk_logp_fwd. */
rlk_status rlk_logp_fwd_noalloc(const rlk_logp_desc* desc, const void* logits,
                                const int32_t* targets, const uint8_t* active_mask, float* logp,
                                float* lse, void* stream);

/* Extended forward: rlk_logp_fwd plus the per-row entropy of the softmax over
 * the real vocabulary,
 *   H_r = -sum_{j < V_real} p_rj log p_rj,  p_rj = exp(x_rj - LSE_r),  0 log 0 = 0.
 * The pages return the LSE as a direct diagnostic beside the selected logp
 * ([PR289] walkthrough: forward_with_lse) and their RL runs log the mean
 * entropy ([H100V] "H100 canonical TP/CP validation", page
 * docs/usage/h100-matrix-validation.md: log metrics such as mean
 * loss/entropy).  Each tile also yields sum exp(x - max) (x - max) over its real
 * columns, merged in the same ascending tile order, so H is bitwise identical
 * for every num_virtual_shards, and logp and LSE are bitwise those of
 * rlk_logp_fwd.
 *   entropy     (device) float [N] out, non-NULL: H_r for every row; NaN where
 *               LSE is not finite (no distribution, or NaN / +inf logits).
 *   workspace   >= rlk_logp_ex_workspace_bytes(desc): the layout of
 *               rlk_logp_workspace_bytes followed by a third [N][T] float array
 *               (the entropy statistic) at [256 + 2P, 256 + 3P).
 * Other arguments and errors as for rlk_logp_fwd. */
size_t rlk_logp_ex_workspace_bytes(const rlk_logp_desc* desc);
rlk_status rlk_logp_fwd_ex(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                           const uint8_t* active_mask, float* logp, float* lse, float* entropy,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Extended backward: the gradient of a loss that reads logp, LSE and the
 * entropy H of rlk_logp_fwd_ex,
 *   dX[r, j] = a_r g_r ([j == target[r]] - p_rj) + gl_r p_rj - gh_r p_rj (log p_rj + H_r)
 * on the real columns (+0 on padded ones), where g = grad_logp, gl = grad_lse,
 * gh = grad_ent and a_r is effective-active.  The logp term applies to
 * effective-active rows only (logp is a constant +0 elsewhere); the LSE and
 * entropy terms apply to every row, since both outputs are defined on every
 * row (reading: the pages return the LSE of every row).  A column at -inf
 * contributes 0 (0 log 0 = 0); a row whose LSE is not finite gets NaN from any
 * LSE or entropy term that reaches it.  A row that no term reaches is +0 and
 * its logits are not read.
 *   lse         (device) float [N]: the forward's LSE.
 *   entropy     (device) float [N]: the forward's H; needed when grad_ent is
 *               non-NULL, otherwise unused (may be NULL).
 *   grad_logp, grad_lse, grad_ent  (device) float [N] each, or NULL for zero;
 *               at least one must be given.  With grad_lse and grad_ent both
 *               NULL the result is bitwise rlk_logp_bwd's.
 *   other arguments, dlogits layout and errors as for rlk_logp_bwd. */
rlk_status rlk_logp_bwd_ex(const rlk_logp_desc* desc, const void* logits, const int32_t* targets,
                           const uint8_t* active_mask, const float* lse, const float* entropy,
                           const float* grad_logp, const float* grad_lse, const float* grad_ent,
                           void* dlogits, int64_t ld_dlogits, rlk_dtype dlogits_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Forward and backward in one launch, for a caller that has the upstream
 * gradient g before the forward (for instance a policy-gradient loss whose
 * per-token weights are fixed in advance).  The outputs are bitwise those of
 * rlk_logp_fwd followed by rlk_logp_bwd on the same arguments -- the same tile
 * partials, the same ascending merge, the same gradient arithmetic -- for every
 * num_virtual_shards; HBM sees one read of the logits and one write of dX
 * instead of two reads and one write.  This single-pass schedule is not on the
 * pages; the contract is [PR289]'s.
 *
 * Two schedules, the same bits:
 *   - units (T <= 64 tiles of 8 to about 2,500 columns, e.g. 64 tiles over a
 *     152,576-column row): a block takes 8 consecutive tiles of a row, keeps
 *     their logits on chip, exchanges its tiles' (max, sumexp) partials
 *     with the row's other blocks through 64-bit slots in the workspace, and
 *     writes dX from what it kept.  A block waits for its row's slots a
 *     bounded number of polls (environment variable RLK_FB_SPIN_LIMIT, read
 *     once per process, default 16384; 0 skips the wait) and past it computes
 *     the row's partials itself.
 *   - rows (any other geometry, or a workspace of only the status words): one
 *     block per row, its second read served by the caches.
 *   desc        as for rlk_logp_fwd, with num_vocab_tiles <= 1024 (the row's
 *               partials live in on-chip memory); num_virtual_shards is
 *               validated and, as everywhere, changes nothing.
 *   logits, targets, active_mask       as for rlk_logp_fwd.
 *   grad_logp   (device) float [N]: g, read on effective-active rows only.
 *   logp, lse   (device) float [N] out, as for rlk_logp_fwd.
 *   dlogits, ld_dlogits, dlogits_dtype  out, as for rlk_logp_bwd.
 *   workspace   >= 256 bytes (the status words), 256-byte aligned; with
 *               rlk_logp_fwd_bwd_workspace_bytes(desc) bytes (256 + 8 N T
 *               where the unit schedule takes the geometry, else 256) the
 *               unit schedule runs.  Its slots are overwritten on every call:
 *               calls that share a workspace must not overlap.
 * Errors as for rlk_logp_fwd (RLK_ERR_BAD_TILING also for T > 1024) and
 * rlk_logp_bwd. */
size_t rlk_logp_fwd_bwd_workspace_bytes(const rlk_logp_desc* desc);
rlk_status rlk_logp_fwd_bwd(const rlk_logp_desc* desc, const void* logits,
                            const int32_t* targets, const uint8_t* active_mask,
                            const float* grad_logp, float* logp, float* lse, void* dlogits,
                            int64_t ld_dlogits, rlk_dtype dlogits_dtype, void* workspace,
                            size_t workspace_bytes, void* stream);

/* The extended forward and backward in one launch: bitwise the outputs of
 * rlk_logp_fwd_ex followed by rlk_logp_bwd_ex on the same arguments (logp,
 * LSE, entropy H, and the gradient of a loss reading all three), for a caller
 * that has the three upstream gradients before the forward.  Where the geometry
 * takes the unit schedule (as for rlk_logp_fwd_bwd) and the workspace holds its
 * slots, one launch reads the logits once; otherwise the two extended calls
 * run, with the same bits.  This single-pass schedule is not on the pages; the
 * contract is [PR289]'s, with the extensions of rlk_logp_fwd_ex/_bwd_ex.
 *   desc, logits, targets, active_mask   as for rlk_logp_fwd_ex.
 *   grad_logp, grad_lse, grad_ent        (device) float [N] each, or NULL
 *               (zero); at least one non-NULL; as for rlk_logp_bwd_ex.
 *   logp, lse, entropy                   (device) float [N] out.
 *   dlogits, ld_dlogits, dlogits_dtype   out, as for rlk_logp_bwd_ex.
 *   workspace   >= rlk_logp_fwd_bwd_ex_workspace_bytes(desc) bytes, 256-byte
 *               aligned: 256 + 16 N T with the unit schedule (two slot
 *               arrays), else rlk_logp_ex_workspace_bytes(desc); with less
 *               than the first but at least the second the two calls run.
 * Errors as for rlk_logp_fwd_ex and rlk_logp_bwd_ex, all returned before any
 * launch; with RLK_FLAG_VALIDATE the status words are checked once, after
 * both steps (target range and non-finite LSE). */
size_t rlk_logp_fwd_bwd_ex_workspace_bytes(const rlk_logp_desc* desc);
rlk_status rlk_logp_fwd_bwd_ex(const rlk_logp_desc* desc, const void* logits,
                               const int32_t* targets, const uint8_t* active_mask,
                               const float* grad_logp, const float* grad_lse,
                               const float* grad_ent, float* logp, float* lse, float* entropy,
                               void* dlogits, int64_t ld_dlogits, rlk_dtype dlogits_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Fused LM-head variant: the logits are z = hidden . weight^T, taken in fp32
 * from bf16 MFMA products and never written to memory.  The pages name an
 * optional fused kernel without describing it ([I323] "Validation Boundary");
 * this one keeps [PR289]'s contract -- per-tile fp32 (max, sumexp) over the real
 * columns, the (-inf, 0) identity, the merge in ascending tile order, fp32 logp
 * and LSE -- with the statistics and the target logit read from the fp32
 * accumulators (no rounding of z to bf16).
 *   desc        num_tokens, real_vocab, padded_vocab, num_vocab_tiles,
 *               num_virtual_shards, ignore_index and flags as for rlk_logp_fwd;
 *               ld_logits is not used; every tile must be at least 256 columns
 *               wide (padded_vocab / num_vocab_tiles >= 256).  Each virtual
 *               shard is computed by its own launches over its own weight rows
 *               only, as one GPU of a vocabulary-parallel LM head would be; logp,
 *               LSE and the per-tile partials are bitwise the same for every
 *               num_virtual_shards in [1, num_vocab_tiles] ([PR289] PR1:
 *               tile-aligned vocabulary shards, fixed-order merge).
 *   hidden      (device) bf16 [num_tokens, hidden_dim], row-major, 16-byte aligned.
 *   weight      (device) bf16 [padded_vocab, hidden_dim], row-major, 16-byte
 *               aligned; rows >= real_vocab are never read.
 *   hidden_dim  a positive multiple of 64, at most 2^21 (RLK_ERR_BAD_SHAPE
 *               otherwise).
 *   targets, active_mask, logp, lse   as for rlk_logp_fwd.
 *   workspace   >= rlk_logp_fused_lmhead_workspace_bytes(desc), 256-byte
 *               aligned.  Its status words and per-tile partials sit where
 *               rlk_logp_fwd puts them; the rest is scratch.
 * Errors as for rlk_logp_fwd; RLK_ERR_BAD_TILING also for tiles narrower than
 * 256 columns. */
size_t rlk_logp_fused_lmhead_workspace_bytes(const rlk_logp_desc* desc);
rlk_status rlk_logp_fused_lmhead(const rlk_logp_desc* desc, const void* hidden,
                                 const void* weight, int64_t hidden_dim, const int32_t* targets,
                                 const uint8_t* active_mask, float* logp, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Host-only geometry (no device access): writes T+1 tile bounds
 * floor(t*V_pad/T) to `bounds` and S+1 shard starts floor(s*T/S) to
 * `shard_first_tile` (either may be NULL).  Same limits as the descriptor. */
rlk_status rlk_logp_tile_geometry(int64_t padded_vocab, int32_t num_vocab_tiles,
                                  int32_t num_virtual_shards, int64_t* bounds,
                                  int32_t* shard_first_tile);

/* Static name of a status code. */
const char* rlk_status_string(rlk_status status);

/* Reason text for the last non-OK status returned on the calling thread
 * ("" if none).  Valid until the next call on that thread. */
const char* rlk_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* RLK_LOGP_H_ */
