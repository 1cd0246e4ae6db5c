// rlk_lmhead.hip -- fused LM-head variant for gfx950: selected-token logp of
// z = h . W^T without writing the logits to memory.
//
// The pages name an optional fused kernel without describing it (Issue #323
// "[WS2][Logprob] H100 validation and reproduction guide for Issue #241
// PR1-PR5", "Validation Boundary": the optional PR6 fused kernel).  This file
// keeps the contract of the materialised path (PR #289 "[WS2][PR4][Logp] feat:
// add distributed TP/CP logprob drift report", PR1 commit messages: per-tile
// fp32 (max, sumexp) over real columns, the (-inf, 0) identity, a merge in
// fixed global tile order) and takes the statistics straight from the fp32
// GEMM accumulators.
//
// Two kernels run before the ordinary stage-2 merge:
//   lmhead_segments  bf16 MFMA GEMM of a 256-vocab x 256-token block over the
//                    whole hidden dimension, then, per token, the (max, sumexp)
//                    of each "segment" -- the part of the block's vocabulary
//                    that lies in one tile (a block holds at most one tile
//                    bound, since tiles are at least 256 columns wide) -- and
//                    the fp32 target logit of every token whose target falls in
//                    the block.
//   lmhead_tiles     per (token, tile): merge the tile's segments in ascending
//                    column order into the tile partial, in the same [N][T]
//                    layout that stage 1 of the materialised path writes.
//
// GEMM layout.  The accumulator is C[vocab][token] = W . h^T: W rows are the
// MFMA "A" operand and hidden rows the "B" operand, both K-contiguous.  With
// v_mfma_f32_16x16x32_bf16, lane l supplies row/col l%16 and k in
// [8*(l/16), 8*(l/16)+8) of a 32-wide k-step; accumulator i of lane l is
// C[4*(l/16) + i][l%16].  So each lane holds 4 vocab rows of one token per
// 16x16 tile, and a wave's rows of one token sit in the four lanes
// l%16 + 16g.  The 512 threads form 2 x 4 waves of 128 vocab x 64 tokens
// (8 x 4 MFMA tiles, 128 fp32 accumulators per lane), two waves per SIMD, so
// one wave's MFMAs run while the other waits on memory.
//
// K advances in slabs of 64 (two k-steps) through two LDS stages filled by
// direct global-to-LDS loads (buffer_load_dwordx4 ... lds: lane i of an
// instruction writes bytes [16i, 16i + 16) after the wave's LDS base; the
// address is a buffer resource per operand based at the block's first row, a
// fixed 32-bit byte offset per lane and the slab's offset in a scalar
// register, so a load needs no address arithmetic).  LDS
// rows are 128 bytes with the 16-byte chunks XOR-swizzled by row -- chunk c of
// row r sits at position c ^ ((r >> 1) & 7) -- so that fragment reads of
// consecutive rows at one chunk spread over the bank groups; each load lane
// fetches the chunk that belongs at its position.  One barrier per slab, placed
// before the slab's last k-step: by then every wave has read the slab's
// fragments into registers, so the DMA for slab s+2 can go into the stage just
// released, and the first fragments of slab s+1 are read while the last k-step's
// MFMAs run.  Inside each k-step the next fragment reads (and the slab loads)
// are spread between the MFMAs.
//
// Determinism: every reduction has a fixed order -- each lane over its rows in
// register order, then the four lanes of a token by xor-shuffles over 16 and
// 32 lanes (commutative additions, so all four lanes hold the same bits), then
// the two vocab halves of the block (the lower half first), then the segments
// of a tile in ascending column order, then the tiles in stage 2.  No atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_internal.h"

namespace rlk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector: arrays of it stay in registers (HIP's uint4 is
// a struct around a union, which keeps arrays of it in scratch memory)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBV = 256;  // vocabulary rows per block (= kLmheadBlockVocab)
constexpr int kBT = 256;  // tokens per block
constexpr int kBK = 64;   // hidden-dimension slab per LDS stage
constexpr int kRowBytes = kBK * 2;           // 128: one row of a slab, 8 chunks
constexpr int kSlabBytes = kBV * kRowBytes;  // one operand, one stage
constexpr int kRowsPerLoad = 64 / (kRowBytes / 16);  // 8 rows per load instruction
constexpr int kRowsPerWave = kBV / kWaves;           // 32 rows of each operand per wave
constexpr int kLoads = kRowsPerWave / kRowsPerLoad;  // 4 instructions per operand per slab

static_assert(kBV == kLmheadBlockVocab, "block width shared with the boundary");
static_assert(kBV == kBT, "the load mapping assumes square blocks");

typedef __attribute__((address_space(3))) void* lds_ptr;

// Word 3 of a raw (untyped) buffer resource on gfx9: 32-bit data format, no
// swizzle, no thread-id addressing.
constexpr int kBufferWord3 = 0x00020000;

// LDS position (in 16-byte units) of chunk c of row r inside one operand stage.
__device__ __forceinline__ int swizzled(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

__device__ __forceinline__ float maxnan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int64_t xcd_local_block(int64_t b, int64_t nb) {
  constexpr int64_t kXcds = 8;
  const int64_t per = nb / kXcds, rem = nb % kXcds, x = b % kXcds, l = b / kXcds;
  return x * per + (x < rem ? x : rem) + l;
}

// Column bound of the first tile boundary strictly inside [v0, v0 + kBV), or
// v0 + kBV if there is none.  Tile t spans [floor(t*V/T), floor((t+1)*V/T)).
__device__ __forceinline__ int32_t inner_tile_bound(int32_t v0, int32_t padded_vocab,
                                                    int32_t num_tiles) {
  // the tile holding column v0 is the largest t with floor(t*V/T) <= v0
  const int64_t t = ((int64_t)(v0 + 1) * num_tiles - 1) / padded_vocab;
  const int32_t b = (int32_t)(((t + 1) * padded_vocab) / num_tiles);
  return (b > v0 && b < v0 + kBV) ? b : v0 + kBV;
}

// ---------------------------------------------------------------------------
// lmhead_segments
//   h          bf16 [num_tokens, K] (16-byte chunks, K/8 per row)
//   w          bf16 [>= real_vocab, K]; only rows [row_lo, row_hi) are read
//   seg_m/s    [num_tokens][2 * n_vb]: slot 2*vb holds the block's columns
//              before its inner tile bound (all of them if there is none), slot
//              2*vb+1 those from the bound on ((-inf, 0) if there is none)
//   tlogit     [num_tokens] fp32 target logit, written for effective-active
//              tokens whose target is a column of this block in [row_lo, row_hi)
// One launch covers one virtual shard: the vocabulary blocks vb_begin ..
// vb_begin + n_vbs - 1 of the global 256-column block grid that overlap the
// shard's real columns [row_lo, row_hi).  Rows outside that range are neither
// read nor counted, and a segment slot is written only by the shard whose
// columns [col_lo, col_hi) hold the slot's first column.  A segment lies
// inside one tile, so it holds the same rows, summed in the same order, under
// every grouping of the tiles: the slots, and so the partials, do not depend
// on the shard count.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void lmhead_segments(
    const u32x4* __restrict__ h, const u32x4* __restrict__ w, int32_t hidden_dim,
    int32_t num_tokens, int32_t padded_vocab, int32_t num_tiles,
    int32_t n_vb, int32_t n_tb, int32_t vb_begin, int32_t n_vbs, int32_t row_lo,
    int32_t row_hi, int32_t col_lo, int32_t col_hi, const int32_t* __restrict__ targets,
    const uint8_t* __restrict__ mask, int32_t ignore_index, float* __restrict__ seg_m,
    float* __restrict__ seg_s, float* __restrict__ tlogit, int64_t blk_begin) {
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * kSlabBytes];
  static_assert(2 * 2 * kSlabBytes >= kBT * 4 * (int)sizeof(float), "epilogue exchange fits");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave >> 2;  // vocabulary half of the block
  const int wt = wave & 3;   // token quarter of the block

  // Block order for L2 reuse.  Consecutive work indices land on one XCD (the
  // XCD-local renumbering), and 32 consecutive indices -- one XCD's worth of
  // resident blocks -- cover kGroupV vocabulary blocks x 8 token blocks: work
  // index l sits in strip l / (kGroupV * n_tb) of kGroupV vocabulary blocks,
  // token-block major inside the strip.  So each W slice is read by 8 resident
  // blocks and each hidden slice by kGroupV, instead of every vocabulary block
  // re-streaming all hidden states.
  constexpr int32_t kGroupV = 4;
  const int64_t blk = blk_begin + xcd_local_block(blockIdx.x, gridDim.x);
  const int64_t strip = blk / ((int64_t)kGroupV * n_tb);
  const int32_t r_in = (int32_t)(blk - strip * kGroupV * n_tb);
  const int32_t strip_w = min(kGroupV, n_vbs - (int32_t)strip * kGroupV);  // last strip may be narrow
  const int32_t vb = vb_begin + (int32_t)strip * kGroupV + r_in % strip_w;
  const int32_t tb = r_in / strip_w;
  const int32_t v0 = vb * kBV;
  const int32_t t0 = tb * kBT;
  const int32_t ldc = hidden_dim / 8;  // 16-byte chunks per row

  // Direct loads: wave w moves rows [32w, 32w + 32) of both operands, 8 rows per
  // instruction; lane i of instruction j fetches row 32w + 8j + i/8 at the chunk
  // that belongs at LDS position i%8.  Rows of W outside [row_lo, row_hi) --
  // padding, other shards -- and rows past the last token are never read: the
  // row is clamped, and each operand's buffer resource covers only the block's
  // rows (at most 256 rows of 2 * hidden_dim bytes, under 2^31 bytes by the
  // boundary's limit on hidden_dim), starting at its first row read.
  const int32_t w_first = max(v0, row_lo);
  const int64_t row_bytes = (int64_t)ldc * 16;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w + (int64_t)w_first * ldc), 0,
      (int)((int64_t)(min(v0 + kBV, row_hi) - w_first) * row_bytes), kBufferWord3);
  const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(h + (int64_t)t0 * ldc), 0,
      (int)((int64_t)(min(t0 + kBT, num_tokens) - t0) * row_bytes), kBufferWord3);
  uint32_t woff[kLoads], hoff[kLoads];  // byte offsets from the resources' bases
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int row = wave * kRowsPerWave + j * kRowsPerLoad + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    woff[j] = (uint32_t)((min(max(v0 + row, row_lo), row_hi - 1) - w_first) * row_bytes + c * 16);
    hoff[j] = (uint32_t)((min(t0 + row, num_tokens - 1) - t0) * row_bytes + c * 16);
  }

  constexpr int kVS = 8;  // 16-row vocabulary tiles per wave
  constexpr int kTS = 4;  // 16-token tiles per wave
  f32x4 acc[kVS][kTS];
#pragma unroll
  for (int a = 0; a < kVS; ++a)
#pragma unroll
    for (int b = 0; b < kTS; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[a][b][i] = 0.0f;

  const int nslab = hidden_dim / kBK;
  // slab `slab` into LDS stage `stage` (A = W rows at the stage base, B = hidden rows after)
  auto issue = [&](int slab, int stage) __attribute__((always_inline)) {
    char* base = smem + stage * 2 * kSlabBytes + (wave * kRowsPerWave) * kRowBytes;
    const uint32_t soff = (uint32_t)slab * kRowBytes;  // the slab's bytes in a row
    // all W rows, then all hidden rows (about 0.6% faster than alternating)
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr)(base + j * kRowsPerLoad * kRowBytes),
                                               16, woff[j], soff, 0, 0);
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          hrs, (lds_ptr)(base + kSlabBytes + j * kRowsPerLoad * kRowBytes), 16, hoff[j], soff, 0, 0);
  };
  // fragment reads of k-step ks: lane l takes row l%16 of each 16-row tile at
  // chunk 4ks + l/16 (k in [32ks + 8(l/16), +8))
  const int frag_row = lane & 15;
  const int frag_c = lane >> 4;
  auto fetch = [&](const char* As, int ks, bf16x8 (&af)[kVS], bf16x8 (&bf)[kTS])
      __attribute__((always_inline)) {
    const char* Bs = As + kSlabBytes;
#pragma unroll
    for (int vs = 0; vs < kVS; ++vs)
      af[vs] = *reinterpret_cast<const bf16x8*>(
          As + swizzled(wv * 128 + vs * 16 + frag_row, ks * 4 + frag_c) * 16);
#pragma unroll
    for (int ts = 0; ts < kTS; ++ts)
      bf[ts] = *reinterpret_cast<const bf16x8*>(
          Bs + swizzled(wt * 64 + ts * 16 + frag_row, ks * 4 + frag_c) * 16);
  };
  auto mma = [&](const bf16x8 (&af)[kVS], const bf16x8 (&bf)[kTS]) __attribute__((always_inline)) {
#pragma unroll
    for (int vs = 0; vs < kVS; ++vs)
#pragma unroll
      for (int ts = 0; ts < kTS; ++ts)
        acc[vs][ts] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[vs], bf[ts], acc[vs][ts], 0, 0, 0);
  };
  // Instruction order inside a k-step: 4 MFMAs, then one fragment read (and,
  // after the barrier, one slab load) per 2 MFMAs, then the remaining MFMAs.
  // The reads thus overlap the MFMAs that do not need them.
  constexpr int kReads = kVS + kTS, kMfmas = kVS * kTS, kLead = 4, kPer = 2;
  static_assert(kLead + kPer * kReads <= kMfmas, "the reads fit inside the step");
  static_assert(2 * kLoads <= kReads, "one load per read at most");
  auto order_step = [&](bool with_loads) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x008, kLead, 0);  // MFMA
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      if (with_loads && i < 2 * kLoads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM
      __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - kLead - kPer * kReads, 0);
  };
  // s_waitcnt immediate with lgkmcnt = 0 and the other counters at their maxima
  constexpr int kWaitLds = 0xC07F;

  issue(0, 0);
  if (nslab > 1) issue(1, 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bf16x8 a0[kVS], b0[kTS], a1[kVS], b1[kTS];
  fetch(smem, 0, a0, b0);
  for (int s = 0; s < nslab; ++s) {
    const char* cur = smem + (s & 1) * 2 * kSlabBytes;
    const char* nxt = smem + ((s + 1) & 1) * 2 * kSlabBytes;
    // the fragments of this k-step were read during the previous one; wait for
    // them before more reads go out (the LDS counter holds at most 15)
    __builtin_amdgcn_s_waitcnt(kWaitLds);
    fetch(cur, 1, a1, b1);
    mma(a0, b0);
    order_step(false);
    __builtin_amdgcn_sched_barrier(0);
    // every wave has read slab s into registers, and slab s+1 (issued one
    // slab ago) has landed in the other stage
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // slab s+2 into the stage just released.  The last two steps reload slab
    // nslab-1 there and read the other stage's first fragments, which nothing
    // uses: the loads and reads stay unconditional, so they can be interleaved
    // with the MFMAs, and stay in bounds.
    issue(min(s + 2, nslab - 1), s & 1);
    fetch(nxt, 0, a0, b0);
    mma(a1, b1);
    order_step(true);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the reloads of the last two steps land before the epilogue reuses the stages
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- epilogue -------------------------------------------------------------
  const int32_t bnd = inner_tile_bound(v0, padded_vocab, num_tiles);
  const int32_t vw0 = v0 + wv * 128;            // first vocabulary row of this wave
  const int32_t row_lane = 4 * (lane >> 4);     // lane-group offset inside a 16-row tile
  float* xch = reinterpret_cast<float*>(smem);  // [256 tokens][4]
  // every row of the block is in [row_lo, row_hi) and no tile bound cuts it:
  // one segment, no masks
  const bool simple = (v0 >= row_lo) && (v0 + kBV <= row_hi) && (bnd == v0 + kBV);

#pragma unroll
  for (int ts = 0; ts < kTS; ++ts) {
    const int32_t tok = t0 + wt * 64 + ts * 16 + (lane & 15);
    int32_t trow = -1;  // the target's column if this wave holds it
    if (tok < num_tokens && (mask == nullptr || mask[tok] != 0)) {
      const int32_t tg = targets[tok];
      if (tg != ignore_index && tg >= vw0 && tg < vw0 + 128 && tg >= row_lo && tg < row_hi)
        trow = tg;
    }
    if (__any(trow >= 0)) {  // rare: some token of this wave has its target here
      float tz = 0.0f;
      bool have_t = false;
#pragma unroll
      for (int vs = 0; vs < kVS; ++vs)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t row = vw0 + vs * 16 + row_lane + i;
          if (row == trow) {
            tz = acc[vs][ts][i];
            have_t = true;
          }
        }
      if (have_t) tlogit[tok] = tz;
    }
    float m0 = kNegInf, m1 = kNegInf, s0 = 0.0f, s1 = 0.0f;
    if (simple) {
#pragma unroll
      for (int vs = 0; vs < kVS; ++vs)
#pragma unroll
        for (int i = 0; i < 4; ++i) m0 = maxnan(m0, acc[vs][ts][i]);
      // the lanes l%16 + 16g hold the other rows of the same token
      m0 = maxnan(m0, __shfl_xor(m0, 16));
      m0 = maxnan(m0, __shfl_xor(m0, 32));
      const float b0 = (m0 == kNegInf) ? 0.0f : m0;
#pragma unroll
      for (int vs = 0; vs < kVS; ++vs)
#pragma unroll
        for (int i = 0; i < 4; ++i) s0 += exp2_hw((acc[vs][ts][i] - b0) * kLog2e);
    } else {
      // Segment 0 is the rows [row_lo, min(row_hi, bnd)), segment 1 the rows
      // [max(row_lo, bnd), row_hi).  A 16-row tile wholly inside one segment
      // takes its rows without per-row tests; only a tile that a bound cuts
      // tests each row.  Rows outside both segments add nothing, exactly as
      // the per-row form's exp(-inf) = +0 addends do, so the sums keep their
      // bits; the maxima do not depend on the order.
      const int32_t end0 = min(row_hi, bnd), beg1 = max(row_lo, bnd);
      // pass 1: per-segment maxima over this lane's rows
#pragma unroll
      for (int vs = 0; vs < kVS; ++vs) {
        const int32_t r0 = vw0 + vs * 16;
        if (r0 >= row_lo && r0 + 16 <= end0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) m0 = maxnan(m0, acc[vs][ts][i]);
        } else if (r0 >= beg1 && r0 + 16 <= row_hi) {
#pragma unroll
          for (int i = 0; i < 4; ++i) m1 = maxnan(m1, acc[vs][ts][i]);
        } else if (r0 + 16 > row_lo && r0 < row_hi) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int32_t row = r0 + row_lane + i;
            const float z = acc[vs][ts][i];
            const bool in = row >= row_lo && row < row_hi;
            if (in && row < bnd) m0 = maxnan(m0, z);
            if (in && row >= bnd) m1 = maxnan(m1, z);
          }
        }
      }
      m0 = maxnan(m0, __shfl_xor(m0, 16));
      m0 = maxnan(m0, __shfl_xor(m0, 32));
      m1 = maxnan(m1, __shfl_xor(m1, 16));
      m1 = maxnan(m1, __shfl_xor(m1, 32));
      // pass 2: sums of exp(z - max) relative to the token's maxima, in the
      // same row order as the one-segment form
      const float b0 = (m0 == kNegInf) ? 0.0f : m0;
      const float b1 = (m1 == kNegInf) ? 0.0f : m1;
#pragma unroll
      for (int vs = 0; vs < kVS; ++vs) {
        const int32_t r0 = vw0 + vs * 16;
        if (r0 >= row_lo && r0 + 16 <= end0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s0 += exp2_hw((acc[vs][ts][i] - b0) * kLog2e);
        } else if (r0 >= beg1 && r0 + 16 <= row_hi) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s1 += exp2_hw((acc[vs][ts][i] - b1) * kLog2e);
        } else if (r0 + 16 > row_lo && r0 < row_hi) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int32_t row = r0 + row_lane + i;
            const float z = (row >= row_lo && row < row_hi) ? acc[vs][ts][i] : kNegInf;
            const bool hi = row >= bnd;
            const float e = exp2_hw((z - (hi ? b1 : b0)) * kLog2e);
            s0 += hi ? 0.0f : e;
            s1 += hi ? e : 0.0f;
          }
        }
      }
    }
    // the four lanes of the token: pairs over 16 lanes, then over 32; each
    // addition has the same two addends in both lanes, so all four agree
    s0 += __shfl_xor(s0, 16);
    s1 += __shfl_xor(s1, 16);
    s0 += __shfl_xor(s0, 32);
    s1 += __shfl_xor(s1, 32);
    if (wv == 1 && lane < 16) {
      float* x = xch + ((wt * 64 + ts * 16 + lane) * 4);
      x[0] = m0;
      x[1] = s0;
      x[2] = m1;
      x[3] = s1;
    }
    // keep this token's values in registers of the lower-half wave
    if (wv == 0) {
      acc[0][ts][0] = m0;
      acc[0][ts][1] = s0;
      acc[0][ts][2] = m1;
      acc[0][ts][3] = s1;
    }
  }
  __syncthreads();
  // slot 0 starts at v0; slot 1 at the inner bound, or (an identity slot that
  // nothing reads) at v0 when there is none
  const int32_t c_slot1 = (bnd < v0 + kBV) ? bnd : v0;
  const bool own0 = v0 >= col_lo && v0 < col_hi;
  const bool own1 = c_slot1 >= col_lo && c_slot1 < col_hi;
  if (wv == 0 && lane < 16) {
    const int64_t seg_ld = 2 * (int64_t)n_vb;
#pragma unroll
    for (int ts = 0; ts < kTS; ++ts) {
      const int32_t tok = t0 + wt * 64 + ts * 16 + lane;
      if (tok >= num_tokens) continue;
      const float* x = xch + ((wt * 64 + ts * 16 + lane) * 4);
      float out_m[2], out_s[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        // lower vocabulary half first, then the upper half
        const float ma = acc[0][ts][2 * g], sa_ = acc[0][ts][2 * g + 1];
        const float mb = x[2 * g], sb_ = x[2 * g + 1];
        const float M = maxnan(ma, mb);
        float S = 0.0f;
        if (M != kNegInf) {
          if (ma != kNegInf) S = sa_ * exp2_hw((ma - M) * kLog2e);
          if (mb != kNegInf) S = fmaf(sb_, exp2_hw((mb - M) * kLog2e), S);
        }
        out_m[g] = M;
        out_s[g] = S;
      }
      float* om = seg_m + (int64_t)tok * seg_ld + 2 * vb;
      float* os = seg_s + (int64_t)tok * seg_ld + 2 * vb;
      if (own0) {
        om[0] = out_m[0];
        os[0] = out_s[0];
      }
      if (own1) {
        om[1] = out_m[1];
        os[1] = out_s[1];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// lmhead_tiles: one thread per (token, tile) of the tiles [tile_begin,
// tile_begin + n_tiles); segments in ascending columns.  A tile that starts at
// or past real_vocab has no real column: the identity (-inf, 0), with no read.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lmhead_tiles(
    const float* __restrict__ seg_m, const float* __restrict__ seg_s, int32_t num_tokens,
    int32_t n_vb, int32_t real_vocab, int32_t padded_vocab, int32_t num_tiles,
    int32_t tile_begin, int32_t n_tiles, float* __restrict__ pmax, float* __restrict__ psum,
    int64_t idx_begin) {
  const int64_t idx = idx_begin + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_tokens * n_tiles) return;
  const int32_t tok = (int32_t)(idx / n_tiles);
  const int32_t t = tile_begin + (int32_t)(idx - (int64_t)tok * n_tiles);
  const int32_t c0 = (int32_t)(((int64_t)t * padded_vocab) / num_tiles);
  const int32_t c1 = (int32_t)(((int64_t)(t + 1) * padded_vocab) / num_tiles);
  const int64_t out = (int64_t)tok * num_tiles + t;
  float M = kNegInf, S = 0.0f;
  // fold one segment into (M, S): identity segments are skipped
  auto fold = [&](float m, float s) __attribute__((always_inline)) {
    if (m == kNegInf) return;
    if (M == kNegInf) {
      M = m;
      S = s;
      return;
    }
    const float nm = maxnan(M, m);
    S = fmaf(s, exp2_hw((m - nm) * kLog2e), S * exp2_hw((M - nm) * kLog2e));
    M = nm;
  };
  if (c0 < real_vocab) {
    const int32_t vb_first = c0 / kBV;
    const int32_t vb_last = min((min(c1, real_vocab) - 1) / kBV, n_vb - 1);
    const int32_t nseg = vb_last - vb_first + 1;
    const int64_t base = (int64_t)tok * 2 * n_vb + 2 * (int64_t)vb_first;
    const int first_slot = (c0 > vb_first * kBV) ? 1 : 0;  // the tile starts inside its first block
    // the first kPre segments' loads all go out before the first fold; the
    // folds then run in ascending column order as before
    constexpr int kPre = 12;
    float pm[kPre], ps[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      if (i < nseg) {
        const int64_t at = base + 2 * i + (i == 0 ? first_slot : 0);
        pm[i] = seg_m[at];
        ps[i] = seg_s[at];
      }
    }
#pragma unroll
    for (int i = 0; i < kPre; ++i)
      if (i < nseg) fold(pm[i], ps[i]);
    for (int32_t i = kPre; i < nseg; ++i) fold(seg_m[base + 2 * i], seg_s[base + 2 * i]);
  }
  pmax[out] = M;
  psum[out] = (M == kNegInf) ? 0.0f : S;
}

}  // namespace

int64_t lmhead_grid_blocks(int32_t num_tokens, int32_t real_vocab) {
  const int64_t n_vb = ((int64_t)real_vocab + kBV - 1) / kBV;
  const int64_t n_tb = ((int64_t)num_tokens + kBT - 1) / kBT;
  return n_vb * n_tb;
}

hipError_t launch_lmhead(const LmheadArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int32_t n_vb = (a.real_vocab + kBV - 1) / kBV;
  const int32_t n_tb = (a.num_tokens + kBT - 1) / kBT;
  const int64_t limit = launch_thread_limit();
  const int64_t max_blocks = limit / kThreads;
  const int64_t max_items = limit / 256 * 256;
  auto bound = [&](int64_t t) { return (int32_t)((t * a.padded_vocab) / a.num_tiles); };
  // Virtual shard s owns tiles [floor(s*T/S), floor((s+1)*T/S)): its GEMM
  // blocks, then its tiles' partials.  A block cut by a shard bound is
  // computed by both shards, each over its own rows.
  for (int32_t s = 0; s < a.num_shards; ++s) {
    const int32_t ta = (int32_t)(((int64_t)s * a.num_tiles) / a.num_shards);
    const int32_t tb = (int32_t)(((int64_t)(s + 1) * a.num_tiles) / a.num_shards);
    const int32_t col_lo = bound(ta), col_hi = bound(tb);
    const int32_t row_hi = col_hi < a.real_vocab ? col_hi : a.real_vocab;
    if (col_lo < row_hi) {  // a shard of padding only has no GEMM block
      const int32_t vb_begin = col_lo / kBV;
      const int32_t n_vbs = (row_hi - 1) / kBV + 1 - vb_begin;
      // launches of at most limit / kThreads blocks; a block's work index (and
      // so its tile) does not depend on the split
      const int64_t blocks = (int64_t)n_vbs * n_tb;
      for (int64_t b0 = 0; b0 < blocks; b0 += max_blocks) {
        const int64_t nb = blocks - b0 < max_blocks ? blocks - b0 : max_blocks;
        hipLaunchKernelGGL(lmhead_segments, dim3((unsigned)nb), dim3(kThreads), 0, stream,
                           reinterpret_cast<const u32x4*>(a.hidden),
                           reinterpret_cast<const u32x4*>(a.weight), a.hidden_dim, a.num_tokens,
                           a.padded_vocab, a.num_tiles, n_vb, n_tb, vb_begin, n_vbs, col_lo,
                           row_hi, col_lo, col_hi, a.targets, a.mask, a.ignore_index, a.seg_m,
                           a.seg_s, a.target_logit, b0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
    const int64_t items = (int64_t)a.num_tokens * (tb - ta);
    for (int64_t i0 = 0; i0 < items; i0 += max_items) {
      const int64_t ni = items - i0 < max_items ? items - i0 : max_items;
      hipLaunchKernelGGL(lmhead_tiles, dim3((unsigned)((ni + 255) / 256)), dim3(256), 0, stream,
                         a.seg_m, a.seg_s, a.num_tokens, n_vb, a.real_vocab, a.padded_vocab,
                         a.num_tiles, ta, tb - ta, a.pmax, a.psum, i0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace rlk
