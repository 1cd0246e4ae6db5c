// rlk_kernels.hip -- gfx950 kernels for deterministic selected-token logp.
//
// Three kernels, one per step of the path:
//   stage1_partials  per (row, vocab tile) fp32 (max, sumexp) over the tile's
//                    real columns ("masked per-tile partials"); optionally the
//                    entropy statistic sum exp(x - max) (x - max) as well.
//   stage2_merge     per row: merge the T partials in ascending tile order into
//                    LSE (and the entropy H), gather the target logit, apply the
//                    active mask and ignore_index, flag bad targets / non-finite
//                    LSE.
//   bwd_dlogits      dX = g * (onehot - exp(X - LSE)) on effective-active rows;
//                    optionally plus the LSE and entropy gradients.
// plus two one-launch forms for when g is known up front, each giving the bits
// of the three kernels above:
//   fwd_bwd_rows     one block per row: reads the row twice (partials, then dX).
//   fwd_bwd_units    blocks of 8 tiles of a row keep their logits on chip, post
//                    their tile partials to 64-bit slots in the workspace, wait
//                    (bounded) for the row's other tiles, then write dX: one HBM
//                    read and one write per element.  With the entropy flag it
//                    also carries the entropy statistic and its gradients.
//
// Sources (web pages, by title and section): PR #289 "[WS2][PR4][Logp] feat:
// add distributed TP/CP logprob drift report", stacked PR1 commit messages
// (padding columns take no part in any tile's (max, sumexp) statistic; the
// (-inf, 0) identity partial; fp32 merge in fixed global tile order; fp32 logp
// and LSE outputs) and the review excerpt of the op's apply() (active-target
// range check, non-finite-LSE check).  Issue #323 "[WS2][Logprob] H100
// validation and reproduction guide for Issue #241 PR1-PR5", "4. Cross-Topology
// Bitwise Check" (outputs identical whatever the tile grouping).
//
// Determinism: no atomic arithmetic on any result (the unit schedule's slots
// are written by plain 64-bit atomic stores, each by one tile, and its only
// atomic add counts fallback blocks in a status word); every tile is reduced
// by the same 16-lane lane mapping (lane l of the group takes the tile's full
// 16-byte chunks l, l+16, ...) and the same fixed DPP tree whatever launch or
// shard computes it; the merge runs in ascending tile order.  The file is built with
// -ffp-contract=off so that only the fmaf calls written here fuse.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_internal.h"

namespace rlk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr uint32_t kNegInfPair = 0xFF80FF80u;  // two bf16 -inf

// Stage-1 geometry: a wave of 64 lanes reduces 4 tiles at once, 16 lanes
// (one DPP row) per tile; each lane holds kChunks 16-byte chunks per pass.
constexpr int kGroupLanes = 16;
constexpr int kGroupsPerWave = 4;
constexpr int kWavesPerBlock = 4;
constexpr int kChunks = 5;
constexpr int kPassChunks = kChunks * kGroupLanes;  // 80 chunks = 640 columns

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// NaN-propagating maximum (IEEE 754-2019 maximum).
__device__ __forceinline__ float maxnan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// 16 bytes of logits.  Streaming loads of the logits carry the nontemporal
// hint: every byte is read once per kernel, so it should not displace lines
// that neighbouring tiles will still use.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// A load whose line should stay in the caches (the fused forward+backward
// reads every chunk a second time shortly afterwards).
__device__ __forceinline__ uint4 load_keep(const uint4* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <bool kNt>
__device__ __forceinline__ uint4 load_chunk(const uint4* p) {
  if constexpr (kNt) return load_stream(p);
  else return load_keep(p);
}
__device__ __forceinline__ void store_stream(uint4* p, const uint4& w) {
  __builtin_nontemporal_store(u32x4{w.x, w.y, w.z, w.w}, reinterpret_cast<u32x4*>(p));
}

// Block index -> work index so that consecutive work indices run on the same
// XCD.  The hardware hands blocks to the 8 XCDs round-robin; each XCD has its
// own L2, and neighbouring tiles share the 128-byte line at their bound, so
// keeping a row's blocks on one XCD lets the second tile find that line in L2.
// A bijection on [0, gridDim.x).
__device__ __forceinline__ int64_t xcd_local_block(int64_t b, int64_t nb) {
  constexpr int64_t kXcds = 8;
  const int64_t per = nb / kXcds, rem = nb % kXcds, x = b % kXcds, l = b / kXcds;
  return x * per + (x < rem ? x : rem) + l;
}

// Rotate right by N lanes within each row of 16 lanes (DPP row_ror:N).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}

// Fold 8 unpacked values into a lane's running (m, s) pair; the values are a
// pass of kChunks*8 columns held in registers (max first, then the sum).
//
// With kEnt the lane also keeps a = sum exp(x - m) (x - m), the entropy's
// statistic relative to the running max: when the max moves from m to nm,
// a becomes (a + (m - nm) s) exp(m - nm).  A column at -inf adds exp(-inf) = 0
// to s and, through the clamp of x - m to -FLT_MAX, exactly 0 to a.  The (m, s)
// arithmetic is the same with or without kEnt.
template <int NV, bool kEnt = false>
__device__ __forceinline__ void fold_values(const float (&v)[NV], float& m, float& s, float& a) {
  float bm = v[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) bm = maxnan(bm, v[i]);
  const float nm = maxnan(m, bm);
  if (nm == kNegInf) return;  // everything so far is -inf: (m, s) stays (-inf, 0)
  // rescale the running sum to the new max (exp2(0) == 1 leaves it unchanged)
  const float r = exp2_hw((m - nm) * kLog2e);
  if (kEnt) a = (m == kNegInf) ? 0.0f : (a + (m - nm) * s) * r;
  s = s * r;
  const float nml = nm;
#pragma unroll
  for (int c = 0; c < NV / 8; ++c) {
    float cs = 0.0f, ca = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = v[c * 8 + e] - nml;
      const float ex = exp2_hw(t * kLog2e);
      cs += ex;
      if (kEnt) ca = fmaf(ex, __builtin_fmaxf(t, -__FLT_MAX__), ca);
    }
    s += cs;
    if (kEnt) a += ca;
  }
  m = nm;
}

__device__ __forceinline__ void unpack8(const uint4& q, float* v) {
  v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
  v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
  v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
}

// NC consecutive bf16 logits of one row as loaded: 8 from a 16-byte load, or
// 4 from an 8-byte load
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int NC>
struct Cols;
template <>
struct Cols<8> {
  typedef uint4 T;
  static __device__ __forceinline__ void unpack(const uint4& q, float* v) { unpack8(q, v); }
};
template <>
struct Cols<4> {
  typedef u32x2 T;
  static __device__ __forceinline__ void unpack(const u32x2& q, float* v) {
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  }
};

// A pass: slot k (k < kChunks) of lane gl of the group is chunk b + 16k + gl.
// Slots outside the tile's full chunks [lo_c, hi_c) are loaded from a clamped
// address (nothing outside the tile is read) and hold -inf, which adds
// exactly 0: fold_values gives the same bits as if the slot were absent.
template <bool kNt>
__device__ __forceinline__ void load_pass(uint4 (&q)[kChunks], const uint4* __restrict__ rowp,
                                          int32_t b, int32_t lo_c, int32_t hi_c, int gl) {
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int32_t c = b + k * kGroupLanes + gl;
    q[k] = load_chunk<kNt>(rowp + min(max(c, lo_c), hi_c - 1));
  }
}

template <bool kEnt>
__device__ __forceinline__ void fold_pass(const uint4 (&q)[kChunks], int32_t b, int32_t lo_c,
                                          int32_t hi_c, int gl, float& m, float& s, float& a) {
  float v[kChunks * 8];
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int32_t c = b + k * kGroupLanes + gl;
    uint4 w = q[k];
    if (c < lo_c || c >= hi_c)
      w = make_uint4(kNegInfPair, kNegInfPair, kNegInfPair, kNegInfPair);
    unpack8(w, &v[k * 8]);
  }
  fold_values<kChunks * 8, kEnt>(v, m, s, a);
}

// The chunk cut by a tile bound, masked to the columns [e_lo, e_hi) that
// belong to the tile, folded into (m, s, a).
template <bool kEnt>
__device__ __forceinline__ void fold_edge(const uint4& qe, int32_t e_lo, int32_t e_hi, float& m,
                                          float& s, float& a) {
  float v[8];
  unpack8(qe, v);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e < e_lo || e >= e_hi) v[e] = kNegInf;
  fold_values<8, kEnt>(v, m, s, a);
}

// The 16 lanes of a group combined: an exact max, then each lane's sums
// rescaled to it and added over a fixed rotate tree; (-inf, 0) (and la = 0)
// when the whole tile is -inf.  Every lane of the group returns the result.
template <bool kEnt>
__device__ __forceinline__ void group_reduce(float m, float s, float a, float& gm_out,
                                             float& ls_out, float& la_out) {
  float gm = m;
  gm = maxnan(gm, row_ror<8>(gm));
  gm = maxnan(gm, row_ror<4>(gm));
  gm = maxnan(gm, row_ror<2>(gm));
  gm = maxnan(gm, row_ror<1>(gm));
  float ls = 0.0f, la = 0.0f;
  if (gm != kNegInf && m != kNegInf) {
    const float r = exp2_hw((m - gm) * kLog2e);
    ls = s * r;
    if (kEnt) la = (a + (m - gm) * s) * r;
  }
  ls += row_ror<8>(ls);
  ls += row_ror<4>(ls);
  ls += row_ror<2>(ls);
  ls += row_ror<1>(ls);
  if (kEnt) {
    la += row_ror<8>(la);
    la += row_ror<4>(la);
    la += row_ror<2>(la);
    la += row_ror<1>(la);
  }
  if (gm == kNegInf) {  // the (-inf, 0) identity partial
    ls = 0.0f;
    la = 0.0f;
  }
  gm_out = gm;
  ls_out = ls;
  la_out = la;
}

// Columns [lo, hi) of tile `tile`: floor(t * V_pad / T) bounds (tile_width =
// V_pad / T when T divides V_pad, else 0), cut at V_real so that padded
// columns never count; an all-padding tile is empty.
__device__ __forceinline__ void tile_range(int32_t tile, int32_t tile_width, int32_t padded_vocab,
                                           int32_t num_tiles, int32_t real_vocab, int32_t& lo,
                                           int32_t& hi) {
  if (tile_width) {
    lo = tile * tile_width;
    hi = lo + tile_width;
  } else {
    lo = (int32_t)(((int64_t)tile * padded_vocab) / num_tiles);
    hi = (int32_t)(((int64_t)(tile + 1) * padded_vocab) / num_tiles);
  }
  if (hi > real_vocab) hi = real_vocab;
  if (hi < lo) hi = lo;
}

// (max, sumexp) of the columns [lo, hi) of one row, reduced by the 16 lanes of
// a group (gl = lane within the group); every lane of the group returns the
// result.  The lane mapping and the order of every operation depend only on
// (lo, hi), so a tile gives the same bits in whatever kernel, launch or block
// computes it:
//   1. the chunks cut by a tile bound (head on lane 0, tail on lane 1), masked
//      by column;
//   2. passes of kChunks slots per lane starting on the 128-byte line (8
//      chunks, counted from the row start) that holds the first full chunk, so
//      that each 16-lane load covers whole lines; slots outside the full
//      chunks are masked (leading and trailing passes);
//   3. the 16 lanes combined by an exact max and a fixed rotate tree.
// kNt selects the nontemporal load hint and kDepth the number of passes whose
// loads are in flight (1, 2 or 3); neither changes the arithmetic.  With kEnt the
// group also returns la = sum exp(x - gm) (x - gm) over the tile (0 for the
// identity partial); gm and ls are the same bits with or without it.
template <bool kNt, int kDepth, bool kEnt = false>
__device__ __forceinline__ void tile_partial(const uint4* __restrict__ rowp, int32_t lo,
                                             int32_t hi, int gl, float& gm_out, float& ls_out,
                                             float& la_out) {
  static_assert(kDepth >= 1 && kDepth <= 3, "prefetch depth is 1, 2 or 3 passes");
  float m = kNegInf, s = 0.0f, a = 0.0f;
  const int32_t cf_lo = (lo + 7) >> 3;  // first full chunk
  int32_t cf_hi = hi >> 3;              // end of full chunks
  if (cf_hi < cf_lo) cf_hi = cf_lo;
  const int32_t base0 = cf_lo & ~7;
  const int32_t npass = cf_hi > cf_lo ? (cf_hi - base0 + kPassChunks - 1) / kPassChunks : 0;

  // the chunk cut by a tile bound, if this lane has one: its load goes out
  // first, so that waiting for it does not wait for the passes' loads (the
  // load counter completes in order)
  int32_t c = -1, e_lo = 0, e_hi = 0;
  if (gl == 0 && hi > lo && (lo & 7)) {
    c = lo >> 3;
    e_lo = lo & 7;
    e_hi = min(hi - (c << 3), 8);
  } else if (gl == 1 && hi > lo && (hi & 7) && (hi >> 3) >= cf_lo) {
    c = hi >> 3;
    e_lo = 0;
    e_hi = hi & 7;
  }
  uint4 qe;
  if (c >= 0) qe = load_chunk<kNt>(rowp + c);
  uint4 qa[kChunks], qb[kChunks], qc[kChunks];
  if (kDepth >= 2) {
    if (npass > 0) load_pass<kNt>(qa, rowp, base0, cf_lo, cf_hi, gl);
    if (npass > 1) load_pass<kNt>(qb, rowp, base0 + kPassChunks, cf_lo, cf_hi, gl);
  }
  if (kDepth == 3 && npass > 2) load_pass<kNt>(qc, rowp, base0 + 2 * kPassChunks, cf_lo, cf_hi, gl);
  if (c >= 0) fold_edge<kEnt>(qe, e_lo, e_hi, m, s, a);
  if (kDepth == 1) {
    for (int32_t p = 0; p < npass; ++p) {
      const int32_t b = base0 + p * kPassChunks;
      load_pass<kNt>(qa, rowp, b, cf_lo, cf_hi, gl);
      fold_pass<kEnt>(qa, b, cf_lo, cf_hi, gl, m, s, a);
    }
  } else if (kDepth == 3) {
    // three passes in flight: pass p + 3 is issued as soon as pass p has folded
    for (int32_t p = 0; p < npass; p += 3) {
      const int32_t b = base0 + p * kPassChunks;
      fold_pass<kEnt>(qa, b, cf_lo, cf_hi, gl, m, s, a);
      if (p + 3 < npass) load_pass<kNt>(qa, rowp, b + 3 * kPassChunks, cf_lo, cf_hi, gl);
      if (p + 1 >= npass) break;
      fold_pass<kEnt>(qb, b + kPassChunks, cf_lo, cf_hi, gl, m, s, a);
      if (p + 4 < npass) load_pass<kNt>(qb, rowp, b + 4 * kPassChunks, cf_lo, cf_hi, gl);
      if (p + 2 >= npass) break;
      fold_pass<kEnt>(qc, b + 2 * kPassChunks, cf_lo, cf_hi, gl, m, s, a);
      if (p + 5 < npass) load_pass<kNt>(qc, rowp, b + 5 * kPassChunks, cf_lo, cf_hi, gl);
    }
  } else {
    // two passes in flight: pass p + 2 is issued as soon as pass p has folded
    for (int32_t p = 0; p < npass; p += 2) {
      const int32_t b = base0 + p * kPassChunks;
      fold_pass<kEnt>(qa, b, cf_lo, cf_hi, gl, m, s, a);
      if (p + 2 < npass) load_pass<kNt>(qa, rowp, b + 2 * kPassChunks, cf_lo, cf_hi, gl);
      if (p + 1 >= npass) break;
      fold_pass<kEnt>(qb, b + kPassChunks, cf_lo, cf_hi, gl, m, s, a);
      if (p + 3 < npass) load_pass<kNt>(qb, rowp, b + 3 * kPassChunks, cf_lo, cf_hi, gl);
    }
  }

  group_reduce<kEnt>(m, s, a, gm_out, ls_out, la_out);
}

// ---------------------------------------------------------------------------
// Stage 1: masked per-tile partials.
//   logits      [N, ld] bf16 as 16-byte chunks (ld_chunks = ld / 8)
//   tiles       [tile_begin, tile_begin + tile_count) of T, for every row
//   tile_width  V_pad / T when T divides V_pad, else 0 (floor formula)
//   pmax, psum  [N][T] fp32
//   pent        [N][T] fp32, the entropy statistic (kEnt only)
// Work item i = row * tile_count + (tile - tile_begin); group q of wave w of
// work block b (the XCD-local renumbering of blockIdx.x) takes item
// item_begin + 4 (kWPB b + w) + q, where item_begin > 0 when a large batch
// takes several launches.  Columns >= V_real never enter the arithmetic;
// chunks that straddle a tile bound are masked by column index.  Neither kWPB
// (waves per block: one-wave blocks spread a small batch over every CU) nor the
// split into launches changes what a tile computes, so all give the same bits.
// ---------------------------------------------------------------------------
template <bool kEnt, int kWPB>
__global__ __launch_bounds__(kWPB * 64) void stage1_partials(
    const uint4* __restrict__ logits, int64_t ld_chunks, int32_t num_rows, int32_t real_vocab,
    int32_t padded_vocab, int32_t num_tiles, int32_t tile_width, int32_t tile_begin,
    int32_t tile_count, int64_t item_begin, float* __restrict__ pmax, float* __restrict__ psum,
    float* __restrict__ pent) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int gl = lane & 15;
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t block = xcd_local_block(blockIdx.x, gridDim.x);
  const int64_t item0 = item_begin + (block * kWPB + wave_in_block) * kGroupsPerWave;
  const int64_t n_items = (int64_t)num_rows * tile_count;

  // item -> (row, tile) once per wave on the scalar unit, then step by grp
  int32_t row = (int32_t)(item0 / tile_count);
  int32_t tq = (int32_t)(item0 - (int64_t)row * tile_count) + grp;
  while (tq >= tile_count) {
    tq -= tile_count;
    ++row;
  }
  const bool have = item0 + grp < n_items;
  const int32_t tile = tile_begin + tq;

  int32_t lo = 0, hi = 0;
  if (have) tile_range(tile, tile_width, padded_vocab, num_tiles, real_vocab, lo, hi);
  const uint4* __restrict__ rowp = logits + (int64_t)row * ld_chunks;

  float gm, ls, la;
  tile_partial<true, 3, kEnt>(rowp, lo, hi, gl, gm, ls, la);

  if (have && gl == 0) {
    const int64_t o = (int64_t)row * num_tiles + tile;
    pmax[o] = gm;
    psum[o] = ls;
    if (kEnt) pent[o] = la;
  }
}

// ---------------------------------------------------------------------------
// Stage 2: per-row merge in ascending tile order, target gather, mask.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 64;  // one row per lane; small blocks spread rows over every CU
constexpr int kMergeVec = 64;      // most tiles the vectorised (16-byte load) path takes

// The merge accumulates S = sum_t s_t exp(m_t - M) in fp64, in ascending tile
// order: a running fp32 sum of T terms drifts by up to T half-ulps, which at
// T = 1024 tiles moves LSE by a few 1e-6 and an fp32 dX entry g (1 - p) by about
// 1e-5.  The exponentials are fp32 (each term's own error averages out) and
// s_t exp(m_t - M) is exact in fp64.  LSE = M + log S is formed in fp64 and
// rounded to fp32 once.
__device__ __forceinline__ float lse_of(float M, double S) {
  return (float)((double)M + log(S));
}

// LSE from a row's T partials: exact max first, then the rescaled sum in
// ascending tile order (fp32 exponentials, an fp64 fma chain), skipping
// identity partials, rounded to fp32 once in lse_of; -inf if every partial is
// the identity.  pm/ps point at the row's T values.
__device__ __forceinline__ float merge_row(const float* __restrict__ pm,
                                           const float* __restrict__ ps, int32_t num_tiles) {
  float M = kNegInf;
  double S = 0.0;
  if (num_tiles <= kMergeVec && (num_tiles & 3) == 0) {
    // the same arithmetic with 16-byte loads: every maximum in flight at once,
    // then the sum over four tiles per load of each array, a few loads ahead
    // (a row's partials are in the cache by then; holding all 2T values in
    // registers cost 201 VGPRs)
#pragma unroll
    for (int t = 0; t < kMergeVec; t += 4) {
      if (t < num_tiles) {
        const float4 a = *reinterpret_cast<const float4*>(pm + t);
        M = maxnan(M, a.x); M = maxnan(M, a.y); M = maxnan(M, a.z); M = maxnan(M, a.w);
      }
    }
    if (M == kNegInf) return kNegInf;
#pragma unroll 2
    for (int32_t t = 0; t < num_tiles; t += 4) {
      const float4 a = *reinterpret_cast<const float4*>(pm + t);
      const float4 b = *reinterpret_cast<const float4*>(ps + t);
      const float mv[4] = {a.x, a.y, a.z, a.w}, sv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (mv[j] != kNegInf) S = fma((double)sv[j], (double)expf(mv[j] - M), S);
    }
    return lse_of(M, S);
  }
  for (int32_t t = 0; t < num_tiles; ++t) M = maxnan(M, pm[t]);
  if (M == kNegInf) return kNegInf;
  for (int32_t t = 0; t < num_tiles; ++t) {
    const float mt = pm[t];
    if (mt != kNegInf) S = fma((double)ps[t], (double)expf(mt - M), S);
  }
  return lse_of(M, S);
}

// merge_row's arithmetic plus the entropy: alongside S it accumulates, in the
// same ascending order and also in fp64, A = sum_t exp(m_t - M) (a_t + (m_t - M)
// s_t), which is sum_j exp(x_j - M) (x_j - M) over the row.  Then LSE = M + log S
// (the same bits as merge_row) and H = log S - A / S, rounded to fp32 once; H is
// NaN where LSE is not finite (no distribution).
__device__ __forceinline__ void merge_step_entropy(float mt, float st, float at, float M,
                                                   double& S, double& A) {
  if (mt != kNegInf) {
    const float d = mt - M;
    const double e = (double)expf(d);
    S = fma((double)st, e, S);
    A = fma(e, fma((double)d, (double)st, (double)at), A);
  }
}

__device__ __forceinline__ float merge_row_entropy(const float* __restrict__ pm,
                                                   const float* __restrict__ ps,
                                                   const float* __restrict__ pa,
                                                   int32_t num_tiles, float& H) {
  H = __builtin_nanf("");
  float M = kNegInf;
  double S = 0.0, A = 0.0;
  if (num_tiles <= kMergeVec && (num_tiles & 3) == 0) {
    // the same arithmetic with 16-byte loads, as in merge_row
#pragma unroll
    for (int t = 0; t < kMergeVec; t += 4) {
      if (t < num_tiles) {
        const float4 a = *reinterpret_cast<const float4*>(pm + t);
        M = maxnan(M, a.x); M = maxnan(M, a.y); M = maxnan(M, a.z); M = maxnan(M, a.w);
      }
    }
    if (M == kNegInf) return kNegInf;
#pragma unroll 2
    for (int32_t t = 0; t < num_tiles; t += 4) {
      const float4 a4 = *reinterpret_cast<const float4*>(pm + t);
      const float4 b4 = *reinterpret_cast<const float4*>(ps + t);
      const float4 c4 = *reinterpret_cast<const float4*>(pa + t);
      merge_step_entropy(a4.x, b4.x, c4.x, M, S, A);
      merge_step_entropy(a4.y, b4.y, c4.y, M, S, A);
      merge_step_entropy(a4.z, b4.z, c4.z, M, S, A);
      merge_step_entropy(a4.w, b4.w, c4.w, M, S, A);
    }
  } else {
    for (int32_t t = 0; t < num_tiles; ++t) M = maxnan(M, pm[t]);
    if (M == kNegInf) return kNegInf;
    for (int32_t t = 0; t < num_tiles; ++t) merge_step_entropy(pm[t], ps[t], pa[t], M, S, A);
  }
  const float L = lse_of(M, S);
  if (__builtin_isfinite(L)) H = (float)(log(S) - A / S);
  return L;
}

template <bool kEnt>
__global__ __launch_bounds__(kMergeThreads) void stage2_merge(
    const uint16_t* __restrict__ logits, const float* __restrict__ target_logit, int64_t ld,
    int32_t num_rows, int32_t real_vocab,
    int32_t num_tiles, const float* __restrict__ pmax, const float* __restrict__ psum,
    const float* __restrict__ pent, const int32_t* __restrict__ targets,
    const uint8_t* __restrict__ mask, int32_t ignore_index, float* __restrict__ logp,
    float* __restrict__ lse, float* __restrict__ entropy, uint32_t* __restrict__ status) {
  const int32_t r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= num_rows) return;
  float L;
  if (kEnt) {
    float H;
    L = merge_row_entropy(pmax + (int64_t)r * num_tiles, psum + (int64_t)r * num_tiles,
                          pent + (int64_t)r * num_tiles, num_tiles, H);
    entropy[r] = H;
  } else {
    L = merge_row(pmax + (int64_t)r * num_tiles, psum + (int64_t)r * num_tiles, num_tiles);
  }
  lse[r] = L;

  const bool act = (mask == nullptr || mask[r] != 0);
  const int32_t tgt = act ? targets[r] : 0;
  if (!act || tgt == ignore_index) {
    logp[r] = 0.0f;
    return;
  }
  if (tgt < 0 || tgt >= real_vocab) {
    logp[r] = __builtin_nanf("");
    status[0] = 1u;
    return;
  }
  const float x = target_logit ? target_logit[r]
                               : __uint_as_float((uint32_t)logits[(int64_t)r * ld + tgt] << 16);
  logp[r] = x - L;
  if (!__builtin_isfinite(L)) status[1] = 1u;
}

// ---------------------------------------------------------------------------
// Backward: one block covers kBwdCols consecutive columns of one row.
// ---------------------------------------------------------------------------
constexpr int kBwdThreads = 128;
constexpr int kBwdUnroll = 2;
constexpr int kBwdCols = kBwdThreads * 8 * kBwdUnroll;  // 2048 columns

// bf16 dX of 8 columns (the fp32 kernels write 4-column pieces, store_quad)
template <typename OutT>
struct Store8;

__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  // two fp32 -> two bf16, round to nearest even (one v_cvt_pk_bf16_f32)
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

template <>
struct Store8<uint16_t> {
  static __device__ __forceinline__ void store(uint16_t* out, const float* d, int n) {
    const uint4 w = make_uint4(pack_bf16_rne(d[0], d[1]), pack_bf16_rne(d[2], d[3]),
                               pack_bf16_rne(d[4], d[5]), pack_bf16_rne(d[6], d[7]));
    if (n == 8) {
      store_stream(reinterpret_cast<uint4*>(out), w);
    } else {
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      for (int e = 0; e < n; ++e) out[e] = (uint16_t)(ws[e >> 1] >> ((e & 1) * 16));
    }
  }
};

// fp32 dX of 4 columns at out (16-byte aligned); n = columns to write (1..4).
// In the 4-column layout a wave's stores cover 1 KB contiguous, so the
// nontemporal hint costs nothing.
__device__ __forceinline__ void store_quad(float* out, const float (&d)[4], int n) {
  if (n == 4) {
    __builtin_nontemporal_store(u32x4{__float_as_uint(d[0]), __float_as_uint(d[1]),
                                      __float_as_uint(d[2]), __float_as_uint(d[3])},
                                reinterpret_cast<u32x4*>(out));
  } else {
    for (int e = 0; e < n; ++e) out[e] = d[e];
  }
}

// dX of the NC columns [j0, j0 + NC) of one row (q = their logits, read only on
// an effective-active row with a good target and j0 < V_real):
//   inactive row                 +0
//   bad target                   NaN on real columns, +0 on padded ones
//   real column j                -g * exp(x_j - L), and g * (1 - exp(x_t - L))
//                                at the target t
//   padded column                +0
// exp(y) is taken as exp2(y * log2 e) on the hardware unit, in one fixed form.
template <int NC>
__device__ __forceinline__ void dlogits_chunk(const typename Cols<NC>::T& q, int32_t j0, bool act,
                                              bool bad, float L, float g, int32_t tgt,
                                              int32_t real_vocab, float (&d)[NC]) {
  if (!act) {
#pragma unroll
    for (int e = 0; e < NC; ++e) d[e] = 0.0f;
  } else if (bad) {
#pragma unroll
    for (int e = 0; e < NC; ++e) d[e] = (j0 + e < real_vocab) ? __builtin_nanf("") : 0.0f;
  } else if (j0 >= real_vocab) {
#pragma unroll
    for (int e = 0; e < NC; ++e) d[e] = 0.0f;
  } else {
    float x[NC];
    Cols<NC>::unpack(q, x);
    const float ng = -g;
#pragma unroll
    for (int e = 0; e < NC; ++e) d[e] = ng * exp2_hw((x[e] - L) * kLog2e);
    if (j0 + NC > real_vocab) {
#pragma unroll
      for (int e = 0; e < NC; ++e)
        if (j0 + e >= real_vocab) d[e] = 0.0f;
    }
    if (tgt >= j0 && tgt < j0 + NC) {
      const int e = tgt - j0;
      d[e] = g * (1.0f - exp2_hw((x[e] - L) * kLog2e));
    }
  }
}

// The extended gradient of the NC columns [j0, j0 + NC) of one row, with the
// LSE and entropy terms (the derivatives of LSE and of H = -sum p log p):
//   d_j = g ([j == t] - p_j) + gl p_j - gh p_j (log p_j + H),  log p_j = x_j - L
// computed off the target as p_j fma(-gh, u_j, k) with k = gl - g - gh H fixed
// for the row, and at the target as fma(p_t, fma(-gh, u_t, k), g), where
// u_j = max(x_j - L, kLogpFloor): a column at -inf has p = 0 and adds 0 to every
// term (0 log 0 = 0), and the floor keeps gh u finite.  Without an entropy term
// (gh == 0, uniform over the row) it is p_j c, c = gl - g, and g (1 - p_t) + p_t gl
// (H is not read there, so a row whose H is NaN keeps its other terms).  `need` is false on a row that no
// term reaches (it stays +0 and is not read); `bad` marks an effective-active
// row with a target outside [0, V_real) (NaN on its real columns).
// Below every exponent whose exponential is nonzero in fp32 (about -103.3):
// clamping log p there changes no column with p > 0.
constexpr float kLogpFloor = -256.0f;

template <int NC>
__device__ __forceinline__ void dlogits_chunk_ex(const typename Cols<NC>::T& q, int32_t j0,
                                                 bool need, bool bad, float L, float g, float gl,
                                                 float gh, float H, int32_t tgt,
                                                 int32_t real_vocab, float (&d)[NC]) {
  if (!need) {
#pragma unroll
    for (int e = 0; e < NC; ++e) d[e] = 0.0f;
  } else if (bad) {
#pragma unroll
    for (int e = 0; e < NC; ++e) d[e] = (j0 + e < real_vocab) ? __builtin_nanf("") : 0.0f;
  } else if (j0 >= real_vocab) {
#pragma unroll
    for (int e = 0; e < NC; ++e) d[e] = 0.0f;
  } else {
    float x[NC];
    Cols<NC>::unpack(q, x);
    const float c = gl - g;
    float p[NC], q[NC];
    if (gh != 0.0f) {  // uniform over the row
      const float k = c - gh * H;
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        const float t = x[e] - L;
        p[e] = exp2_hw(t * kLog2e);
        q[e] = fmaf(-gh, __builtin_fmaxf(t, kLogpFloor), k);
        d[e] = p[e] * q[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        p[e] = exp2_hw((x[e] - L) * kLog2e);
        q[e] = 0.0f;
        d[e] = p[e] * c;
      }
    }
    if (j0 + NC > real_vocab) {
#pragma unroll
      for (int e = 0; e < NC; ++e)
        if (j0 + e >= real_vocab) d[e] = 0.0f;
    }
    if (tgt >= j0 && tgt < j0 + NC) {
      const int e = tgt - j0;
      d[e] = gh != 0.0f ? fmaf(p[e], q[e], g) : g * (1.0f - p[e]) + p[e] * gl;
    }
  }
}

// kEx: the extended gradient (grad_lse, grad_ent, entropy may be given; any
// of grad, grad_lse, grad_ent may be null = zero).  Without kEx the kernel is
// the plain backward and the extra pointers are unused.
template <typename OutT, bool kEx>
__global__ __launch_bounds__(kBwdThreads) void bwd_dlogits(
    const uint4* __restrict__ logits, int64_t ld_chunks, int32_t num_rows, int32_t real_vocab,
    int32_t padded_vocab, int32_t col_blocks, const int32_t* __restrict__ targets,
    const uint8_t* __restrict__ mask, int32_t ignore_index, const float* __restrict__ lse,
    const float* __restrict__ grad, const float* __restrict__ grad_lse,
    const float* __restrict__ grad_ent, const float* __restrict__ entropy,
    OutT* __restrict__ dlogits, int64_t ld_d, uint32_t* __restrict__ status,
    int64_t block_begin) {
  // block index over the whole batch (a large batch takes several launches)
  const int64_t gb = block_begin + blockIdx.x;
  const int32_t row = (int32_t)(gb / col_blocks);
  const int32_t cb = (int32_t)(gb - (int64_t)row * col_blocks);
  const bool act_mask = (mask == nullptr || mask[row] != 0);
  const int32_t tgt = act_mask ? targets[row] : 0;
  const bool act = act_mask && tgt != ignore_index;
  const bool bad = act && (tgt < 0 || tgt >= real_vocab);
  if (bad && cb == 0 && threadIdx.x == 0) status[0] = 1u;
  float gl = 0.0f, gh = 0.0f, H = 0.0f;
  if (kEx) {
    gl = grad_lse ? grad_lse[row] : 0.0f;
    gh = grad_ent ? grad_ent[row] : 0.0f;
    if (gh != 0.0f) H = entropy[row];
  }
  const bool need = act || gl != 0.0f || gh != 0.0f;
  const float L = need ? lse[row] : 0.0f;
  const float g = (act && (!kEx || grad)) ? grad[row] : 0.0f;
  OutT* __restrict__ orow = dlogits + (int64_t)row * ld_d;
  if constexpr (sizeof(OutT) == 4) {
    // fp32 dX in 4-column pieces from 8-byte loads: each lane's 16-byte store
    // then lands next to its neighbours', and a wave's store instruction writes
    // 1 KB contiguous.  (Two 16-byte stores per lane at a 32-byte lane stride,
    // nontemporal, ran the read-write mix at about 4.0 TB/s against 5.8.)
    constexpr int kPieces = kBwdCols / 4 / kBwdThreads;
    const u32x2* __restrict__ xq =
        reinterpret_cast<const u32x2*>(logits) + (int64_t)row * (ld_chunks * 2);
    const int32_t p0 = cb * (kBwdCols / 4) + threadIdx.x;
    u32x2 q[kPieces];
    if (need && !bad) {
#pragma unroll
      for (int k = 0; k < kPieces; ++k) {
        const int32_t pc = p0 + k * kBwdThreads;
        if ((pc << 2) < real_vocab) q[k] = __builtin_nontemporal_load(xq + pc);
      }
    }
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
      const int32_t j0 = (p0 + k * kBwdThreads) << 2;
      if (j0 >= padded_vocab) continue;
      float d[4];
      if (kEx)
        dlogits_chunk_ex(q[k], j0, need, bad, L, g, gl, gh, H, act ? tgt : -1, real_vocab, d);
      else
        dlogits_chunk(q[k], j0, act, bad, L, g, tgt, real_vocab, d);
      store_quad(reinterpret_cast<float*>(orow) + j0, d, min(4, padded_vocab - j0));
    }
  } else {
    // bf16 dX: 2 chunks of 8 columns per thread, 16-byte loads and stores
    const uint4* __restrict__ xrow = logits + (int64_t)row * ld_chunks;
    const int32_t c0 = cb * (kBwdCols / 8) + threadIdx.x;
    uint4 q[kBwdUnroll];
    if (need && !bad) {
#pragma unroll
      for (int k = 0; k < kBwdUnroll; ++k) {
        const int32_t c = c0 + k * kBwdThreads;
        if ((c << 3) < real_vocab) q[k] = xrow[c];
      }
    }
#pragma unroll
    for (int k = 0; k < kBwdUnroll; ++k) {
      const int32_t c = c0 + k * kBwdThreads;
      const int32_t j0 = c << 3;
      if (j0 >= padded_vocab) continue;
      float d[8];
      if (kEx)
        dlogits_chunk_ex(q[k], j0, need, bad, L, g, gl, gh, H, act ? tgt : -1, real_vocab, d);
      else
        dlogits_chunk(q[k], j0, act, bad, L, g, tgt, real_vocab, d);
      Store8<OutT>::store(orow + j0, d, min(8, padded_vocab - j0));
    }
  }
}

// ---------------------------------------------------------------------------
// Forward and backward in one launch, for a caller that knows g before the
// forward.  One block owns one row:
//   1. its 4 * kFbWaves groups compute the row's T tile partials with the
//      stage-1 code (tile t on group t mod groups), into LDS; the target logit
//      is gathered first and the first batch of phase-3 loads is issued before
//      the barrier, so both are in flight during the merge;
//   2. wave 0 merges the partials in ascending tile order (the stage-2
//      arithmetic) and writes LSE, logp and the status words;
//   3. the whole block streams the row again, one batch of loads ahead, and
//      writes dX.
// The second read follows the first within tens of microseconds, so it is
// served by the caches (the first read does not carry the nontemporal hint)
// and HBM sees one read and one write of the row.  Every value is computed by
// the same code, in the same order, as in stage1_partials, stage2_merge and
// bwd_dlogits, so the outputs are bitwise those of the separate launches.
// ---------------------------------------------------------------------------
constexpr int kFbWaves = 8;
constexpr int kFbThreads = kFbWaves * 64;
constexpr int kFbGroups = kFbWaves * kGroupsPerWave;
constexpr int kFbUnroll = 4;

// The stage-2 merge of T <= 64 partials held one per lane of a wave (lane t
// holds tile t; lanes >= T hold the identity).  The max is exact in any order
// and the exponentials are taken in parallel; the fma chain then runs in
// ascending tile order over LDS copies, in fp64 as in merge_row.  An identity
// partial enters the chain as fma(0, 0, S), which is S (S >= +0), exactly as if
// it were skipped.  Every lane returns the LSE.
__device__ __forceinline__ float merge_lanes(float mt, float st, int32_t num_tiles, int lane,
                                             float* s_e, float* s_sv) {
  float M = mt;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = maxnan(M, __shfl_xor(M, o));
  if (M == kNegInf) return kNegInf;
  const bool live = lane < num_tiles && mt != kNegInf;
  s_e[lane] = live ? expf(mt - M) : 0.0f;
  s_sv[lane] = live ? st : 0.0f;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double S = 0.0;
#pragma unroll
  for (int t = 0; t < 64; t += 4) {
    const float4 e4 = *reinterpret_cast<const float4*>(s_e + t);
    const float4 s4 = *reinterpret_cast<const float4*>(s_sv + t);
    S = fma((double)s4.x, (double)e4.x, S);
    S = fma((double)s4.y, (double)e4.y, S);
    S = fma((double)s4.z, (double)e4.z, S);
    S = fma((double)s4.w, (double)e4.w, S);
  }
  return lse_of(M, S);
}

// merge_row_entropy with the T <= 64 partials held one per lane: the max and the
// exponentials as in merge_lanes, then the fp64 chains for S and A in ascending
// tile order over LDS copies.  An identity lane enters both chains as
// fma(0, 0, .), which leaves S (>= +0) and A (+0 or negative) unchanged, exactly
// as if it were skipped.  Every lane returns the LSE and H.
__device__ __forceinline__ float merge_lanes_entropy(float mt, float st, float at,
                                                     int32_t num_tiles, int lane, float* s_e,
                                                     float* s_sv, float* s_d, float* s_a,
                                                     float& H) {
  H = __builtin_nanf("");
  float M = mt;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = maxnan(M, __shfl_xor(M, o));
  if (M == kNegInf) return kNegInf;
  const bool live = lane < num_tiles && mt != kNegInf;
  const float d = live ? mt - M : 0.0f;
  s_e[lane] = live ? expf(d) : 0.0f;
  s_sv[lane] = live ? st : 0.0f;
  s_d[lane] = d;
  s_a[lane] = live ? at : 0.0f;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double S = 0.0, A = 0.0;
  // two groups of LDS loads ahead: fully unrolled, all 256 values were held
  // in registers at once (256 VGPRs, occupancy 1)
#pragma unroll 2
  for (int t = 0; t < 64; t += 4) {
    const float4 e4 = *reinterpret_cast<const float4*>(s_e + t);
    const float4 s4 = *reinterpret_cast<const float4*>(s_sv + t);
    const float4 d4 = *reinterpret_cast<const float4*>(s_d + t);
    const float4 a4 = *reinterpret_cast<const float4*>(s_a + t);
    const float ev[4] = {e4.x, e4.y, e4.z, e4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
    const float dv[4] = {d4.x, d4.y, d4.z, d4.w}, av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      S = fma((double)sv[j], (double)ev[j], S);
      A = fma((double)ev[j], fma((double)dv[j], (double)sv[j], (double)av[j]), A);
    }
  }
  const float L = lse_of(M, S);
  if (__builtin_isfinite(L)) H = (float)(log(S) - A / S);
  return L;
}

// ---------------------------------------------------------------------------
// Stage 2 with one wave per row, for T <= 64: lane t holds tile t's partial and
// merge_lanes (merge_lanes_entropy with the entropy output) takes the
// exponentials in parallel, so a row costs one exp per lane instead of T in one
// thread; the arithmetic, and so every output bit, is that of stage2_merge.
// Rows [row_begin, row_begin + gridDim.x * kMergeRows) of the batch; a wave past
// num_rows returns at once.
// ---------------------------------------------------------------------------
constexpr int kMergeRows = 4;  // rows (waves) per block
// Batches up to this many rows take stage2_merge_waves.  Measured against one
// thread per row on 152576-column rows (forward times; same bits): 32 rows 9.9
// against 13.4 us, 1024 rows 52.3 against 55.6 us, 4096 rows 187.8 against 190.0
// us, 8192 rows level, 16384 rows 741 against 735 us (each wave's serial fp64
// chain then costs more than the exponentials it spreads over lanes).
constexpr int64_t kMergeWaveMaxRows = 4096;
// With the entropy output a wave runs two fp64 chains, so the crossover comes
// earlier: forward_ex times 11.4 against 16.1 us at 32 rows, 62.4 against 66.5 us
// at 1024 rows, 219.9 against 215.1 us at 4096 rows.
constexpr int64_t kMergeWaveMaxRowsEnt = 2048;
template <bool kEnt>
__global__ __launch_bounds__(kMergeRows * 64) void stage2_merge_waves(
    const uint16_t* __restrict__ logits, const float* __restrict__ target_logit, int64_t ld,
    int32_t num_rows, int32_t real_vocab, int32_t num_tiles, const float* __restrict__ pmax,
    const float* __restrict__ psum, const float* __restrict__ pent,
    const int32_t* __restrict__ targets, const uint8_t* __restrict__ mask, int32_t ignore_index,
    float* __restrict__ logp, float* __restrict__ lse, float* __restrict__ entropy,
    uint32_t* __restrict__ status, int64_t row_begin) {
  __shared__ __align__(16) float s_e[kMergeRows][64];
  __shared__ __align__(16) float s_sv[kMergeRows][64];
  __shared__ __align__(16) float s_d[kEnt ? kMergeRows : 1][64];
  __shared__ __align__(16) float s_a[kEnt ? kMergeRows : 1][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t r = row_begin + (int64_t)blockIdx.x * kMergeRows + w;
  if (r >= num_rows) return;  // uniform over the wave
  const bool act_mask = (mask == nullptr || mask[r] != 0);
  const int32_t tgt = act_mask ? targets[r] : 0;
  const bool act = act_mask && tgt != ignore_index;
  const bool bad = act && (tgt < 0 || tgt >= real_vocab);
  // the target logit goes out first, so that its latency overlaps the merge
  float x = 0.0f;
  if (lane == 0 && act && !bad)
    x = target_logit ? target_logit[r]
                     : __uint_as_float((uint32_t)logits[r * ld + tgt] << 16);
  const float mt = lane < num_tiles ? pmax[r * num_tiles + lane] : kNegInf;
  const float st = lane < num_tiles ? psum[r * num_tiles + lane] : 0.0f;
  float L, H = 0.0f;
  if constexpr (kEnt) {
    const float at = lane < num_tiles ? pent[r * num_tiles + lane] : 0.0f;
    L = merge_lanes_entropy(mt, st, at, num_tiles, lane, s_e[w], s_sv[w], s_d[w], s_a[w], H);
  } else {
    L = merge_lanes(mt, st, num_tiles, lane, s_e[w], s_sv[w]);
  }
  if (lane == 0) {
    lse[r] = L;
    if (kEnt) entropy[r] = H;
    if (!act) {
      logp[r] = 0.0f;
    } else if (bad) {
      logp[r] = __builtin_nanf("");
      status[0] = 1u;
    } else {
      logp[r] = x - L;
      if (!__builtin_isfinite(L)) status[1] = 1u;
    }
  }
}

template <typename OutT>
__global__ __launch_bounds__(kFbThreads) void fwd_bwd_rows(
    const uint4* __restrict__ logits, int64_t ld_chunks, int32_t real_vocab,
    int32_t padded_vocab, int32_t num_tiles, int32_t tile_width,
    const int32_t* __restrict__ targets, const uint8_t* __restrict__ mask, int32_t ignore_index,
    const float* __restrict__ grad, float* __restrict__ logp, float* __restrict__ lse,
    OutT* __restrict__ dlogits, int64_t ld_d, uint32_t* __restrict__ status, int32_t row_begin) {
  __shared__ float s_m[kFbMaxTiles];
  __shared__ float s_s[kFbMaxTiles];
  __shared__ __align__(16) float s_e[64];
  __shared__ __align__(16) float s_sv[64];
  __shared__ float s_lse;
  // XCD x takes a contiguous eighth of the launch's rows, in order: runs of
  // inactive rows (a prompt), which only write zeros, then spread over the
  // launch instead of reaching the whole chip at once (32K workload: 4.08 ->
  // 3.99 ms together with the three-pass phase 1 below)
  const int32_t row = row_begin + (int32_t)xcd_local_block(blockIdx.x, gridDim.x);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave * kGroupsPerWave + (lane >> 4);
  const int gl = lane & 15;
  const uint4* __restrict__ rowp = logits + (int64_t)row * ld_chunks;

  const bool act_mask = (mask == nullptr || mask[row] != 0);
  const int32_t tgt = act_mask ? targets[row] : 0;
  const bool act = act_mask && tgt != ignore_index;
  const bool bad = act && (tgt < 0 || tgt >= real_vocab);
  const bool reread = act && !bad;
  float x_t = 0.0f;
  if (wave == 0 && reread)
    x_t = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(rowp)[tgt] << 16);
  const float g = act ? grad[row] : 0.0f;

  // 1. tile partials (the loop bound is uniform: all groups of a wave call
  //    tile_partial together)
  for (int32_t t0 = 0; t0 < num_tiles; t0 += kFbGroups) {
    const int32_t tile = t0 + grp;
    int32_t lo = 0, hi = 0;
    if (tile < num_tiles) tile_range(tile, tile_width, padded_vocab, num_tiles, real_vocab, lo, hi);
    float gm, ls, la;
    // three passes in flight (125 VGPRs, two blocks per CU): bitwise the same
    tile_partial<false, 3>(rowp, lo, hi, gl, gm, ls, la);
    if (tile < num_tiles && gl == 0) {
      s_m[tile] = gm;
      s_s[tile] = ls;
    }
  }
  // the first batch of phase-3 loads: 16-byte chunks of 8 columns, or for fp32
  // dX 8-byte pieces of 4 columns (see bwd_dlogits)
  constexpr bool kQuad = sizeof(OutT) == 4;
  constexpr int kPieces = 2 * kFbUnroll;
  const u32x2* __restrict__ rowq = reinterpret_cast<const u32x2*>(rowp);
  const int32_t n_chunks = (padded_vocab + 7) >> 3;
  int32_t c0 = threadIdx.x;
  uint4 qa[kFbUnroll], qb[kFbUnroll];
  u32x2 pa[kPieces], pb[kPieces];
  if (reread) {
    if constexpr (kQuad) {
#pragma unroll
      for (int k = 0; k < kPieces; ++k) {
        const int32_t pc = c0 + k * kFbThreads;
        if ((pc << 2) < real_vocab) pa[k] = __builtin_nontemporal_load(rowq + pc);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kFbUnroll; ++k) {
        const int32_t c = c0 + k * kFbThreads;
        if ((c << 3) < real_vocab) qa[k] = load_stream(rowp + c);
      }
    }
  }
  __syncthreads();

  // 2. merge, LSE, logp (wave 0)
  if (wave == 0) {
    float L;
    if (num_tiles <= 64) {
      const float mt = lane < num_tiles ? s_m[lane] : kNegInf;
      const float st = lane < num_tiles ? s_s[lane] : 0.0f;
      L = merge_lanes(mt, st, num_tiles, lane, s_e, s_sv);
    } else {
      L = merge_row(s_m, s_s, num_tiles);
    }
    if (lane == 0) {
      s_lse = L;
      lse[row] = L;
      if (!act) {
        logp[row] = 0.0f;
      } else if (bad) {
        logp[row] = __builtin_nanf("");
        status[0] = 1u;
      } else {
        logp[row] = x_t - L;
        if (!__builtin_isfinite(L)) status[1] = 1u;
      }
    }
  }
  __syncthreads();

  // 3. dX over the row's V_pad columns (the logits of inactive or bad rows
  //    are not read again)
  const float L = act ? s_lse : 0.0f;
  OutT* __restrict__ orow = dlogits + (int64_t)row * ld_d;
  if constexpr (kQuad) {
    const int32_t n_quads = (padded_vocab + 3) >> 2;
    for (int32_t p0 = threadIdx.x; p0 < n_quads; p0 += kFbThreads * kPieces) {
      const int32_t p1 = p0 + kFbThreads * kPieces;
      if (reread && p1 < n_quads) {
#pragma unroll
        for (int k = 0; k < kPieces; ++k) {
          const int32_t pc = p1 + k * kFbThreads;
          if ((pc << 2) < real_vocab) pb[k] = __builtin_nontemporal_load(rowq + pc);
        }
      }
#pragma unroll
      for (int k = 0; k < kPieces; ++k) {
        const int32_t j0 = (p0 + k * kFbThreads) << 2;
        if (j0 >= padded_vocab) continue;
        float d[4];
        dlogits_chunk(pa[k], j0, act, bad, L, g, tgt, real_vocab, d);
        store_quad(reinterpret_cast<float*>(orow) + j0, d, min(4, padded_vocab - j0));
      }
#pragma unroll
      for (int k = 0; k < kPieces; ++k) pa[k] = pb[k];
    }
  } else {
    for (; c0 < n_chunks; c0 += kFbThreads * kFbUnroll) {
      const int32_t c1 = c0 + kFbThreads * kFbUnroll;
      if (reread && c1 < n_chunks) {
#pragma unroll
        for (int k = 0; k < kFbUnroll; ++k) {
          const int32_t c = c1 + k * kFbThreads;
          if ((c << 3) < real_vocab) qb[k] = load_stream(rowp + c);
        }
      }
#pragma unroll
      for (int k = 0; k < kFbUnroll; ++k) {
        const int32_t c = c0 + k * kFbThreads;
        const int32_t j0 = c << 3;
        if (j0 >= padded_vocab) continue;
        float d[8];
        dlogits_chunk(qa[k], j0, act, bad, L, g, tgt, real_vocab, d);
        Store8<OutT>::store(orow + j0, d, min(8, padded_vocab - j0));
      }
#pragma unroll
      for (int k = 0; k < kFbUnroll; ++k) qa[k] = qb[k];
    }
  }
}

// ---------------------------------------------------------------------------
// Forward and backward in one launch, split across blocks: one block owns a
// unit of kUnitWaves * 4 consecutive tiles of one row and keeps them on chip
// (registers, and LDS for part of them) from the read to the dX write, so HBM
// sees exactly one read of the logits and one write of dX.
//   1. each 16-lane group reduces its tile with the stage-1 code (lane
//      mapping, fold order and rotate tree of tile_partial), holding every
//      chunk it loads;
//   2. the group publishes the tile's (max, sumexp) pair as one 64-bit relaxed
//      atomic store at agent scope into the row's slot for that tile, which a
//      fill kernel has set to kSlotEmpty;
//   3. wave 0 polls the row's T <= 64 slots (one per lane, relaxed atomic
//      loads at agent scope) until none is empty, then merges them with the
//      stage-2 arithmetic;
//   4. the block writes dX of its columns from what it kept.
// A pair is a single 64-bit access, so a reader sees either the sentinel or
// both halves of the partial: no fence is needed between the data and a flag
// (a device-scope release would write back the L2 full of dX lines), only the
// per-location coherence that relaxed atomics have across the XCDs.  The
// sentinel is not a pair the reduction can produce: its max half would be a NaN
// whose low 16 bits are set, and a tile max is an input logit (a bf16 value
// widened, low 16 bits zero), -inf or the hardware's default NaN.
//
// Progress: a block waits only for the other units of its row, which are the
// neighbouring block indices.  The poll is bounded: after spin_limit polls
// (or at once when spin_limit <= 0) the block computes all T partials of the
// row itself, with the same code, and goes on -- the same bits whatever the
// schedule, and no block waits for ever.
//
// Every value is computed by the code of stage1_partials, stage2_merge_waves
// and bwd_dlogits in the same order, so the outputs are bitwise those of the
// separate launches.  Each dX chunk has one writer: the tile that holds the
// chunk's first column (a full chunk in its passes, or its tail chunk, which
// may reach into the next tile or the padding); chunks that start at or past
// V_real are zeros written by the tile whose padded bounds hold their first
// column.  That needs tiles of at least 8 columns (the launcher checks it).
// ---------------------------------------------------------------------------
constexpr uint64_t kSlotEmpty = ~0ull;
constexpr int kUnitMaxPass = 4;  // tiles of up to 4 passes (80 chunks each) per lane group
constexpr int kUnitWaves = 2;    // waves per block: 8 tiles per unit
// Passes a lane keeps in registers; the rest wait in LDS.  With bf16 dX two
// passes in LDS free 40 VGPRs (117 against 156), for 4 waves per SIMD instead of
// 3 (32K rows: 3.28 against 3.45 ms).  With fp32 dX, whose stores are twice as
// many, the registers win (5.43 against 5.99 ms).
template <typename OutT>
constexpr int kUnitRegPass = sizeof(OutT) == 2 ? 2 : kUnitMaxPass;

typedef __attribute__((address_space(3))) void* lds_ptr;

// 16 bytes per lane from global memory straight into LDS (nontemporal): lane i
// of the wave writes bytes [16i, 16i + 16) after dst, which is the same for
// the whole wave.  Completion is counted by vmcnt, like any load.
__device__ __forceinline__ void load_chunk_to_lds(const uint4* src, char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr)dst, 16, 0, 2);
}

// The chunks one lane holds for its tile: slot (p, k) is chunk
// base0 + p * kPassChunks + k * 16 + gl, plus the chunk cut by a tile bound
// (lane 0: the head chunk, lane 1: the tail chunk) in qe.  Passes below kRegPass
// are kept in registers, the others in the wave's LDS area: slot (p, k) at
// lds + ((p - kRegPass) * kChunks + k) * 1024 + 16 * lane.
template <int kMaxPass, int kRegPass>
struct TileRegs {
  uint4 q[kRegPass][kChunks];
  uint4 qe;
  char* lds;       // this wave's LDS area (unused when kRegPass == kMaxPass)
  int32_t c_tail;  // this lane's tail chunk (its dX is written here), or -1
  int32_t base0, cf_lo, cf_hi, npass;
  __device__ __forceinline__ uint4 chunk(int p, int k) const {
    if (p < kRegPass) return q[p < kRegPass ? p : 0][k];
    return *reinterpret_cast<const uint4*>(lds + ((p - kRegPass) * kChunks + k) * 1024 +
                                           (threadIdx.x & 63) * 16);
  }
};

// tile_partial's loads and arithmetic with every pass loaded up front and kept
// (npass <= kMaxPass); the same fold order -- the cut chunk, then the passes in
// ascending order -- and the same group reduction, so the same bits.  The
// register passes' loads go out first, so that folding them waits only for
// them; the LDS passes are read back after all loads have landed.
template <int kMaxPass, int kRegPass, bool kEnt>
__device__ __forceinline__ void tile_partial_regs(const uint4* __restrict__ rowp, int32_t lo,
                                                  int32_t hi, int gl,
                                                  TileRegs<kMaxPass, kRegPass>& r, float& gm_out,
                                                  float& ls_out, float& la_out) {
  float m = kNegInf, s = 0.0f, a = 0.0f;
  r.cf_lo = (lo + 7) >> 3;
  r.cf_hi = hi >> 3;
  if (r.cf_hi < r.cf_lo) r.cf_hi = r.cf_lo;
  r.base0 = r.cf_lo & ~7;
  r.npass = r.cf_hi > r.cf_lo ? (r.cf_hi - r.base0 + kPassChunks - 1) / kPassChunks : 0;
  int32_t c = -1, e_lo = 0, e_hi = 0;
  r.c_tail = -1;
  if (gl == 0 && hi > lo && (lo & 7)) {
    c = lo >> 3;
    e_lo = lo & 7;
    e_hi = min(hi - (c << 3), 8);
  } else if (gl == 1 && hi > lo && (hi & 7) && (hi >> 3) >= r.cf_lo) {
    c = hi >> 3;
    e_lo = 0;
    e_hi = hi & 7;
    r.c_tail = c;
  }
  if (c >= 0) r.qe = load_stream(rowp + c);
#pragma unroll
  for (int p = 0; p < kRegPass; ++p)
    if (p < r.npass) load_pass<true>(r.q[p], rowp, r.base0 + p * kPassChunks, r.cf_lo, r.cf_hi, gl);
#pragma unroll
  for (int p = kRegPass; p < kMaxPass; ++p)
    if (p < r.npass) {
#pragma unroll
      for (int k = 0; k < kChunks; ++k) {  // load_pass's clamped addresses
        const int32_t cc = r.base0 + p * kPassChunks + k * kGroupLanes + gl;
        load_chunk_to_lds(rowp + min(max(cc, r.cf_lo), r.cf_hi - 1),
                          r.lds + ((p - kRegPass) * kChunks + k) * 1024);
      }
    }
  if (c >= 0) fold_edge<kEnt>(r.qe, e_lo, e_hi, m, s, a);
#pragma unroll
  for (int p = 0; p < kRegPass; ++p)
    if (p < r.npass)
      fold_pass<kEnt>(r.q[p], r.base0 + p * kPassChunks, r.cf_lo, r.cf_hi, gl, m, s, a);
  if (kRegPass < kMaxPass) {
    __builtin_amdgcn_s_waitcnt(0);  // the LDS passes have landed
#pragma unroll
    for (int p = kRegPass; p < kMaxPass; ++p)
      if (p < r.npass) {
        uint4 q[kChunks];
#pragma unroll
        for (int k = 0; k < kChunks; ++k) q[k] = r.chunk(p, k);
        fold_pass<kEnt>(q, r.base0 + p * kPassChunks, r.cf_lo, r.cf_hi, gl, m, s, a);
      }
  }
  group_reduce<kEnt>(m, s, a, gm_out, ls_out, la_out);
}

// dX of 8 columns at out; n = columns to write (1..8).  bf16: one 16-byte
// nontemporal store.  fp32: two 16-byte stores; a lane's 32 bytes sit between
// its neighbours', so each store instruction covers every other 16 bytes of
// its span, and without the nontemporal hint the L2 joins the two halves of
// each line (32K rows: 5.46 against 5.80 ms with the hint).
template <typename OutT>
__device__ __forceinline__ void store_chunk(OutT* out, const float (&d)[8], int n) {
  if constexpr (sizeof(OutT) == 2) {
    Store8<uint16_t>::store(out, d, n);
  } else if (n == 8) {
    *reinterpret_cast<u32x4*>(out) = u32x4{__float_as_uint(d[0]), __float_as_uint(d[1]),
                                           __float_as_uint(d[2]), __float_as_uint(d[3])};
    *reinterpret_cast<u32x4*>(out + 4) = u32x4{__float_as_uint(d[4]), __float_as_uint(d[5]),
                                               __float_as_uint(d[6]), __float_as_uint(d[7])};
  } else {
    for (int e = 0; e < n; ++e) out[e] = d[e];
  }
}

// dX of the tile's chunks from what the lane kept.  A full chunk lies inside the
// real columns, so dlogits_chunk reduces to one of three forms, chosen once per
// row (act and bad are the same for the whole block): +0 on an inactive row,
// NaN on a row with a bad target, else -g exp(x - L) per column with the
// target's column g (1 - exp(x_t - L)) -- dlogits_chunk's arithmetic.  The
// tail chunk, which may reach past V_real, takes dlogits_chunk itself.
// With kExGrad the extended gradient instead (dlogits_chunk_ex's arithmetic,
// the same forms per full chunk: +0 on a row no term reaches, NaN on a bad
// target, else the LSE, entropy and logp terms); act then means "some term
// reaches the row" and tgt is -1 on a row that is not effective-active.
template <int kMaxPass, int kRegPass, typename OutT, bool kExGrad = false>
__device__ __forceinline__ void tile_dx_regs(const TileRegs<kMaxPass, kRegPass>& r, int gl,
                                             OutT* __restrict__ orow, bool act, bool bad, float L,
                                             float g, int32_t tgt, int32_t real_vocab,
                                             int32_t padded_vocab, float gl_ = 0.0f,
                                             float gh = 0.0f, float H = 0.0f) {
  const float ng = -g;
  const float cc = gl_ - g;
  const float kk = cc - gh * H;  // read only where gh != 0
#pragma unroll
  for (int p = 0; p < kMaxPass; ++p) {
    if (p >= r.npass) break;
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int32_t c = r.base0 + p * kPassChunks + k * kGroupLanes + gl;
      if (c < r.cf_lo || c >= r.cf_hi) continue;
      const int32_t j0 = c << 3;
      float d[8];
      if (act && !bad && kExGrad) {
        float x[8], pv[8], qv[8];
        unpack8(r.chunk(p, k), x);
        if (gh != 0.0f) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float t = x[e] - L;
            pv[e] = exp2_hw(t * kLog2e);
            qv[e] = fmaf(-gh, __builtin_fmaxf(t, kLogpFloor), kk);
            d[e] = pv[e] * qv[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = exp2_hw((x[e] - L) * kLog2e);
            qv[e] = 0.0f;
            d[e] = pv[e] * cc;
          }
        }
        if (tgt >= j0 && tgt < j0 + 8) {
          const int e = tgt - j0;
          d[e] = gh != 0.0f ? fmaf(pv[e], qv[e], g) : g * (1.0f - pv[e]) + pv[e] * gl_;
        }
      } else if (act && !bad) {
        float x[8];
        unpack8(r.chunk(p, k), x);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = ng * exp2_hw((x[e] - L) * kLog2e);
        if (tgt >= j0 && tgt < j0 + 8) {
          const int e = tgt - j0;
          d[e] = g * (1.0f - exp2_hw((x[e] - L) * kLog2e));
        }
      } else {
        const float v = act ? __builtin_nanf("") : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = v;
      }
      store_chunk<OutT>(orow + j0, d, 8);
    }
  }
  if (r.c_tail >= 0) {
    const int32_t j0 = r.c_tail << 3;
    float d[8];
    if (kExGrad)
      dlogits_chunk_ex(r.qe, j0, act, bad, L, g, gl_, gh, H, tgt, real_vocab, d);
    else
      dlogits_chunk(r.qe, j0, act, bad, L, g, tgt, real_vocab, d);
    store_chunk<OutT>(orow + j0, d, min(8, padded_vocab - j0));
  }
}

__device__ __forceinline__ uint64_t pack_partial(float m, float s) {
  return ((uint64_t)__float_as_uint(s) << 32) | __float_as_uint(m);
}

// Sets every slot to kSlotEmpty and clears the fallback counter (status[2]).
__global__ __launch_bounds__(256) void fill_slots(uint64_t* __restrict__ slots, int64_t n,
                                                  uint32_t* __restrict__ status) {
  if (blockIdx.x == 0 && threadIdx.x == 0) status[2] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    slots[i] = kSlotEmpty;
}

// kEnt: the forward also gives each row's entropy (stage1_partials<true> and
// stage2's merge_lanes_entropy); the third statistic of a tile travels in a
// second slot array [N][T] right after the first, as the pair (a, max) -- the
// max half keeps that slot, too, from ever holding the sentinel.
// kExGrad: dX is rlk_logp_bwd_ex's extended gradient (grad_lse or grad_ent
// given; any of grad, grad_lse and grad_ent may be null = zero), else the plain
// gradient, as the separate extended backward chooses.
template <typename OutT, int kMaxPass, int kRegPass, int kUnitWaves, bool kEnt, bool kExGrad>
__global__ __launch_bounds__(kUnitWaves * 64) void fwd_bwd_units(
    const uint4* __restrict__ logits, int64_t ld_chunks, int32_t real_vocab,
    int32_t padded_vocab, int32_t num_tiles, int32_t tile_width, int32_t units_per_row,
    const int32_t* __restrict__ targets, const uint8_t* __restrict__ mask, int32_t ignore_index,
    const float* __restrict__ grad, const float* __restrict__ grad_lse,
    const float* __restrict__ grad_ent, float* __restrict__ logp, float* __restrict__ lse,
    float* __restrict__ entropy, OutT* __restrict__ dlogits, int64_t ld_d,
    uint32_t* __restrict__ status, uint64_t* __restrict__ slots, int64_t slots_b,
    int32_t spin_limit, int64_t unit_begin) {
  static_assert(kEnt || !kExGrad, "the extended gradient needs the entropy");
  constexpr int kGroups = kUnitWaves * kGroupsPerWave;  // tiles per unit
  __shared__ float s_m[64];
  __shared__ float s_s[64];
  __shared__ float s_a[kEnt ? 64 : 1];
  __shared__ __align__(16) float s_e[64];
  __shared__ __align__(16) float s_sv[64];
  __shared__ __align__(16) float s_d[kEnt ? 64 : 1];
  __shared__ __align__(16) float s_av[kEnt ? 64 : 1];
  __shared__ float s_lse;
  __shared__ float s_ent;
  __shared__ int s_fallback;
  constexpr int kLdsPass = kMaxPass - kRegPass;
  __shared__ __attribute__((aligned(16))) char s_pass[kUnitWaves * (kLdsPass > 0 ? kLdsPass : 1) *
                                                      kChunks * 1024];
  const int64_t u = unit_begin + blockIdx.x;
  const int32_t row = (int32_t)(u / units_per_row);
  const int32_t unit = (int32_t)(u - (int64_t)row * units_per_row);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave * kGroupsPerWave + (lane >> 4);
  const int gl = lane & 15;
  const int32_t tile = unit * kGroups + grp;
  const uint4* __restrict__ rowp = logits + (int64_t)row * ld_chunks;

  // row values, the same in every lane (kept in scalar registers)
  const bool act_mask = (mask == nullptr || mask[row] != 0);
  const int32_t tgt = __builtin_amdgcn_readfirstlane(act_mask ? targets[row] : 0);
  const bool act = __builtin_amdgcn_readfirstlane(act_mask && tgt != ignore_index);
  const bool bad = act && (tgt < 0 || tgt >= real_vocab);
  float x_t = 0.0f;
  if (unit == 0 && threadIdx.x == 0 && act && !bad)
    x_t = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(rowp)[tgt] << 16);
  const float g = (act && (!kExGrad || grad)) ? grad[row] : 0.0f;
  float g_l = 0.0f, g_h = 0.0f;
  if (kExGrad) {
    g_l = grad_lse ? grad_lse[row] : 0.0f;
    g_h = grad_ent ? grad_ent[row] : 0.0f;
  }

  // 1. this unit's tiles, kept on chip
  int32_t lo = 0, hi = 0;
  if (tile < num_tiles) tile_range(tile, tile_width, padded_vocab, num_tiles, real_vocab, lo, hi);
  TileRegs<kMaxPass, kRegPass> tr;
  tr.lds = s_pass + wave * kLdsPass * kChunks * 1024;
  float gm, ls, la;
  tile_partial_regs<kMaxPass, kRegPass, kEnt>(rowp, lo, hi, gl, tr, gm, ls, la);
  uint64_t* __restrict__ rs = slots + (int64_t)row * num_tiles;
  uint64_t* __restrict__ rsb = slots + slots_b + (int64_t)row * num_tiles;
  // 2. publish
  if (tile < num_tiles && gl == 0) {
    __hip_atomic_store(rs + tile, pack_partial(gm, ls), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (kEnt)
      __hip_atomic_store(rsb + tile, pack_partial(gm, la), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  // 3. the row's partials, merged in ascending tile order (wave 0)
  if (wave == 0) {
    bool ok = false;
    uint64_t v = kSlotEmpty, vb = kSlotEmpty;
    for (int32_t it = 0; it < spin_limit; ++it) {
      if (lane < num_tiles) {
        v = __hip_atomic_load(rs + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (kEnt) vb = __hip_atomic_load(rsb + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (__all(lane >= num_tiles || (v != kSlotEmpty && (!kEnt || vb != kSlotEmpty)))) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (ok) {
      const float mt = lane < num_tiles ? __uint_as_float((uint32_t)v) : kNegInf;
      const float st = lane < num_tiles ? __uint_as_float((uint32_t)(v >> 32)) : 0.0f;
      if (kEnt) {
        const float at = lane < num_tiles ? __uint_as_float((uint32_t)(vb >> 32)) : 0.0f;
        float H;
        const float L = merge_lanes_entropy(mt, st, at, num_tiles, lane, s_e, s_sv, s_d, s_av, H);
        if (lane == 0) {
          s_lse = L;
          s_ent = H;
        }
      } else {
        const float L = merge_lanes(mt, st, num_tiles, lane, s_e, s_sv);
        if (lane == 0) s_lse = L;
      }
    }
    if (lane == 0) s_fallback = ok ? 0 : 1;
  }
  __syncthreads();
  if (s_fallback) {
    // the row's T partials from the logits, by this block alone (counted in
    // status[2], which fill_slots cleared)
    if (threadIdx.x == 0) atomicAdd(status + 2, 1u);
    for (int32_t t0 = 0; t0 < num_tiles; t0 += kGroups) {
      const int32_t t = t0 + grp;
      int32_t flo = 0, fhi = 0;
      if (t < num_tiles) tile_range(t, tile_width, padded_vocab, num_tiles, real_vocab, flo, fhi);
      float fm, fs, fa;
      tile_partial<true, 1, kEnt>(rowp, flo, fhi, gl, fm, fs, fa);
      if (t < num_tiles && gl == 0) {
        s_m[t] = fm;
        s_s[t] = fs;
        if (kEnt) s_a[kEnt ? t : 0] = fa;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const float mt = lane < num_tiles ? s_m[lane] : kNegInf;
      const float st = lane < num_tiles ? s_s[lane] : 0.0f;
      if (kEnt) {
        const float at = lane < num_tiles ? s_a[kEnt ? lane : 0] : 0.0f;
        float H;
        const float L = merge_lanes_entropy(mt, st, at, num_tiles, lane, s_e, s_sv, s_d, s_av, H);
        if (lane == 0) {
          s_lse = L;
          s_ent = H;
        }
      } else {
        const float L = merge_lanes(mt, st, num_tiles, lane, s_e, s_sv);
        if (lane == 0) s_lse = L;
      }
    }
    __syncthreads();
  }
  const float Lrow = s_lse;
  const float Hrow = kEnt ? s_ent : 0.0f;
  if (unit == 0 && threadIdx.x == 0) {
    lse[row] = Lrow;
    if (kEnt) entropy[row] = Hrow;
    if (!act) {
      logp[row] = 0.0f;
    } else if (bad) {
      logp[row] = __builtin_nanf("");
      status[0] = 1u;
    } else {
      logp[row] = x_t - Lrow;
      if (!__builtin_isfinite(Lrow)) status[1] = 1u;
    }
  }

  // 4. dX of this unit's columns
  if (tile >= num_tiles) return;
  OutT* __restrict__ orow = dlogits + (int64_t)row * ld_d;
  if (kExGrad) {
    // the separate extended backward's row values: a row is reached by the logp
    // term when effective-active, by the LSE and entropy terms when theirs are
    // nonzero; the target term only on an effective-active row
    const bool need = act || g_l != 0.0f || g_h != 0.0f;
    const float L = need ? Lrow : 0.0f;
    const float H = g_h != 0.0f ? Hrow : 0.0f;
    tile_dx_regs<kMaxPass, kRegPass, OutT, true>(tr, gl, orow, need, bad, L, g, act ? tgt : -1,
                                                 real_vocab, padded_vocab, g_l, g_h, H);
  } else {
    const float L = act ? Lrow : 0.0f;
    tile_dx_regs<kMaxPass, kRegPass, OutT>(tr, gl, orow, act, bad, L, g, tgt, real_vocab,
                                           padded_vocab);
  }
  // chunks that start at or past V_real inside this tile's padded bounds: +0
  int32_t plo, phi;
  if (tile_width) {
    plo = tile * tile_width;
    phi = plo + tile_width;
  } else {
    plo = (int32_t)(((int64_t)tile * padded_vocab) / num_tiles);
    phi = (int32_t)(((int64_t)(tile + 1) * padded_vocab) / num_tiles);
  }
  const int32_t z_end = (phi + 7) >> 3;
  const float zero[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int32_t c = max((plo + 7) >> 3, (real_vocab + 7) >> 3) + gl; c < z_end; c += kGroupLanes)
    store_chunk<OutT>(orow + (c << 3), zero, min(8, padded_vocab - (c << 3)));
}

__global__ void clear_status(uint32_t* status) {
  if (threadIdx.x < 2) status[threadIdx.x] = 0u;
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers (called by the boundary after it has validated every argument).
// ---------------------------------------------------------------------------
int64_t stage1_blocks(int64_t items) {
  const int64_t per_block = (int64_t)kWavesPerBlock * kGroupsPerWave;
  return (items + per_block - 1) / per_block;
}

// Below this many 4-wave blocks a launch would leave CUs idle (two per CU on
// the 256-CU part); smaller launches use one-wave blocks instead.
constexpr int64_t kStage1SmallBlocks = 512;

hipError_t launch_stage1(const Stage1Args& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.num_rows * a.tile_count;
  if (items == 0) return hipSuccess;
  const int64_t blocks4 = stage1_blocks(items);
  const bool small = blocks4 < kStage1SmallBlocks;
  const int wpb = small ? 1 : kWavesPerBlock;
  const int64_t items_per_block = (int64_t)wpb * kGroupsPerWave;
  const int64_t blocks = (items + items_per_block - 1) / items_per_block;
  const int64_t max_blocks = launch_thread_limit() / (wpb * 64);
  const uint4* x = reinterpret_cast<const uint4*>(a.logits);
  for (int64_t b0 = 0; b0 < blocks; b0 += max_blocks) {
    const dim3 grid((unsigned)(blocks - b0 < max_blocks ? blocks - b0 : max_blocks));
    const int64_t item_begin = b0 * items_per_block;
#define RLK_LAUNCH_S1(ENT, WPB, PENT)                                                           \
  hipLaunchKernelGGL((stage1_partials<ENT, WPB>), grid, dim3((WPB) * 64), 0, stream, x,       \
                     a.ld / 8, a.num_rows, a.real_vocab, a.padded_vocab, a.num_tiles,         \
                     a.tile_width, a.tile_begin, a.tile_count, item_begin, a.pmax, a.psum, PENT)
    if (a.pent) {
      if (small) RLK_LAUNCH_S1(true, 1, a.pent);
      else RLK_LAUNCH_S1(true, kWavesPerBlock, a.pent);
    } else {
      if (small) RLK_LAUNCH_S1(false, 1, nullptr);
      else RLK_LAUNCH_S1(false, kWavesPerBlock, nullptr);
    }
#undef RLK_LAUNCH_S1
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_stage2(const Stage2Args& a, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  if (a.num_tiles <= 64 &&
      a.num_rows <= (a.entropy ? kMergeWaveMaxRowsEnt : kMergeWaveMaxRows)) {
    // one wave per row, in launches of at most launch_thread_limit() threads
    const int64_t rows_per_launch = launch_thread_limit() / 64 / kMergeRows * kMergeRows;
    for (int64_t r0 = 0; r0 < a.num_rows; r0 += rows_per_launch) {
      const int64_t nr = a.num_rows - r0 < rows_per_launch ? a.num_rows - r0 : rows_per_launch;
      const dim3 grid((unsigned)((nr + kMergeRows - 1) / kMergeRows));
      if (a.entropy)
        hipLaunchKernelGGL(stage2_merge_waves<true>, grid, dim3(kMergeRows * 64), 0, stream,
                           reinterpret_cast<const uint16_t*>(a.logits), a.target_logit, a.ld,
                           a.num_rows, a.real_vocab, a.num_tiles, a.pmax, a.psum, a.pent,
                           a.targets, a.mask, a.ignore_index, a.logp, a.lse, a.entropy,
                           a.status, r0);
      else
        hipLaunchKernelGGL(stage2_merge_waves<false>, grid, dim3(kMergeRows * 64), 0, stream,
                           reinterpret_cast<const uint16_t*>(a.logits), a.target_logit, a.ld,
                           a.num_rows, a.real_vocab, a.num_tiles, a.pmax, a.psum, nullptr,
                           a.targets, a.mask, a.ignore_index, a.logp, a.lse, nullptr, a.status,
                           r0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const dim3 grid((unsigned)((a.num_rows + kMergeThreads - 1) / kMergeThreads));
  if (a.entropy) {
    hipLaunchKernelGGL(stage2_merge<true>, grid, dim3(kMergeThreads), 0, stream,
                       reinterpret_cast<const uint16_t*>(a.logits), a.target_logit, a.ld,
                       a.num_rows, a.real_vocab, a.num_tiles, a.pmax, a.psum, a.pent, a.targets,
                       a.mask, a.ignore_index, a.logp, a.lse, a.entropy, a.status);
  } else {
    hipLaunchKernelGGL(stage2_merge<false>, grid, dim3(kMergeThreads), 0, stream,
                       reinterpret_cast<const uint16_t*>(a.logits), a.target_logit, a.ld,
                       a.num_rows, a.real_vocab, a.num_tiles, a.pmax, a.psum, nullptr,
                       a.targets, a.mask, a.ignore_index, a.logp, a.lse, nullptr, a.status);
  }
  return hipGetLastError();
}

int64_t bwd_col_blocks(int32_t padded_vocab) {
  return ((int64_t)padded_vocab + kBwdCols - 1) / kBwdCols;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  const int32_t cbs = (int32_t)bwd_col_blocks(a.padded_vocab);
  const int64_t blocks = (int64_t)a.num_rows * cbs;
  const int64_t max_blocks = launch_thread_limit() / kBwdThreads;
  const uint4* x = reinterpret_cast<const uint4*>(a.logits);
  const bool ex = a.grad_lse || a.grad_ent;
  for (int64_t b0 = 0; b0 < blocks; b0 += max_blocks) {
    const dim3 grid((unsigned)(blocks - b0 < max_blocks ? blocks - b0 : max_blocks));
#define RLK_LAUNCH_BWD(OUT_T, EX)                                                              \
  hipLaunchKernelGGL((bwd_dlogits<OUT_T, EX>), grid, dim3(kBwdThreads), 0, stream, x,         \
                     a.ld / 8, a.num_rows, a.real_vocab, a.padded_vocab, cbs, a.targets,     \
                     a.mask, a.ignore_index, a.lse, a.grad, a.grad_lse, a.grad_ent,          \
                     a.entropy, reinterpret_cast<OUT_T*>(a.dlogits), a.ld_d, a.status, b0)
    if (a.out_bf16) {
      if (ex) RLK_LAUNCH_BWD(uint16_t, true);
      else RLK_LAUNCH_BWD(uint16_t, false);
    } else {
      if (ex) RLK_LAUNCH_BWD(float, true);
      else RLK_LAUNCH_BWD(float, false);
    }
#undef RLK_LAUNCH_BWD
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

bool fwd_bwd_units_fit(int32_t real_vocab, int32_t padded_vocab, int32_t num_tiles) {
  if (num_tiles < 1 || num_tiles > 64 || padded_vocab / num_tiles < 8) return false;
  // the passes tile_partial_regs takes for each tile (its geometry, on the host)
  for (int32_t t = 0; t < num_tiles; ++t) {
    const int64_t lo = (int64_t)t * padded_vocab / num_tiles;
    int64_t hi = (int64_t)(t + 1) * padded_vocab / num_tiles;
    if (hi > real_vocab) hi = real_vocab;
    if (hi < lo) hi = lo;
    const int64_t cf_lo = (lo + 7) >> 3;
    int64_t cf_hi = hi >> 3;
    if (cf_hi < cf_lo) cf_hi = cf_lo;
    const int64_t base0 = cf_lo & ~int64_t{7};
    const int64_t npass = cf_hi > cf_lo ? (cf_hi - base0 + kPassChunks - 1) / kPassChunks : 0;
    if (npass > kUnitMaxPass) return false;
  }
  return true;
}

namespace {

template <typename OutT, bool kEnt, bool kExGrad>
hipError_t launch_units(const FwdBwdArgs& a, OutT* dl, hipStream_t stream) {
  constexpr int kGroups = kUnitWaves * kGroupsPerWave;
  const int64_t n_slots = (int64_t)a.num_rows * a.num_tiles * (kEnt ? 2 : 1);
  const int64_t fill_blocks = (n_slots + 255) / 256 < 8192 ? (n_slots + 255) / 256 : 8192;
  hipLaunchKernelGGL(fill_slots, dim3((unsigned)fill_blocks), dim3(256), 0, stream, a.slots,
                     n_slots, a.status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // whole rows per launch: a row's units wait only for each other
  const int32_t upr = (a.num_tiles + kGroups - 1) / kGroups;
  const int64_t rows_per_launch = launch_thread_limit() / (kUnitWaves * 64) / upr;
  const int32_t spin = fwd_bwd_spin_limit();
  const uint4* x = reinterpret_cast<const uint4*>(a.logits);
  const int64_t slots_b = (int64_t)a.num_rows * a.num_tiles;
  for (int64_t r0 = 0; r0 < a.num_rows; r0 += rows_per_launch) {
    const int64_t nr = a.num_rows - r0 < rows_per_launch ? a.num_rows - r0 : rows_per_launch;
    hipLaunchKernelGGL(
        (fwd_bwd_units<OutT, kUnitMaxPass, kUnitRegPass<OutT>, kUnitWaves, kEnt, kExGrad>),
        dim3((unsigned)(nr * upr)), dim3(kUnitWaves * 64), 0, stream, x, a.ld / 8, a.real_vocab,
        a.padded_vocab, a.num_tiles, a.tile_width, upr, a.targets, a.mask, a.ignore_index, a.grad,
        a.grad_lse, a.grad_ent, a.logp, a.lse, a.entropy, dl, a.ld_d, a.status, a.slots, slots_b,
        spin, r0 * upr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename OutT>
hipError_t launch_units_for(const FwdBwdArgs& a, OutT* dl, hipStream_t stream) {
  if (!a.entropy) return launch_units<OutT, false, false>(a, dl, stream);
  if (a.grad_lse || a.grad_ent) return launch_units<OutT, true, true>(a, dl, stream);
  return launch_units<OutT, true, false>(a, dl, stream);
}

}  // namespace

hipError_t launch_fwd_bwd(const FwdBwdArgs& a, hipStream_t stream) {
  if (a.num_rows == 0) return hipSuccess;
  if (a.slots) {
    if (a.out_bf16) return launch_units_for(a, reinterpret_cast<uint16_t*>(a.dlogits), stream);
    return launch_units_for(a, reinterpret_cast<float*>(a.dlogits), stream);
  }
  const int64_t rows_per_launch = launch_thread_limit() / kFbThreads;
  const uint4* x = reinterpret_cast<const uint4*>(a.logits);
  for (int64_t r0 = 0; r0 < a.num_rows; r0 += rows_per_launch) {
    const int64_t nr = a.num_rows - r0 < rows_per_launch ? a.num_rows - r0 : rows_per_launch;
    const dim3 grid((unsigned)nr);
    const int32_t row_begin = (int32_t)r0;
    if (a.out_bf16) {
      hipLaunchKernelGGL(fwd_bwd_rows<uint16_t>, grid, dim3(kFbThreads), 0, stream, x,
                         a.ld / 8, a.real_vocab, a.padded_vocab, a.num_tiles, a.tile_width,
                         a.targets, a.mask, a.ignore_index, a.grad, a.logp, a.lse,
                         reinterpret_cast<uint16_t*>(a.dlogits), a.ld_d, a.status, row_begin);
    } else {
      hipLaunchKernelGGL(fwd_bwd_rows<float>, grid, dim3(kFbThreads), 0, stream, x,
                         a.ld / 8, a.real_vocab, a.padded_vocab, a.num_tiles, a.tile_width,
                         a.targets, a.mask, a.ignore_index, a.grad, a.logp, a.lse,
                         reinterpret_cast<float*>(a.dlogits), a.ld_d, a.status, row_begin);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_clear_status(uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(clear_status, dim3(1), dim3(64), 0, stream, status);
  return hipGetLastError();
}

}  // namespace rlk
