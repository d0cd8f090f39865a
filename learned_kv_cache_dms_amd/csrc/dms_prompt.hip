// DMS attention of several queries per sequence for gfx950 (MI355X):
//   * prefill_attention_kernel: every prompt query over its own visible set,
//     from the compressed cache (positions below q - w) and the dense prompt
//     (the window), right after the prompt's compression;
//   * chunk_attention_kernel + append_chunk_kernel: the queries of a chunk of
//     tokens over the cache as it stands plus the chunk's own rows, then the
//     chunk's appends in order.
#include "dms_device.h"

namespace dms {
// ---------------------------------------------------------------------------
// attention of the prompt's own queries, after the prompt's compression
// ---------------------------------------------------------------------------

// Query q attends Vis(q) = { j < q - w : j unmarked } + [q - w, q] (every
// token of the last w + 1 positions is visible, marked or not).  The first
// part is exactly the cache slots whose position is below q - w: right after
// the compression the cache holds every unmarked prompt token, and the marked
// tokens it still holds sit at positions >= P - 1 - w >= q - w; its slots are
// in position order.  The second part is read from the dense prompt.  The two
// parts are disjoint and the decisions themselves are never needed.
//

// Fragment (the cache block order) of 16 consecutive dense rows row0 ..
// row0 + 15 of one (sequence, KV head), rows clamped to `last` (the clamped
// rows are masked out by the caller; they only have to be finite).
template <int ES, int D>
__device__ __forceinline__ void load_frag_dense(Frag<ES, D>& f, const uint8_t* __restrict__ K,
                                                const uint8_t* __restrict__ V, int row0, int last, int lane,
                                                int zero_ch = -1) {
  using G = Geo<ES, D>;
  // K: lane l carries row l % 16, 16-byte piece 4c + l / 16 of the row
  // (key channel zero_ch, when >= 0, is read as 0, as the cache stores it)
  const uint8_t* krow = K + (int64_t)min(row0 + (lane & 15), last) * D * ES;
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    f.k[c] = *(const u32x4*)(krow + c * 64 + 16 * (lane >> 4));
    clear_channel<ES>(f.k[c], 4 * c + (lane >> 4), zero_ch);
  }
  // V: lane l carries rows 4 (l / 16) + e, channel 16 (c kNJ + jj) + l % 16
  const uint8_t* vrow[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) vrow[e] = V + (int64_t)min(row0 + 4 * (lane >> 4) + e, last) * D * ES;
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    u32x4 val = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int jj = 0; jj < G::kNJ; ++jj) {
      const int ch = 16 * (c * G::kNJ + jj) + (lane & 15);
      if constexpr (ES == 2) {
        // two 16-bit loads per register, joined as a vector (one v_perm_b32
        // instead of a shift and an or)
        typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          u16x2 t;
          t.x = *(const uint16_t*)(vrow[2 * h2] + ch * 2);
          t.y = *(const uint16_t*)(vrow[2 * h2 + 1] + ch * 2);
          val[jj * 2 + h2] = __builtin_bit_cast(uint32_t, t);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = *(const uint32_t*)(vrow[e] + ch * 4);
      }
    }
    f.v[c] = val;
  }
}

// Softmax step and P.V of a pair of blocks for the compute-bound attention
// of several queries per sequence (the masks as softmax_pv_masked).  A
// column's reference max moves only when a score exceeds it by more than
// 2^kPromptSlack in the exp2 domain, so the accumulators are rescaled a few
// times per column rather than whenever its max creeps up; the weights
// exp2(s - m) stay below 2^kPromptSlack and o / l is unchanged.  (A state
// kept this way and one kept by softmax_pv_masked are the same kind: o and l
// relative to the reference m.)  HILO: the weights enter P.V as bf16 hi + lo
// pairs (about 2^-17, as the decode kernels); else as bf16 (nearest even), one
// product per tile: an output element is then off by at most 2^-8 of
// sum_i p_i |v_i| / sum_i p_i (the sum l stays fp32).
//  - prompt attention: bf16 weights; hi + lo cost 22 % of the kernel's time on
//    the 32B-shaped layer (276.8 against 220.2 ms with both changes);
//  - chunk attention: hi + lo, so that a chunk's outputs match the one-token
//    steps' to their precision; the stale max took C = 16 from 0.390 to
//    0.372 ms and C = 64 from 1.170 to 1.141 ms.
// On gfx950 the VALU and MFMA work of a SIMD add up rather than overlap, so
// the step is written for few VALU instructions:
//  - the lane's 8 scores are reduced with the NaN-propagating maximum
//    (v_maximum3_f32 takes its operands as they are; fmaxf quiets each one
//    first).  Scores are finite or -inf here, where the two agree;
//  - each lane first tests its own 8 scores against the reference; only when
//    some lane of the wave exceeds it does the wave form the column max
//    across the four lane groups and rescale;
//  - MASKED = false skips the key masks (pairs whose 32 keys are all live
//    and visible to every column).
// Together: prompt attention 219.4 -> 205.8 ms on the 32B-shaped layer.
constexpr float kPromptSlack = 8.0f;
template <int D, bool HILO, bool MASKED = true>
__device__ __forceinline__ void softmax_pv_stale(const PairFrag<2, D>& f, const f32x4& SA, const f32x4& SB,
                                                 uint32_t ma, uint32_t mb, int lane, float sl2e, Acc<D>& a) {
  using G = Geo<2, D>;
  const int tb = 4 * (lane >> 4);
  float s[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s[r] = !MASKED || ((ma >> (tb + r)) & 1u) ? SA[r] : -INFINITY;
    s[4 + r] = !MASKED || ((mb >> (tb + r)) & 1u) ? SB[r] : -INFINITY;
  }
  auto mx = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
  const float lm = mx(mx(mx(s[0], s[1]), mx(s[2], s[3])), mx(mx(s[4], s[5]), mx(s[6], s[7])));
  // the scale is > 0, so scaling and the max commute
  if (__builtin_amdgcn_ballot_w64(lm * sl2e > a.m + kPromptSlack) != 0) {
    // a column with no key yet has m = -inf and o = l = 0: its first finite
    // score moves the reference, and alpha = 0 leaves o and l at 0; the other
    // columns keep theirs (alpha = 1, also when m is still -inf)
    const float bm2 = max_over_groups(lm) * sl2e;
    const bool grow = bm2 > a.m + kPromptSlack;
    const float mn = grow ? bm2 : a.m;
    const float alpha = grow ? exp2_fast(a.m - mn) : 1.0f;
    a.l *= alpha;
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) a.o[j] *= alpha;
    a.m = mn;
  }
  const float mref = (a.m == -INFINITY) ? 0.f : a.m;
  float pr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) pr[r] = exp2_fast(fmaf(s[r], sl2e, -mref));
  a.l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
  unsigned hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) hi[i] = pack_bf16x2(pr[2 * i], pr[2 * i + 1]);
  const u32x4 hv = {hi[0], hi[1], hi[2], hi[3]};
  const bf16x8 PH = __builtin_bit_cast(bf16x8, hv);
  if constexpr (HILO) {
    unsigned lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lo[i] = pack_bf16x2(pr[2 * i] - bf16_lo_to_f32(hi[i]), pr[2 * i + 1] - bf16_hi_to_f32(hi[i]));
    const u32x4 lv = {lo[0], lo[1], lo[2], lo[3]};
    const bf16x8 PL = __builtin_bit_cast(bf16x8, lv);
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) {
      const bf16x8 A = __builtin_bit_cast(bf16x8, f.v[j]);
      a.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, PH, a.o[j], 0, 0, 0);
      a.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, PL, a.o[j], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j)
      a.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.v[j]), PH, a.o[j], 0, 0, 0);
  }
}

// attend_pair with the prompt attention's softmax step for bf16 rows.
template <int ES, int D>
__device__ __forceinline__ void attend_pair_prompt(const PairFrag<ES, D>& f, const u32x4 (&qf)[Geo<ES, D>::kChunks],
                                                   uint32_t ma, uint32_t mb, int lane, float sl2e, Acc<D>& a) {
  if constexpr (ES != 2) {
    attend_pair<ES, D>(f, qf, ma, mb, lane, sl2e, a);
  } else {
    f32x4 SA, SB;
    score_pair<D>(f, qf, SA, SB);
    softmax_pv_stale<D, false>(f, SA, SB, ma, mb, lane, sl2e, a);
  }
}

// Column tiles per wave of the prompt attention for rows of ES-byte elements:
// fp32 rows at d = 128 take twice the registers of bf16 ones, and three tiles
// of them spill (93 registers); two do not.
template <int ES, int D>
constexpr int pf_cols() {
  return ES == 4 && D == 128 ? 2 : kPfCols;
}
template <int ES, int D>
constexpr int pf_tile() {
  return 16 * pf_cols<ES, D>() * kWavesPerWG;
}

// Grid (ceil(max_len_used / pf_tile<ES, D>()), Hq, B), read as one list of work items.
template <int ES, int D>
__global__ __launch_bounds__(256) void prefill_attention_kernel(Dev p, const uint8_t* __restrict__ q,
                                                                const uint8_t* __restrict__ k,
                                                                const uint8_t* __restrict__ v, int32_t max_len,
                                                                int zero_ch, float* __restrict__ out) {
  using G = Geo<ES, D>;
  constexpr int NCOL = pf_cols<ES, D>(), TILE = pf_tile<ES, D>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Work item (sequence, query head, query tile) of this work-group.  Work-group
  // i runs on XCD i mod 8; each XCD takes a contiguous run of the items, which
  // are in unit order, so that a unit's blocks are read into one XCD's L2 by
  // the query tiles of all its heads; within a (sequence, query head) the
  // last query tiles (the longest far parts) go first.  (Against the grid's
  // own order on the 32B-shaped layer: 172.6 -> 168.6 ms; tiles in ascending
  // order 169.5.)
  const int ntile = gridDim.x, nitems = ntile * gridDim.y * gridDim.z;
  const int lin = blockIdx.x + ntile * (blockIdx.y + gridDim.y * blockIdx.z);
  const int xcd = lin & 7, base = nitems >> 3, rem = nitems & 7;
  const int item = xcd * base + min(xcd, rem) + (lin >> 3);
  const int tile = ntile - 1 - item % ntile, hq = (item / ntile) % gridDim.y, b = item / (ntile * gridDim.y);
  const int h = hq / p.G, u = b * p.Hkv + h;
  const int P = __builtin_amdgcn_readfirstlane(p.pos[u]);
  const int q0 = tile * TILE;
  if (q0 >= P) return;
  const int w = p.R - 1;
  const int qmax = min(q0 + TILE, P) - 1;
  const int64_t unit_rows = ((int64_t)b * p.Hkv + h) * max_len;
  const uint8_t* Ku = k + unit_rows * D * ES;
  const uint8_t* Vu = v + unit_rows * D * ES;
  const uint8_t* Qh = q + ((int64_t)b * p.Hq + hq) * max_len * D * ES;

  int qc[NCOL];
  u32x4 qf[NCOL][G::kChunks];
  Acc<D> acc[NCOL];
#pragma unroll
  for (int t = 0; t < NCOL; ++t) {
    qc[t] = q0 + 16 * (NCOL * wave + t) + (lane & 15);
    const uint8_t* qrow = Qh + (int64_t)min(qc[t], P - 1) * D * ES;
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) qf[t][c] = *(const u32x4*)(qrow + c * 64 + 16 * (lane >> 4));
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) acc[t].o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[t].m = -INFINITY;
    acc[t].l = 0.f;
  }
  const int tb = 4 * (lane >> 4);

  // Far part: the cache blocks whose first slot lies below qmax - w (slot
  // positions increase, so they are a prefix); counted with one round of
  // independent loads of the blocks' first positions.
  const int n = __builtin_amdgcn_readfirstlane(p.n[u]);
  const int nb = (n + 15) >> 4;
  const int32_t* bt = p.btab + (int64_t)u * p.max_blocks;
  const int lim = qmax - w;
  // nfar: blocks whose first slot lies below qmax - w.  nfull: blocks j whose
  // next block starts at or below q0 - w; all 16 slots of such a block lie
  // below q0 - w, so every key in it is far for every query of the tile.
  // Slot positions increase, so both are prefixes; one round of independent
  // loads of the blocks' first positions counts them.
  int nfar = 0, nlow = 0;
  for (int j0 = 0; j0 < nb; j0 += 64) {
    const int j = j0 + lane;
    int c = 0, d2 = 0;
    if (j < nb) {
      const int first = p.blk_pos[(int64_t)bt[j] * 16];
      c = first < lim ? 1 : 0;
      d2 = first <= q0 - w ? 1 : 0;
    }
    nfar += wave_sum_i(c);
    nlow += wave_sum_i(d2);
  }
  nfar = __builtin_amdgcn_readfirstlane(nfar);
  // (rounded down to whole pairs; the odd block, if any, goes with the
  // straddling blocks, whose per-slot masks also hold for it)
  const int nfull = min(max(__builtin_amdgcn_readfirstlane(nlow) - 1, 0), nfar) & ~1;
  auto blk_at = [&](int j, int jmax) { return __builtin_amdgcn_readfirstlane(bt[min(j, jmax)]); };
  if (nfull > 0) {
    // Whole blocks, in pairs, one pair loaded ahead of the one computed; all
    // 32 keys of a pair are live and far for every query of the tile, so
    // the softmax takes no masks.  Loads are unconditional: the prefetch past
    // the last pair re-reads it and goes unused.  The scheduling barriers
    // keep each pair's loads issued ahead of the previous pair's arithmetic
    // (left alone, the scheduler sinks them next to their use, exposing
    // their latency).
    const int npair = nfull >> 1;
    auto fetch = [&](PairFrag<ES, D>& f, int i) {
      const int ba = blk_at(2 * i, nfull - 1), bb = blk_at(2 * i + 1, nfull - 1);
      load_pair<ES, D, false>(f, p.pool + (int64_t)ba * p.block_bytes, p.pool + (int64_t)bb * p.block_bytes, lane);
    };
    auto compute = [&](const PairFrag<ES, D>& f, int i) {
      if constexpr (ES == 2) {
        // column t + 1's score products issued before column t's softmax
        f32x4 SA[2], SB[2];
        score_pair<D>(f, qf[0], SA[0], SB[0]);
#pragma unroll
        for (int t = 0; t < NCOL; ++t) {
          if (t + 1 < NCOL) score_pair<D>(f, qf[t + 1], SA[(t + 1) & 1], SB[(t + 1) & 1]);
          softmax_pv_stale<D, false, false>(f, SA[t & 1], SB[t & 1], 0xffffu, 0xffffu, lane, p.scale_log2e,
                                           acc[t]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < NCOL; ++t) attend_pair_prompt<ES, D>(f, qf[t], 0xffffu, 0xffffu, lane, p.scale_log2e, acc[t]);
      }
    };
    PairFrag<ES, D> f0, f1;
    fetch(f0, 0);
    for (int i = 0; i < npair; i += 2) {
      fetch(f1, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(f0, i);
      if (i + 1 >= npair) break;
      fetch(f0, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(f1, i + 1);
    }
  }
  // The far blocks that straddle q - w for some query of the tile: masked
  // per slot position (a key is far for query q when its position is < q - w).
  for (int j = nfull; j < nfar; j += 2) {
    const int ba = blk_at(j, nfar - 1), bb = blk_at(j + 1, nfar - 1);
    PairFrag<ES, D> f;
    load_pair<ES, D, false>(f, p.pool + (int64_t)ba * p.block_bytes, p.pool + (int64_t)bb * p.block_bytes, lane);
    const int4 pa = *(const int4*)(p.blk_pos + (int64_t)ba * 16 + tb);
    const int4 pb = *(const int4*)(p.blk_pos + (int64_t)bb * 16 + tb);
    const int lva = n - 16 * j, lvb = j + 1 < nfar ? n - 16 * (j + 1) : 0;  // live slots
#pragma unroll
    for (int t = 0; t < NCOL; ++t) {
      const int lt = qc[t] - w;
      uint32_t ma = 0, mb = 0;
      const int xa[4] = {pa.x, pa.y, pa.z, pa.w}, xb[4] = {pb.x, pb.y, pb.z, pb.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (tb + r < lva && xa[r] < lt) ma |= 1u << (tb + r);
        if (tb + r < lvb && xb[r] < lt) mb |= 1u << (tb + r);
      }
      attend_pair_prompt<ES, D>(f, qf[t], ma, mb, lane, p.scale_log2e, acc[t]);
    }
  }

  // Near part: the dense rows within the window of the wave's own queries,
  // max(0, qw0 - w) .. qw1, 32 rows per softmax step.  (The work-group's whole
  // range, as one loop shared by the waves, took about 4 % longer on the
  // 32B-shaped layer; a second, mask-free softmax path for the pairs that all
  // of a tile's queries see took 18 % longer, its code and registers costing
  // more than the masks.)
  auto near_mask = [&](int r0, int t) -> uint32_t {
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = r0 + tb + r;
      if (pos <= qc[t] && pos >= qc[t] - w && pos < P) m |= 1u << (tb + r);
    }
    return m;
  };
  const int qw0 = q0 + 16 * NCOL * wave, qw1 = min(qw0 + 16 * NCOL - 1, qmax);
  for (int r0 = max(0, qw0 - w); r0 <= qw1; r0 += 32) {
    Frag<ES, D> fa, fb;
    load_frag_dense<ES, D>(fa, Ku, Vu, r0, P - 1, lane, zero_ch);
    load_frag_dense<ES, D>(fb, Ku, Vu, r0 + 16, P - 1, lane, zero_ch);
    PairFrag<ES, D> f;
    make_pair<ES, D>(f, fa, fb);
#pragma unroll
    for (int t = 0; t < NCOL; ++t)
      attend_pair_prompt<ES, D>(f, qf[t], near_mask(r0, t), near_mask(r0 + 16, t), lane, p.scale_log2e, acc[t]);
  }

#pragma unroll
  for (int t = 0; t < NCOL; ++t) {
    // each lane's l sums its own 4 keys of every block: add the 4 lane groups
    // of the column (all share the column's running max)
    float lt = acc[t].l + __shfl_xor(acc[t].l, 16);
    lt = lt + __shfl_xor(lt, 32);
    if (qc[t] >= P) continue;
    const float inv = 1.0f / lt;
    float* orow = out + (((int64_t)b * p.Hq + hq) * max_len + qc[t]) * D + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) *(f32x4*)(orow + 16 * j) = acc[t].o[j] * inv;
  }
}

// `chunk` consecutive tokens per unit, in order, as that many append_kernel
// launches would: k, v [U, chunk, d]; the logit of token j from `logit` at
// position j.
template <int ES, int D>
__global__ __launch_bounds__(256) void append_chunk_kernel(Dev p, const uint8_t* __restrict__ k,
                                                           const uint8_t* __restrict__ v, LogitSrc logit,
                                                           int zero_ch, int chunk) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int u = blockIdx.x * kWavesPerWG + wave;
  unsigned long long live = 0;
  if (u < p.U) {
    const int b = u / p.Hkv, h = u - b * p.Hkv;
    for (int j = 0; j < chunk; ++j) {
      const int64_t row = (int64_t)u * chunk + j;
      live += append_token<ES, D>(p, u, lane, k + row * D * ES, v + row * D * ES, load_logit(logit, b, h, j),
                                  zero_ch);
    }
  }
  add_live_token_steps(p, live);
}

// ---------------------------------------------------------------------------
// decode of a chunk of consecutive tokens: attention, then the appends
// ---------------------------------------------------------------------------

// Chunk query j (position q0 + j, q0 = the unit's length before the chunk)
// attends Vis(q0 + j), read before any token of the chunk is appended:
//  - every cached token that is not a pending marked one (an unmarked token
//    stays visible for good);
//  - a pending marked token (a slot held by the ring) while its position is
//    >= q0 + j - w;
//  - chunk row i <= j when it is unmarked or i >= j - w.
// Marked tokens that left the cache before the chunk are invisible to every
// chunk query too, so this is exactly the visible set of each step.  The
// pending slots come from the ring into a per-block bitmap in LDS: bit s of
// word i is slot 16 i + s, and bit 16 flags a block holding a pending token
// at a position below q0 + chunk - 1 - w, which some chunk query cannot see.
// A pair of full blocks without that flag is visible to every column whole,
// so its per-column masks are skipped (at most chunk such tokens exist,
// against thousands of blocks).
//
// Work-group = 4 waves = one (sequence, KV head) unit and up to 64 NC
// columns; column c = j G + g carries query head h G + g of chunk position j,
// so the group's heads share every loaded block as in the decode kernel.
constexpr int kChunkMaxBlocks = 8192;

// NC tiles of 16 columns per wave.  One work-group per (unit, group of 64 NC
// columns), ceil(chunk G / (64 NC)) groups per unit; grid 8 ceil(items / 8).
// q [B, Hq, chunk, d]; k, v [B, Hkv,
// chunk, d]; logit [B, Hkv, chunk]; out [B, Hq, chunk, d].
//
// The work-group's columns need 1 to 4 waves of NC tiles each.  When
// they fit in one or two waves, the idle waves split the key stream instead
// (4 or 2 ways: wave w takes every nsplit-th pair of blocks and of chunk
// rows), and the waves of one tile group merge their softmax states through
// LDS at the end, tile by tile.  CACHED: the cache blocks are loaded without
// the streaming hint (load_pair).
template <int ES, int D, int NC, bool CACHED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NC == 1 && ES == 2 ? 2 : 1))) void chunk_attention_kernel(Dev p, const uint8_t* __restrict__ q,
                                                              const uint8_t* __restrict__ k,
                                                              const uint8_t* __restrict__ v, LogitSrc logit,
                                                              int zero_ch, int chunk, float* __restrict__ out) {
  using G = Geo<ES, D>;
  __shared__ uint32_t pend[kChunkMaxBlocks];
  __shared__ f32x4 mo[kWavesPerWG - 1][G::kTiles][64];
  __shared__ float mm[kWavesPerWG - 1][64], ml[kWavesPerWG - 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Work item (unit, column group) of this work-group.  Work-group i runs on
  // XCD i mod 8; the items are dealt so that each XCD takes a run of
  // consecutive items: the column groups of a unit one after another (its
  // blocks are then re-read from that XCD's L2) and neighbouring units, whose
  // blocks the prefill allocated next to each other.  (Measured on the
  // 32B-shaped layer against one work-group per item in unit order: 1-5 %
  // faster for chunks of 4 to 64.)
  const int ytiles = (chunk * p.G + 64 * NC - 1) / (64 * NC);
  const int items = p.U * ytiles, per_xcd = (items + 7) / 8;
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (item >= items) return;  // before any barrier
  const int u = item / ytiles, ytile = item - u * ytiles;
  const int b = u / p.Hkv, h = u - b * p.Hkv;
  const int n = __builtin_amdgcn_readfirstlane(p.n[u]);
  const int nb = (n + 15) >> 4;
  const int q0 = __builtin_amdgcn_readfirstlane(p.pos[u]);
  const int w = p.R - 1;
  // the first and last block holding a pending token hidden from some column
  __shared__ int hid_lo, hid_hi;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) pend[i] = 0u;
  if (threadIdx.x == 0) {
    hid_lo = 1 << 30;
    hid_hi = -1;
  }
  __syncthreads();
  const int32_t* ring = p.ring + (int64_t)u * p.R;
  const int hide_lim = q0 + chunk - 1 - w;
  for (int r = threadIdx.x; r < p.R; r += blockDim.x) {
    const int sl = ring[r];
    if (sl >= 0 && sl < n) {
      const int blk = p.btab[(int64_t)u * p.max_blocks + (sl >> 4)];
      const int pos = p.blk_pos[(int64_t)blk * 16 + (sl & 15)];
      const bool hidden = pos < hide_lim;
      atomicOr(&pend[sl >> 4], (1u << (sl & 15)) | (hidden ? 0x10000u : 0u));
      if (hidden) {
        atomicMin(&hid_lo, sl >> 4);
        atomicMax(&hid_hi, sl >> 4);
      }
    }
  }
  __syncthreads();

  const int ncol = chunk * p.G;
  const int cwg = ytile * (16 * NC * kWavesPerWG);
  const int wg_cols = min((16 * NC * kWavesPerWG), ncol - cwg);
  const int need = (wg_cols + 16 * NC - 1) / (16 * NC);  // waves with columns
  const int nsplit = need == 1 ? 4 : (need == 2 ? 2 : 1);
  const int tg = wave / nsplit, sp = wave - tg * nsplit;
  if (tg >= need) return;  // only when nsplit == 1: no barrier follows for this work-group
  const int c0 = cwg + 16 * NC * tg;
  const int tb = 4 * (lane >> 4);
  int qj[NC], qg[NC];
  u32x4 qf[NC][G::kChunks];
  Acc<D> acc[NC];
#pragma unroll
  for (int t = 0; t < NC; ++t) {
    const int col = min(c0 + 16 * t + (lane & 15), ncol - 1);
    qj[t] = col / p.G;
    qg[t] = col - qj[t] * p.G;
    const uint8_t* qrow = q + (((int64_t)b * p.Hq + h * p.G + qg[t]) * chunk + qj[t]) * D * ES;
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) qf[t][c] = *(const u32x4*)(qrow + c * 64 + 16 * (lane >> 4));
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) acc[t].o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[t].m = -INFINITY;
    acc[t].l = 0.f;
  }

  // Cached tokens, in pairs of blocks.  The pairs of two full blocks with no
  // token hidden from any column ("plain": every key visible to every
  // column) go through their own loop and a softmax without masks; the rest
  // (every pair from the first to the last block holding a hidden token, a
  // short range near the tail of the cache, since pending tokens take the
  // tail's slots or slots freed by recent retirements; and a last pair that
  // is not two full blocks) through the masked one.  Each wave
  // takes every nsplit-th pair of each list, from its sp-th on.  (One loop
  // for both, the masks all ones for plain pairs: C = 16 0.359 -> 0.342 ms,
  // C = 64 1.101 -> 0.976 ms on the 32B-shaped layer with the split.)
  const int32_t* bt = p.btab + (int64_t)u * p.max_blocks;
  const int npair = (nb + 1) >> 1;
  const int plast = npair - ((n & 31) != 0 ? 1 : 0);  // pairs [0, plast) hold two full blocks
  const int hlo = __builtin_amdgcn_readfirstlane(hid_lo), hhi = __builtin_amdgcn_readfirstlane(hid_hi);
  const int mlo = hhi >= 0 ? min(hlo >> 1, plast) : plast;       // masked pairs [mlo, mhi) ...
  const int mhi = hhi >= 0 ? min((hhi >> 1) + 1, plast) : plast;  // ... and [plast, npair)
  const int nplain = plast - (mhi - mlo), nmasked = npair - nplain;
  auto load_blocks = [&](PairFrag<ES, D>& f, int i) {
    // The block ids through the scalar cache (an index the compiler can
    // see is uniform): a vector load here, its value needed at once for
    // the addresses, made the wave wait for every load in flight, the
    // prefetched pair's included (measured: C = 16 0.469 -> 0.408 ms).
    const int ja = 2 * i, jb = min(2 * i + 1, nb - 1);
    const int ba = scalar_load(bt + ja), bb = scalar_load(bt + jb);
    load_pair<ES, D, !CACHED>(f, p.pool + (int64_t)ba * p.block_bytes, p.pool + (int64_t)bb * p.block_bytes, lane);
    return int2{ba, bb};
  };
  const int cnt_plain = sp < nplain ? (nplain - sp + nsplit - 1) / nsplit : 0;
  if (cnt_plain > 0) {
    // plain pair kk of this wave: index sp + nsplit kk of the plain list
    auto pair_id = [&](int kk) {
      const int x = __builtin_amdgcn_readfirstlane(min(sp + nsplit * kk, nplain - 1));
      return x < mlo ? x : x + (mhi - mlo);
    };
    auto compute = [&](const PairFrag<ES, D>& f) {
      if constexpr (ES == 2) {
        // column t + 1's score products are issued before column t's softmax
        f32x4 SA[2], SB[2];
        score_pair<D>(f, qf[0], SA[0], SB[0]);
#pragma unroll
        for (int t = 0; t < NC; ++t) {
          if (t + 1 < NC) score_pair<D>(f, qf[t + 1], SA[(t + 1) & 1], SB[(t + 1) & 1]);
          softmax_pv_stale<D, true, false>(f, SA[t & 1], SB[t & 1], 0xffffu, 0xffffu, lane, p.scale_log2e, acc[t]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < NC; ++t) attend_pair<ES, D>(f, qf[t], 0xffffu, 0xffffu, lane, p.scale_log2e, acc[t]);
      }
    };
    // one pair loaded ahead of the one computed (the load past the wave's
    // last pair re-reads it and goes unused)
    PairFrag<ES, D> f0, f1;
    load_blocks(f0, pair_id(0));
    for (int kk = 0; kk < cnt_plain; kk += 2) {
      load_blocks(f1, pair_id(kk + 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(f0);
      if (kk + 1 >= cnt_plain) break;
      load_blocks(f0, pair_id(kk + 2));
      __builtin_amdgcn_sched_barrier(0);
      compute(f1);
    }
  }
  for (int x = sp; x < nmasked; x += nsplit) {
    const int i = x < mhi - mlo ? mlo + x : plast + (x - (mhi - mlo));
    PairFrag<ES, D> f;
    const int2 bl = load_blocks(f, i);
    const int4 pa = *(const int4*)(p.blk_pos + (int64_t)bl.x * 16 + tb);
    const int4 pb = *(const int4*)(p.blk_pos + (int64_t)bl.y * 16 + tb);
    const int ja = 2 * i;
    const uint32_t wa = pend[ja], wb = pend[min(ja + 1, nb - 1)];
    const int lva = n - 16 * ja, lvb = ja + 1 < nb ? n - 16 * (ja + 1) : 0;  // live slots
    const int xa[4] = {pa.x, pa.y, pa.z, pa.w}, xb[4] = {pb.x, pb.y, pb.z, pb.w};
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int lt = q0 + qj[t] - w;  // a pending token is visible from position >= lt
      uint32_t ma = 0, mb = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int bit = tb + r;
        if (bit < lva && (!((wa >> bit) & 1u) || xa[r] >= lt)) ma |= 1u << bit;
        if (bit < lvb && (!((wb >> bit) & 1u) || xb[r] >= lt)) mb |= 1u << bit;
      }
      if constexpr (ES == 2) {
        f32x4 SA, SB;
        score_pair<D>(f, qf[t], SA, SB);
        softmax_pv_stale<D, true>(f, SA, SB, ma, mb, lane, p.scale_log2e, acc[t]);
      } else {
        attend_pair<ES, D>(f, qf[t], ma, mb, lane, p.scale_log2e, acc[t]);
      }
    }
  }

  // The chunk's own rows, 32 per step, every nsplit-th step for this wave.
  const uint8_t* Ku = k + (int64_t)u * chunk * D * ES;
  const uint8_t* Vu = v + (int64_t)u * chunk * D * ES;
  for (int r0 = 32 * sp; r0 < chunk; r0 += 32 * nsplit) {
    Frag<ES, D> fa, fb;
    load_frag_dense<ES, D>(fa, Ku, Vu, r0, chunk - 1, lane, zero_ch);
    load_frag_dense<ES, D>(fb, Ku, Vu, r0 + 16, chunk - 1, lane, zero_ch);
    PairFrag<ES, D> f;
    make_pair<ES, D>(f, fa, fb);
    bool unmarked_a[4], unmarked_b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      unmarked_a[r] = !(load_logit(logit, b, h, min(r0 + tb + r, chunk - 1)) > 0.0f);
      unmarked_b[r] = !(load_logit(logit, b, h, min(r0 + 16 + tb + r, chunk - 1)) > 0.0f);
    }
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      uint32_t ma = 0, mb = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ia = r0 + tb + r, ib = r0 + 16 + tb + r;
        if (ia <= qj[t] && (unmarked_a[r] || ia >= qj[t] - w)) ma |= 1u << (tb + r);
        if (ib <= qj[t] && (unmarked_b[r] || ib >= qj[t] - w)) mb |= 1u << (tb + r);
      }
      attend_pair<ES, D>(f, qf[t], ma, mb, lane, p.scale_log2e, acc[t]);
    }
  }

  // Merge the split waves' states (per lane: same column, same lane group),
  // then normalise and write.  nsplit is uniform over the work-group, so every
  // wave takes the same barriers.
#pragma unroll
  for (int t = 0; t < NC; ++t) {
    if (nsplit > 1) {
      if (sp > 0) {
        const int slot = (tg * nsplit + sp) - tg - 1;  // the split waves' LDS slots: 0 .. 4 - need - 1
#pragma unroll
        for (int j = 0; j < G::kTiles; ++j) mo[slot][j][lane] = acc[t].o[j];
        mm[slot][lane] = acc[t].m;
        ml[slot][lane] = acc[t].l;
      }
      __syncthreads();
      if (sp == 0) {
        float M = acc[t].m;
        for (int x = 1; x < nsplit; ++x) M = fmaxf(M, mm[tg * (nsplit - 1) + x - 1][lane]);
        const float Mr = M == -INFINITY ? 0.f : M;
        const float w0 = exp2_fast(acc[t].m - Mr);
        float L = acc[t].l * w0;
#pragma unroll
        for (int j = 0; j < G::kTiles; ++j) acc[t].o[j] *= w0;
        for (int x = 1; x < nsplit; ++x) {
          const int slot = tg * (nsplit - 1) + x - 1;
          const float wx = exp2_fast(mm[slot][lane] - Mr);
          L += ml[slot][lane] * wx;
#pragma unroll
          for (int j = 0; j < G::kTiles; ++j) acc[t].o[j] += mo[slot][j][lane] * wx;
        }
        acc[t].l = L;
      }
      __syncthreads();
    }
    float lt = acc[t].l + __shfl_xor(acc[t].l, 16);
    lt = lt + __shfl_xor(lt, 32);
    if (sp != 0 || c0 + 16 * t + (lane & 15) >= ncol) continue;
    const float inv = 1.0f / lt;
    float* orow = out + (((int64_t)b * p.Hq + h * p.G + qg[t]) * chunk + qj[t]) * D + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) *(f32x4*)(orow + 16 * j) = acc[t].o[j] * inv;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <int ES, int D>
static hipError_t prefill_attention_t(const Dev& p, const void* q, const void* k, const void* v, int32_t max_len,
                                      int32_t max_prompt, int zero_ch, float* out, hipStream_t s) {
  constexpr int TILE = pf_tile<ES, D>();
  const dim3 grid((unsigned)((max_prompt + TILE - 1) / TILE), (unsigned)p.Hq, (unsigned)p.B);
  return launch(prefill_attention_kernel<ES, D>, grid, dim3(64 * kWavesPerWG), s, p, (const uint8_t*)q,
                (const uint8_t*)k, (const uint8_t*)v, max_len, zero_ch, out);
}

hipError_t launch_prefill_attention(const Dev& p, int dtype, int d, const void* q, const void* k, const void* v,
                                    int32_t max_len, int32_t max_prompt, int zero_ch, float* out, hipStream_t s) {
  if (max_prompt < 1) return hipSuccess;
  if (dtype == 1)
    return d == 128 ? prefill_attention_t<2, 128>(p, q, k, v, max_len, max_prompt, zero_ch, out, s)
                    : prefill_attention_t<2, 64>(p, q, k, v, max_len, max_prompt, zero_ch, out, s);
  return d == 128 ? prefill_attention_t<4, 128>(p, q, k, v, max_len, max_prompt, zero_ch, out, s)
                  : prefill_attention_t<4, 64>(p, q, k, v, max_len, max_prompt, zero_ch, out, s);
}

// Column tiles per wave of the chunk attention, by the chunk's tiles of 16
// columns (chunk x G): one tile when they fit in it (every wave then streams
// a quarter of the keys, and two work-groups stay resident per CU); as many
// tiles as the columns need, up to 4, so that no wave computes a padding
// tile and one wave holds every column of the pairs it loads; 3 beyond (5
// tiles at d = 128 spill).  Measured on the 32B-shaped layer (G = 5), against
// 3 tiles whenever more than one was needed: 2 tiles at C = 4 0.249 -> 0.237
// ms, 4 tiles at C = 12 0.383 -> 0.281 ms.  fp32 rows: two tiles at d = 128
// (three spill), three at d = 64.
template <int ES, int D>
constexpr int chunk_cols() {
  return ES == 4 && D == 128 ? 2 : 3;
}

template <int ES, int D, int NC, bool CACHED = false>
static hipError_t chunk_attention_t(const Dev& p, const void* q, const void* k, const void* v, const LogitSrc& logit,
                                    int zero_ch, int chunk, float* out, hipStream_t s) {
  const int ytiles = (chunk * p.G + 64 * NC - 1) / (64 * NC);
  const int items = p.U * ytiles;
  return launch(chunk_attention_kernel<ES, D, NC, CACHED>, dim3((unsigned)(8 * ((items + 7) / 8))), dim3(64 * kWavesPerWG), s,
                p, (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, logit, zero_ch, chunk, out);
}

template <int ES, int D>
static hipError_t decode_chunk_t(const Dev& p, const void* q, const void* k, const void* v, const LogitSrc& logit,
                                 int zero_ch, int chunk, float* out, hipStream_t s) {
  const int tiles = (chunk * p.G + 15) / 16;
  hipError_t e;
  if (tiles <= 1) e = chunk_attention_t<ES, D, 1>(p, q, k, v, logit, zero_ch, chunk, out, s);
  else if constexpr (ES == 4) e = chunk_attention_t<ES, D, chunk_cols<ES, D>()>(p, q, k, v, logit, zero_ch, chunk, out, s);
  else if (tiles == 2) e = chunk_attention_t<ES, D, 2>(p, q, k, v, logit, zero_ch, chunk, out, s);
  else if (tiles == 3) e = chunk_attention_t<ES, D, 3>(p, q, k, v, logit, zero_ch, chunk, out, s);
  else if (tiles == 4) e = chunk_attention_t<ES, D, 4>(p, q, k, v, logit, zero_ch, chunk, out, s);
  // two groups of three column tiles, each reading every pair of the
  // work-group's unit: plain loads (see load_pair)
  else if (tiles <= 6) e = chunk_attention_t<ES, D, 3, true>(p, q, k, v, logit, zero_ch, chunk, out, s);
  else e = chunk_attention_t<ES, D, 3>(p, q, k, v, logit, zero_ch, chunk, out, s);
  if (e != hipSuccess) return e;
  const int blocks = (p.U + kWavesPerWG - 1) / kWavesPerWG;
  return launch(append_chunk_kernel<ES, D>, dim3(blocks), dim3(64 * kWavesPerWG), s, p, (const uint8_t*)k,
                (const uint8_t*)v, logit, zero_ch, chunk);
}

hipError_t launch_decode_chunk(const Dev& p, int dtype, int d, const void* q, const void* k, const void* v,
                               const LogitSrc& logit, int zero_ch, int chunk, float* out, hipStream_t s) {
  if (dtype == 1)
    return d == 128 ? decode_chunk_t<2, 128>(p, q, k, v, logit, zero_ch, chunk, out, s)
                    : decode_chunk_t<2, 64>(p, q, k, v, logit, zero_ch, chunk, out, s);
  return d == 128 ? decode_chunk_t<4, 128>(p, q, k, v, logit, zero_ch, chunk, out, s)
                  : decode_chunk_t<4, 64>(p, q, k, v, logit, zero_ch, chunk, out, s);
}

int chunk_max_blocks() { return kChunkMaxBlocks; }

}  // namespace dms
