// The DMS decode path for gfx950 (MI355X): cache state, the append (decide,
// retire position q - w - 1, store), the prompt's compression, the decode
// attention over the visible tokens, the split merge, and the state export.
//
// Decode attention (attention_kernel): a persistent launch of 4-wave
// work-groups.  In whole-unit mode each work-group takes whole (sequence,
// KV head) units; in split mode every work-group takes an equal share of
// all live blocks, and the pieces of a cut unit are merged by reduce_kernel
// (log-sum-exp).  The decode step (dms_decode_step) runs the append inside
// the same launch in whole-unit mode, and inside the merge launch in split
// mode.
#include "dms_device.h"

namespace dms {
// ---------------------------------------------------------------------------
// state initialisation (create / reset)
// ---------------------------------------------------------------------------

__global__ void init_kernel(Dev p) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t nring = (int64_t)p.U * p.R;
  for (int64_t i = tid; i < nring; i += stride) p.ring[i] = -1;
  // whole-unit mode's default layout: work-group g takes units g, g + grid,
  // g + 2 grid, ... (its range of the unit order starts after the units of
  // the work-groups before it)
  const int per = p.U / p.grid, extra = p.U % p.grid;
  for (int64_t i = tid; i < p.U; i += stride) {
    p.n[i] = 0;
    p.pos[i] = 0;
    p.plan[2 * i] = 0;
    p.plan[2 * i + 1] = 0;
    const int g = (int)(i % p.grid), k = (int)(i / p.grid);
    p.order[g * per + min(g, extra) + k] = (int32_t)i;
  }
  for (int64_t g = tid; g <= p.grid; g += stride) p.wg_range[g] = (int32_t)(g * per + min<int64_t>(g, extra));
  for (int64_t g = tid; g < kMaxAttnWGs; g += stride) p.wg_live[g] = 0;
  if (tid == 0) {
    p.ctr->bump = 0;
    p.ctr->live_token_steps = 0;
    p.ctr->sticky_error = 0;
  }
}

// One token per (sequence, KV head): one wave per unit, 4 units per work-group.
template <int ES, int D>
__global__ __launch_bounds__(256) void append_kernel(Dev p, const uint8_t* __restrict__ k,
                                                     const uint8_t* __restrict__ v, LogitSrc logit,
                                                     int zero_ch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int u = blockIdx.x * kWavesPerWG + wave;
  unsigned live = 0;
  if (u < p.U)
    live = append_token<ES, D>(p, u, lane, k + (int64_t)u * D * ES, v + (int64_t)u * D * ES,
                               load_logit(logit, u / p.Hkv, u % p.Hkv, 0), zero_ch);
  add_live_token_steps(p, live);
}

// ---------------------------------------------------------------------------
// prefill compress
// ---------------------------------------------------------------------------

__device__ __forceinline__ int block_sum_1024(int x, int* s_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum_i(x);
  __syncthreads();
  if (lane == 0) s_tmp[wave] = x;
  __syncthreads();
  int t = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += s_tmp[i];
  return t;
}

// Prefill allocates in three launches, so that each unit's blocks are one
// contiguous run of the pool and the runs follow unit order: the attention
// streams many units at once, and runs at regularly spaced addresses spread
// its concurrent reads evenly over the memory channels (runs placed in
// arbitrary order were measured about 4 % slower).

// One work-group of 1024 threads per (sequence, KV head): n[u] = the tokens
// visible at the last prompt position.
__global__ __launch_bounds__(1024) void prefill_count_kernel(Dev p, LogitSrc logit, int32_t b0,
                                                             PromptLens lens) {
  __shared__ int s_tmp[16];
  const int u = b0 * p.Hkv + blockIdx.x;
  const int b = u / p.Hkv, h = u % p.Hkv;
  const int P = lens.v[blockIdx.x / p.Hkv];
  const int w = p.R - 1;
  int cnt = 0;
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    const bool alpha = load_logit(logit, b, h, i) > 0.0f;
    cnt += (!alpha || (P - 1 - i) <= w) ? 1 : 0;
  }
  const int n = block_sum_1024(cnt, s_tmp);
  if (threadIdx.x == 0) p.n[u] = n;
}

// One work-group of 1024 threads: base[u] = first pool block of unit u, an
// exclusive scan of the units' block counts in unit order after one atomic
// reservation of them all.  A unit whose run does not fit in the pool gets
// no blocks and no tokens, and sets the sticky error.
__global__ __launch_bounds__(1024) void prefill_alloc_kernel(Dev p, int32_t* __restrict__ base) {
  __shared__ long long s_sum[16];
  __shared__ int s_wave[16];
  __shared__ long long s_b0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  long long t = 0;
  for (int u = tid; u < p.U; u += blockDim.x) t += (p.n[u] + 15) >> 4;
  t = wave_sum_ll(t);
  if (lane == 0) s_sum[wave] = t;
  __syncthreads();
  if (tid == 0) {
    long long tot = 0;
    for (int i = 0; i < nw; ++i) tot += s_sum[i];
    s_b0 = tot > 0 ? (long long)atomicAdd(&p.ctr->bump, (unsigned long long)tot) : 0;
  }
  __syncthreads();
  long long running = s_b0;
  for (int c0 = 0; c0 < p.U; c0 += blockDim.x) {
    const int u = c0 + tid;
    const int nb = u < p.U ? (p.n[u] + 15) >> 4 : 0;
    const int incl = wave_incl_scan_i(nb, lane);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int i = 0; i < nw; ++i) {
      const int y = s_wave[i];
      if (i < wave) before += y;
      total += y;
    }
    const long long start = running + before + incl - nb;
    if (u < p.U) {
      if (start + nb > p.pool_blocks) {
        p.n[u] = 0;
        base[u] = 0;
        atomicCAS(&p.ctr->sticky_error, 0, kErrOutOfBlocks);
      } else {
        base[u] = (int32_t)start;
      }
    }
    running += total;
    __syncthreads();  // s_wave is reused by the next chunk
  }
}

// One work-group of 1024 threads per (sequence, KV head): assigns the
// visible tokens slots 0 .. n-1 in position order and fills block table,
// slot positions, masks and the pending-eviction ring.
__global__ __launch_bounds__(1024) void prefill_scan_kernel(Dev p, LogitSrc logit, int32_t b0,
                                                            PromptLens lens, const int32_t* __restrict__ bases) {
  __shared__ int s_wave_pre[16];
  const int u = b0 * p.Hkv + blockIdx.x;
  const int b = u / p.Hkv, h = u % p.Hkv;
  const int P = lens.v[blockIdx.x / p.Hkv];
  const int w = p.R - 1;
  int32_t* ring = p.ring + (int64_t)u * p.R;
  for (int i = threadIdx.x; i < p.R; i += blockDim.x) ring[i] = -1;
  const int n = p.n[u];
  const long long base = bases[u];
  const int nb = (n + 15) >> 4;
  int32_t* bt = p.btab + (int64_t)u * p.max_blocks;
  for (int j = threadIdx.x; j < nb; j += blockDim.x) {
    bt[j] = (int32_t)(base + j);
    const int fill = (j < nb - 1 || (n & 15) == 0) ? 16 : (n & 15);
    p.blk_mask[base + j] = (fill == 16) ? 0xffffu : ((1u << fill) - 1u);
  }
  if (n > 0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int running = 0;
    for (int i0 = 0; i0 < P; i0 += blockDim.x) {
      const int i = i0 + threadIdx.x;
      bool alpha = false;
      int vis = 0;
      if (i < P) {
        alpha = load_logit(logit, b, h, i) > 0.0f;
        vis = (!alpha || (P - 1 - i) <= w) ? 1 : 0;
      }
      const int incl = wave_incl_scan_i(vis, lane);
      __syncthreads();
      if (lane == 63) s_wave_pre[wave] = incl;
      __syncthreads();
      int before = 0, total = 0;
      for (int x = 0; x < nw; ++x) {
        const int y = s_wave_pre[x];
        if (x < wave) before += y;
        total += y;
      }
      if (vis) {
        const int slot = running + before + incl - 1;
        const int64_t blk = base + (slot >> 4);
        p.blk_pos[blk * 16 + (slot & 15)] = i;
        if (alpha) ring[i % p.R] = slot;  // marked and visible: eviction pending
      }
      running += total;
    }
  }
  if (threadIdx.x == 0) p.pos[u] = P;
}

// Gathers the visible rows of the dense prompt into the unit's blocks, in
// fragment order.  Grid (U, S); each wave handles whole blocks.
template <int ES, int D>
__global__ __launch_bounds__(256) void prefill_scatter_kernel(Dev p, const uint8_t* __restrict__ k,
                                                              const uint8_t* __restrict__ v,
                                                              int32_t max_len, int zero_ch) {
  using G = Geo<ES, D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int u = blockIdx.x;
  const int n = p.n[u];
  const int nb = (n + 15) >> 4;
  const int64_t row0 = (int64_t)u * max_len;
  const int32_t* bt = p.btab + (int64_t)u * p.max_blocks;
  for (int j = blockIdx.y * kWavesPerWG + wave; j < nb; j += gridDim.y * kWavesPerWG) {
    const int blk = bt[j];
    const uint32_t msk = p.blk_mask[blk];
    uint8_t* dst = p.pool + (int64_t)blk * p.block_bytes;
    const int32_t* bpos = p.blk_pos + (int64_t)blk * 16;
    // K: lane l carries token l % 16
    {
      const int t = lane & 15;
      const int sp = ((msk >> t) & 1u) ? bpos[t] : -1;
      const uint8_t* src = k + (row0 + (sp < 0 ? 0 : sp)) * D * ES;
#pragma unroll
      for (int c = 0; c < G::kChunks; ++c) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (sp >= 0) {
          val = *(const u32x4*)(src + (c * 4 * G::kE + G::kE * (lane >> 4)) * ES);
          clear_channel<ES>(val, c * 4 + (lane >> 4), zero_ch);
        }
        *(u32x4*)(dst + c * 1024 + lane * 16) = val;
      }
    }
    // V: lane l carries tokens 4*(l/16) + e
    {
      int sp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * (lane >> 4) + e;
        sp[e] = ((msk >> t) & 1u) ? bpos[t] : -1;
      }
#pragma unroll
      for (int c = 0; c < G::kChunks; ++c) {
        u32x4 val = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int jj = 0; jj < G::kNJ; ++jj) {
          const int ch = 16 * (c * G::kNJ + jj) + (lane & 15);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (sp[e] < 0) continue;
            const uint8_t* src = v + ((row0 + sp[e]) * D + ch) * ES;
            if constexpr (ES == 2) {
              const unsigned x = *(const uint16_t*)src;
              val[jj * 2 + (e >> 1)] |= x << (16 * (e & 1));
            } else {
              val[e] = *(const uint32_t*)src;
            }
          }
        }
        *(u32x4*)(dst + G::kHalf + c * 1024 + lane * 16) = val;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode attention
// ---------------------------------------------------------------------------

// A work item: plan blocks [jb, je) of one (sequence, KV head) unit, i.e. its
// logical blocks jb .. je - 1.  A unit with no live token counts one plan
// block and holds no real one, so that every unit belongs to some item.
struct Item {
  int u;          // the unit
  int nblk;       // the unit's blocks that hold live tokens
  int tail;       // live slots of the unit's last block, 0 when it is full
  int jb, je;     // plan blocks of the unit covered by this item
  int pidx;       // partial slot of the item, or -1 when it is the whole unit
  int plan_cnt;   // split mode, the unit's first item: the unit's item count, else 0
};

__device__ __forceinline__ uint32_t wave_incl_scan_u(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Split mode.  Every work-group derives the same plan from the live counts:
// unit u counts nb_u = max(1, ceil(n_u / 16)) plan blocks, the units' plan
// blocks lie end to end in unit order (P[u] = plan blocks of the units before
// u, P[U] = T), and work-group g of the R taking part takes plan blocks
// [floor(g T / R), floor((g + 1) T / R)).  Every work-group therefore streams
// the same number of blocks, within one, whatever compression ratio each
// head has reached.  Its items are the pieces of that range in each unit it
// meets.  An item that is not its whole unit leaves a partial in slot u + g:
// distinct pieces have distinct slots, and the pieces of one unit occupy
// consecutive slots, which reduce_kernel merges.  Every unit of a split call
// has its item count recorded by its first item (1 when it is not cut).
struct SplitPlan {
  uint32_t P[kPlanLdsUnits + 1];
  int32_t n[kPlanLdsUnits];
  uint32_t wsum[kWavesPerWG];
};

// Work-group-wide (256 threads); ends with a barrier.  n[] is read with
// coalesced loads (unit u by thread u % 256); thread t then scans the
// ceil(U / 256) consecutive units from t * ceil(U / 256) on.  The pool holds
// fewer than 2^31 blocks and U <= 4096, so T < 2^32.
__device__ void split_plan_build(const Dev& p, SplitPlan& pl) {
  constexpr int kThreads = 64 * kWavesPerWG;
  constexpr int kPer = kPlanLdsUnits / kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = p.U;
  // unconditional loads with clamped indices, so that all issue before the first wait
  int x[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) x[k] = p.n[min(tid + kThreads * k, U - 1)];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int u = tid + kThreads * k;
    if (u < U) pl.n[u] = x[k];
  }
  __syncthreads();
  const int per = (U + kThreads - 1) / kThreads;  // <= kPer
  const int u0 = tid * per;
  uint32_t nb[kPer];
  uint32_t s = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    nb[k] = (k < per && u0 + k < U) ? (uint32_t)max(1, (pl.n[u0 + k] + 15) >> 4) : 0u;
    s += nb[k];
  }
  const uint32_t incl = wave_incl_scan_u(s, lane);
  if (lane == 63) pl.wsum[wave] = incl;
  __syncthreads();
  uint32_t run = incl - s;
  for (int w = 0; w < wave; ++w) run += pl.wsum[w];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (k < per && u0 + k < U) pl.P[u0 + k] = run;
    run += nb[k];
  }
  if (tid == kThreads - 1) pl.P[U] = run;  // the last thread's running sum is the total
  __syncthreads();
}

// The last unit u with P[u] <= b (b < T), by a 64-way search (two rounds for
// 4096 units).  P is strictly increasing and P[0] = 0.
__device__ __forceinline__ int split_unit_at(const SplitPlan& pl, int U, uint32_t b, int lane) {
  int lo = 0, len = U;
  while (len > 64) {
    const int step = (len + 63) >> 6;
    const int off = lane * step;
    const unsigned long long bal = __ballot(off < len && pl.P[lo + off] <= b);  // bit 0 is always set
    const int k = 63 - __clzll((long long)bal);
    lo += k * step;
    len = min(step, len - k * step);
  }
  const unsigned long long bal = __ballot(lane < len && pl.P[lo + lane] <= b);
  return __builtin_amdgcn_readfirstlane(lo + 63 - __clzll((long long)bal));
}

// One work-group's share of a call: in split mode its range of plan blocks,
// in whole-unit mode its range of the unit order.
struct Share {
  int g;               // work-group index
  int R;               // split: work-groups taking part
  uint32_t T, b0, b1;  // split: total plan blocks, this work-group's [b0, b1)
  int u0;              // split: the unit holding plan block b0
  int w0, w1;          // whole-unit: the units order[w0 .. w1)
};

// The k-th item of a work-group in split mode; false past its range.
__device__ __forceinline__ bool split_item(const Dev& p, const SplitPlan& pl, const Share& s, int k, Item& it) {
  const int u = s.u0 + k;
  if (u >= p.U) return false;
  // readfirstlane: the compiler does not know an LDS value is uniform, and a
  // branch on it would make every item value a per-lane (vector) value
  const uint32_t pu = __builtin_amdgcn_readfirstlane(pl.P[u]);
  if (pu >= s.b1) return false;
  const uint32_t pe = __builtin_amdgcn_readfirstlane(pl.P[u + 1]);
  const int n = __builtin_amdgcn_readfirstlane(pl.n[u]);
  it.u = u;
  it.nblk = (n + 15) >> 4;
  it.tail = n & 15;
  it.jb = (int)(max(s.b0, pu) - pu);
  it.je = (int)(min(s.b1, pe) - pu);
  it.pidx = (it.jb == 0 && it.je == (int)(pe - pu)) ? -1 : u + s.g;
  // the work-group holding the unit's last plan block: the largest g with
  // floor(g T / R) <= pe - 1
  const int glast = (int)(((uint64_t)pe * (uint64_t)s.R - 1ull) / s.T);
  it.plan_cnt = it.jb == 0 ? glast - s.g + 1 : 0;
  return true;
}

// The eviction logit of unit (b, h) of a one-token step, as a scalar load of
// the aligned dword that holds it (an exact upcast for bf16).
__device__ __forceinline__ float scalar_logit(const LogitSrc& ls, int b, int h) {
  const int64_t e = (int64_t)b * ls.sb + (int64_t)h * ls.sh + ls.off;
  if (ls.bf16) {
    const int64_t byte = e * 2;
    const unsigned w = (unsigned)scalar_load((const int32_t*)((const uint8_t*)ls.base + (byte & ~(int64_t)3)));
    return __uint_as_float(((byte & 2) ? (w >> 16) : (w & 0xffffu)) << 16);
  }
  return __int_as_float(scalar_load((const int32_t*)ls.base + e));
}

// The k-th item of a work-group in whole-unit mode: a whole unit, the next
// of its range of the unit order; false past the range.
__device__ __forceinline__ bool whole_item(const Dev& p, const Share& s, int k, Item& it) {
  const int i = s.w0 + k;
  if (i >= s.w1) return false;
  const int u = scalar_load(p.order + i);
  const int n = scalar_load(p.n + u);
  it.u = u;
  it.nblk = (n + 15) >> 4;
  it.tail = n & 15;
  it.jb = 0;
  it.je = it.nblk;
  it.pidx = -1;
  it.plan_cnt = 0;
  return true;
}

// Decode attention.  A work item is a run of one (sequence, KV head)'s
// blocks, processed by one work-group of 4 waves: wave w takes the run's
// blocks w, w+4, w+8, ... so the work-group streams one contiguous run.  The
// waves' softmax states are merged through LDS; an item that is its whole
// unit writes the output there, otherwise the merged partial goes to
// reduce_kernel.
//
// The loads do not stop at item boundaries.  While a wave computes item A it
// already holds the block ids of its next item B, and the loads that run past
// A's last block fetch B's first two blocks; the LDS merge of A overlaps
// them.
//
// FUSED (the decode step in whole-unit mode): each work-group also appends
// the new token of every unit it owns.  The attention reads the cache as it
// was before the step, without the slot of the token that retires now, and
// takes the new token from the step's input rows; the append's stores land
// in slots no one reads during the launch.  So the visible set is the one
// after the append, Vis(q) = Vis(q - 1) - {q - w - 1 if marked} + {q}, with
// no ordering between work-groups.
template <int ES, int D, bool FUSED>
struct AttnShared {
  // staging buffers of the per-item inputs: the next item's are stored
  // while the current one streams.  The fused append reads the current
  // item's new row after the merge, so the rows have a third buffer that
  // keeps them from being overwritten meanwhile.
  static constexpr int kRowBufs = 3;
  static constexpr int kRowPieces = 2 * D * ES / 16;  // 16-byte pieces of the K row then the V row
  f32x4 o[kWavesPerWG][Geo<ES, D>::kTiles][64];
  float m[kWavesPerWG][16], l[kWavesPerWG][16];
  u32x4 q[2][Geo<ES, D>::kChunks][64];           // Q fragments
  u32x4 row[FUSED ? kRowBufs : 1][kRowPieces];  // the new token's K then V row (FUSED)
};

// One work item as one wave sees it.  Block ids are read through the scalar
// cache (waiting for a scalar load never waits for the vector loads in
// flight): the first two when the item is set up, one item ahead, and the
// rest inside the block loop, one iteration ahead.
struct WaveItem {
  int u;         // (sequence, KV head) unit
  int nblk;      // the unit's blocks
  int tail;      // live slots of the unit's last block, 0 when it is full
  int pidx;      // partial slot of the item, or -1 when it is the unit's only item
  int j0;        // the unit's logical block of this wave's block 0 (jb + wave)
  int cnt;       // this wave's blocks: the unit's blocks j0 + 4i, i < cnt
  int vs;        // visit stride: the wave's i-th load is its block (i * vs) mod cnt
  int pf0, pf1;  // pool ids of the first two blocks visited (pool block 0 if absent)
  int n;         // the unit's live slots before the step
  int first;     // 1 when the item begins at the unit's first block (it takes the new token when FUSED)
  // FUSED: the token appended to the unit (wave_item_step)
  int q;         // its position
  int rs;        // slot of position q - w - 1 if that token was marked (it retires now), else -1
  int rj;        // logical block of the retiring slot (masked out), else -1
  uint32_t rbit; // its bit in that block's mask
  int tblk;      // pool block of the slot the token goes to, -1 when it starts a new block
  int alpha;     // its eviction decision
};

__device__ __forceinline__ int padded3(int c) { return (c + 2) / 3 * 3; }

// Visit order.  Every work-group streams its runs at the same pace, so if
// the waves walked their blocks in address order, the addresses read at any
// moment would be the runs' start addresses shifted by a common offset: how
// evenly they spread over the memory channels would be fixed by where the
// runs happen to start, for the whole launch.  Walking each wave's blocks at
// a stride coprime to their count keeps those offsets changing (measured:
// about 4 % faster on prefilled caches, as fast as the best start layouts).
__device__ __forceinline__ int visit_stride(int cnt) {
  if (cnt <= 1) return 0;
  // the first of these primes that does not divide cnt (their product exceeds
  // any block count, so one always qualifies)
  constexpr int kPrimes[8] = {7, 11, 13, 17, 19, 23, 29, 31};
  int a = 37;
  for (int i = 7; i >= 0; --i)
    if (cnt % kPrimes[i]) a = kPrimes[i];
  return a % cnt;
}

// Position in the wave's block list of its i-th visit (i < cnt).  A unit
// holds at most 2^31 / 16 blocks (token counts are int32), a wave at most a
// quarter of them, so i * vs < 2^25 * 37 stays within 32 unsigned bits.
__device__ __forceinline__ int visit_pos(const WaveItem& w, int i) {
  return (int)((unsigned)i * (unsigned)w.vs % (unsigned)w.cnt);
}

// Pool id of this wave's i-th visited block, i clamped to cnt - 1 (cnt >= 1).
__device__ __forceinline__ int wave_item_id(const int32_t* __restrict__ btab, int max_blocks, const WaveItem& w,
                                            int i) {
  const int j = __builtin_amdgcn_readfirstlane(w.j0 + kWavesPerWG * visit_pos(w, min(i, w.cnt - 1)));
  return scalar_load(btab + (int64_t)w.u * max_blocks + j);
}

// Sets up item `it` for this wave; in split mode the first wave of a unit's
// first item also records the unit's item range for reduce_kernel.
__device__ __forceinline__ void wave_item_setup(const Dev& p, const int32_t* __restrict__ btab, int wave, int lane,
                                                const Item& it, WaveItem& w) {
  // readfirstlane: all of these are uniform, and must live in scalar
  // registers, or the block-id loads computed from them would be vector loads
  const int je = min(it.je, it.nblk);  // plan blocks past the live ones (an empty unit's) load nothing
  w.u = __builtin_amdgcn_readfirstlane(it.u);
  w.nblk = __builtin_amdgcn_readfirstlane(it.nblk);
  w.tail = __builtin_amdgcn_readfirstlane(it.tail);
  w.pidx = __builtin_amdgcn_readfirstlane(it.pidx);
  w.j0 = __builtin_amdgcn_readfirstlane(it.jb + wave);
  w.cnt = __builtin_amdgcn_readfirstlane(max(0, (je - it.jb - wave + kWavesPerWG - 1) / kWavesPerWG));
  w.vs = visit_stride(w.cnt);
  w.pf0 = w.cnt > 0 ? wave_item_id(btab, p.max_blocks, w, 0) : 0;
  w.pf1 = w.cnt > 1 ? wave_item_id(btab, p.max_blocks, w, 1) : 0;
  w.n = __builtin_amdgcn_readfirstlane(it.nblk > 0 ? (it.nblk - 1) * 16 + (it.tail ? it.tail : 16) : 0);
  w.first = __builtin_amdgcn_readfirstlane(it.jb == 0 ? 1 : 0);
  w.q = 0;
  w.rs = -1;
  w.rj = -1;
  w.rbit = 0;
  w.tblk = -1;
  w.alpha = 0;
  if (it.plan_cnt > 0 && wave == 0 && lane == 0) {
    p.plan[2 * it.u] = it.pidx < 0 ? 0 : it.pidx;
    p.plan[2 * it.u + 1] = it.plan_cnt;
  }
}

// An empty item on unit 0: stands for "no next item", so that the loads that
// would start the next item stay unconditional.
__device__ __forceinline__ void wave_item_none(WaveItem& w) {
  w.u = 0;
  w.nblk = 0;
  w.tail = 0;
  w.pidx = -1;
  w.j0 = 0;
  w.cnt = 0;
  w.vs = 0;
  w.pf0 = 0;
  w.pf1 = 0;
  w.n = 0;
  w.first = 0;
  w.q = 0;
  w.rs = -1;
  w.rj = -1;
  w.rbit = 0;
  w.tblk = -1;
  w.alpha = 0;
}

// FUSED: reads what the step's append to item w's unit needs: the new
// token's position q, the slot that retires with it (ring entry q mod R), the
// pool block of the slot the token goes to and its decision.  Each wave reads
// them one item ahead (the first item's after its first block loads are
// issued, so that those do not wait for this chain of dependent loads);
// only wave 0 of the work-group that owns the unit writes the unit's state,
// after every wave has passed a barrier that follows these reads.
__device__ __forceinline__ void wave_item_step(const Dev& p, const LogitSrc& logit, WaveItem& w) {
  w.q = scalar_load(p.pos + w.u);
  w.rs = scalar_load(p.ring + (int64_t)w.u * p.R + w.q % p.R);
  w.rj = w.rs >= 0 ? (w.rs >> 4) : -1;
  w.rbit = 1u << (w.rs & 15);
  const int slot = w.rs >= 0 ? w.rs : w.n;
  // the slot's block exists unless the token starts a new one
  w.tblk = (w.rs >= 0 || (w.n & 15) != 0) ? scalar_load(p.btab + (int64_t)w.u * p.max_blocks + (slot >> 4)) : -1;
  const int b = w.u / p.Hkv;
  w.alpha = scalar_logit(logit, b, w.u - b * p.Hkv) > 0.0f ? 1 : 0;  // NaN compares false
}

// Live-slot mask of this wave's i-th visited block of item w.  Live slots are
// always the dense prefix [0, n) of the unit's slots (an append reuses the
// slot it retires or takes slot n; prefill assigns 0 .. n-1), so only the
// unit's last block can be partly filled.  FUSED: the retiring slot is
// masked out as well.
template <bool FUSED>
__device__ __forceinline__ uint32_t wave_item_mask(const WaveItem& w, int i) {
  const int j = w.j0 + kWavesPerWG * visit_pos(w, i);
  uint32_t m = (j == w.nblk - 1 && w.tail != 0) ? ((1u << w.tail) - 1u) : 0xffffu;
  if constexpr (FUSED) m &= (j == w.rj) ? ~w.rbit : 0xffffffffu;
  return m;
}

// Per-item inputs, staged through LDS: wave w loads chunks w, w+4, ... of the
// next item's Q fragment (B operand of S = K Q^T: head g = lane % 16 of the
// item's group, the channels this lane's K fragment elements carry) while
// the current item streams, and, when FUSED, the pieces of the new token's
// K and V rows.  The pieces are stored before the merge and read after it.
// No wait for a K/V load is ever also a wait for these, nor the other way
// round.
template <int ES, int D, bool FUSED>
struct QPart {
  static constexpr int kN = (Geo<ES, D>::kChunks + kWavesPerWG - 1) / kWavesPerWG;
  u32x4 v[kN];
  u32x4 row;  // FUSED: piece min(lane, kRowPieces - 1) of the new K row then V row
};

template <int ES, int D, bool FUSED>
__device__ __forceinline__ void load_q_part(const Dev& p, const uint8_t* __restrict__ q, const StepIn& in, int u,
                                            int lane, int wave, QPart<ES, D, FUSED>& part) {
  using G = Geo<ES, D>;
  const int b = u / p.Hkv, h = u - b * p.Hkv;
  const int g = lane & 15;
  // Columns g >= G (unused heads) load head 0 of the group: every column is
  // an independent softmax, and those columns are never written out.
  const uint8_t* qrow = q + ((int64_t)b * p.Hq + h * p.G + (g < p.G ? g : 0)) * D * ES;
#pragma unroll
  for (int j = 0; j < QPart<ES, D, FUSED>::kN; ++j) {
    const int c = min(wave + kWavesPerWG * j, G::kChunks - 1);
    part.v[j] = *(const u32x4*)(qrow + (c * 4 * G::kE + G::kE * (lane >> 4)) * ES);
  }
  if constexpr (FUSED) {
    constexpr int kRowPieces = AttnShared<ES, D, FUSED>::kRowPieces;
    constexpr int kHalf = kRowPieces / 2;
    const int r = min(lane, kRowPieces - 1);
    const uint8_t* src = r < kHalf ? in.k + (int64_t)u * D * ES + r * 16 : in.v + (int64_t)u * D * ES + (r - kHalf) * 16;
    part.row = *(const u32x4*)src;  // the key channel is cleared when stored (store_q_part)
  }
}

template <int ES, int D, bool FUSED>
__device__ __forceinline__ void store_q_part(AttnShared<ES, D, FUSED>& sh, int buf, int rbuf, int lane, int wave,
                                             const QPart<ES, D, FUSED>& part, int zero_ch) {
  // Clamped like the load: waves past the last chunk store that chunk again,
  // with the same values (an unconditional store keeps the load waits exact).
#pragma unroll
  for (int j = 0; j < QPart<ES, D, FUSED>::kN; ++j)
    sh.q[buf][min(wave + kWavesPerWG * j, Geo<ES, D>::kChunks - 1)][lane] = part.v[j];
  if constexpr (FUSED) {
    // every wave stores the same row pieces; the key row with channel
    // zero_ch cleared (here, where the loaded value is consumed anyway: a
    // change of it right after its load would wait for every load before it)
    constexpr int kRowPieces = AttnShared<ES, D, FUSED>::kRowPieces;
    const int r = min(lane, kRowPieces - 1);
    u32x4 v = part.row;
    if (r < kRowPieces / 2) clear_channel<ES>(v, r, zero_ch);
    sh.row[rbuf][r] = v;
  }
}

template <int ES, int D, bool FUSED>
__device__ __forceinline__ void read_q(const AttnShared<ES, D, FUSED>& sh, int buf, int lane,
                                       u32x4 (&qf)[Geo<ES, D>::kChunks]) {
#pragma unroll
  for (int c = 0; c < Geo<ES, D>::kChunks; ++c) qf[c] = sh.q[buf][c][lane];
}

__device__ __forceinline__ float sum_over_groups(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Raw score <q_g, k_new> of the new token for head g = lane % 16 (every lane
// of the head gets it): each lane multiplies the channels of its Q fragment
// with the same channels of the staged K row, then the four lane groups add.
template <int ES, int D>
__device__ __forceinline__ float new_token_score(const u32x4* krow, const u32x4 (&qf)[Geo<ES, D>::kChunks],
                                                 int lane) {
  using G = Geo<ES, D>;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    const u32x4 kk = krow[c * 4 + (lane >> 4)];  // channels c * 4E + E * (lane / 16) + e
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (ES == 2) {
        acc = fmaf(bf16_lo_to_f32(qf[c][e]), bf16_lo_to_f32(kk[e]), acc);
        acc = fmaf(bf16_hi_to_f32(qf[c][e]), bf16_hi_to_f32(kk[e]), acc);
      } else {
        acc = fmaf(__uint_as_float(qf[c][e]), __uint_as_float(kk[e]), acc);
      }
    }
  }
  return sum_over_groups(acc);
}

// Channels 16 j + 4 (lane / 16) + r (r < 4) of the staged V row, as fp32.
template <int ES, int D>
__device__ __forceinline__ f32x4 new_token_values(const u32x4* vrow_pieces, int j, int lane) {
  const uint8_t* vrow = (const uint8_t*)vrow_pieces;
  const int ch = 16 * j + 4 * (lane >> 4);
  if constexpr (ES == 2) {
    const u32x2 w = *(const u32x2*)(vrow + ch * 2);
    return f32x4{bf16_lo_to_f32(w[0]), bf16_hi_to_f32(w[0]), bf16_lo_to_f32(w[1]), bf16_hi_to_f32(w[1])};
  } else {
    return *(const f32x4*)(vrow + ch * 4);
  }
}

// Computes this wave's blocks of item A.  The wave reads one stream of
// blocks: A's, each item padded to a multiple of three blocks, then B's.
// The three buffers rotate, so with the padding every item starts with its
// blocks 0 and 1 in buffers 0 and 1, and ends with B's blocks 0 and 1 loading
// there.  Padding slots, and stream positions past B, load pool block 0 (any
// valid address does) and are not computed.  When A has no blocks, buffers 0
// and 1 were filled before B was known and are loaded again here.
template <int ES, int D, bool FUSED, typename Early>
__device__ __forceinline__ void run_item(const Dev& p, Frag<ES, D>& f0, Frag<ES, D>& f1, Frag<ES, D>& f2,
                                         const WaveItem& A, const WaveItem& B,
                                         const u32x4 (&qf)[Geo<ES, D>::kChunks], int lane, Acc<D>& acc,
                                         Early&& early) {
#pragma unroll
  for (int j = 0; j < Geo<ES, D>::kTiles; ++j) acc.o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc.m = -INFINITY;
  acc.l = 0.f;
  const uint8_t* pool = p.pool;
  const int64_t BB = p.block_bytes;
  const float sl2e = p.scale_log2e;
  const int cnt = A.cnt, cpad = padded3(A.cnt);
  // Pool id of stream position s, given the id `own` of A's block s when s < cnt.
  auto stream_id = [&](int s, int own) { return s < cnt ? own : (s == cpad ? B.pf0 : (s == cpad + 1 ? B.pf1 : 0)); };
  const int32_t* __restrict__ btab = p.btab;
  auto fetch = [&](Frag<ES, D>& fr, int blk) { load_frag<ES, D>(fr, pool + (int64_t)blk * BB, lane); };
  // A's ids of the blocks fetched next (scalar-cache hits: the same lines as
  // blocks 0 and 1)
  int n2 = 0, n3 = 0, n4 = 0;
  if (cnt > 0) {
    n2 = wave_item_id(btab, p.max_blocks, A, 2);
    n3 = wave_item_id(btab, p.max_blocks, A, 3);
    n4 = wave_item_id(btab, p.max_blocks, A, 4);
  }
  // Blocks i, i+1, i+2 (i a multiple of 3 below cpad, so block i is one of A's).
  auto body = [&](int i) {
    const int b2 = stream_id(i + 2, n2), b3 = stream_id(i + 3, n3), b4 = stream_id(i + 4, n4);
    if (i + 5 < cnt) {  // the next iteration's ids
      n2 = wave_item_id(btab, p.max_blocks, A, i + 5);
      n3 = wave_item_id(btab, p.max_blocks, A, i + 6);
      n4 = wave_item_id(btab, p.max_blocks, A, i + 7);
    }
    fetch(f2, b2);
    attend_block<ES, D>(f0, qf, wave_item_mask<FUSED>(A, i), lane, sl2e, acc);
    fetch(f0, b3);
    if (i + 1 < cnt) attend_block<ES, D>(f1, qf, wave_item_mask<FUSED>(A, i + 1), lane, sl2e, acc);
    fetch(f1, b4);
    if (i + 2 < cnt) attend_block<ES, D>(f2, qf, wave_item_mask<FUSED>(A, i + 2), lane, sl2e, acc);
  };
  // The first group is peeled: it is the one that waits for the item's Q
  // (loaded after blocks 0 and 1), and keeping that wait out of the loop
  // keeps the loop's own load waits exact.
  // `early` consumes values loaded before this function: it runs right after
  // the first group of loads, where the compiler counts the loads issued
  // since exactly (after a loop it would assume none and wait for all).
  if (cpad == 0) {
    fetch(f0, B.pf0);
    fetch(f1, B.pf1);
    early();
  } else {
    body(0);
    early();
    for (int i = 3; i < cpad; i += 3) body(i);
  }
}

// Merges the four waves' states of item `it` through LDS and writes the
// output (an item that is its whole unit) or the item's partial.  FUSED: the
// new token (staged in row buffer `buf`) joins the merge as one more key.
// Contains two work-group barriers; LDS stores made before the call (the next
// item's staged inputs) are visible to every wave on return.
template <int ES, int D, bool FUSED>
__device__ __forceinline__ void merge_item(const Dev& p, float* __restrict__ out, const WaveItem& it,
                                           const Acc<D>& acc, int lane, int wave, AttnShared<ES, D, FUSED>& sh,
                                           int buf, const u32x4 (&qf)[Geo<ES, D>::kChunks]) {
  using G = Geo<ES, D>;
  constexpr int kW = kWavesPerWG;
  constexpr int kTilesPerWave = (G::kTiles + kW - 1) / kW;
  if (!FUSED && it.nblk == 0) {  // a unit with no live token (uniform): nothing to write
    __syncthreads();             // but the next item's Q must still be visible on return
    return;
  }
  const int u = it.u;
  const int b = u / p.Hkv, h = u - b * p.Hkv;
  const int g = lane & 15;
  const bool gvalid = g < p.G;
  const int hq = h * p.G + g;

  // lane-local l holds 4 of the 16 tokens per block; add the four groups
  float lt = acc.l + __shfl_xor(acc.l, 16);
  lt = lt + __shfl_xor(lt, 32);
  if (lane < 16) {
    sh.m[wave][lane] = acc.m;
    sh.l[wave][lane] = lt;
  }
#pragma unroll
  for (int j = 0; j < G::kTiles; ++j) sh.o[wave][j][lane] = acc.o[j];
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kW; ++w) M = fmaxf(M, sh.m[w][g]);
  // wave w finishes tiles w * kTilesPerWave ...
  const int j0 = wave * kTilesPerWave;
  float sn = -INFINITY;  // the new token's score: only the unit's first item takes it
  if constexpr (FUSED) {
    if (it.first) {
      sn = new_token_score<ES, D>(&sh.row[buf][0], qf, lane) * p.scale_log2e;
      M = fmaxf(M, sn);
    }
  }
  const float Mr = (M == -INFINITY) ? 0.f : M;
  float wt[kW];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    wt[w] = exp2_fast(sh.m[w][g] - Mr);
    L += wt[w] * sh.l[w][g];
  }
  f32x4 O[kTilesPerWave];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (j0 + t < G::kTiles) {
#pragma unroll
      for (int w = 0; w < kW; ++w) O[t] += wt[w] * sh.o[w][j0 + t][lane];
    }
  }
  if constexpr (FUSED) {
    const float wn = exp2_fast(sn - Mr);  // 0 for an item without the new token
    L += wn;
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t)
      if (j0 + t < G::kTiles)
        O[t] += wn * new_token_values<ES, D>(&sh.row[buf][AttnShared<ES, D, FUSED>::kRowPieces / 2], j0 + t, lane);
  }
  __syncthreads();  // the LDS of this item may be overwritten after this
  if (it.pidx < 0) {
    if (gvalid) {
      float* orow = out + ((int64_t)b * p.Hq + hq) * D + 4 * (lane >> 4);
      const float inv = 1.0f / L;
#pragma unroll
      for (int t = 0; t < kTilesPerWave; ++t)
        if (j0 + t < G::kTiles) *(f32x4*)(orow + 16 * (j0 + t)) = O[t] * inv;
    }
    return;
  }
  // several items: publish the merged partial; reduce_kernel combines them
  const int IF = p.item_floats;
  float* mine = p.part + (int64_t)it.pidx * IF;
  if (gvalid) {
    if (wave == 0 && lane < 16) {
      mine[g] = M;
      mine[16 + g] = L;
    }
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t)
      if (j0 + t < G::kTiles) *(f32x4*)(mine + 32 + g * D + 16 * (j0 + t) + 4 * (lane >> 4)) = O[t];
  }
}

// Persistent launch: one work-group per resident slot.  Whole-unit mode:
// work-group g takes the units of its range of the unit order, each as one
// item (the host deals the units so that the ranges carry about equal live
// blocks).  Split mode: it takes its equal share of all plan blocks, cut at
// unit boundaries (SplitPlan).  Either way each work-group knows its next item
// in advance: its block ids are read while the item before it is computed.
//
// The loop is written so that the compiler's load-counter waits stay exact:
// every load is unconditional (an absent next item is an empty one on unit
// 0), block ids come through the scalar cache, and values loaded before an
// item's block loop are consumed right after its first group of loads.  A
// wait for one value then never drains the K/V blocks in flight behind it.
// What an attention launch does: kAttend, the attention alone (whole units
// or split, as p.split says); kStepWhole, a decode step in whole-unit mode
// (the append inside); kStepSplit, a decode step in split mode (reduce_kernel
// appends).  The whole-unit step carries no split plan.
constexpr int kAttend = 0, kStepWhole = 1, kStepSplit = 2;

template <int ES, int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ES == 2 ? 2 : 1))) void attention_kernel(
    Dev p, const int32_t* __restrict__ btab, const uint8_t* __restrict__ q, float* __restrict__ out, StepIn in) {
  using G = Geo<ES, D>;
  constexpr bool FUSED = MODE != kAttend;
  __shared__ AttnShared<ES, D, FUSED> sh;
  __shared__ typename std::conditional<MODE == kStepWhole, int, SplitPlan>::type pl;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Share s;
  s.g = blockIdx.x;
  s.R = 1;
  s.T = 1;
  s.b0 = 0;
  s.b1 = 0;
  s.u0 = 0;
  s.w0 = 0;
  s.w1 = 0;
  const bool split = MODE == kStepSplit || (MODE == kAttend && p.split != 0);
  if constexpr (MODE != kStepWhole) {
    if (split) {
      split_plan_build(p, pl);
      const uint32_t T = __builtin_amdgcn_readfirstlane(pl.P[p.U]);
      const int R = (int)min((uint32_t)p.split_wgs, (T + kMinSplitBlocks - 1) / kMinSplitBlocks);
      if (s.g >= R) return;  // uniform over the work-group
      s.R = R;
      s.T = T;
      s.b0 = (uint32_t)((uint64_t)s.g * T / (uint64_t)R);
      s.b1 = (uint32_t)((uint64_t)(s.g + 1) * T / (uint64_t)R);
      s.u0 = split_unit_at(pl, p.U, s.b0, lane);
    }
  }
  if (!split) {
    s.w0 = scalar_load(p.wg_range + s.g);
    s.w1 = scalar_load(p.wg_range + s.g + 1);
  }
  auto find_item = [&](int k, Item& it) -> bool {
    if constexpr (MODE != kStepWhole) {
      if (split) return split_item(p, pl, s, k, it);
    }
    return whole_item(p, s, k, it);
  };

  int k = 0;
  WaveItem W0, W1;
  QPart<ES, D, FUSED> q0;
  {
    Item it;
    if (!find_item(k, it)) return;  // uniform over the work-group
    // Q first: it is stored to LDS below, and a wait for it must not also
    // wait for the first blocks (loads complete in issue order)
    load_q_part<ES, D, FUSED>(p, q, in, it.u, lane, wave, q0);
    wave_item_setup(p, btab, wave, lane, it, W0);
  }
  bool has_next;
  {
    Item it;
    has_next = find_item(k + 1, it);
    if (has_next)
      wave_item_setup(p, btab, wave, lane, it, W1);
    else
      wave_item_none(W1);
  }
  Frag<ES, D> f0, f1, f2;
  load_frag<ES, D>(f0, p.pool + (int64_t)W0.pf0 * p.block_bytes, lane);
  load_frag<ES, D>(f1, p.pool + (int64_t)W0.pf1 * p.block_bytes, lane);
  unsigned long long live = 0;  // FUSED: live tokens after this work-group's appends (wave 0)
  if constexpr (FUSED) {
    // after the first block loads: their addresses do not depend on these
    __builtin_amdgcn_sched_barrier(0);
    wave_item_step(p, in.logit, W0);
    if (has_next) wave_item_step(p, in.logit, W1);
    // this work-group's running sum of live tokens, continued below
    live = (unsigned long long)(uint32_t)scalar_load((const int32_t*)(p.wg_live + s.g)) |
           ((unsigned long long)(uint32_t)scalar_load((const int32_t*)(p.wg_live + s.g) + 1) << 32);
  }
  store_q_part<ES, D, FUSED>(sh, 0, 0, lane, wave, q0, in.zero_ch);
  __syncthreads();
  u32x4 qf[G::kChunks];
  read_q<ES, D, FUSED>(sh, 0, lane, qf);
  int qbuf = 0, rbuf = 0;  // staging buffers of the current item (Q: 2, rows: 3)

  // W0 is the item being computed, W1 the next one (both held in scalar
  // registers, so moving W1 into W0 waits for no load).
  for (;;) {
    const int nrbuf = rbuf + 1 == AttnShared<ES, D, FUSED>::kRowBufs ? 0 : rbuf + 1;
    QPart<ES, D, FUSED> qn;
    load_q_part<ES, D, FUSED>(p, q, in, W1.u, lane, wave, qn);  // W1's inputs, stored to LDS early in W0's block loop
    Acc<D> acc;  // set by run_item
    run_item<ES, D, FUSED>(p, f0, f1, f2, W0, W1, qf, lane, acc, [&]() {
      store_q_part<ES, D, FUSED>(sh, qbuf ^ 1, nrbuf, lane, wave, qn, in.zero_ch);
    });
    merge_item<ES, D, FUSED>(p, out, W0, acc, lane, wave, sh, rbuf, qf);
    if constexpr (FUSED) {
      // The append, by wave 0 after the merge: the new row (staged in row
      // buffer rbuf, which the staging of the next two items leaves alone) goes to a
      // slot this launch never reads, the retiring one (masked) or slot n
      // (past the live prefix).  (Done inside the block stream instead, right
      // after the item's first blocks, the call took 197 against 191 us.)
      // In split mode several work-groups read a unit's state, so the split
      // merge that follows appends instead.
      if (MODE == kStepWhole && wave == 0) {
        const uint8_t* krow = (const uint8_t*)&sh.row[rbuf][0];
        live += store_token<ES, D>(p, W0.u, lane, krow, krow + D * ES, W0.alpha != 0, W0.q, W0.rs, W0.n,
                                   W0.tblk, -1);
      }
    }
    if (!has_next) break;
    qbuf ^= 1;
    rbuf = nrbuf;
    read_q<ES, D, FUSED>(sh, qbuf, lane, qf);
    W0 = W1;
    ++k;
    Item it;
    has_next = find_item(k + 1, it);
    if (has_next) {
      wave_item_setup(p, btab, wave, lane, it, W1);
      if constexpr (FUSED) wave_item_step(p, in.logit, W1);
    } else {
      wave_item_none(W1);
    }
  }
  if constexpr (FUSED) {
    // one slot per work-group, written only by it: no contended atomic
    if (wave == 0 && lane == 0) p.wg_live[s.g] = live;
  }
}

// Split merge: one wave per (sequence, KV head) whose attention was split
// into several work items; merges their (m, l, o) partials by log-sum-exp,
//   M = max_s m_s,  L = sum_s 2^(m_s - M) l_s,  o = sum_s 2^(m_s - M) o_s / L,
// in one online pass: the partials are loaded four items at a time (all
// loads of a group before any use), each group's max updates M and rescales
// what was summed so far.  Lane l handles head l % 16 and the channels
// 16j + 4(l/16) + r.
template <int D>
__device__ __forceinline__ void merge_partials(const Dev& p, int u, int lane, float* __restrict__ out) {
  const int base = p.plan[2 * u], items = p.plan[2 * u + 1];
  const int g = lane & 15;
  if (items <= 1 || g >= p.G) return;
  constexpr int kJ = D / 16, kU = 4;
  const int IF = p.item_floats;
  const float* pb = p.part + (int64_t)base * IF;
  const int c0 = 4 * (lane >> 4);
  float M = -INFINITY, L = 0.f;
  f32x4 O[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < items; s0 += kU) {
    float ms[kU], ls[kU];
    f32x4 os[kU][kJ];
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const float* ps = pb + (int64_t)min(s0 + k, items - 1) * IF;  // clamped: past the end weighs 0
      ms[k] = ps[g];
      ls[k] = ps[16 + g];
#pragma unroll
      for (int j = 0; j < kJ; ++j) os[k][j] = *(const f32x4*)(ps + 32 + g * D + 16 * j + c0);
    }
    float mg = -INFINITY;
#pragma unroll
    for (int k = 0; k < kU; ++k)
      if (s0 + k < items) mg = fmaxf(mg, ms[k]);
    const float Mn = fmaxf(M, mg);
    const float Mr = (Mn == -INFINITY) ? 0.f : Mn;
    const float a = exp2_fast(M - Mr);  // 0 before the first finite max
    L *= a;
#pragma unroll
    for (int j = 0; j < kJ; ++j) O[j] *= a;
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const float w = (s0 + k < items) ? exp2_fast(ms[k] - Mr) : 0.f;
      L += w * ls[k];
#pragma unroll
      for (int j = 0; j < kJ; ++j) O[j] += w * os[k][j];
    }
    M = Mn;
  }
  const int b = u / p.Hkv, h = u - b * p.Hkv;
  const float inv = 1.0f / L;
  float* orow = out + ((int64_t)b * p.Hq + h * p.G + g) * D + c0;
#pragma unroll
  for (int j = 0; j < kJ; ++j) *(f32x4*)(orow + 16 * j) = O[j] * inv;
}

// After a split attention: one wave per (sequence, KV head) merges its
// partials (when it was cut).  STEP (a decode step in split mode): a second
// wave per unit appends the unit's new token, which the attention has
// already taken from the step's input rows; the unit's state is written only
// now, so every work-group of the attention read the state from before the
// step.  The merge and the append touch disjoint data, so their chains of
// dependent loads run side by side in the two waves.
template <int ES, int D, bool STEP>
__global__ __launch_bounds__(256) void reduce_kernel(Dev p, float* __restrict__ out, StepIn in) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kUnitsPerWG = STEP ? kWavesPerWG / 2 : kWavesPerWG;
  const int u = blockIdx.x * kUnitsPerWG + (STEP ? (wave >> 1) : wave);
  unsigned long long live = 0;
  if (u < p.U) {
    if (!STEP || (wave & 1) == 0) {
      merge_partials<D>(p, u, lane, out);
    } else {
      const int b = u / p.Hkv;
      live = append_token<ES, D>(p, u, lane, in.k + (int64_t)u * D * ES, in.v + (int64_t)u * D * ES,
                                 load_logit(in.logit, b, u - b * p.Hkv, 0), in.zero_ch);
    }
  }
  if constexpr (STEP) add_live_token_steps(p, live);
}

// ---------------------------------------------------------------------------
// export: slot -> position of units [u0, u0 + count) into a staging area
// ---------------------------------------------------------------------------

// Flat index f = (u - u0) * max_tokens + slot, for f in [f0, f0 + len).
__global__ void export_kernel(Dev p, int32_t u0, int64_t f0, int64_t len, int32_t* __restrict__ stage) {
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < len; k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = f0 + k;
    const int iu = (int)(i / p.max_tokens);
    const int slot = (int)(i - (int64_t)iu * p.max_tokens);
    const int u = u0 + iu;
    int32_t val = -1;
    if (slot < p.n[u]) {
      const int blk = p.btab[(int64_t)u * p.max_blocks + (slot >> 4)];
      if ((p.blk_mask[blk] >> (slot & 15)) & 1u) val = p.blk_pos[(int64_t)blk * 16 + (slot & 15)];
    }
    stage[k] = val;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_init(const Dev& p, hipStream_t s) {
  const int64_t work = std::max<int64_t>((int64_t)p.U * p.R, p.U);
  const int threads = 256;
  const int blocks = (int)std::min<int64_t>((work + threads - 1) / threads, 4096);
  return launch(init_kernel, dim3(std::max(blocks, 1)), dim3(threads), s, p);
}

hipError_t launch_export(const Dev& p, int32_t u0, int64_t f0, int64_t len, int32_t* stage, hipStream_t s) {
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((len + 255) / 256, 8192));
  return launch(export_kernel, dim3(blocks), dim3(256), s, p, u0, f0, len, stage);
}

template <int ES, int D>
static hipError_t append_t(const Dev& p, const void* k, const void* v, const LogitSrc& logit, int zero_ch,
                           hipStream_t s) {
  const int blocks = (p.U + kWavesPerWG - 1) / kWavesPerWG;
  return launch(append_kernel<ES, D>, dim3(blocks), dim3(64 * kWavesPerWG), s, p, (const uint8_t*)k,
                (const uint8_t*)v, logit, zero_ch);
}

hipError_t launch_append(const Dev& p, int dtype, int d, const void* k, const void* v,
                         const LogitSrc& logit, int zero_ch, hipStream_t s) {
  if (dtype == 1)
    return d == 128 ? append_t<2, 128>(p, k, v, logit, zero_ch, s) : append_t<2, 64>(p, k, v, logit, zero_ch, s);
  return d == 128 ? append_t<4, 128>(p, k, v, logit, zero_ch, s) : append_t<4, 64>(p, k, v, logit, zero_ch, s);
}

template <int ES, int D>
static hipError_t prefill_t(const Dev& p, const void* k, const void* v, const LogitSrc& logit, int zero_ch,
                            const int32_t* h_lengths, int32_t max_len, hipStream_t s) {
  // The partial area is free between attention calls: it holds the bases.
  int32_t* bases = (int32_t*)p.part;
  for (int pass = 0; pass < 2; ++pass) {
    for (int b0 = 0; b0 < p.B; b0 += PromptLens::kMax) {
      const int nb = std::min(PromptLens::kMax, p.B - b0);
      PromptLens lens;
      for (int i = 0; i < nb; ++i) lens.v[i] = h_lengths[b0 + i];
      const hipError_t e =
          pass == 0 ? launch(prefill_count_kernel, dim3(nb * p.Hkv), dim3(1024), s, p, logit, b0, lens)
                    : launch(prefill_scan_kernel, dim3(nb * p.Hkv), dim3(1024), s, p, logit, b0, lens,
                             (const int32_t*)bases);
      if (e != hipSuccess) return e;
    }
    if (pass == 0) {
      const hipError_t e = launch(prefill_alloc_kernel, dim3(1), dim3(1024), s, p, bases);
      if (e != hipSuccess) return e;
    }
  }
  const int ysplit = 8;
  return launch(prefill_scatter_kernel<ES, D>, dim3(p.U, ysplit), dim3(64 * kWavesPerWG), s, p,
                (const uint8_t*)k, (const uint8_t*)v, max_len, zero_ch);
}

hipError_t launch_prefill(const Dev& p, int dtype, int d, const void* k, const void* v,
                          const LogitSrc& logit, int zero_ch, const int32_t* h_lengths, int32_t max_len,
                          hipStream_t s) {
  if (dtype == 1)
    return d == 128 ? prefill_t<2, 128>(p, k, v, logit, zero_ch, h_lengths, max_len, s)
                    : prefill_t<2, 64>(p, k, v, logit, zero_ch, h_lengths, max_len, s);
  return d == 128 ? prefill_t<4, 128>(p, k, v, logit, zero_ch, h_lengths, max_len, s)
                  : prefill_t<4, 64>(p, k, v, logit, zero_ch, h_lengths, max_len, s);
}

template <int ES, int D>
static hipError_t attention_t(const Dev& p, const void* q, float* out, hipStream_t s, hipEvent_t start,
                              hipEvent_t stop) {
  // whole-unit mode: no unit is split, so there is nothing for reduce_kernel
  const dim3 grid((unsigned)p.grid), block(64 * kWavesPerWG);
  const dim3 rgrid((p.U + kWavesPerWG - 1) / kWavesPerWG);
  const StepIn none{};
  const hipError_t e = launch_timed(attention_kernel<ES, D, kAttend>, grid, block, s, start, p.split ? nullptr : stop,
                                    p, (const int32_t*)p.btab, (const uint8_t*)q, out, none);
  if (e != hipSuccess || !p.split) return e;
  return launch_timed(reduce_kernel<ES, D, false>, rgrid, block, s, nullptr, stop, p, out, none);
}

template <typename K>
static int resident_of(K kernel, int num_cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * kWavesPerWG, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return per_cu * num_cus;
}

// The launch size serves every attention kernel (the attention alone and the
// two decode steps): the smallest of their resident counts.
template <int ES, int D>
static int resident_t(int num_cus) {
  return std::min({resident_of(attention_kernel<ES, D, kAttend>, num_cus),
                   resident_of(attention_kernel<ES, D, kStepWhole>, num_cus),
                   resident_of(attention_kernel<ES, D, kStepSplit>, num_cus)});
}

int attention_resident_wgs(int dtype, int d, int num_cus) {
  if (dtype == 1) return d == 128 ? resident_t<2, 128>(num_cus) : resident_t<2, 64>(num_cus);
  return d == 128 ? resident_t<4, 128>(num_cus) : resident_t<4, 64>(num_cus);
}

hipError_t launch_attention(const Dev& p, int dtype, int d, const void* q, float* out, hipStream_t s,
                            hipEvent_t start, hipEvent_t stop) {
  if (dtype == 1)
    return d == 128 ? attention_t<2, 128>(p, q, out, s, start, stop) : attention_t<2, 64>(p, q, out, s, start, stop);
  return d == 128 ? attention_t<4, 128>(p, q, out, s, start, stop) : attention_t<4, 64>(p, q, out, s, start, stop);
}

template <int ES, int D>
static hipError_t decode_step_t(const Dev& p, const void* q, const StepIn& in, float* out, hipStream_t s,
                                hipEvent_t start, hipEvent_t stop) {
  const dim3 block(64 * kWavesPerWG);
  // whole-unit mode: one launch (the append inside); split mode: the
  // attention, then the split merge with the appends
  if (!p.split)
    return launch_timed(attention_kernel<ES, D, kStepWhole>, dim3((unsigned)p.grid), block, s, start, stop, p,
                        (const int32_t*)p.btab, (const uint8_t*)q, out, in);
  const hipError_t e = launch_timed(attention_kernel<ES, D, kStepSplit>, dim3((unsigned)p.grid), block, s, start,
                                    nullptr, p, (const int32_t*)p.btab, (const uint8_t*)q, out, in);
  if (e != hipSuccess) return e;
  const dim3 rgrid((p.U + kWavesPerWG / 2 - 1) / (kWavesPerWG / 2));  // two waves per unit
  return launch_timed(reduce_kernel<ES, D, true>, rgrid, block, s, nullptr, stop, p, out, in);
}

hipError_t launch_decode_step(const Dev& p, int dtype, int d, const void* q, const StepIn& in, float* out,
                              hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (dtype == 1)
    return d == 128 ? decode_step_t<2, 128>(p, q, in, out, s, start, stop)
                    : decode_step_t<2, 64>(p, q, in, out, s, start, stop);
  return d == 128 ? decode_step_t<4, 128>(p, q, in, out, s, start, stop)
                  : decode_step_t<4, 64>(p, q, in, out, s, start, stop);
}

}  // namespace dms
