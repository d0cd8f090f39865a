// HIP kernels of the DMS decode path for gfx950 (MI355X).
//
// Method: "Inference-Time Hyper-Scaling with KV Cache Compression", paper
// summary page, "Key claims" and "Method" (paper section 3.2, section 5.3,
// Fig. 5).  Each KV head decides per token whether to evict it (alpha = 1
// when the eviction logit is > 0); a marked token stays attendable for w more
// steps, then leaves the cache.  Attention reads only what is still visible,
// so the additive mask of the paper is never built.
//
// Cache layout (all inside the caller's workspace, see dms_internal.h)
//   * Per (sequence, KV head) "unit": n live slots, always the dense prefix
//     [0, n) of the unit's slot space (an append reuses the slot of the token
//     it retires, else takes slot n), a block table mapping logical block
//     j = slot / 16 to a physical pool block, and a ring of R = w + 1 slots
//     of marked tokens whose eviction is pending (entry q mod R belongs to
//     position q).
//   * Pool blocks hold 16 tokens of K and V in MFMA-fragment order, so the
//     decode attention loads each operand with one 16-byte load per lane
//     and 1 KiB contiguous per wave instruction:
//       K half, chunk c, lane l (16 bytes):
//         token l % 16, channels c*4*E + E*(l/16) + e  (E = 16/sizeof(T))
//       V half, chunk c, lane l (16 bytes):
//         tokens 4*(l/16) + e (e < 4), channel 16*(c*NJ + jj) + l % 16
//         at byte jj*8 + e*sizeof(T)  (NJ = 2 for bf16, 1 for fp32)
//   * Per block: 16 slot positions and a 16-bit live mask.
//
// Decode attention per (unit, block range) work item, one work-group of four
// waves each (waves take every fourth block and merge through LDS):
//   S[t][g]  = K_blk[t] . Q[g]     MFMA, A = K fragment, B = Q fragment
//   online softmax on S in the MFMA output layout (lane l holds tokens
//            4*(l/16)+r of head l % 16), exp2 domain
//   O^T[c][g] += V^T[c][t] P[t][g]  MFMA, A = V fragment, B = P taken in
//            place from the S registers (bf16: P split into hi + lo parts)
// A unit whose blocks were split over several work items gets its partials
// merged by reduce_kernel in a second launch (log-sum-exp).  With at least as
// many units as resident work-groups no unit is split and that launch is
// skipped.
//
// The other kernels, in file order:
//   * append_kernel / append_chunk_kernel: one token (or a chunk of tokens, in
//     order) per unit: decision, retirement of position q - w - 1, store.
//   * prefill_{count,alloc,scan,scatter}_kernel: a dense prompt compressed to
//     the state of one append per token.
//   * prefill_attention_kernel: every prompt query over its own visible set,
//     from the compressed cache (positions below q - w) and the dense prompt
//     (the window).
//   * chunk_attention_kernel: the queries of a chunk of tokens over the cache
//     as it stands plus the chunk's own rows, before the chunk's appends.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <tuple>
#include <utility>

#include "dms_internal.h"

namespace dms {

// Launches `kernel` and returns the status of this launch alone (a stale
// error left in the thread by an unrelated earlier HIP call is not reported).
template <typename... KArgs, typename... Args>
static hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, Args&&... args) {
  auto tup = [](auto&&... a) { return std::tuple<KArgs...>(a...); }(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... a) {
    int i = 0;
    ((ptrs[i++] = (void*)&a), ...);
  }, tup);
  return hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, s);
}

// As launch, through hipExtLaunchKernel with events that the runtime stamps
// with the start and the end of this kernel (either may be null).
template <typename... KArgs, typename... Args>
static hipError_t launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, hipEvent_t start,
                               hipEvent_t stop, Args&&... args) {
  auto tup = [](auto&&... a) { return std::tuple<KArgs...>(a...); }(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... a) {
    int i = 0;
    ((ptrs[i++] = (void*)&a), ...);
  }, tup);
  if (!start && !stop) return hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, s);
  return hipExtLaunchKernel((const void*)kernel, grid, block, ptrs, 0, s, start, stop, 0);
}

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned int))));
typedef unsigned int u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));

template <int ES, int D>
struct Geo {
  static constexpr int kE = 16 / ES;                // elements per 16-byte chunk
  static constexpr int kChunks = D * 16 * ES / 1024;  // chunks per lane per K (or V) half
  static constexpr int kHalf = D * 16 * ES;         // bytes of one half-block
  static constexpr int kTiles = D / 16;             // output tiles of 16 channels
  static constexpr int kNJ = ES == 2 ? 2 : 1;       // V channel groups per chunk
};

// ---------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ long long wave_sum_ll(long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups that hold
// one MFMA column's rows).  The gfx950 permlane swaps exchange those lane
// groups within the VALU; a shuffle would go through the LDS crossbar.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ float bf16_lo_to_f32(unsigned x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(unsigned x) { return __uint_as_float(x & 0xffff0000u); }

// Eviction logit of unit (b, h) at position i (an exact upcast for bf16).
__device__ __forceinline__ float load_logit(const LogitSrc& ls, int b, int h, int64_t i) {
  const int64_t e = (int64_t)b * ls.sb + (int64_t)h * ls.sh + i * ls.si + ls.off;
  if (ls.bf16) return __uint_as_float((unsigned)((const uint16_t*)ls.base)[e] << 16);
  return ((const float*)ls.base)[e];
}

// Clears key channel zc (none when zc < 0) if it lies in 16-byte piece r of
// a row (channels r * 16 / ES .. (r + 1) * 16 / ES - 1).
template <int ES>
__device__ __forceinline__ void clear_channel(u32x4& val, int r, int zc) {
  constexpr int kE = 16 / ES;
  if (zc < 0 || zc / kE != r) return;
  const int byte = (zc % kE) * ES;
  const unsigned keep = ES == 4 ? 0u : ((byte & 2) ? 0x0000ffffu : 0xffff0000u);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i == (byte >> 2)) val[i] &= keep;
}

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

// ---------------------------------------------------------------------------
// append + evict: one wave per (sequence, KV head)
// ---------------------------------------------------------------------------

// Stores one token row into slot t of an existing block.
template <int ES, int D>
__device__ __forceinline__ void write_row(uint8_t* blkp, int t, const uint8_t* krow,
                                          const uint8_t* vrow, int lane, int zero_ch) {
  using G = Geo<ES, D>;
  if (lane < D / G::kE) {
    const int r = lane;  // 16-byte piece of the row: channels r*E .. r*E+E-1
    u32x4 val = *(const u32x4*)(krow + r * 16);
    clear_channel<ES>(val, r, zero_ch);
    *(u32x4*)(blkp + (r >> 2) * 1024 + (t + 16 * (r & 3)) * 16) = val;
  }
#pragma unroll
  for (int ch = lane; ch < D; ch += 64) {
    const int c = ch / (16 * G::kNJ), jj = (ch >> 4) % G::kNJ, nn = ch & 15;
    const int l = nn + 16 * (t >> 2), e = t & 3;
    uint8_t* dst = blkp + G::kHalf + c * 1024 + l * 16 + jj * 8 + e * ES;
    if constexpr (ES == 2)
      *(uint16_t*)dst = *(const uint16_t*)(vrow + ch * 2);
    else
      *(uint32_t*)dst = *(const uint32_t*)(vrow + ch * 4);
  }
}

// Writes a whole fresh block: the row in slot 0, zeros in slots 1..15 (the
// attention multiplies masked slots by zero weights, so they must be finite).
template <int ES, int D>
__device__ __forceinline__ void write_fresh(uint8_t* blkp, const uint8_t* krow,
                                            const uint8_t* vrow, int lane, int zero_ch) {
  using G = Geo<ES, D>;
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    u32x4 val = {0u, 0u, 0u, 0u};
    if ((lane & 15) == 0) {
      val = *(const u32x4*)(krow + (c * 4 + (lane >> 4)) * 16);
      clear_channel<ES>(val, c * 4 + (lane >> 4), zero_ch);
    }
    *(u32x4*)(blkp + c * 1024 + lane * 16) = val;
  }
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    u32x4 val = {0u, 0u, 0u, 0u};
    if (lane < 16) {
      if constexpr (ES == 2) {
        val[0] = *(const uint16_t*)(vrow + (16 * (2 * c) + lane) * 2);
        val[2] = *(const uint16_t*)(vrow + (16 * (2 * c + 1) + lane) * 2);
      } else {
        val[0] = *(const uint32_t*)(vrow + (16 * c + lane) * 4);
      }
    }
    *(u32x4*)(blkp + G::kHalf + c * 1024 + lane * 16) = val;
  }
}

// Stores the token at position q of unit u (one wave), once its decision and
// destination are known: rs = the slot of position q - R if that token was
// marked (it retires now and the new token takes its slot), else -1 (the new
// token takes slot n); blk = the pool block of that slot, or -1 when the
// slot starts a new block, which is then claimed from the pool (on
// exhaustion the sticky error is set and nothing is stored).  Writes the
// row, the slot's position and mask bit, the ring entry of q, n and pos, all
// from lane 0 except the row.  Returns the unit's live count afterwards.
template <int ES, int D>
__device__ __forceinline__ unsigned store_token(const Dev& p, int u, int lane, const uint8_t* krow,
                                                const uint8_t* vrow, bool alpha, int q, int rs, int n, int blk,
                                                int zero_ch) {
  int32_t* ring = p.ring + (int64_t)u * p.R;
  const int r = q % p.R;
  const int slot = rs >= 0 ? rs : n;
  bool fresh = false, ok = true;
  if (blk < 0) {
    unsigned long long nb = 0;
    if (lane == 0) nb = atomicAdd(&p.ctr->bump, 1ull);
    nb = __shfl(nb, 0);
    if (nb >= (unsigned long long)p.pool_blocks) {
      ok = false;
      if (lane == 0) atomicCAS(&p.ctr->sticky_error, 0, kErrOutOfBlocks);
    } else {
      blk = (int)nb;
      fresh = true;
      if (lane == 0) p.btab[(int64_t)u * p.max_blocks + (slot >> 4)] = blk;
    }
  }
  const int t = slot & 15;
  unsigned live;
  if (ok) {
    uint8_t* dst = p.pool + (int64_t)blk * p.block_bytes;
    if (fresh)
      write_fresh<ES, D>(dst, krow, vrow, lane, zero_ch);
    else
      write_row<ES, D>(dst, t, krow, vrow, lane, zero_ch);
    if (lane == 0) {
      p.blk_pos[(int64_t)blk * 16 + t] = q;
      // live slots are the dense prefix [0, n): taking slot n leaves slots
      // 0 .. t of its block live (no read of the old mask); a reused slot
      // was live already
      if (rs < 0) p.blk_mask[blk] = (2u << t) - 1u;
      ring[r] = alpha ? slot : -1;
      if (rs < 0) p.n[u] = n + 1;
    }
    live = (rs < 0) ? (unsigned)(n + 1) : (unsigned)n;
  } else {
    if (lane == 0) ring[r] = -1;
    live = (unsigned)n;
  }
  if (lane == 0) p.pos[u] = q + 1;
  return live;
}

// Appends the token at unit u's next position (one wave): decides alpha,
// retires position q - R if it was marked (its slot is reused), stores the
// row.  Returns the unit's live count afterwards.  Every per-unit value is
// read through lane 0, the lane that writes it, so that consecutive calls of
// one wave (a chunk) see their own updates in program order.
template <int ES, int D>
__device__ __forceinline__ unsigned append_token(const Dev& p, int u, int lane, const uint8_t* krow,
                                                 const uint8_t* vrow, float lg, int zero_ch) {
  const bool alpha = lg > 0.0f;  // NaN compares false
  const int q = __builtin_amdgcn_readfirstlane(p.pos[u]);
  const int rs = __builtin_amdgcn_readfirstlane(p.ring[(int64_t)u * p.R + q % p.R]);  // slot of q - R if marked
  const int n = __builtin_amdgcn_readfirstlane(p.n[u]);
  const int slot = rs >= 0 ? rs : n;
  // the slot's block exists unless the token starts a new one
  const int blk = (rs >= 0 || (n & 15) != 0)
                      ? __builtin_amdgcn_readfirstlane(p.btab[(int64_t)u * p.max_blocks + (slot >> 4)])
                      : -1;
  return store_token<ES, D>(p, u, lane, krow, vrow, alpha, q, rs, n, blk, zero_ch);
}

// Adds each work-group's live counts to live_token_steps (one atomic).
__device__ __forceinline__ void add_live_token_steps(const Dev& p, unsigned long long live) {
  __shared__ unsigned long long s_live[kWavesPerWG];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_live[wave] = live;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long sum = 0;
#pragma unroll
    for (int i = 0; i < kWavesPerWG; ++i) sum += s_live[i];
    atomicAdd(&p.ctr->live_token_steps, sum);
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

// A load of a uniform address through the scalar cache (constant address
// space): the address must not be written by this kernel before the load.
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ int scalar_load(const int32_t* a) { return *(const_i32*)(uintptr_t)a; }

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

template <int ES, int D>
struct Frag {
  u32x4 k[Geo<ES, D>::kChunks];
  u32x4 v[Geo<ES, D>::kChunks];
};

template <int ES, int D>
__device__ __forceinline__ void load_frag(Frag<ES, D>& f, const uint8_t* blkp, int lane) {
  using G = Geo<ES, D>;
  const uint8_t* a = blkp + lane * 16;
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) f.k[c] = __builtin_nontemporal_load((const u32x4*)(a + c * 1024));
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c)
    f.v[c] = __builtin_nontemporal_load((const u32x4*)(a + G::kHalf + c * 1024));
}

// Running softmax state of one wave: lane l tracks head l % 16.
template <int D>
struct Acc {
  f32x4 o[D / 16];  // O^T tiles: lane l, reg r -> channel 16j + 4(l/16) + r of head l % 16
  float m, l;
};

template <int ES, int D>
__device__ __forceinline__ void attend_block(const Frag<ES, D>& f, const u32x4 (&qf)[Geo<ES, D>::kChunks],
                                             uint32_t mask, int lane, float sl2e, Acc<D>& a) {
  using G = Geo<ES, D>;
  f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    if constexpr (ES == 2) {
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.k[c]),
                                                 __builtin_bit_cast(bf16x8, qf[c]), S, 0, 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.k[c][e]), __uint_as_float(qf[c][e]),
                                                 S, 0, 0, 0);
    }
  }
  const int tb = 4 * (lane >> 4);
  float s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) s[r] = ((mask >> (tb + r)) & 1u) ? S[r] * sl2e : -INFINITY;
  float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  bm = fmaxf(bm, __shfl_xor(bm, 16));
  bm = fmaxf(bm, __shfl_xor(bm, 32));
  const float mn = fmaxf(a.m, bm);
  const float mref = (mn == -INFINITY) ? 0.f : mn;
  const float alpha = exp2_fast(a.m - mref);
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = exp2_fast(s[r] - mref);
  a.l = a.l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
  a.m = mn;
#pragma unroll
  for (int j = 0; j < G::kTiles; ++j) a.o[j] *= alpha;
  if constexpr (ES == 2) {
    const unsigned h01 = pack_bf16x2(pr[0], pr[1]), h23 = pack_bf16x2(pr[2], pr[3]);
    const unsigned l01 = pack_bf16x2(pr[0] - bf16_lo_to_f32(h01), pr[1] - bf16_hi_to_f32(h01));
    const unsigned l23 = pack_bf16x2(pr[2] - bf16_lo_to_f32(h23), pr[3] - bf16_hi_to_f32(h23));
    const u32x2 hv = {h01, h23}, lv = {l01, l23};
    const s16x4 PH = __builtin_bit_cast(s16x4, hv), PL = __builtin_bit_cast(s16x4, lv);
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x2 vv = {f.v[c][2 * jj], f.v[c][2 * jj + 1]};
        const s16x4 A = __builtin_bit_cast(s16x4, vv);
        a.o[2 * c + jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, PH, a.o[2 * c + jj], 0, 0, 0);
        a.o[2 * c + jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, PL, a.o[2 * c + jj], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a.o[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.v[c][e]), pr[e], a.o[c], 0, 0, 0);
    }
  }
}

// Two blocks (32 keys) per softmax step.  For bf16, S of both blocks, one
// running-max update and rescale, then O^T += V^T P^T with 16x16x32 MFMAs.
// Their k index runs over the lane group's 4 keys of block A, then the same 4
// keys of block B, for both operands alike (a permutation of the sum).  The V
// operand of channel tile j is therefore 8 bytes of block A next to 8 bytes
// of block B, and it is loaded straight into that order.  For fp32 the pair
// is two blocks computed one after the other.
template <int ES, int D>
struct PairFrag {
  Frag<ES, D> a, b;
};

template <int D>
struct PairFrag<2, D> {
  u32x4 ka[Geo<2, D>::kChunks], kb[Geo<2, D>::kChunks];
  u32x4 v[Geo<2, D>::kTiles];  // tile 2c + jj: {A keys tb..tb+3, B keys tb..tb+3} of channel 16(2c+jj) + l%16
};

// Loads blocks A and B of the pool (fragment order) as a pair.
template <int ES, int D>
__device__ __forceinline__ void load_pair(PairFrag<ES, D>& f, const uint8_t* blka, const uint8_t* blkb, int lane) {
  using G = Geo<ES, D>;
  if constexpr (ES == 2) {
    const uint8_t* a = blka + lane * 16;
    const uint8_t* b = blkb + lane * 16;
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) f.ka[c] = __builtin_nontemporal_load((const u32x4*)(a + c * 1024));
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) f.kb[c] = __builtin_nontemporal_load((const u32x4*)(b + c * 1024));
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x2 x = __builtin_nontemporal_load((const u32x2*)(a + G::kHalf + c * 1024 + jj * 8));
        const u32x2 y = __builtin_nontemporal_load((const u32x2*)(b + G::kHalf + c * 1024 + jj * 8));
        f.v[2 * c + jj] = u32x4{x[0], x[1], y[0], y[1]};
      }
    }
  } else {
    load_frag<ES, D>(f.a, blka, lane);
    load_frag<ES, D>(f.b, blkb, lane);
  }
}

// The same pair order from two fragments already in registers.
template <int ES, int D>
__device__ __forceinline__ void make_pair(PairFrag<ES, D>& f, const Frag<ES, D>& fa, const Frag<ES, D>& fb) {
  using G = Geo<ES, D>;
  if constexpr (ES == 2) {
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) {
      f.ka[c] = fa.k[c];
      f.kb[c] = fb.k[c];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        f.v[2 * c + jj] = u32x4{fa.v[c][2 * jj], fa.v[c][2 * jj + 1], fb.v[c][2 * jj], fb.v[c][2 * jj + 1]};
    }
  } else {
    f.a = fa;
    f.b = fb;
  }
}

template <int D>
__device__ __forceinline__ void score_pair(const PairFrag<2, D>& f, const u32x4 (&qf)[Geo<2, D>::kChunks], f32x4& SA,
                                           f32x4& SB) {
  using G = Geo<2, D>;
  SA = f32x4{0.f, 0.f, 0.f, 0.f};
  SB = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    SA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.ka[c]),
                                                  __builtin_bit_cast(bf16x8, qf[c]), SA, 0, 0, 0);
    SB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.kb[c]),
                                                  __builtin_bit_cast(bf16x8, qf[c]), SB, 0, 0, 0);
  }
}

// Softmax step and P.V of a pair of blocks from its raw scores (score_pair):
// masks ma, mb select the live keys (bit i = key i of the block).
template <int D>
__device__ __forceinline__ void softmax_pv_masked(const PairFrag<2, D>& f, const f32x4& SA, const f32x4& SB,
                                                  uint32_t ma, uint32_t mb, int lane, float sl2e, Acc<D>& a) {
  using G = Geo<2, D>;
  const int tb = 4 * (lane >> 4);
  // Raw scores, masked to -inf; the scale (> 0) is applied to the max and
  // inside the exponent's fma, which keeps the max exact.
  float s[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s[r] = ((ma >> (tb + r)) & 1u) ? SA[r] : -INFINITY;
    s[4 + r] = ((mb >> (tb + r)) & 1u) ? SB[r] : -INFINITY;
  }
  const float bm = max_over_groups(
      fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]))));
  const float mn = fmaxf(a.m, bm * sl2e);
  const float mref = (mn == -INFINITY) ? 0.f : mn;
  float pr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) pr[r] = exp2_fast(fmaf(s[r], sl2e, -mref));
  const float psum = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
  // Rescale only when some column's running max moved (after the first
  // blocks it rarely does).  An unmoved max gives alpha = 1 exactly; a
  // column with no key yet has o = l = 0, which any alpha leaves at 0.
  if (__builtin_amdgcn_ballot_w64(mn != a.m) != 0) {
    const float alpha = exp2_fast(a.m - mref);
    a.l *= alpha;
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) a.o[j] *= alpha;
  }
  a.l += psum;
  a.m = mn;
  unsigned hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = pack_bf16x2(pr[2 * i], pr[2 * i + 1]);
    lo[i] = pack_bf16x2(pr[2 * i] - bf16_lo_to_f32(hi[i]), pr[2 * i + 1] - bf16_hi_to_f32(hi[i]));
  }
  const u32x4 hv = {hi[0], hi[1], hi[2], hi[3]}, lv = {lo[0], lo[1], lo[2], lo[3]};
  const bf16x8 PH = __builtin_bit_cast(bf16x8, hv), PL = __builtin_bit_cast(bf16x8, lv);
#pragma unroll
  for (int j = 0; j < G::kTiles; ++j) {
    const bf16x8 A = __builtin_bit_cast(bf16x8, f.v[j]);
    a.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, PH, a.o[j], 0, 0, 0);
    a.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, PL, a.o[j], 0, 0, 0);
  }
}

template <int ES, int D>
__device__ __forceinline__ void attend_pair(const PairFrag<ES, D>& f, const u32x4 (&qf)[Geo<ES, D>::kChunks],
                                            uint32_t ma, uint32_t mb, int lane, float sl2e, Acc<D>& a) {
  if constexpr (ES != 2) {
    attend_block<ES, D>(f.a, qf, ma, lane, sl2e, a);
    attend_block<ES, D>(f.b, qf, mb, lane, sl2e, a);
  } else {
    f32x4 SA, SB;
    score_pair<D>(f, qf, SA, SB);
    softmax_pv_masked<D>(f, SA, SB, ma, mb, lane, sl2e, a);
  }
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
// partials (when it was cut).  STEP (a decode step in split mode): the wave
// then appends the unit's new token, which the attention has already taken
// from the step's input rows; the unit's state is written only now, so every
// work-group of the attention read the state from before the step.
template <int ES, int D, bool STEP>
__global__ __launch_bounds__(256) void reduce_kernel(Dev p, float* __restrict__ out, StepIn in) {
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * kWavesPerWG + (threadIdx.x >> 6);
  unsigned long long live = 0;
  if (u < p.U) {
    merge_partials<D>(p, u, lane, out);
    if constexpr (STEP) {
      const int b = u / p.Hkv;
      live = append_token<ES, D>(p, u, lane, in.k + (int64_t)u * D * ES, in.v + (int64_t)u * D * ES,
                                 load_logit(in.logit, b, u - b * p.Hkv, 0), in.zero_ch);
    }
  }
  if constexpr (STEP) add_live_token_steps(p, live);
}

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
// Work-group = 4 waves = kPfTile consecutive queries of one query head; wave
// w owns kPfCols tiles of 16 queries, one query per MFMA column (where the
// decode packs the group's heads), and streams the same key blocks as the
// other waves.
constexpr int kPfCols = 3;
constexpr int kPfTile = 16 * kPfCols * kWavesPerWG;

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
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (ES == 2) {
          const unsigned x = *(const uint16_t*)(vrow[e] + ch * 2);
          val[jj * 2 + (e >> 1)] |= x << (16 * (e & 1));
        } else {
          val[e] = *(const uint32_t*)(vrow[e] + ch * 4);
        }
      }
    }
    f.v[c] = val;
  }
}

// Grid (ceil(max_len_used / kPfTile), Hq, B).
template <int ES, int D>
__global__ __launch_bounds__(256) void prefill_attention_kernel(Dev p, const uint8_t* __restrict__ q,
                                                                const uint8_t* __restrict__ k,
                                                                const uint8_t* __restrict__ v, int32_t max_len,
                                                                int zero_ch, float* __restrict__ out) {
  using G = Geo<ES, D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.z, hq = blockIdx.y;
  const int h = hq / p.G, u = b * p.Hkv + h;
  const int P = __builtin_amdgcn_readfirstlane(p.pos[u]);
  const int q0 = blockIdx.x * kPfTile;
  if (q0 >= P) return;
  const int w = p.R - 1;
  const int qmax = min(q0 + kPfTile, P) - 1;
  const int64_t unit_rows = ((int64_t)b * p.Hkv + h) * max_len;
  const uint8_t* Ku = k + unit_rows * D * ES;
  const uint8_t* Vu = v + unit_rows * D * ES;
  const uint8_t* Qh = q + ((int64_t)b * p.Hq + hq) * max_len * D * ES;

  int qc[kPfCols];
  u32x4 qf[kPfCols][G::kChunks];
  Acc<D> acc[kPfCols];
#pragma unroll
  for (int t = 0; t < kPfCols; ++t) {
    qc[t] = q0 + 16 * (kPfCols * wave + t) + (lane & 15);
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
  const int nfull = min(max(__builtin_amdgcn_readfirstlane(nlow) - 1, 0), nfar);
  auto blk_at = [&](int j, int jmax) { return __builtin_amdgcn_readfirstlane(bt[min(j, jmax)]); };
  if (nfull > 0) {
    // Whole blocks, in pairs, one pair loaded ahead of the one computed.
    // Loads are unconditional: an index past the last whole block re-reads
    // it, and its keys are masked out.  The scheduling barriers keep each
    // pair's loads issued ahead of the previous pair's arithmetic (left alone,
    // the scheduler sinks them next to their use, exposing their latency).
    const int npair = (nfull + 1) >> 1;
    auto fetch = [&](PairFrag<ES, D>& f, int i) {
      const int ba = blk_at(2 * i, nfull - 1), bb = blk_at(2 * i + 1, nfull - 1);
      load_pair<ES, D>(f, p.pool + (int64_t)ba * p.block_bytes, p.pool + (int64_t)bb * p.block_bytes, lane);
    };
    auto compute = [&](const PairFrag<ES, D>& f, int i) {
      const uint32_t mb = 2 * i + 1 < nfull ? 0xffffu : 0u;
      if constexpr (ES == 2) {
        // column t + 1's score products issued before column t's softmax
        f32x4 SA[2], SB[2];
        score_pair<D>(f, qf[0], SA[0], SB[0]);
#pragma unroll
        for (int t = 0; t < kPfCols; ++t) {
          if (t + 1 < kPfCols) score_pair<D>(f, qf[t + 1], SA[(t + 1) & 1], SB[(t + 1) & 1]);
          softmax_pv_masked<D>(f, SA[t & 1], SB[t & 1], 0xffffu, mb, lane, p.scale_log2e, acc[t]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < kPfCols; ++t) attend_pair<ES, D>(f, qf[t], 0xffffu, mb, lane, p.scale_log2e, acc[t]);
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
    load_pair<ES, D>(f, p.pool + (int64_t)ba * p.block_bytes, p.pool + (int64_t)bb * p.block_bytes, lane);
    const int4 pa = *(const int4*)(p.blk_pos + (int64_t)ba * 16 + tb);
    const int4 pb = *(const int4*)(p.blk_pos + (int64_t)bb * 16 + tb);
    const int lva = n - 16 * j, lvb = j + 1 < nfar ? n - 16 * (j + 1) : 0;  // live slots
#pragma unroll
    for (int t = 0; t < kPfCols; ++t) {
      const int lt = qc[t] - w;
      uint32_t ma = 0, mb = 0;
      const int xa[4] = {pa.x, pa.y, pa.z, pa.w}, xb[4] = {pb.x, pb.y, pb.z, pb.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (tb + r < lva && xa[r] < lt) ma |= 1u << (tb + r);
        if (tb + r < lvb && xb[r] < lt) mb |= 1u << (tb + r);
      }
      attend_pair<ES, D>(f, qf[t], ma, mb, lane, p.scale_log2e, acc[t]);
    }
  }

  // Near part: dense rows max(0, q0 - w) .. qmax, all visible within the
  // window, 32 rows per softmax step.
  auto near_mask = [&](int r0, int t) -> uint32_t {
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = r0 + tb + r;
      if (pos <= qc[t] && pos >= qc[t] - w && pos < P) m |= 1u << (tb + r);
    }
    return m;
  };
  for (int r0 = max(0, q0 - w); r0 <= qmax; r0 += 32) {
    Frag<ES, D> fa, fb;
    load_frag_dense<ES, D>(fa, Ku, Vu, r0, P - 1, lane, zero_ch);
    load_frag_dense<ES, D>(fb, Ku, Vu, r0 + 16, P - 1, lane, zero_ch);
    PairFrag<ES, D> f;
    make_pair<ES, D>(f, fa, fb);
#pragma unroll
    for (int t = 0; t < kPfCols; ++t)
      attend_pair<ES, D>(f, qf[t], near_mask(r0, t), near_mask(r0 + 16, t), lane, p.scale_log2e, acc[t]);
  }

#pragma unroll
  for (int t = 0; t < kPfCols; ++t) {
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

// ---------------------------------------------------------------------------
// training-time relaxed attention (Gumbel-sigmoid decisions as a soft mask)
// ---------------------------------------------------------------------------

// Soft decision of key i: x = (logit + gamma + noise) / tau, alpha = sigmoid(x).
// Query q >= i adds log(1 - alpha) = -softplus(x) to the score of key i when
// q - i > w, nothing inside the window (the hard rule when alpha is 0 or 1).
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// The x of key i of unit (b, h).
__device__ __forceinline__ float soft_x(const SoftArgs& a, const float* __restrict__ logit,
                                        const float* __restrict__ noise, int64_t unit_row0, int i) {
  return (logit[unit_row0 + i] + a.gamma + noise[unit_row0 + i]) * a.inv_tau;
}

// The softmax step and P.V of a pair of blocks from its raw scores
// (score_pair), with an additive score per key and column in the exp2 domain:
// badd[0..3] for this lane's keys of block A, badd[4..7] of block B (-inf for
// keys the column may not see).  Split from the score products so that the
// next column's can be issued ahead of this column's softmax.
template <int D>
__device__ __forceinline__ void softmax_pv_biased(const PairFrag<2, D>& f, const f32x4& SA, const f32x4& SB,
                                                  const float (&badd)[8], float sl2e, Acc<D>& a) {
  using G = Geo<2, D>;
  float s[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s[r] = fmaf(SA[r], sl2e, badd[r]);
    s[4 + r] = fmaf(SB[r], sl2e, badd[4 + r]);
  }
  const float bm = max_over_groups(
      fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]))));
  const float mn = fmaxf(a.m, bm);
  const float mref = (mn == -INFINITY) ? 0.f : mn;
  float pr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) pr[r] = exp2_fast(s[r] - mref);
  const float psum = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
  if (__builtin_amdgcn_ballot_w64(mn != a.m) != 0) {
    const float alpha = exp2_fast(a.m - mref);
    a.l *= alpha;
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) a.o[j] *= alpha;
  }
  a.l += psum;
  a.m = mn;
  unsigned hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = pack_bf16x2(pr[2 * i], pr[2 * i + 1]);
    lo[i] = pack_bf16x2(pr[2 * i] - bf16_lo_to_f32(hi[i]), pr[2 * i + 1] - bf16_hi_to_f32(hi[i]));
  }
  const u32x4 hv = {hi[0], hi[1], hi[2], hi[3]}, lv = {lo[0], lo[1], lo[2], lo[3]};
  const bf16x8 PH = __builtin_bit_cast(bf16x8, hv), PL = __builtin_bit_cast(bf16x8, lv);
#pragma unroll
  for (int j = 0; j < G::kTiles; ++j) {
    const bf16x8 A = __builtin_bit_cast(bf16x8, f.v[j]);
    a.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, PH, a.o[j], 0, 0, 0);
    a.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, PL, a.o[j], 0, 0, 0);
  }
}

// attend_pair (bf16) with the additive scores badd (as softmax_pv_biased).
template <int D>
__device__ __forceinline__ void attend_pair_biased(const PairFrag<2, D>& f, const u32x4 (&qf)[Geo<2, D>::kChunks],
                                                   const float (&badd)[8], float sl2e, Acc<D>& a) {
  f32x4 SA, SB;
  score_pair<D>(f, qf, SA, SB);
  softmax_pv_biased<D>(f, SA, SB, badd, sl2e, a);
}

// Forward: out = softmax(scale q k^T + bias) v and lse (natural log of each
// row's softmax denominator) for every position.  q [B, Hq, T, d], k [B, Hkv,
// T, d] bf16 rows; vt the pairT copy of v; bias2 the keys' far bias
// (exp2 domain, soft_bias_kernel); out [B, Hq, T, d], lse [B, Hq, T] fp32.
// Each wave holds kPfCols tiles of 16 queries and streams the causal keys in
// pairs of 16-row blocks, one pair loaded ahead of the one computed.  Grid
// (ceil(T / kPfTile), Hq, B).
template <int D>
__global__ __launch_bounds__(256) void soft_forward_kernel(SoftArgs a, const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ k,
                                                           const uint8_t* __restrict__ vt,
                                                           const float* __restrict__ bias2, float* __restrict__ out,
                                                           float* __restrict__ lse);

// Bias of key i in the exp2 domain, log2e * log(1 - sigmoid(x)) =
// -(max(x, 0) log2e + log2(1 + 2^(-|x| log2e))).  It is added to a score, so
// its absolute error (a few 1e-7) is what matters, not a relative one.
__device__ __forceinline__ float soft_bias2(float x) {
  constexpr float kLog2e = 1.4426950408889634f;
  return -(fmaxf(x, 0.f) * kLog2e + __builtin_amdgcn_logf(1.f + exp2_fast(-fabsf(x) * kLog2e)));
}

// Transposed pair copy ("pairT") of a row-major [R, D] bf16 matrix, the
// operand layout of a product that contracts over its rows: for row pair p
// (rows 32p .. 32p + 31), channel tile j and lane l, 16 bytes at
// ((p * D / 16 + j) * 64 + l) * 16 holding rows 32p + 4(l/16) + e, then rows
// 32p + 16 + 4(l/16) + e (e = 0..3), of channel 16j + l % 16.  Rows >= R are
// 0.  With `out` set, also the row dot products delta[r] = sum_c src[r][c] *
// out[r][c] (out fp32, [R, D]).  Grid (matrices, ceil(R / 32)), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void soft_pack_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                        int R, const float* __restrict__ out,
                                                        float* __restrict__ delta) {
  __shared__ uint16_t tile[32][D + 2];
  const int p = blockIdx.y, m = blockIdx.x, tid = threadIdx.x;
  const int64_t mrow0 = (int64_t)m * R;
  const int npairs = (R + 31) / 32;
  for (int e = tid; e < 32 * D / 2; e += 256) {
    const int r = e / (D / 2), c2 = e % (D / 2);
    const int row = 32 * p + r;
    uint32_t x = 0u;
    if (row < R) x = *(const uint32_t*)(src + (mrow0 + row) * D + 2 * c2);
    tile[r][2 * c2] = (uint16_t)(x & 0xffffu);
    tile[r][2 * c2 + 1] = (uint16_t)(x >> 16);
  }
  __syncthreads();
  uint8_t* d0 = dst + ((int64_t)m * npairs + p) * (D / 16) * 64 * 16;
  for (int o = tid; o < (D / 16) * 64; o += 256) {
    const int j = o >> 6, l = o & 63, g = l >> 4, ch = 16 * j + (l & 15);
    u32x4 val;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int r = 16 * h + 4 * g + 2 * e2;
        val[2 * h + e2] = (uint32_t)tile[r][ch] | ((uint32_t)tile[r + 1][ch] << 16);
      }
    *(u32x4*)(d0 + (int64_t)o * 16) = val;
  }
  if (out != nullptr) {
    // 8 threads per row, D / 8 channels each
    const int r = tid >> 3, part = tid & 7, row = 32 * p + r;
    float acc = 0.f;
    if (row < R) {
      const float* orow = out + (mrow0 + row) * D;
#pragma unroll
      for (int c = part * (D / 8); c < (part + 1) * (D / 8); ++c)
        acc = fmaf(__uint_as_float((uint32_t)tile[r][c] << 16), orow[c], acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (row < R && part == 0) delta[mrow0 + row] = acc;
  }
}

// 16 consecutive rows row0 .. row0 + 15 of a row-major [*, D] bf16 matrix as
// an MFMA operand whose rows are the matrix rows: lane l carries row l % 16
// (clamped to `last`), 16-byte piece 4c + l / 16.
template <int D>
__device__ __forceinline__ void load_rows(u32x4 (&f)[D / 32], const uint8_t* __restrict__ M, int row0, int last,
                                          int lane) {
  const uint8_t* r = M + (int64_t)min(row0 + (lane & 15), last) * D * 2 + 16 * (lane >> 4);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) f[c] = *(const u32x4*)(r + c * 64);
}

template <int D>
__device__ __forceinline__ void load_pairT(u32x4 (&f)[D / 16], const uint8_t* __restrict__ Mt, int pair, int lane) {
  const uint8_t* a = Mt + ((int64_t)pair * (D / 16) * 64 + lane) * 16;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) f[j] = *(const u32x4*)(a + j * 1024);
}

// 8 fp32 values in the pair order as bf16 hi and lo parts (x = hi + lo to
// about 2^-17 relative), the B operand of a product over the pair's rows.
__device__ __forceinline__ void split_pair(const float (&x)[8], bf16x8& H, bf16x8& L) {
  unsigned hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    lo[i] = pack_bf16x2(x[2 * i] - bf16_lo_to_f32(hi[i]), x[2 * i + 1] - bf16_hi_to_f32(hi[i]));
  }
  const u32x4 hv = {hi[0], hi[1], hi[2], hi[3]}, lv = {lo[0], lo[1], lo[2], lo[3]};
  H = __builtin_bit_cast(bf16x8, hv);
  L = __builtin_bit_cast(bf16x8, lv);
}

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Far bias of every key, bias2[u][i] = log2e * log(1 - sigmoid(x_i)) for
// unit u = b * Hkv + h, rows padded to a multiple of 32 with 0.
__global__ __launch_bounds__(256) void soft_bias_kernel(SoftArgs a, const float* __restrict__ logit,
                                                        const float* __restrict__ noise, float* __restrict__ bias2) {
  const int rows = (a.T + 31) / 32 * 32;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)a.B * a.Hkv * rows) return;
  const int64_t u = e / rows;
  const int i = (int)(e - u * rows);
  bias2[e] = i < a.T ? soft_bias2(soft_x(a, logit, noise, u * a.T, i)) : 0.f;
}

template <int D>
struct SoftPair {
  PairFrag<2, D> f;
  f32x4 ba, bb;  // far bias of this lane's keys tb..tb+3 of blocks A and B
};

template <int D>
__global__ __launch_bounds__(256) void soft_forward_kernel(SoftArgs a, const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ k,
                                                           const uint8_t* __restrict__ vt,
                                                           const float* __restrict__ bias2, float* __restrict__ out,
                                                           float* __restrict__ lse) {
  using G = Geo<2, D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.z, hq = blockIdx.y, h = hq / a.G;
  const int T = a.T, w = a.w;
  const int npairs = (T + 31) / 32;
  const int q0 = blockIdx.x * kPfTile;
  const int qmax = min(q0 + kPfTile, T) - 1;
  const int64_t unit = (int64_t)b * a.Hkv + h;
  const uint8_t* Ku = k + unit * T * D * 2;
  const uint8_t* Vt = vt + unit * npairs * 32 * D * 2;
  const float* bu = bias2 + unit * npairs * 32;
  const uint8_t* Qh = q + ((int64_t)b * a.Hq + hq) * T * D * 2;
  const int tb = 4 * (lane >> 4);
  int qc[kPfCols];
  u32x4 qf[kPfCols][G::kChunks];
  Acc<D> acc[kPfCols];
#pragma unroll
  for (int t = 0; t < kPfCols; ++t) {
    const int c0 = q0 + 16 * (kPfCols * wave + t);
    qc[t] = c0 + (lane & 15);
    load_rows<D>(qf[t], Qh, c0, T - 1, lane);
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) acc[t].o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[t].m = -INFINITY;
    acc[t].l = 0.f;
  }
  const int npair = qmax / 32 + 1;
  // Loads are unconditional: an index past the last pair re-reads it (not
  // computed).  The scheduling barriers keep a pair's loads ahead of the
  // previous pair's arithmetic.
  auto fetch = [&](SoftPair<D>& x, int i) {
    i = min(i, npair - 1);
    load_rows<D>(x.f.ka, Ku, 32 * i, T - 1, lane);
    load_rows<D>(x.f.kb, Ku, 32 * i + 16, T - 1, lane);
    load_pairT<D>(x.f.v, Vt, i, lane);
    x.ba = *(const f32x4*)(bu + 32 * i + tb);
    x.bb = *(const f32x4*)(bu + 32 * i + 16 + tb);
  };
  const int cw0 = q0 + 16 * kPfCols * wave;  // the wave's first query
  auto compute = [&](const SoftPair<D>& x, int i) {
    if (32 * i + 31 + w < cw0) {
      // every key of the pair is past the window of every query of the wave
      const float badd[8] = {x.ba[0], x.ba[1], x.ba[2], x.ba[3], x.bb[0], x.bb[1], x.bb[2], x.bb[3]};
      // column t + 1's score products are issued before column t's softmax,
      // so they run while its VALU work does (each column's lazy-rescale
      // test is a branch the scheduler does not move work across)
      f32x4 SA[2], SB[2];
      score_pair<D>(x.f, qf[0], SA[0], SB[0]);
#pragma unroll
      for (int t = 0; t < kPfCols; ++t) {
        if (t + 1 < kPfCols) score_pair<D>(x.f, qf[t + 1], SA[(t + 1) & 1], SB[(t + 1) & 1]);
        softmax_pv_biased<D>(x.f, SA[t & 1], SB[t & 1], badd, a.scale_log2e, acc[t]);
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < kPfCols; ++t) {
      float badd[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int key = 32 * i + (r >> 2) * 16 + tb + (r & 3);
        const float fb = r < 4 ? x.ba[r] : x.bb[r - 4];
        badd[r] = key > qc[t] ? -INFINITY : (qc[t] - key > w ? fb : 0.f);
      }
      attend_pair_biased<D>(x.f, qf[t], badd, a.scale_log2e, acc[t]);
    }
  };
  SoftPair<D> f0, f1;
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
  constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
  for (int t = 0; t < kPfCols; ++t) {
    float lt = acc[t].l + __shfl_xor(acc[t].l, 16);
    lt = lt + __shfl_xor(lt, 32);
    if (qc[t] >= T) continue;
    const float inv = 1.0f / lt;
    const int64_t row = ((int64_t)b * a.Hq + hq) * T + qc[t];
    float* orow = out + row * D + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) *(f32x4*)(orow + 16 * j) = acc[t].o[j] * inv;
    if (lane < 16) lse[row] = (acc[t].m + log2f(lt)) / kLog2e;
  }
}

// Waves per work-group of the backward kernels.  The waves of a work-group
// share every staged step, so more waves re-read the streamed operands less
// often; measured on the 32B-shaped training layer, 8 waves made dq slower
// and dkv no faster than 4.
constexpr int kSoftQWaves = 4;
constexpr int kSoftKWaves = 4;
constexpr int kSoftQCols = 1;              // query tiles of 16 per wave (dQ)
constexpr int kSoftQTile = 16 * kSoftQCols * kSoftQWaves;  // queries per work-group (dQ)
constexpr int kSoftKT = 1;                   // key tiles of 16 per wave (dK, dV)
constexpr int kSoftKTile = 16 * kSoftKT * kSoftKWaves;      // keys per work-group (dK, dV)
constexpr int kSoftDqWavesPerEu = 2;  // waves per SIMD soft_dq_kernel's registers are sized for

// Backward, query-stationary: dq = scale * dS k with dS = P (dP - delta), P
// recomputed from the forward's lse, dP = dO v^T.  Each wave holds
// kSoftQCols tiles of 16 queries (columns) and streams the causal keys in
// pairs of 16-row blocks: S^T = k q^T and dP^T = v dO^T with the keys as rows,
// then dq^T += k^T dS^T with k^T from its pairT copy.  The 4 waves share each
// key pair: the work-group stages k and v rows (operand order), k^T and the
// keys' bias in LDS, double-buffered as in soft_dkv_kernel.  Grid (ceil(T /
// kSoftQTile), Hq, B).
// Pieces of one staged operand this thread moves (32 rows of D bf16 = 4 D
// pieces, NTH threads): row operands in fragment order, piece (blk * D / 32 +
// c) * 64 + l = row 16 blk + l % 16, bytes 64 c + 16 (l / 16); pairT
// operands are contiguous already.  Row offsets and piece slots are fixed per
// thread.
template <int D, int NTH>
struct SoftStagePieces {
  static constexpr int kN = (4 * D + NTH - 1) / NTH;  // pieces per thread per operand (slot < 4 D)
  int slot[kN];                           // piece index in the operand
  int row[kN];                            // row within the 32 (row operands)
  int col_bytes[kN];                      // byte offset within the row
  // Only when the threads outnumber the pieces does a slot fall outside.
  static __device__ __forceinline__ bool valid(int slot) { return (4 * D) % NTH == 0 || slot < 4 * D; }
  __device__ __forceinline__ SoftStagePieces(int tid) {
    constexpr int NCH = D / 32;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const int pc = tid + NTH * n, l = pc & 63;
      slot[n] = pc;
      row[n] = 16 * (pc / (NCH * 64)) + (l & 15);
      col_bytes[n] = 64 * ((pc / 64) % NCH) + 16 * (l >> 4);
    }
  }
};

template <int D>
struct SoftQStage {
  static constexpr int kOps = 3;                       // k rows, v rows, k^T
  static constexpr int kOpPieces = 32 * D * 2 / 16;
  u32x4 op[kOps][kOpPieces];
  float bias[32];
};

template <int D>
__global__ __launch_bounds__(64 * kSoftQWaves) __attribute__((amdgpu_waves_per_eu(kSoftDqWavesPerEu))) void soft_dq_kernel(
    SoftArgs a, const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const uint8_t* __restrict__ kt, const uint8_t* __restrict__ dO, const float* __restrict__ bias2,
    const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dq) {
  using St = SoftQStage<D>;
  using Pc = SoftStagePieces<D, 64 * kSoftQWaves>;
  constexpr int NCH = D / 32, NT = D / 16, NP = Pc::kN;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ St st[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z, hq = blockIdx.y, h = hq / a.G;
  const int T = a.T, w = a.w;
  const int npairs = (T + 31) / 32;
  const int q0 = blockIdx.x * kSoftQTile;
  const int qmax = min(q0 + kSoftQTile, T) - 1;
  const int cw0 = q0 + 16 * kSoftQCols * wave;  // the wave's first query
  const int64_t unit = (int64_t)b * a.Hkv + h;
  const int64_t urow = unit * T;
  const int64_t hrow = ((int64_t)b * a.Hq + hq) * T;
  const uint8_t* Ku = k + urow * D * 2;
  const uint8_t* Vu = v + urow * D * 2;
  const uint8_t* Kt = kt + unit * npairs * 32 * D * 2;
  const float* bu = bias2 + unit * npairs * 32;
  const int tb = 4 * (lane >> 4);
  const int nsteps = qmax / 32 + 1;
  const Pc pcs(tid);

  auto gload = [&](u32x4 (&r)[3][NP], float& bx, int s) {
    const int r0 = 32 * s;
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      if (!Pc::valid(pcs.slot[n])) continue;
      const int off = min(r0 + pcs.row[n], T - 1) * D * 2 + pcs.col_bytes[n];
      r[0][n] = *(const u32x4*)(Ku + off);
      r[1][n] = *(const u32x4*)(Vu + off);
      r[2][n] = *(const u32x4*)(Kt + (int64_t)s * 32 * D * 2 + pcs.slot[n] * 16);
    }
    if (tid < 32) bx = bu[r0 + tid];
  };
  auto lds_store = [&](St& S, const u32x4 (&r)[3][NP], float bx) {
#pragma unroll
    for (int o = 0; o < 3; ++o)
#pragma unroll
      for (int n = 0; n < NP; ++n)
        if (Pc::valid(pcs.slot[n])) S.op[o][pcs.slot[n]] = r[o][n];
    if (tid < 32) S.bias[tid] = bx;
  };

  int qc[kSoftQCols];
  float lse2[kSoftQCols], dl[kSoftQCols];
  u32x4 qf[kSoftQCols][NCH], of[kSoftQCols][NCH];
  f32x4 acc[kSoftQCols][NT];
#pragma unroll
  for (int t = 0; t < kSoftQCols; ++t) {
    const int c0 = q0 + 16 * (kSoftQCols * wave + t);
    qc[t] = c0 + (lane & 15);
    load_rows<D>(qf[t], q + hrow * D * 2, c0, T - 1, lane);
    load_rows<D>(of[t], dO + hrow * D * 2, c0, T - 1, lane);
    const int64_t r = hrow + min(qc[t], T - 1);
    lse2[t] = lse[r] * kLog2e;
    dl[t] = delta[r];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  u32x4 pre[3][NP];
  float prb = 0.f;
  gload(pre, prb, 0);
  lds_store(st[0], pre, prb);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) gload(pre, prb, s + 1);
    const St& S = st[s & 1];
    const int r0 = 32 * s;
    // every key of the pair is past the window of every query of the wave
    const bool far = r0 + 31 + w < cw0;
    u32x4 ka[NCH], kb[NCH], va[NCH], vb[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      ka[c] = S.op[0][c * 64 + lane];
      kb[c] = S.op[0][(NCH + c) * 64 + lane];
      va[c] = S.op[1][c * 64 + lane];
      vb[c] = S.op[1][(NCH + c) * 64 + lane];
    }
    const f32x4 ba = *(const f32x4*)&S.bias[tb], bb = *(const f32x4*)&S.bias[16 + tb];
#pragma unroll
    for (int t = 0; t < kSoftQCols; ++t) {
      f32x4 SA = {0.f, 0.f, 0.f, 0.f}, SB = SA, PA = SA, PB = SA;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        SA = mfma_bf16(ka[c], qf[t][c], SA);
        SB = mfma_bf16(kb[c], qf[t][c], SB);
        PA = mfma_bf16(va[c], of[t][c], PA);
        PB = mfma_bf16(vb[c], of[t][c], PB);
      }
      float ds[8];
      if (far) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float kb2 = r < 4 ? ba[r] : bb[r - 4];
          const float sv = r < 4 ? SA[r] : SB[r - 4];
          const float dp = r < 4 ? PA[r] : PB[r - 4];
          ds[r] = exp2_fast(fmaf(sv, a.scale_log2e, kb2 - lse2[t])) * (dp - dl[t]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int i = r0 + (r >> 2) * 16 + tb + (r & 3);
          const float kb2 = r < 4 ? ba[r] : bb[r - 4];
          const float badd = i > qc[t] ? -INFINITY : (qc[t] - i > w ? kb2 : 0.f);
          const float sv = r < 4 ? SA[r] : SB[r - 4];
          const float dp = r < 4 ? PA[r] : PB[r - 4];
          ds[r] = exp2_fast(fmaf(sv, a.scale_log2e, badd) - lse2[t]) * (dp - dl[t]);
        }
      }
      bf16x8 DH, DL;
      split_pair(ds, DH, DL);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const bf16x8 KT = __builtin_bit_cast(bf16x8, S.op[2][j * 64 + lane]);
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KT, DH, acc[t][j], 0, 0, 0);
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KT, DL, acc[t][j], 0, 0, 0);
      }
    }
    if (s + 1 < nsteps) lds_store(st[(s + 1) & 1], pre, prb);
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < kSoftQCols; ++t) {
    if (qc[t] >= T) continue;
    float* orow = dq + (hrow + qc[t]) * D + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NT; ++j) *(f32x4*)(orow + 16 * j) = acc[t][j] * a.scale;
  }
}

// Backward, key-stationary: for 16 keys per wave, over the G query heads of
// its KV head and every query at or after them, dv = P^T dO, dk = scale dS^T
// q and dlogit = -sigmoid(x) / tau * (sum of dS over the far queries).  S =
// q k^T and dP = dO v^T with the queries as rows (k, v rows stay in
// registers); dv^T += dO^T P and dk^T += q^T dS with dO^T, q^T from their
// pairT copies.  The 4 waves share each step's 32 queries: the work-group
// stages q and dO (rows and pairT, in operand order) and the rows' lse and
// delta in LDS, double-buffered, the next step's loads in flight during the
// current step's products.  No atomics: every key has one owner.  Grid
// (ceil(T / kSoftKTile), Hkv, B); the work-groups with the most queries
// start first.
template <int D>
struct SoftKvStage {
  static constexpr int kOps = 4;                       // q rows, dO rows, q^T, dO^T
  static constexpr int kOpPieces = 32 * D * 2 / 16;    // 16-byte pieces of one operand
  u32x4 op[kOps][kOpPieces];
  float lse2[32], delta[32];
};

template <int D>
__global__ __launch_bounds__(64 * kSoftKWaves) void soft_dkv_kernel(SoftArgs a, const uint8_t* __restrict__ q,
                                                       const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                                       const uint8_t* __restrict__ qt, const uint8_t* __restrict__ dO,
                                                       const uint8_t* __restrict__ dOt,
                                                       const float* __restrict__ logit,
                                                       const float* __restrict__ noise, const float* __restrict__ lse,
                                                       const float* __restrict__ delta, float* __restrict__ dk,
                                                       float* __restrict__ dv, float* __restrict__ dlogit) {
  using St = SoftKvStage<D>;
  using Pc = SoftStagePieces<D, 64 * kSoftKWaves>;
  constexpr int NCH = D / 32, NT = D / 16, NP = Pc::kN;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ St st[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z, h = blockIdx.y;
  const int T = a.T, w = a.w;
  const int nkt = (T + kSoftKTile - 1) / kSoftKTile;
  const int kbase = (nkt - 1 - (int)blockIdx.x) * kSoftKTile;
  constexpr int KT = kSoftKT;
  const int k0 = kbase + 16 * KT * wave;  // the wave's first key
  const int64_t urow = ((int64_t)b * a.Hkv + h) * T;
  const int npairs = (T + 31) / 32;
  const int tb = 4 * (lane >> 4);
  const int per_head = (T - kbase + 31) / 32;  // steps of 32 queries per query head
  const int nsteps = a.G * per_head;
  const Pc pcs(tid);

  // Step state (hq, q0), advanced without divisions.
  struct Pos {
    int hq, q0;
  };
  auto next = [&](Pos p) -> Pos {
    p.q0 += 32;
    if (p.q0 >= T) {
      p.q0 = kbase;
      ++p.hq;
    }
    return p;
  };
  auto gload = [&](u32x4 (&r)[4][NP], float& x, Pos p) {
    const int64_t head = (int64_t)b * a.Hq + p.hq;
    const uint8_t* Qh = q + head * T * D * 2;
    const uint8_t* Oh = dO + head * T * D * 2;
    const uint8_t* Qt = qt + (head * npairs + p.q0 / 32) * 32 * D * 2;
    const uint8_t* Ot = dOt + (head * npairs + p.q0 / 32) * 32 * D * 2;
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      if (!Pc::valid(pcs.slot[n])) continue;
      const int off = min(p.q0 + pcs.row[n], T - 1) * D * 2 + pcs.col_bytes[n];
      r[0][n] = *(const u32x4*)(Qh + off);
      r[1][n] = *(const u32x4*)(Oh + off);
      r[2][n] = *(const u32x4*)(Qt + pcs.slot[n] * 16);
      r[3][n] = *(const u32x4*)(Ot + pcs.slot[n] * 16);
    }
    if (tid < 64) {  // lse (0..31) and delta (32..63) of the step's rows
      // (scaled only when stored: arithmetic on a just-loaded value would
      // make the wave wait here for every load of the step)
      const int64_t row = head * T + min(p.q0 + (tid & 31), T - 1);
      x = (tid < 32 ? lse : delta)[row];
    }
  };
  auto lds_store = [&](St& S, const u32x4 (&r)[4][NP], float x) {
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
      for (int n = 0; n < NP; ++n)
        if (Pc::valid(pcs.slot[n])) S.op[o][pcs.slot[n]] = r[o][n];
    if (tid < 32) S.lse2[tid] = x * kLog2e;
    else if (tid < 64) S.delta[tid - 32] = x;
  };

  u32x4 kf[KT][NCH], vf[KT][NCH];
  int key[KT];
  float x[KT], kb2[KT], far_ds[KT];
  f32x4 ak[KT][NT], av[KT][NT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    key[kt] = k0 + 16 * kt + (lane & 15);
    load_rows<D>(kf[kt], k + urow * D * 2, k0 + 16 * kt, T - 1, lane);
    load_rows<D>(vf[kt], v + urow * D * 2, k0 + 16 * kt, T - 1, lane);
    x[kt] = soft_x(a, logit, noise, urow, min(key[kt], T - 1));
    kb2[kt] = soft_bias2(x[kt]);
    far_ds[kt] = 0.f;
#pragma unroll
    for (int j = 0; j < NT; ++j) ak[kt][j] = av[kt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  u32x4 pre[4][NP];
  float prx = 0.f;
  Pos cur{h * a.G, kbase};
  gload(pre, prx, cur);
  lds_store(st[0], pre, prx);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const Pos nx = next(cur);
    if (s + 1 < nsteps) gload(pre, prx, nx);
    const St& S = st[s & 1];
    const int q0 = cur.q0;
    u32x4 qa[NCH], qb[NCH], oa[NCH], ob[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qa[c] = S.op[0][c * 64 + lane];
      qb[c] = S.op[0][(NCH + c) * 64 + lane];
      oa[c] = S.op[1][c * 64 + lane];
      ob[c] = S.op[1][(NCH + c) * 64 + lane];
    }
    const f32x4 la = *(const f32x4*)&S.lse2[tb], lb = *(const f32x4*)&S.lse2[16 + tb];
    const f32x4 da = *(const f32x4*)&S.delta[tb], db = *(const f32x4*)&S.delta[16 + tb];
    bf16x8 PH[KT], PL[KT], DH[KT], DL[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      f32x4 SA = {0.f, 0.f, 0.f, 0.f}, SB = SA, PA = SA, PB = SA;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        SA = mfma_bf16(qa[c], kf[kt][c], SA);
        SB = mfma_bf16(qb[c], kf[kt][c], SB);
        PA = mfma_bf16(oa[c], vf[kt][c], PA);
        PB = mfma_bf16(ob[c], vf[kt][c], PB);
      }
      float pr[8], ds[8];
      if (q0 >= k0 + 16 * kt + 16 + w && q0 + 32 <= T) {
        // every query of the step is past the window of every key of the tile
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float sv = r < 4 ? SA[r] : SB[r - 4];
          const float dp = r < 4 ? PA[r] : PB[r - 4];
          const float l2 = r < 4 ? la[r] : lb[r - 4];
          const float dl = r < 4 ? da[r] : db[r - 4];
          pr[r] = exp2_fast(fmaf(sv, a.scale_log2e, kb2[kt] - l2));
          ds[r] = pr[r] * (dp - dl);
        }
        far_ds[kt] += ((ds[0] + ds[1]) + (ds[2] + ds[3])) + ((ds[4] + ds[5]) + (ds[6] + ds[7]));
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int qi = q0 + (r >> 2) * 16 + tb + (r & 3);
          const float badd = (qi < key[kt] || qi >= T) ? -INFINITY : (qi - key[kt] > w ? kb2[kt] : 0.f);
          const float sv = r < 4 ? SA[r] : SB[r - 4];
          const float dp = r < 4 ? PA[r] : PB[r - 4];
          const float l2 = r < 4 ? la[r] : lb[r - 4];
          const float dl = r < 4 ? da[r] : db[r - 4];
          pr[r] = exp2_fast(fmaf(sv, a.scale_log2e, badd) - l2);
          ds[r] = pr[r] * (dp - dl);
          if (qi - key[kt] > w) far_ds[kt] += ds[r];
        }
      }
      split_pair(pr, PH[kt], PL[kt]);
      split_pair(ds, DH[kt], DL[kt]);
    }
    // Raised issue priority over the gradient products, so that another
    // wave's softmax arithmetic on the same SIMD does not delay their issue
    // (measured: the backward pass about 3% faster than without).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const bf16x8 OT = __builtin_bit_cast(bf16x8, S.op[3][j * 64 + lane]);
      const bf16x8 QT = __builtin_bit_cast(bf16x8, S.op[2][j * 64 + lane]);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        av[kt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(OT, PH[kt], av[kt][j], 0, 0, 0);
        av[kt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(OT, PL[kt], av[kt][j], 0, 0, 0);
        ak[kt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(QT, DH[kt], ak[kt][j], 0, 0, 0);
        ak[kt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(QT, DL[kt], ak[kt][j], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (s + 1 < nsteps) lds_store(st[(s + 1) & 1], pre, prx);
    __syncthreads();
    cur = nx;
  }
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    float fd = far_ds[kt] + __shfl_xor(far_ds[kt], 16);
    fd += __shfl_xor(fd, 32);
    if (key[kt] >= T) continue;
    float* krow = dk + (urow + key[kt]) * D + 4 * (lane >> 4);
    float* vrow = dv + (urow + key[kt]) * D + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      *(f32x4*)(krow + 16 * j) = ak[kt][j] * a.scale;
      *(f32x4*)(vrow + 16 * j) = av[kt][j];
    }
    if (lane < 16) dlogit[urow + key[kt]] = -sigmoid_f(x[kt]) * a.inv_tau * fd;
  }
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
// pending slots come from the ring into a per-block bitmap in LDS.
//
// Work-group = 4 waves = one (sequence, KV head) unit and kPfTile columns;
// column c = j G + g carries query head h G + g of chunk position j, so the
// group's heads share every loaded block as in the decode kernel.
constexpr int kChunkMaxBlocks = 8192;

// NC tiles of 16 columns per wave.  Grid (U, ceil(chunk G / (64 NC))).
// q [B, Hq, chunk, d]; k, v [B, Hkv,
// chunk, d]; logit [B, Hkv, chunk]; out [B, Hq, chunk, d].
//
// The work-group's columns need 1 to 4 waves of NC tiles each.  When
// they fit in one or two waves, the idle waves split the key stream instead
// (4 or 2 ways: wave w takes every nsplit-th pair of blocks and of chunk
// rows), and the waves of one tile group merge their softmax states through
// LDS at the end, tile by tile.
template <int ES, int D, int NC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NC == 1 && ES == 2 ? 2 : 1))) void chunk_attention_kernel(Dev p, const uint8_t* __restrict__ q,
                                                              const uint8_t* __restrict__ k,
                                                              const uint8_t* __restrict__ v, LogitSrc logit,
                                                              int zero_ch, int chunk, float* __restrict__ out) {
  using G = Geo<ES, D>;
  __shared__ uint32_t pend[kChunkMaxBlocks];
  __shared__ f32x4 mo[kWavesPerWG - 1][G::kTiles][64];
  __shared__ float mm[kWavesPerWG - 1][64], ml[kWavesPerWG - 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int u = blockIdx.x;
  const int b = u / p.Hkv, h = u - b * p.Hkv;
  const int n = __builtin_amdgcn_readfirstlane(p.n[u]);
  const int nb = (n + 15) >> 4;
  const int q0 = __builtin_amdgcn_readfirstlane(p.pos[u]);
  const int w = p.R - 1;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) pend[i] = 0u;
  __syncthreads();
  const int32_t* ring = p.ring + (int64_t)u * p.R;
  for (int r = threadIdx.x; r < p.R; r += blockDim.x) {
    const int sl = ring[r];
    if (sl >= 0 && sl < n) atomicOr(&pend[sl >> 4], 1u << (sl & 15));
  }
  __syncthreads();

  const int ncol = chunk * p.G;
  const int cwg = blockIdx.y * (16 * NC * kWavesPerWG);
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

  // Cached tokens: this wave's pairs of blocks i = sp, sp + nsplit, ...,
  // one pair loaded ahead of the one computed.  Loads are unconditional
  // (clamped indices; a pair past the wave's last is masked out).
  const int32_t* bt = p.btab + (int64_t)u * p.max_blocks;
  const int npair = (nb + 1) >> 1;
  const int cnt = sp < npair ? (npair - sp + nsplit - 1) / nsplit : 0;
  if (cnt > 0) {
    struct Meta {
      int4 pa, pb;
      uint32_t wa, wb;
    };
    auto fetch = [&](PairFrag<ES, D>& f, Meta& m, int kk) {
      const int i = min(sp + nsplit * kk, npair - 1);
      const int ja = 2 * i, jb = min(2 * i + 1, nb - 1);
      const int ba = __builtin_amdgcn_readfirstlane(bt[ja]), bb = __builtin_amdgcn_readfirstlane(bt[jb]);
      load_pair<ES, D>(f, p.pool + (int64_t)ba * p.block_bytes, p.pool + (int64_t)bb * p.block_bytes, lane);
      m.pa = *(const int4*)(p.blk_pos + (int64_t)ba * 16 + tb);
      m.pb = *(const int4*)(p.blk_pos + (int64_t)bb * 16 + tb);
      m.wa = pend[ja];
      m.wb = pend[jb];
    };
    auto compute = [&](const PairFrag<ES, D>& f, const Meta& m, int kk) {
      const int i = sp + nsplit * kk;
      const bool ok = i < npair;
      const int ja = 2 * i;
      const int lva = ok ? n - 16 * ja : 0, lvb = ok && ja + 1 < nb ? n - 16 * (ja + 1) : 0;
      const int xa[4] = {m.pa.x, m.pa.y, m.pa.z, m.pa.w}, xb[4] = {m.pb.x, m.pb.y, m.pb.z, m.pb.w};
#pragma unroll
      for (int t = 0; t < NC; ++t) {
        const int lt = q0 + qj[t] - w;  // a pending token is visible from position >= lt
        uint32_t ma = 0, mb = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int bit = tb + r;
          if (bit < lva && (!((m.wa >> bit) & 1u) || xa[r] >= lt)) ma |= 1u << bit;
          if (bit < lvb && (!((m.wb >> bit) & 1u) || xb[r] >= lt)) mb |= 1u << bit;
        }
        attend_pair<ES, D>(f, qf[t], ma, mb, lane, p.scale_log2e, acc[t]);
      }
    };
    PairFrag<ES, D> f0, f1;
    Meta m0, m1;
    fetch(f0, m0, 0);
    for (int kk = 0; kk < cnt; kk += 2) {
      fetch(f1, m1, kk + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(f0, m0, kk);
      if (kk + 1 >= cnt) break;
      fetch(f0, m0, kk + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(f1, m1, kk + 1);
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

template <int ES, int D>
static hipError_t prefill_attention_t(const Dev& p, const void* q, const void* k, const void* v, int32_t max_len,
                                      int32_t max_prompt, int zero_ch, float* out, hipStream_t s) {
  const dim3 grid((unsigned)((max_prompt + kPfTile - 1) / kPfTile), (unsigned)p.Hq, (unsigned)p.B);
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

// Columns per wave of the chunk attention: one tile when the chunk's columns
// (chunk x G) fit in it; every wave then streams a quarter of the keys, and
// two work-groups stay resident per CU.  Three tiles beyond, so that more
// columns share every loaded block.  (Measured on the 32B-shaped layer, G =
// 5: one tile was faster for chunks of 1, three tiles for 4 and 12.)
constexpr int kChunkSmallCols = 16;

template <int ES, int D, int NC>
static hipError_t chunk_attention_t(const Dev& p, const void* q, const void* k, const void* v, const LogitSrc& logit,
                                    int zero_ch, int chunk, float* out, hipStream_t s) {
  const int ytiles = (chunk * p.G + 64 * NC - 1) / (64 * NC);
  return launch(chunk_attention_kernel<ES, D, NC>, dim3((unsigned)p.U, (unsigned)ytiles), dim3(64 * kWavesPerWG), s,
                p, (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, logit, zero_ch, chunk, out);
}

template <int ES, int D>
static hipError_t decode_chunk_t(const Dev& p, const void* q, const void* k, const void* v, const LogitSrc& logit,
                                 int zero_ch, int chunk, float* out, hipStream_t s) {
  const hipError_t e = chunk * p.G <= kChunkSmallCols
                           ? chunk_attention_t<ES, D, 1>(p, q, k, v, logit, zero_ch, chunk, out, s)
                           : chunk_attention_t<ES, D, 3>(p, q, k, v, logit, zero_ch, chunk, out, s);
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

static int64_t soft_pairT_bytes(int T, int d) { return (int64_t)((T + 31) / 32) * 32 * d * 2; }
static int64_t soft_bias_bytes(int B, int Hkv, int T) { return (int64_t)B * Hkv * ((T + 31) / 32) * 32 * 4; }

int64_t soft_forward_workspace_bytes(int B, int Hq, int Hkv, int T, int d) {
  (void)Hq;
  return (int64_t)B * Hkv * soft_pairT_bytes(T, d) + soft_bias_bytes(B, Hkv, T);
}

int64_t soft_backward_workspace_bytes(int B, int Hq, int Hkv, int T, int d) {
  // pairT copies of q and dO (per query head) and of k (per KV head), delta, bias
  const int64_t pt = soft_pairT_bytes(T, d);
  const int64_t copies = ((int64_t)B * Hq * 2 + (int64_t)B * Hkv) * pt;
  return copies + (int64_t)B * Hq * T * 4 + soft_bias_bytes(B, Hkv, T);
}

static hipError_t soft_bias(const SoftArgs& a, const float* logit, const float* noise, float* bias2, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.Hkv * ((a.T + 31) / 32) * 32;
  return launch(soft_bias_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), s, a, logit, noise, bias2);
}

template <int D>
static hipError_t soft_forward_t(const SoftArgs& a, const void* q, const void* k, const void* v, const float* logit,
                                 const float* noise, float* out, float* lse, uint8_t* ws, hipStream_t s) {
  uint8_t* vt = ws;
  float* bias2 = (float*)(vt + (int64_t)a.B * a.Hkv * soft_pairT_bytes(a.T, D));
  const unsigned npairs = (unsigned)((a.T + 31) / 32);
  hipError_t e = launch(soft_pack_kernel<D>, dim3((unsigned)(a.B * a.Hkv), npairs), dim3(256), s,
                        (const uint16_t*)v, vt, a.T, (const float*)nullptr, (float*)nullptr);
  if (e == hipSuccess) e = soft_bias(a, logit, noise, bias2, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((a.T + kPfTile - 1) / kPfTile), (unsigned)a.Hq, (unsigned)a.B);
  return launch(soft_forward_kernel<D>, grid, dim3(64 * kWavesPerWG), s, a, (const uint8_t*)q, (const uint8_t*)k,
                (const uint8_t*)vt, (const float*)bias2, out, lse);
}

hipError_t launch_soft_forward(const SoftArgs& a, int d, const void* q, const void* k, const void* v,
                               const float* logit, const float* noise, float* out, float* lse, void* ws,
                               hipStream_t s) {
  return d == 128 ? soft_forward_t<128>(a, q, k, v, logit, noise, out, lse, (uint8_t*)ws, s)
                  : soft_forward_t<64>(a, q, k, v, logit, noise, out, lse, (uint8_t*)ws, s);
}

// Allocation-free relaxed forward: its scratch (v's transposed copy and the
// keys' biases, soft_forward_workspace_bytes) lives in this file-scope device
// array instead of a caller workspace.  Host code never passes the array's
// name to a kernel (there it is a host-side stand-in): its address on each
// device is looked up once, with that device current, and kept.
constexpr int64_t kSoftScratchBytes = 64ll << 20;
static __device__ __align__(256) uint8_t scratch[kSoftScratchBytes];

int64_t soft_scratch_bytes() { return kSoftScratchBytes; }

void* soft_scratch_address(int dev) {
  constexpr int kMaxDevices = 256;
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = ptrs[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(mu);
  ptr = ptrs[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    ptrs[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

template <int D>
static hipError_t soft_backward_t(const SoftArgs& a, const void* q, const void* k, const void* v,
                                  const float* logit, const float* noise, const float* out, const float* lse,
                                  const void* dout, float* dq, float* dk, float* dv, float* dlogit, uint8_t* ws,
                                  hipStream_t s) {
  const int64_t pt = soft_pairT_bytes(a.T, D);
  uint8_t* qt = ws;
  uint8_t* ot = qt + (int64_t)a.B * a.Hq * pt;
  uint8_t* kt = ot + (int64_t)a.B * a.Hq * pt;
  float* delta = (float*)(kt + (int64_t)a.B * a.Hkv * pt);
  float* bias2 = delta + (int64_t)a.B * a.Hq * a.T;
  const unsigned npairs = (unsigned)((a.T + 31) / 32);
  hipError_t e = launch(soft_pack_kernel<D>, dim3((unsigned)(a.B * a.Hq), npairs), dim3(256), s,
                        (const uint16_t*)q, qt, a.T, (const float*)nullptr, (float*)nullptr);
  if (e == hipSuccess)
    e = launch(soft_pack_kernel<D>, dim3((unsigned)(a.B * a.Hq), npairs), dim3(256), s, (const uint16_t*)dout, ot,
               a.T, out, delta);
  if (e == hipSuccess)
    e = launch(soft_pack_kernel<D>, dim3((unsigned)(a.B * a.Hkv), npairs), dim3(256), s, (const uint16_t*)k, kt,
               a.T, (const float*)nullptr, (float*)nullptr);
  if (e == hipSuccess) e = soft_bias(a, logit, noise, bias2, s);
  if (e == hipSuccess)
    e = launch(soft_dq_kernel<D>, dim3((unsigned)((a.T + kSoftQTile - 1) / kSoftQTile), (unsigned)a.Hq, (unsigned)a.B),
               dim3(64 * kSoftQWaves), s, a, (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v,
               (const uint8_t*)kt, (const uint8_t*)dout, (const float*)bias2, lse, (const float*)delta, dq);
  if (e == hipSuccess)
    e = launch(soft_dkv_kernel<D>, dim3((unsigned)((a.T + kSoftKTile - 1) / kSoftKTile), (unsigned)a.Hkv,
                                        (unsigned)a.B),
               dim3(64 * kSoftKWaves), s, a, (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v,
               (const uint8_t*)qt, (const uint8_t*)dout, (const uint8_t*)ot, logit, noise, lse, (const float*)delta,
               dk, dv, dlogit);
  return e;
}

hipError_t launch_soft_backward(const SoftArgs& a, int d, const void* q, const void* k, const void* v,
                                const float* logit, const float* noise, const float* out, const float* lse,
                                const void* dout, float* dq, float* dk, float* dv, float* dlogit, void* ws,
                                hipStream_t s) {
  return d == 128 ? soft_backward_t<128>(a, q, k, v, logit, noise, out, lse, dout, dq, dk, dv, dlogit,
                                         (uint8_t*)ws, s)
                  : soft_backward_t<64>(a, q, k, v, logit, noise, out, lse, dout, dq, dk, dv, dlogit,
                                        (uint8_t*)ws, s);
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
  const dim3 rgrid((p.U + kWavesPerWG - 1) / kWavesPerWG);
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
