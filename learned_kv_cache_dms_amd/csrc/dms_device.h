// Device code shared by the DMS kernels for gfx950 (MI355X): launch helpers,
// wave and lane-group helpers, the cache block's fragment layout with its
// loads and the attention step over one or two blocks, and the token store
// that every append path uses.
//
// Method: "Inference-Time Hyper-Scaling with KV Cache Compression", paper
// summary page, "Key claims" and "Method".  Each KV head decides per token
// whether to evict it (alpha = 1 when the eviction logit is > 0); a marked
// token stays attendable for w more steps, then leaves the cache.  Attention
// reads only what is still visible, so the additive mask is never built.
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
// Attention step over a block (the MFMA output layout: lane l holds tokens
// 4*(l/16)+r of column l % 16, exp2-domain online softmax):
//   S[t][g]  = K_blk[t] . Q[g]      MFMA, A = K fragment, B = Q fragment
//   O^T[c][g] += V^T[c][t] P[t][g]  MFMA, A = V fragment, B = P taken in
//            place from the S registers (bf16: P split into hi + lo parts)
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <tuple>
#include <type_traits>
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

// A load of a uniform address through the scalar cache (constant address
// space): the address must not be written by this kernel before the load.
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ int scalar_load(const int32_t* a) { return *(const_i32*)(uintptr_t)a; }

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

// Loads blocks A and B of the pool (fragment order) as a pair.  kStream: with
// the non-temporal hint, for a stream that reads each block about once;
// false: plain loads, for kernels whose waves and work-groups re-read the
// same blocks close together.  Measured on the 32B-shaped layer: the prompt
// attention 196.7 -> 172.5 ms with plain loads; the chunk attention faster
// with the hint at C = 1, 4, 8, 12 and 64 (3-10 %), and with plain loads at
// C = 16 (0.343 -> 0.325 ms), where two groups of column tiles in a
// work-group each read every pair.
template <int ES, int D, bool kStream = true>
__device__ __forceinline__ void load_pair(PairFrag<ES, D>& f, const uint8_t* blka, const uint8_t* blkb, int lane) {
  using G = Geo<ES, D>;
  auto ld = [](const auto* ptr) {
    if constexpr (kStream) return __builtin_nontemporal_load(ptr);
    else return *ptr;
  };
  if constexpr (ES == 2) {
    const uint8_t* a = blka + lane * 16;
    const uint8_t* b = blkb + lane * 16;
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) f.ka[c] = ld((const u32x4*)(a + c * 1024));
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) f.kb[c] = ld((const u32x4*)(b + c * 1024));
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x2 x = ld((const u32x2*)(a + G::kHalf + c * 1024 + jj * 8));
        const u32x2 y = ld((const u32x2*)(b + G::kHalf + c * 1024 + jj * 8));
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

// Work-group = 4 waves = kPfTile consecutive queries of one query head; wave
// w owns kPfCols tiles of 16 queries, one query per MFMA column (where the
// decode packs the group's heads), and streams the same key blocks as the
// other waves.
constexpr int kPfCols = 3;
constexpr int kPfTile = 16 * kPfCols * kWavesPerWG;

}  // namespace dms
