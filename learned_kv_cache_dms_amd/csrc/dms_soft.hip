// Training-time relaxed DMS attention for gfx950 (MI355X): the decisions as
// a differentiable soft mask (Gumbel-sigmoid), forward and backward, and the
// allocation-free forward whose scratch is a built-in device array.
#include "dms_device.h"

namespace dms {
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
// A column's reference max m moves only when a score exceeds it by more than
// 2^kSoftSlack (exp2 domain): the weights stay below 2^kSoftSlack, o and l are
// kept relative to m, and lse = m + log2 l holds for any such m.  Each lane
// tests its own 8 scores first (NaN-propagating maximum, v_maximum3_f32, which
// takes its operands unquieted; scores are finite or -inf); the column max
// across the four lane groups and the rescale run only when some lane of the
// wave grows.  Measured on the 32B-shaped training layer: forward 1.527 ->
// 1.42-1.47 ms against the running exact max.
constexpr float kSoftSlack = 8.0f;
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
  auto mx = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
  const float lm = mx(mx(mx(s[0], s[1]), mx(s[2], s[3])), mx(mx(s[4], s[5]), mx(s[6], s[7])));
  if (__builtin_amdgcn_ballot_w64(lm > a.m + kSoftSlack) != 0) {
    const float bm = max_over_groups(lm);
    const bool grow = bm > a.m + kSoftSlack;
    const float mn = grow ? bm : a.m;
    const float alpha = grow ? exp2_fast(a.m - mn) : 1.0f;
    a.l *= alpha;
#pragma unroll
    for (int j = 0; j < G::kTiles; ++j) a.o[j] *= alpha;
    a.m = mn;
  }
  const float mref = (a.m == -INFINITY) ? 0.f : a.m;
  float pr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) pr[r] = exp2_fast(s[r] - mref);
  a.l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
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
// (ceil(T / kPfTile), Hq, B), read as one list of work items (xcd_item); the
// last query tiles of a (sequence, head), with the most keys, go first.
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

// 8 fp32 values in the pair order rounded to bf16 (nearest even, 2^-8
// relative at most), the B operand of a product over the pair's rows.  The
// backward's gradient products take P and dS this way: their error is at
// most 2^-8 of the sum of the terms' magnitudes (e.g. of P^T |dO| for dV).
// Measured on the 32B-shaped training layer, keeping a lo part as well (x =
// hi + lo to about 2^-17) made the backward 15 % slower.
__device__ __forceinline__ bf16x8 round_pair(const float (&x)[8]) {
  const u32x4 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, v);
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

// Work item (x, y, z) of this work-group, the grid read as one list of items
// x + X (y + Y z): work-group i runs on XCD i mod 8, and each XCD takes a
// contiguous run of items.  The kernels below put the (sequence, head) in y
// and z, so a unit's work-groups share one XCD's L2 for the operands they all
// stream (its keys and values, or its queries and output gradients).
// Against the grid's own order on the 32B-shaped training layer: forward
// 1.48 -> 1.32-1.38 ms, backward 5.36 -> 3.77 ms.
__device__ __forceinline__ int3 xcd_item() {
  const int X = gridDim.x, Y = gridDim.y, n = X * Y * gridDim.z;
  const int lin = blockIdx.x + X * (blockIdx.y + Y * blockIdx.z);
  const int xcd = lin & 7, it = xcd * (n >> 3) + min(xcd, n & 7) + (lin >> 3);
  return int3{it % X, (it / X) % Y, it / (X * Y)};
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
  const int3 wi = xcd_item();
  const int b = wi.z, hq = wi.y, h = hq / a.G;
  const int T = a.T, w = a.w;
  const int npairs = (T + 31) / 32;
  const int q0 = ((int)gridDim.x - 1 - wi.x) * kPfTile;
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
// share every staged step, so more waves stage the streamed operands less
// often; measured on the 32B-shaped training layer, 8 waves made dkv about
// 4 % faster than 4 (and 4 waves, or 2 key tiles per wave at 4 waves, 12-16 %
// slower in the XCD-aware order), and dq 3 % faster once the work items were
// dealt XCD-aware (3.48 against 3.60 ms; before, 8 waves had made it slower).
// dq then took 12 waves (three per SIMD, which its registers allow): the
// backward 2 % faster again (3.52 against 3.59 ms).  With the staged key
// fragments read one channel chunk at a time (48 registers fewer), two query
// tiles per dq wave fit the registers of two waves per SIMD: each staged
// fragment then feeds twice the products, and the backward went from 3.49 to
// 3.36 ms against the twelve-wave, one-tile dq (the chunked reads alone
// changed nothing).
constexpr int kSoftQWaves = 8;
constexpr int kSoftKWaves = 8;
constexpr int kSoftQCols = 2;              // query tiles of 16 per wave (dQ)
constexpr int kSoftQTile = 16 * kSoftQCols * kSoftQWaves;  // queries per work-group (dQ)
constexpr int kSoftKT = 1;                   // key tiles of 16 per wave (dK, dV)
constexpr int kSoftKTile = 16 * kSoftKT * kSoftKWaves;      // keys per work-group (dK, dV)
constexpr int kSoftDqWavesPerEu = 2;  // waves per SIMD soft_dq_kernel's registers are sized for

// Backward, query-stationary: dq = scale * dS k with dS = P (dP - delta), P
// recomputed from the forward's lse, dP = dO v^T.  Each wave holds
// kSoftQCols tiles of 16 queries (columns) and streams the causal keys in
// pairs of 16-row blocks: S^T = k q^T and dP^T = v dO^T with the keys as rows,
// then dq^T += k^T dS^T with k^T from its pairT copy (dS rounded to bf16).
// The kSoftQWaves waves share each key pair: the work-group stages k and v rows
// (operand order), k^T and the keys' bias in LDS, double-buffered as in
// soft_dkv_kernel.  Grid (ceil(T / kSoftQTile), Hq, B), read as one list of
// work items (xcd_item), the last query tiles of a (sequence, head) first.
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
  const int3 wi = xcd_item();
  const int b = wi.z, hq = wi.y, h = hq / a.G;
  const int T = a.T, w = a.w;
  const int npairs = (T + 31) / 32;
  const int q0 = ((int)gridDim.x - 1 - wi.x) * kSoftQTile;
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
    const f32x4 ba = *(const f32x4*)&S.bias[tb], bb = *(const f32x4*)&S.bias[16 + tb];
    f32x4 SA[kSoftQCols], SB[kSoftQCols], PA[kSoftQCols], PB[kSoftQCols];
#pragma unroll
    for (int t = 0; t < kSoftQCols; ++t) SA[t] = SB[t] = PA[t] = PB[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const u32x4 ka = S.op[0][c * 64 + lane], kb = S.op[0][(NCH + c) * 64 + lane];
      const u32x4 va = S.op[1][c * 64 + lane], vb = S.op[1][(NCH + c) * 64 + lane];
#pragma unroll
      for (int t = 0; t < kSoftQCols; ++t) {
        SA[t] = mfma_bf16(ka, qf[t][c], SA[t]);
        SB[t] = mfma_bf16(kb, qf[t][c], SB[t]);
        PA[t] = mfma_bf16(va, of[t][c], PA[t]);
        PB[t] = mfma_bf16(vb, of[t][c], PB[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < kSoftQCols; ++t) {
      float ds[8];
      if (far) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float kb2 = r < 4 ? ba[r] : bb[r - 4];
          const float sv = r < 4 ? SA[t][r] : SB[t][r - 4];
          const float dp = r < 4 ? PA[t][r] : PB[t][r - 4];
          ds[r] = exp2_fast(fmaf(sv, a.scale_log2e, kb2 - lse2[t])) * (dp - dl[t]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int i = r0 + (r >> 2) * 16 + tb + (r & 3);
          const float kb2 = r < 4 ? ba[r] : bb[r - 4];
          const float badd = i > qc[t] ? -INFINITY : (qc[t] - i > w ? kb2 : 0.f);
          const float sv = r < 4 ? SA[t][r] : SB[t][r - 4];
          const float dp = r < 4 ? PA[t][r] : PB[t][r - 4];
          ds[r] = exp2_fast(fmaf(sv, a.scale_log2e, badd) - lse2[t]) * (dp - dl[t]);
        }
      }
      const bf16x8 DS = round_pair(ds);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const bf16x8 KT = __builtin_bit_cast(bf16x8, S.op[2][j * 64 + lane]);
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KT, DS, acc[t][j], 0, 0, 0);
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
// pairT copies (P and dS rounded to bf16).  The kSoftKWaves waves share
// each step's 32 queries: the work-group
// stages q and dO (rows and pairT, in operand order) and the rows' lse and
// delta in LDS, double-buffered, the next step's loads in flight during the
// current step's products.  No atomics: every key has one owner.  Grid
// (ceil(T / kSoftKTile), Hkv, B), read as one list of work items
// (xcd_item); within a unit the key tiles with the most queries go first
// (backward 3.77 ms, against 4.31 ms the other way round).
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
  const int3 wi = xcd_item();
  const int b = wi.z, h = wi.y;
  const int T = a.T, w = a.w;
  const int nkt = (T + kSoftKTile - 1) / kSoftKTile;
  const int kbase = wi.x * kSoftKTile;
  constexpr int KT = kSoftKT;
  const int k0 = kbase + 16 * KT * wave;  // the wave's first key
  const int64_t urow = ((int64_t)b * a.Hkv + h) * T;
  const int npairs = (T + 31) / 32;
  const int tb = 4 * (lane >> 4);
  const int per_head = (T - kbase + 31) / 32;  // steps of 32 queries per query head
  const int nsteps = a.G * per_head;
  const Pc pcs(tid);

  // Step state (hq, q0), advanced without divisions: the query steps from
  // the last one down to kbase, the G query heads of each step one after
  // another.  Every work-group of a unit walks the same sequence of steps
  // (each stops at its own kbase), so the work-groups of a unit that run at
  // once read each staged step from the XCD's L2 together.
  struct Pos {
    int hq, q0;
  };
  const int hq0 = h * a.G, qtop = 32 * ((T - 1) / 32);
  auto next = [&](Pos p) -> Pos {
    if (++p.hq == hq0 + a.G) {
      p.hq = hq0;
      p.q0 -= 32;
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
  Pos cur{hq0, qtop};
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
    bf16x8 PB16[KT], DS16[KT];
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
      PB16[kt] = round_pair(pr);
      DS16[kt] = round_pair(ds);
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
        av[kt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(OT, PB16[kt], av[kt][j], 0, 0, 0);
        ak[kt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(QT, DS16[kt], ak[kt][j], 0, 0, 0);
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
// launchers
// ---------------------------------------------------------------------------

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

}  // namespace dms
