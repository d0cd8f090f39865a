// Device twin of synth/synth.py: the same counter-based values, bit for bit,
// generated in HBM so large synthetic workloads need no host round trip.
// Holds no arithmetic of the decode path.  See synth.py for the definition.
// Also a plain streaming read (read_kernel) with which the bench measures the
// HBM read ceiling that the decode attention is compared with.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t flat_index(uint64_t layer, uint64_t b, uint64_t head, uint64_t pos,
                                               uint64_t ch) {
  return ((((layer * 1024ull + b) * 64ull + head) * (1ull << 20) + pos) * 128ull + ch);
}

__device__ __forceinline__ float normal_at(uint64_t seed, uint64_t stream, uint64_t idx) {
  const uint64_t base = seed ^ (stream << 56);
  int64_t s = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const uint64_t z = splitmix64(base ^ (3ull * idx + (uint64_t)j));
    s += (int64_t)(z & 0xFFFF) + (int64_t)((z >> 16) & 0xFFFF) + (int64_t)((z >> 32) & 0xFFFF) +
         (int64_t)(z >> 48);
  }
  return (float)(2 * s - 786420) * 0x1p-17f;
}

__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

struct Shape {
  uint64_t seed;
  int stream, layer, b0, nb, heads, pos0, npos, channels;
  const int32_t* pos_base;  // [nb] per-sequence first position, or null (use pos0)
};

__device__ __forceinline__ void coords(const Shape& s, int64_t i, int& bi, int& h, int& pi, int& c) {
  c = (int)(i % s.channels);
  int64_t r = i / s.channels;
  pi = (int)(r % s.npos);
  r /= s.npos;
  h = (int)(r % s.heads);
  bi = (int)(r / s.heads);
}

__global__ void fill_kernel(Shape s, void* out, int bf16, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    int bi, h, pi, c;
    coords(s, i, bi, h, pi, c);
    const int pos = (s.pos_base ? s.pos_base[bi] : s.pos0) + pi;
    const float x = normal_at(s.seed, (uint64_t)s.stream, flat_index(s.layer, s.b0 + bi, h, pos, c));
    if (bf16)
      ((uint16_t*)out)[i] = bf16_rne_bits(x);
    else
      ((float*)out)[i] = x;
  }
}

struct Mu {
  double before[64];
  double after[64];
};

__global__ void logit_kernel(Shape s, float* out, Mu mu, int pos_threshold, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    int bi, h, pi, c;
    coords(s, i, bi, h, pi, c);
    const int pos = (s.pos_base ? s.pos_base[bi] : s.pos0) + pi;
    const float x = normal_at(s.seed, 3ull, flat_index(s.layer, s.b0 + bi, h, pos, 0));
    const double m = pos < pos_threshold ? mu.before[h] : mu.after[h];
    out[i] = __double2float_rn(m + (double)x);
  }
}

int grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

// Reads n16 16-byte words as a decode attention reads its blocks (16 bytes
// per lane, nontemporal, four loads in flight per thread, the grid striding
// over the buffer) and folds them by XOR into one word per work-group, so
// that no load can be dropped; nothing else.
typedef unsigned int u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned int))));

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t fold = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __shared__ uint32_t part[256];
  part[threadIdx.x] = fold;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int t = 0; t < 256; ++t) x ^= part[t];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

extern "C" {

__attribute__((visibility("default")))
// Fills out[nb][heads][npos][channels] (fp32, or bf16 when bf16 != 0) with
// the values of (seed, stream) at layer, sequences b0.., positions
// pos_base[bi] (device array, may be null -> pos0) + 0..npos-1.
int synth_fill(void* d_out, int bf16, uint64_t seed, int stream, int layer, int b0, int nb, int heads,
               const int32_t* d_pos_base, int pos0, int npos, int channels, void* hip_stream) {
  if (!d_out || nb < 0 || heads < 1 || heads > 64 || npos < 0 || channels < 1 || channels > 128) return -1;
  Shape s{seed, stream, layer, b0, nb, heads, pos0, npos, channels, d_pos_base};
  const int64_t total = (int64_t)nb * heads * npos * channels;
  if (total == 0) return 0;
  void* args[] = {&s, &d_out, &bf16, (void*)&total};
  return hipLaunchKernel((const void*)fill_kernel, dim3(grid_for(total)), dim3(256), args, 0,
                         (hipStream_t)hip_stream) == hipSuccess ? 0 : -6;
}

__attribute__((visibility("default")))
// Eviction logits out[nb][heads][npos] = float32(mu + x), mu per head from
// mu_before (positions < pos_threshold) or mu_after.
int synth_logits(float* d_out, uint64_t seed, int layer, int b0, int nb, int heads, const int32_t* d_pos_base,
                 int pos0, int npos, const double* h_mu_before, const double* h_mu_after, int pos_threshold,
                 void* hip_stream) {
  if (!d_out || !h_mu_before || !h_mu_after || nb < 0 || heads < 1 || heads > 64 || npos < 0) return -1;
  Shape s{seed, 3, layer, b0, nb, heads, pos0, npos, 1, d_pos_base};
  Mu mu;
  for (int h = 0; h < 64; ++h) {
    mu.before[h] = h < heads ? h_mu_before[h] : 0.0;
    mu.after[h] = h < heads ? h_mu_after[h] : 0.0;
  }
  const int64_t total = (int64_t)nb * heads * npos;
  if (total == 0) return 0;
  void* args[] = {&s, &d_out, &mu, &pos_threshold, (void*)&total};
  return hipLaunchKernel((const void*)logit_kernel, dim3(grid_for(total)), dim3(256), args, 0,
                         (hipStream_t)hip_stream) == hipSuccess ? 0 : -6;
}

// Streams n_bytes (a multiple of 16) of d_src once with `grid` work-groups;
// d_sink receives `grid` words.
__attribute__((visibility("default"))) int synth_read(const void* d_src, int64_t n_bytes, int grid,
                                                      uint32_t* d_sink, hipStream_t stream) {
  if (!d_src || !d_sink || n_bytes <= 0 || n_bytes % 16 != 0 || grid < 1) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, stream, (const u32x4*)d_src, n_bytes / 16, d_sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
