// Host runtime behind the C ABI in include/dms.h: argument and state
// validation, workspace layout, launch geometry, status mapping, and the
// host side of stats / export.  All device work is the kernels in
// dms_*.hip; nothing here computes any part of the decode path.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "dms.h"
#include "dms_internal.h"

struct dms_cache {
  dms_config cfg;
  dms::Layout L;
  uint8_t* ws;
  int device;
  int num_cus;
  int grid;   // attention work-groups per launch (resident at once)
  bool split; // the attention's mode: split by live blocks, or whole units
  std::vector<int32_t> len;  // host mirror of each sequence's length
  // True from a successful prefill until the next append or reset: the cache
  // then holds the prompt's visible tokens with slots in position order, which
  // dms_prefill_attention relies on.
  bool prompt_fresh = false;
  int prompt_zero_ch = -1;  // the key channel that prefill stored as 0, or -1
  // Host copies of the whole-unit layout last uploaded (order, wg_range),
  // alive while the upload may still read them.
  std::vector<int32_t> order, wg_range;
};

namespace {

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool valid_config(const dms_config* c) {
  if (!c) return false;
  if (c->batch < 1 || c->batch > 65535) return false;
  if (c->num_kv_heads < 1 || c->num_q_heads < 1) return false;
  if (c->num_q_heads % c->num_kv_heads != 0) return false;
  if (c->num_q_heads / c->num_kv_heads > dms::kMaxGroup) return false;
  if ((int64_t)c->batch * c->num_kv_heads > (1 << 24)) return false;
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  if (c->window < 0) return false;
  if (c->block_tokens != dms::kBlockTokens) return false;
  if (c->max_tokens < 1 || c->max_tokens > (1 << 24)) return false;
  if (c->split_wgs < 0 || c->split_wgs > 65535) return false;
  if (c->pool_blocks < 1 || c->pool_blocks > 0x7fffffffLL) return false;
  if (c->dtype != DMS_F32 && c->dtype != DMS_BF16) return false;
  if (!isfinite(c->scale) || c->scale < 0.0f) return false;
  return true;
}

void make_layout(const dms_config* c, dms::Layout& L) {
  L.B = c->batch;
  L.Hq = c->num_q_heads;
  L.Hkv = c->num_kv_heads;
  L.G = c->num_q_heads / c->num_kv_heads;
  L.d = c->head_dim;
  L.esize = c->dtype == DMS_BF16 ? 2 : 4;
  L.R = std::min(c->window, c->max_tokens) + 1;
  L.max_tokens = c->max_tokens;
  L.max_blocks = (c->max_tokens + dms::kBlockTokens - 1) / dms::kBlockTokens;
  L.U = c->batch * c->num_kv_heads;
  L.pool_blocks = c->pool_blocks;
  L.block_bytes = 2LL * dms::kBlockTokens * L.d * L.esize;
  L.item_floats = 32 + L.G * L.d;
  // split mode writes the partial of work-group g's piece of unit u to slot u + g
  L.max_items = (int64_t)L.U + dms::kMaxAttnWGs;
  int64_t o = 0;
  L.off_pool = o;
  o = align_up(o + L.pool_blocks * L.block_bytes, kAlign);
  L.off_btab = o;
  o = align_up(o + (int64_t)L.U * L.max_blocks * 4, kAlign);
  L.off_blkpos = o;
  o = align_up(o + L.pool_blocks * dms::kBlockTokens * 4, kAlign);
  L.off_blkmask = o;
  o = align_up(o + L.pool_blocks * 4, kAlign);
  L.off_ring = o;
  o = align_up(o + (int64_t)L.U * L.R * 4, kAlign);
  L.off_n = o;
  o = align_up(o + (int64_t)L.U * 4, kAlign);
  L.off_pos = o;
  o = align_up(o + (int64_t)L.U * 4, kAlign);
  L.off_plan = o;
  o = align_up(o + (int64_t)L.U * 8, kAlign);
  L.off_order = o;
  o = align_up(o + (int64_t)L.U * 4, kAlign);
  L.off_wgrange = o;
  o = align_up(o + (int64_t)(dms::kMaxAttnWGs + 1) * 4, kAlign);
  L.off_wglive = o;
  o = align_up(o + (int64_t)dms::kMaxAttnWGs * 8, kAlign);
  L.off_ctr = o;
  o = align_up(o + (int64_t)sizeof(dms::Counters), kAlign);
  L.off_part = o;
  o = align_up(o + L.max_items * L.item_floats * 4, kAlign);
  L.total = o;
}

dms::Dev make_dev(const dms_cache* c) {
  const dms::Layout& L = c->L;
  dms::Dev p;
  p.pool = c->ws + L.off_pool;
  p.btab = (int32_t*)(c->ws + L.off_btab);
  p.blk_pos = (int32_t*)(c->ws + L.off_blkpos);
  p.blk_mask = (uint32_t*)(c->ws + L.off_blkmask);
  p.ring = (int32_t*)(c->ws + L.off_ring);
  p.n = (int32_t*)(c->ws + L.off_n);
  p.pos = (int32_t*)(c->ws + L.off_pos);
  p.plan = (int32_t*)(c->ws + L.off_plan);
  p.order = (int32_t*)(c->ws + L.off_order);
  p.wg_range = (int32_t*)(c->ws + L.off_wgrange);
  p.wg_live = (unsigned long long*)(c->ws + L.off_wglive);
  p.ctr = (dms::Counters*)(c->ws + L.off_ctr);
  p.part = (float*)(c->ws + L.off_part);
  p.B = L.B;
  p.Hq = L.Hq;
  p.Hkv = L.Hkv;
  p.G = L.G;
  p.R = L.R;
  p.max_tokens = L.max_tokens;
  p.max_blocks = L.max_blocks;
  p.U = L.U;
  p.item_floats = L.item_floats;
  p.grid = c->grid;
  p.split = c->split ? 1 : 0;
  // Split mode shares the live blocks over at most one work-group per CU by
  // default: with two per CU (the resident grid) every work-group streams
  // half as many blocks and a cut unit has twice the pieces to merge, and on
  // the layers whose steps are latency-bound that was slower (Llama-3.2-1B-
  // shaped step 0.0266 against 0.0201 ms, Qwen-R1-7B-shaped 0.0443 against
  // 0.0403 ms) while the bandwidth-bound head-skew step was unchanged
  // (0.2842 against 0.2848 ms).  Widths between one and two per CU load
  // some CUs twice and were slower than either.
  p.split_wgs = c->cfg.split_wgs >= 2 ? std::min(c->cfg.split_wgs, c->grid) : std::min(c->grid, c->num_cus);
  p.pool_blocks = L.pool_blocks;
  p.block_bytes = L.block_bytes;
  const float scale = c->cfg.scale == 0.0f ? 1.0f / sqrtf((float)L.d) : c->cfg.scale;
  p.scale_log2e = (float)((double)scale * 1.4426950408889634);
  return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DMS_OK : DMS_ERR_HIP; }

int check_device(const dms_cache* c) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DMS_ERR_HIP;
  return dev == c->device ? DMS_OK : DMS_ERR_STATE;
}

// The current device, if it is a gfx950 (property query cached per device).
int current_gfx950_device(int* dev) {
  static int8_t known[256];  // 0 unknown, 1 gfx950, -1 other
  if (hipGetDevice(dev) != hipSuccess) return DMS_ERR_HIP;
  if (*dev < 0 || *dev >= 256) return DMS_ERR_DEVICE;
  int8_t k = __atomic_load_n(&known[*dev], __ATOMIC_RELAXED);
  if (k == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, *dev) != hipSuccess) return DMS_ERR_HIP;
    k = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    __atomic_store_n(&known[*dev], k, __ATOMIC_RELAXED);
  }
  return k == 1 ? DMS_OK : DMS_ERR_DEVICE;
}

constexpr int32_t kSoftMaxT = 1 << 20;

bool soft_shapes_ok(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d) {
  return B >= 1 && B <= 65535 && Hkv >= 1 && Hq >= Hkv && Hq <= 65535 && Hq % Hkv == 0 && T >= 1 &&
         T <= kSoftMaxT && (d == 64 || d == 128) && (int64_t)B * Hq <= INT32_MAX;
}

int soft_args(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d, int32_t window, float gamma, float tau,
              float scale, dms::SoftArgs* a) {
  if (!soft_shapes_ok(B, Hq, Hkv, T, d) || window < 0 || !(tau > 0.0f) || !std::isfinite(tau) ||
      !std::isfinite(gamma) || !std::isfinite(scale) || scale < 0.0f)
    return DMS_ERR_ARG;
  const float sc = scale == 0.0f ? 1.0f / sqrtf((float)d) : scale;
  *a = dms::SoftArgs{B, Hq, Hkv, Hq / Hkv, T, window, gamma, 1.0f / tau,
                     (float)((double)sc * 1.4426950408889634), sc};
  return DMS_OK;
}

// The attention's mode until dms_cache_balance decides from the live counts:
// split_wgs 1 forces whole units, >= 2 forces the split; otherwise whole units
// when every work-group can have one.
bool default_split(const dms_cache* c) {
  if (c->cfg.split_wgs == 1) return false;
  if (c->cfg.split_wgs >= 2) return true;
  return c->L.U < c->grid && c->L.U <= dms::kPlanLdsUnits;
}

}  // namespace

extern "C" {

size_t dms_workspace_bytes(const dms_config* cfg) {
  if (!valid_config(cfg)) return 0;
  dms::Layout L;
  make_layout(cfg, L);
  return (size_t)L.total;
}

int dms_cache_create(const dms_config* cfg, void* d_workspace, size_t workspace_bytes, void* stream,
                     dms_cache** out) {
  if (!out) return DMS_ERR_ARG;
  *out = nullptr;
  if (!valid_config(cfg) || !d_workspace) return DMS_ERR_ARG;
  dms::Layout L;
  make_layout(cfg, L);
  if ((uintptr_t)d_workspace % kAlign != 0 || workspace_bytes < (size_t)L.total) return DMS_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DMS_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DMS_ERR_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return DMS_ERR_DEVICE;
  dms_cache* c = new dms_cache();
  c->cfg = *cfg;
  c->L = L;
  c->ws = (uint8_t*)d_workspace;
  c->device = dev;
  c->num_cus = prop.multiProcessorCount;
  // Persistent attention grid: as many 4-wave work-groups as fit at once.
  // Whole-unit mode when there are at least as many units as work-groups
  // (each work-group takes whole units: no plan, no partials, no split
  // merge, and the decode step fuses the append into the same launch), split
  // mode with fewer units (the live blocks in equal shares).
  // dms_cache_balance re-decides from the live counts.
  c->grid = std::max(1, std::min(dms::kMaxAttnWGs, dms::attention_resident_wgs(cfg->dtype, L.d, c->num_cus)));
  if (cfg->split_wgs >= 2 && L.U > dms::kPlanLdsUnits) {
    delete c;
    return DMS_ERR_ARG;  // split mode plans at most kPlanLdsUnits units
  }
  c->split = default_split(c);
  c->len.assign(L.B, 0);
  const int st = hip_status(dms::launch_init(make_dev(c), (hipStream_t)stream));
  if (st != DMS_OK) {
    delete c;
    return st;
  }
  *out = c;
  return DMS_OK;
}

int dms_cache_destroy(dms_cache* c) {
  delete c;
  return DMS_OK;
}

int dms_cache_reset(dms_cache* c, void* stream) {
  if (!c) return DMS_ERR_ARG;
  int st = check_device(c);
  if (st != DMS_OK) return st;
  st = hip_status(dms::launch_init(make_dev(c), (hipStream_t)stream));
  if (st == DMS_OK) {
    std::fill(c->len.begin(), c->len.end(), 0);
    c->prompt_fresh = false;
    c->split = default_split(c);
  }
  return st;
}

// Logit source of the plain fp32 arrays: [B, Hkv] per step (positions = 1),
// [B, Hkv, max_len] for a prompt.
static dms::LogitSrc array_logits(const dms_cache* c, const float* d_logit, int64_t positions) {
  dms::LogitSrc ls{};
  ls.base = d_logit;
  ls.sh = positions;
  ls.sb = (int64_t)c->L.Hkv * positions;
  ls.si = 1;
  ls.off = 0;
  ls.bf16 = 0;
  return ls;
}

// Logit source of a projection channel; rows of d elements, `positions` rows
// per head ([B, H, positions, d]).  Returns DMS_ERR_ARG for bad arguments.
static int channel_logits(const dms_cache* c, const void* d_k, const void* d_q, int32_t source,
                          int32_t channel, int32_t zero_channel, int64_t positions, dms::LogitSrc* ls) {
  const int d = c->L.d;
  if (channel < 0 || channel >= d) return DMS_ERR_ARG;
  if (source == DMS_LOGIT_FROM_K) {
    ls->base = d_k;
    ls->sh = positions * d;
    ls->sb = (int64_t)c->L.Hkv * positions * d;
  } else if (source == DMS_LOGIT_FROM_Q) {
    if (!d_q || zero_channel) return DMS_ERR_ARG;
    ls->base = d_q;
    ls->sh = (int64_t)c->L.G * positions * d;  // query head h * G
    ls->sb = (int64_t)c->L.Hq * positions * d;
  } else {
    return DMS_ERR_ARG;
  }
  ls->si = d;
  ls->off = channel;
  ls->bf16 = c->cfg.dtype == DMS_BF16 ? 1 : 0;
  return DMS_OK;
}

// Whole-unit mode: deals the units to the work-groups longest processing
// time first (heaviest unit to the least loaded work-group) by weight wt[u],
// and uploads the layout (order, wg_range) to the workspace.  Returns the
// heaviest work-group's load.
static int64_t deal_units(dms_cache* c, const std::vector<int64_t>& wt, void* stream, int* status) {
  const int U = c->L.U, Gn = c->grid;
  std::vector<int32_t> s(U);
  for (int u = 0; u < U; ++u) s[u] = u;
  std::stable_sort(s.begin(), s.end(), [&](int32_t a, int32_t b) { return wt[a] > wt[b]; });
  // min-heap of (load, work-group)
  std::vector<std::pair<int64_t, int32_t>> heap;
  heap.reserve(Gn);
  for (int g = 0; g < Gn; ++g) heap.push_back({0, g});
  auto cmp = [](const std::pair<int64_t, int32_t>& a, const std::pair<int64_t, int32_t>& b) {
    return a.first != b.first ? a.first > b.first : a.second > b.second;
  };
  std::make_heap(heap.begin(), heap.end(), cmp);
  std::vector<std::vector<int32_t>> lists(Gn);
  for (int32_t u : s) {
    std::pop_heap(heap.begin(), heap.end(), cmp);
    heap.back().first += wt[u];
    lists[heap.back().second].push_back(u);
    std::push_heap(heap.begin(), heap.end(), cmp);
  }
  int64_t worst = 0;
  for (const auto& h : heap) worst = std::max(worst, h.first);
  c->order.clear();
  c->wg_range.assign(1, 0);
  for (int g = 0; g < Gn; ++g) {
    c->order.insert(c->order.end(), lists[g].begin(), lists[g].end());
    c->wg_range.push_back((int32_t)c->order.size());
  }
  const dms::Layout& L = c->L;
  *status = (hipMemcpyAsync(c->ws + L.off_order, c->order.data(), (size_t)U * 4, hipMemcpyHostToDevice,
                            (hipStream_t)stream) != hipSuccess ||
             hipMemcpyAsync(c->ws + L.off_wgrange, c->wg_range.data(), (size_t)(Gn + 1) * 4,
                            hipMemcpyHostToDevice, (hipStream_t)stream) != hipSuccess)
                ? DMS_ERR_HIP
                : DMS_OK;
  return worst;
}

// After a prefill with unequal prompt lengths, whole-unit mode deals the
// units by their sequence's length (the live counts of a sequence's heads
// grow with it; they are not known on the host).  Appends keep the layout
// valid.  Equal lengths keep the default layout.
static int balance_by_length(dms_cache* c, void* stream) {
  if (c->split) return DMS_OK;
  const auto mm = std::minmax_element(c->len.begin(), c->len.end());
  if (*mm.first == *mm.second) return DMS_OK;
  std::vector<int64_t> wt(c->L.U);
  for (int u = 0; u < c->L.U; ++u) wt[u] = c->len[u / c->L.Hkv];
  int st = DMS_OK;
  deal_units(c, wt, stream, &st);
  return st;
}

static int prefill_common(dms_cache* c, const void* d_k, const void* d_v, const dms::LogitSrc& ls, int zero_ch,
                          const int32_t* h_lengths, int32_t max_len, void* stream) {
  int st = check_device(c);
  if (st != DMS_OK) return st;
  for (int32_t x : c->len)
    if (x != 0) return DMS_ERR_STATE;
  for (int b = 0; b < c->L.B; ++b) {
    if (h_lengths[b] < 0 || h_lengths[b] > max_len) return DMS_ERR_ARG;
    if (h_lengths[b] > c->L.max_tokens) return DMS_ERR_CAPACITY;
  }
  st = hip_status(dms::launch_prefill(make_dev(c), c->cfg.dtype, c->L.d, d_k, d_v, ls, zero_ch, h_lengths,
                                      max_len, (hipStream_t)stream));
  if (st == DMS_OK) {
    for (int b = 0; b < c->L.B; ++b) c->len[b] = h_lengths[b];
    c->prompt_fresh = true;
    c->prompt_zero_ch = zero_ch;
    st = balance_by_length(c, stream);
  }
  return st;
}

static int append_common(dms_cache* c, const void* d_k, const void* d_v, const dms::LogitSrc& ls, int zero_ch,
                         void* stream) {
  int st = check_device(c);
  if (st != DMS_OK) return st;
  for (int32_t x : c->len)
    if (x + 1 > c->L.max_tokens) return DMS_ERR_CAPACITY;
  st = hip_status(
      dms::launch_append(make_dev(c), c->cfg.dtype, c->L.d, d_k, d_v, ls, zero_ch, (hipStream_t)stream));
  if (st == DMS_OK) {
    for (auto& x : c->len) ++x;
    c->prompt_fresh = false;
  }
  return st;
}

int dms_prefill_compress(dms_cache* c, const void* d_k, const void* d_v, const float* d_logit,
                         const int32_t* h_lengths, int32_t max_len, void* stream) {
  if (!c || !d_k || !d_v || !d_logit || !h_lengths || max_len < 1) return DMS_ERR_ARG;
  return prefill_common(c, d_k, d_v, array_logits(c, d_logit, max_len), -1, h_lengths, max_len, stream);
}

int dms_prefill_compress_channel(dms_cache* c, const void* d_k, const void* d_v, const void* d_q, int32_t source,
                                 int32_t channel, int32_t zero_channel, const int32_t* h_lengths, int32_t max_len,
                                 void* stream) {
  if (!c || !d_k || !d_v || !h_lengths || max_len < 1) return DMS_ERR_ARG;
  dms::LogitSrc ls{};
  const int st = channel_logits(c, d_k, d_q, source, channel, zero_channel, max_len, &ls);
  if (st != DMS_OK) return st;
  return prefill_common(c, d_k, d_v, ls, zero_channel ? channel : -1, h_lengths, max_len, stream);
}

int dms_append_step(dms_cache* c, const void* d_k, const void* d_v, const float* d_logit, void* stream) {
  if (!c || !d_k || !d_v || !d_logit) return DMS_ERR_ARG;
  return append_common(c, d_k, d_v, array_logits(c, d_logit, 1), -1, stream);
}

int dms_append_step_channel(dms_cache* c, const void* d_k, const void* d_v, const void* d_q, int32_t source,
                            int32_t channel, int32_t zero_channel, void* stream) {
  if (!c || !d_k || !d_v) return DMS_ERR_ARG;
  dms::LogitSrc ls{};
  const int st = channel_logits(c, d_k, d_q, source, channel, zero_channel, 1, &ls);
  if (st != DMS_OK) return st;
  return append_common(c, d_k, d_v, ls, zero_channel ? channel : -1, stream);
}

int dms_prefill_attention(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, int32_t max_len,
                          float* d_out, void* stream) {
  if (!c || !d_q || !d_k || !d_v || !d_out || max_len < 1) return DMS_ERR_ARG;
  int st = check_device(c);
  if (st != DMS_OK) return st;
  if (!c->prompt_fresh) return DMS_ERR_STATE;
  int32_t longest = 0;
  for (int32_t x : c->len) {
    if (x > max_len) return DMS_ERR_ARG;
    longest = std::max(longest, x);
  }
  return hip_status(dms::launch_prefill_attention(make_dev(c), c->cfg.dtype, c->L.d, d_q, d_k, d_v, max_len,
                                                  longest, c->prompt_zero_ch, d_out, (hipStream_t)stream));
}

static int chunk_common(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, const dms::LogitSrc& ls,
                        int zero_ch, int32_t chunk, float* d_out, void* stream) {
  if (c->L.max_blocks > dms::chunk_max_blocks()) return DMS_ERR_ARG;
  int st = check_device(c);
  if (st != DMS_OK) return st;
  for (int32_t x : c->len)
    if ((int64_t)x + chunk > c->L.max_tokens) return DMS_ERR_CAPACITY;
  st = hip_status(dms::launch_decode_chunk(make_dev(c), c->cfg.dtype, c->L.d, d_q, d_k, d_v, ls, zero_ch, chunk,
                                           d_out, (hipStream_t)stream));
  if (st == DMS_OK) {
    for (auto& x : c->len) x += chunk;
    c->prompt_fresh = false;
  }
  return st;
}

int dms_decode_chunk(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, const float* d_logit,
                     int32_t chunk, float* d_out, void* stream) {
  if (!c || !d_q || !d_k || !d_v || !d_logit || !d_out || chunk < 1) return DMS_ERR_ARG;
  return chunk_common(c, d_q, d_k, d_v, array_logits(c, d_logit, chunk), -1, chunk, d_out, stream);
}

int dms_decode_chunk_channel(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, int32_t source,
                             int32_t channel, int32_t zero_channel, int32_t chunk, float* d_out, void* stream) {
  if (!c || !d_q || !d_k || !d_v || !d_out || chunk < 1) return DMS_ERR_ARG;
  dms::LogitSrc ls{};
  const int st = channel_logits(c, d_k, d_q, source, channel, zero_channel, chunk, &ls);
  if (st != DMS_OK) return st;
  return chunk_common(c, d_q, d_k, d_v, ls, zero_channel ? channel : -1, chunk, d_out, stream);
}

int dms_decode_attention(dms_cache* c, const void* d_q, float* d_out, void* stream) {
  if (!c || !d_q || !d_out) return DMS_ERR_ARG;
  int st = check_device(c);
  if (st != DMS_OK) return st;
  for (int32_t x : c->len)
    if (x < 1) return DMS_ERR_STATE;
  return hip_status(dms::launch_attention(make_dev(c), c->cfg.dtype, c->L.d, d_q, d_out, (hipStream_t)stream));
}

int dms_decode_attention_timed(dms_cache* c, const void* d_q, float* d_out, void* start_event, void* stop_event,
                               void* stream) {
  if (!c || !d_q || !d_out || !start_event || !stop_event) return DMS_ERR_ARG;
  int st = check_device(c);
  if (st != DMS_OK) return st;
  for (int32_t x : c->len)
    if (x < 1) return DMS_ERR_STATE;
  return hip_status(dms::launch_attention(make_dev(c), c->cfg.dtype, c->L.d, d_q, d_out, (hipStream_t)stream,
                                          (hipEvent_t)start_event, (hipEvent_t)stop_event));
}

static int step_common(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, const dms::LogitSrc& ls,
                       int zero_ch, float* d_out, void* stream, void* start_event, void* stop_event) {
  int st = check_device(c);
  if (st != DMS_OK) return st;
  for (int32_t x : c->len)
    if (x + 1 > c->L.max_tokens) return DMS_ERR_CAPACITY;
  const dms::StepIn in{(const uint8_t*)d_k, (const uint8_t*)d_v, ls, zero_ch};
  st = hip_status(dms::launch_decode_step(make_dev(c), c->cfg.dtype, c->L.d, d_q, in, d_out, (hipStream_t)stream,
                                          (hipEvent_t)start_event, (hipEvent_t)stop_event));
  if (st == DMS_OK) {
    for (auto& x : c->len) ++x;
    c->prompt_fresh = false;
  }
  return st;
}

int dms_decode_step(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, const float* d_logit,
                    float* d_out, void* stream) {
  if (!c || !d_q || !d_k || !d_v || !d_logit || !d_out) return DMS_ERR_ARG;
  return step_common(c, d_q, d_k, d_v, array_logits(c, d_logit, 1), -1, d_out, stream, nullptr, nullptr);
}

int dms_decode_step_timed(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, const float* d_logit,
                          float* d_out, void* start_event, void* stop_event, void* stream) {
  if (!c || !d_q || !d_k || !d_v || !d_logit || !d_out || !start_event || !stop_event) return DMS_ERR_ARG;
  return step_common(c, d_q, d_k, d_v, array_logits(c, d_logit, 1), -1, d_out, stream, start_event, stop_event);
}

int dms_decode_step_channel(dms_cache* c, const void* d_q, const void* d_k, const void* d_v, int32_t source,
                            int32_t channel, int32_t zero_channel, float* d_out, void* stream) {
  if (!c || !d_q || !d_k || !d_v || !d_out) return DMS_ERR_ARG;
  dms::LogitSrc ls{};
  const int st = channel_logits(c, d_k, d_q, source, channel, zero_channel, 1, &ls);
  if (st != DMS_OK) return st;
  return step_common(c, d_q, d_k, d_v, ls, zero_channel ? channel : -1, d_out, stream, nullptr, nullptr);
}

int dms_cache_balance(dms_cache* c, void* stream) {
  if (!c) return DMS_ERR_ARG;
  int st = check_device(c);
  if (st != DMS_OK) return st;
  const dms::Layout& L = c->L;
  if (c->cfg.split_wgs >= 2) return DMS_OK;  // split mode forced: nothing to plan on the host
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DMS_ERR_HIP;
  std::vector<int32_t> n(L.U);
  if (hipMemcpy(n.data(), c->ws + L.off_n, (size_t)L.U * 4, hipMemcpyDeviceToHost) != hipSuccess) return DMS_ERR_HIP;
  // plan blocks, as the attention counts them (a unit with no live token counts one)
  std::vector<int64_t> nb(L.U);
  int64_t total = 0;
  for (int u = 0; u < L.U; ++u) {
    nb[u] = std::max<int64_t>(1, (n[u] + 15) / 16);
    total += nb[u];
  }
  const bool can_split = c->cfg.split_wgs == 0 && L.U <= dms::kPlanLdsUnits;
  if (can_split && L.U < c->grid) {
    // Fewer units than resident work-groups.  Whole units leave work-groups
    // idle, and one work-group streams the heaviest unit alone; the split
    // streams every block at the chip's rate but adds its plan and the merge
    // launch.  Estimated times, from MI355X measurements of both modes on the
    // Llama-3.2-1B- and Qwen-R1-7B-shaped layers (whole units 16.4 and 34.3 us
    // per step, split 18.9 and 39.8 us): one work-group alone streams about
    // 48 GB/s, the split about 6.2 TB/s with about 6.2 us more fixed work.
    const int64_t heaviest = *std::max_element(nb.begin(), nb.end());
    const double bytes = (double)L.block_bytes;
    const double t_whole = (double)heaviest * bytes / 48e9;
    const double t_split = (double)total * bytes / 6.2e12 + 6.2e-6;
    c->split = t_split < t_whole;
    if (c->split) return DMS_OK;
    deal_units(c, nb, stream, &st);  // each unit its own work-group
    return st;
  }
  const int64_t worst = deal_units(c, nb, stream, &st);
  if (st != DMS_OK) return st;
  // Whole units while the heaviest work-group carries at most 1/16 (plus one
  // block) above the mean; beyond that the split's equal shares win.
  c->split = can_split && 16 * worst * c->grid > 17 * total + 16LL * c->grid;
  return DMS_OK;
}

int dms_cache_stats(dms_cache* c, dms_stats* out, void* stream) {
  if (!c || !out) return DMS_ERR_ARG;
  int st = check_device(c);
  if (st != DMS_OK) return st;
  const dms::Layout& L = c->L;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DMS_ERR_HIP;
  dms::Counters ctr;
  std::vector<int32_t> n(L.U), pos(L.U);
  std::vector<unsigned long long> wg_live(c->grid);
  if (hipMemcpy(&ctr, c->ws + L.off_ctr, sizeof(ctr), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(wg_live.data(), c->ws + L.off_wglive, wg_live.size() * 8, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(n.data(), c->ws + L.off_n, (size_t)L.U * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(pos.data(), c->ws + L.off_pos, (size_t)L.U * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return DMS_ERR_HIP;
  memset(out, 0, sizeof(*out));
  for (int u = 0; u < L.U; ++u) {
    out->live_tokens += n[u];
    out->seen_tokens += pos[u];
  }
  out->allocated_blocks = (int64_t)std::min<unsigned long long>(ctr.bump, (unsigned long long)L.pool_blocks);
  out->live_token_steps = (int64_t)ctr.live_token_steps;
  for (unsigned long long x : wg_live) out->live_token_steps += (int64_t)x;
  out->sticky_error = ctr.sticky_error;
  out->split_mode = c->split ? 1 : 0;
  return DMS_OK;
}

int dms_cache_export(dms_cache* c, int32_t unit_begin, int32_t unit_count, int32_t* h_slot_pos, int32_t* h_ring,
                     int32_t* h_n, void* stream) {
  if (!c) return DMS_ERR_ARG;
  const dms::Layout& L = c->L;
  if (unit_begin < 0 || unit_count < 0 || (int64_t)unit_begin + unit_count > L.U) return DMS_ERR_ARG;
  int st = check_device(c);
  if (st != DMS_OK) return st;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DMS_ERR_HIP;
  if (unit_count == 0) return DMS_OK;
  std::vector<int32_t> n(unit_count);
  if (hipMemcpy(n.data(), c->ws + L.off_n + (int64_t)unit_begin * 4, (size_t)unit_count * 4,
                hipMemcpyDeviceToHost) != hipSuccess)
    return DMS_ERR_HIP;
  if (h_n) memcpy(h_n, n.data(), (size_t)unit_count * 4);
  if (h_ring) {
    if (hipMemcpy(h_ring, c->ws + L.off_ring + (int64_t)unit_begin * L.R * 4, (size_t)unit_count * L.R * 4,
                  hipMemcpyDeviceToHost) != hipSuccess)
      return DMS_ERR_HIP;
  }
  if (h_slot_pos) {
    // Gathered on the device into the attention-partials area (idle between
    // calls on this stream), then copied out piece by piece.
    const int64_t stage_words = L.max_items * L.item_floats;
    const int64_t total = (int64_t)unit_count * L.max_tokens;
    const dms::Dev p = make_dev(c);
    for (int64_t f0 = 0; f0 < total; f0 += stage_words) {
      const int64_t len = std::min(stage_words, total - f0);
      if (dms::launch_export(p, unit_begin, f0, len, (int32_t*)p.part, (hipStream_t)stream) != hipSuccess)
        return DMS_ERR_HIP;
      if (hipMemcpyAsync(h_slot_pos + f0, p.part, (size_t)len * 4, hipMemcpyDeviceToHost, (hipStream_t)stream) !=
              hipSuccess ||
          hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
        return DMS_ERR_HIP;
    }
  }
  return DMS_OK;
}

size_t dms_soft_attention_forward_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d) {
  if (!soft_shapes_ok(B, Hq, Hkv, T, d)) return 0;
  return (size_t)dms::soft_forward_workspace_bytes(B, Hq, Hkv, T, d);
}

int dms_soft_attention_forward(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d, int32_t window,
                               float gamma, float tau, float scale, const void* d_q, const void* d_k,
                               const void* d_v, const float* d_logit, const float* d_noise, float* d_out,
                               float* d_lse, void* d_workspace, size_t workspace_bytes, void* stream) {
  if (!d_q || !d_k || !d_v || !d_logit || !d_noise || !d_out || !d_lse || !d_workspace) return DMS_ERR_ARG;
  dms::SoftArgs a;
  int st = soft_args(B, Hq, Hkv, T, d, window, gamma, tau, scale, &a);
  if (st != DMS_OK) return st;
  if ((uintptr_t)d_workspace % kAlign != 0 ||
      workspace_bytes < (size_t)dms::soft_forward_workspace_bytes(B, Hq, Hkv, T, d))
    return DMS_ERR_WORKSPACE;
  int dev;
  st = current_gfx950_device(&dev);
  if (st != DMS_OK) return st;
  return hip_status(dms::launch_soft_forward(a, d, d_q, d_k, d_v, d_logit, d_noise, d_out, d_lse, d_workspace,
                                             (hipStream_t)stream));
}

int dms_soft_attention_forward_noalloc(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d, int32_t window,
                                       float gamma, float tau, float scale, const void* d_q, const void* d_k,
                                       const void* d_v, const float* d_logit, const float* d_noise, float* d_out,
                                       float* d_lse, void* stream) {
  if (!d_q || !d_k || !d_v || !d_logit || !d_noise || !d_out || !d_lse) return DMS_ERR_ARG;
  dms::SoftArgs a;
  int st = soft_args(B, Hq, Hkv, T, d, window, gamma, tau, scale, &a);
  if (st != DMS_OK) return st;
  if (dms::soft_forward_workspace_bytes(B, Hq, Hkv, T, d) > dms::soft_scratch_bytes()) return DMS_ERR_TOO_LARGE;
  int dev;
  st = current_gfx950_device(&dev);
  if (st != DMS_OK) return st;
  void* ws = dms::soft_scratch_address(dev);
  if (!ws) return DMS_ERR_HIP;
  return hip_status(
      dms::launch_soft_forward(a, d, d_q, d_k, d_v, d_logit, d_noise, d_out, d_lse, ws, (hipStream_t)stream));
}

size_t dms_soft_attention_forward_noalloc_max_bytes(void) { return (size_t)dms::soft_scratch_bytes(); }

size_t dms_soft_attention_backward_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d) {
  if (!soft_shapes_ok(B, Hq, Hkv, T, d)) return 0;
  return (size_t)dms::soft_backward_workspace_bytes(B, Hq, Hkv, T, d);
}

int dms_soft_attention_backward(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d, int32_t window,
                                float gamma, float tau, float scale, const void* d_q, const void* d_k,
                                const void* d_v, const float* d_logit, const float* d_noise, const float* d_out,
                                const float* d_lse, const void* d_dout, float* d_dq, float* d_dk, float* d_dv,
                                float* d_dlogit, void* d_workspace, size_t workspace_bytes, void* stream) {
  if (!d_q || !d_k || !d_v || !d_logit || !d_noise || !d_out || !d_lse || !d_dout || !d_dq || !d_dk || !d_dv ||
      !d_dlogit || !d_workspace)
    return DMS_ERR_ARG;
  dms::SoftArgs a;
  int st = soft_args(B, Hq, Hkv, T, d, window, gamma, tau, scale, &a);
  if (st != DMS_OK) return st;
  if ((uintptr_t)d_workspace % kAlign != 0 ||
      workspace_bytes < (size_t)dms::soft_backward_workspace_bytes(B, Hq, Hkv, T, d))
    return DMS_ERR_WORKSPACE;
  int dev;
  st = current_gfx950_device(&dev);
  if (st != DMS_OK) return st;
  return hip_status(dms::launch_soft_backward(a, d, d_q, d_k, d_v, d_logit, d_noise, d_out, d_lse, d_dout, d_dq,
                                              d_dk, d_dv, d_dlogit, d_workspace, (hipStream_t)stream));
}

const char* dms_status_str(int status) {
  switch (status) {
    case DMS_OK: return "DMS_OK";
    case DMS_ERR_ARG: return "DMS_ERR_ARG: invalid argument";
    case DMS_ERR_WORKSPACE: return "DMS_ERR_WORKSPACE: workspace too small or misaligned";
    case DMS_ERR_OUT_OF_BLOCKS: return "DMS_ERR_OUT_OF_BLOCKS: block pool exhausted";
    case DMS_ERR_CAPACITY: return "DMS_ERR_CAPACITY: a sequence would exceed max_tokens";
    case DMS_ERR_STATE: return "DMS_ERR_STATE: call not valid in the cache's current state";
    case DMS_ERR_HIP: return "DMS_ERR_HIP: HIP runtime or launch failure";
    case DMS_ERR_DEVICE: return "DMS_ERR_DEVICE: current device is not gfx950";
    case DMS_ERR_TOO_LARGE: return "DMS_ERR_TOO_LARGE: the call needs more scratch than the built-in buffer holds";
    default: return "unknown dms status";
  }
}

}  // extern "C"
