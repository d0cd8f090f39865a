// Internal layout of the DMS cache workspace and the launch interface between
// the host runtime (dms_runtime.cpp) and the kernels (dms_decode.hip,
// dms_prompt.hip, dms_soft.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace dms {

constexpr int kBlockTokens = 16;
constexpr int kMaxGroup = 16;      // query heads per KV head held by one MFMA tile
constexpr int kWavesPerWG = 4;     // waves per work-group (attention work item, append, reduce)
constexpr int kPlanLdsUnits = 4096;  // most units the attention's split mode plans for (its plan is in LDS)
constexpr int kMaxAttnWGs = 4096;  // most attention work-groups of a launch (the workspace is sized for it)
constexpr int kMinSplitBlocks = 8;  // split mode: fewest blocks per work-group (2 per wave)

// Device-side counters (one 64-byte line).
struct Counters {
  unsigned long long bump;              // next free pool block (may overshoot on exhaustion)
  unsigned long long live_token_steps;  // sum of live tokens after each append (fused steps: in wg_live)
  int sticky_error;                     // first device-detected dms_status, else 0
  int pad[11];
};

// Byte offsets of every region inside the caller's workspace.  The workspace
// holds no pointers, so a byte copy of it is a complete checkpoint.
struct Layout {
  int32_t B, Hq, Hkv, G, d, esize;
  int32_t R;           // ring entries per unit = min(window, max_tokens) + 1
  int32_t max_tokens, max_blocks, U;
  int64_t pool_blocks, block_bytes;
  int32_t item_floats;  // floats per attention partial: m[16], l[16], o[G][d]
  int64_t max_items;    // partial slots: U + kMaxAttnWGs (split mode uses slots u + g)
  int64_t off_pool, off_btab, off_blkpos, off_blkmask, off_ring, off_n, off_pos, off_plan, off_order,
      off_wgrange, off_wglive, off_ctr, off_part, total;
};

// Device pointers derived from a Layout and the workspace base, passed by
// value to every kernel.
struct Dev {
  uint8_t* pool;       // [pool_blocks][block_bytes]: K fragments then V fragments
  int32_t* btab;       // [U][max_blocks] physical block of each logical block
  int32_t* blk_pos;    // [pool_blocks][16] position held by each slot
  uint32_t* blk_mask;  // [pool_blocks] live-slot bits (low 16)
  int32_t* ring;       // [U][R] slot of a pending marked token, or -1
  int32_t* n;          // [U] slots in use
  int32_t* pos;        // [U] tokens appended so far (next position)
  int32_t* plan;       // [U][2] split mode: first partial slot and item count of each unit
  int32_t* order;      // [U] whole-unit mode: the units, work-group by work-group
  int32_t* wg_range;   // [grid + 1] whole-unit mode: work-group g takes order[wg_range[g] .. wg_range[g+1])
  unsigned long long* wg_live;  // [kMaxAttnWGs] fused steps: live tokens summed by work-group g
  Counters* ctr;
  float* part;         // [max_items][item_floats] attention partials
  int32_t B, Hq, Hkv, G, R, max_tokens, max_blocks, U, item_floats;
  int32_t grid;        // attention work-groups of a launch (resident at once)
  int32_t split;       // 1: split mode (the live blocks in equal shares, then reduce_kernel), 0: whole units
  int32_t split_wgs;   // split mode: at most this many work-groups take part (<= grid)
  int64_t pool_blocks, block_bytes;
  float scale_log2e;   // attention scale times log2(e)
};

// Prompt lengths of up to kMax sequences, passed by value to the prefill kernel.
struct PromptLens {
  static constexpr int kMax = 256;
  int32_t v[kMax];
};

// Where the eviction logit of unit (b, h) at position i is read: element
// b * sb + h * sh + i * si + off of an fp32 or bf16 array.  It covers the
// logit arrays ([B, Hkv] per step, [B, Hkv, max_len] for a prompt) and a
// channel of the keys ([B, Hkv, (max_len,) d]) or of the group's first query
// head ([B, Hq, (max_len,) d], sh = G * row stride).
struct LogitSrc {
  const void* base;
  int64_t sb, sh, si;
  int32_t off;
  int32_t bf16;  // 1: bf16 elements (upcast exactly), 0: fp32
};

// Relaxed (training-time) attention of T positions: shapes, window w, and
// the decision argument x = (logit + gamma + noise) * inv_tau of each key.
struct SoftArgs {
  int32_t B, Hq, Hkv, G, T, w;
  float gamma, inv_tau, scale_log2e, scale;
};

// Inputs of a fused decode step (zero everywhere else): the new token's K
// and V rows [U, d], where its eviction logit is read, and the key channel
// stored as 0 (-1: none).
struct StepIn {
  const uint8_t* k;
  const uint8_t* v;
  LogitSrc logit;
  int32_t zero_ch;
};

// Status codes mirrored from dms.h for device code.
constexpr int kErrOutOfBlocks = -3;

hipError_t launch_init(const Dev& p, hipStream_t s);
// zero_ch >= 0: that key channel is stored as 0; -1: keys are stored as given.
hipError_t launch_append(const Dev& p, int dtype, int d, const void* k, const void* v,
                         const LogitSrc& logit, int zero_ch, hipStream_t s);
hipError_t launch_prefill(const Dev& p, int dtype, int d, const void* k, const void* v,
                          const LogitSrc& logit, int zero_ch, const int32_t* h_lengths, int32_t max_len,
                          hipStream_t s);
// Attention of every prompt query (q, k, v: the dense prompt tensors the
// compression read); max_prompt = the longest prompt (grid size); zero_ch >= 0:
// the key channel the compression stored as 0 (read as 0 from k too).
hipError_t launch_prefill_attention(const Dev& p, int dtype, int d, const void* q, const void* k, const void* v,
                                    int32_t max_len, int32_t max_prompt, int zero_ch, float* out, hipStream_t s);
// Decode of `chunk` consecutive tokens per sequence: attention of the chunk's
// queries over the current cache and the chunk's rows, then the appends.
hipError_t launch_decode_chunk(const Dev& p, int dtype, int d, const void* q, const void* k, const void* v,
                               const LogitSrc& logit, int zero_ch, int chunk, float* out, hipStream_t s);
// Longest block table (blocks per unit) the chunk decode supports.
int chunk_max_blocks();
// Relaxed attention, bf16 q [B, Hq, T, d], k, v [B, Hkv, T, d]; logit, noise
// [B, Hkv, T] fp32.  Forward: out [B, Hq, T, d] and lse [B, Hq, T] fp32.
// ws holds soft_forward_workspace_bytes.
int64_t soft_forward_workspace_bytes(int B, int Hq, int Hkv, int T, int d);
hipError_t launch_soft_forward(const SoftArgs& a, int d, const void* q, const void* k, const void* v,
                               const float* logit, const float* noise, float* out, float* lse, void* ws,
                               hipStream_t s);
// The relaxed forward's built-in scratch (for the allocation-free entry
// point): its size, and its device address on device `dev`, which must be
// current (looked up the first time, then kept; null on failure).
int64_t soft_scratch_bytes();
void* soft_scratch_address(int dev);
// Backward from dout (bf16, like out): dq, dk, dv (fp32, like q, k, v) and
// dlogit (fp32, like logit); ws holds soft_backward_workspace_bytes.
int64_t soft_backward_workspace_bytes(int B, int Hq, int Hkv, int T, int d);
hipError_t launch_soft_backward(const SoftArgs& a, int d, const void* q, const void* k, const void* v,
                                const float* logit, const float* noise, const float* out, const float* lse,
                                const void* dout, float* dq, float* dk, float* dv, float* dlogit, void* ws,
                                hipStream_t s);
hipError_t launch_export(const Dev& p, int32_t u0, int64_t f0, int64_t len, int32_t* stage, hipStream_t s);
// Work-groups of the attention kernels that fit on the device at once.
int attention_resident_wgs(int dtype, int d, int num_cus);
// start / stop (may be null): events stamped with the start of the attention
// launch and the end of the call's last launch.  Split mode adds reduce_kernel.
hipError_t launch_attention(const Dev& p, int dtype, int d, const void* q, float* out, hipStream_t s,
                            hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// One decode step: append + attention.  Whole-unit mode: one fused launch;
// split mode: append_kernel, the attention, reduce_kernel.  start / stop as
// launch_attention, around the step's launches.
hipError_t launch_decode_step(const Dev& p, int dtype, int d, const void* q, const StepIn& in, float* out,
                              hipStream_t s, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

}  // namespace dms
