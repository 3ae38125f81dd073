// Shared device helpers for the HGA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hga.h"

namespace hga {

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kGroup = 8;    // tokens per group
constexpr int kBlockQ = 64;  // queries per routed block
constexpr int kWave = 64;
constexpr int kMaxTopKChunks = 64;
constexpr int kMaxTopKGroups = 512;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 is carried as raw 16-bit words in memory.
__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
// Round-to-nearest-even fp32 -> bf16 (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Loads 8 consecutive elements as fp32 from fp32 or bf16 storage.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static void load8(const float* p, float* out) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
  __device__ __forceinline__ static float to_f32(float x) { return x; }
  __device__ __forceinline__ static float from_f32(float x) { return x; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static void load8(const uint16_t* p, float* out) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
  __device__ __forceinline__ static uint16_t from_f32(float x) { return f32_to_bf16(x); }
};

// Order-preserving map of an fp32 score to uint32: larger score -> larger key.
// NaN maps to the key of -inf and -0 to the key of +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN -> -inf
  if (u == 0x80000000u) u = 0u;                          // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// 64-bit ranking key: score first, then the LOWER index wins.
__device__ __forceinline__ uint64_t rank_key(float s, uint32_t idx) {
  return (static_cast<uint64_t>(score_key(s)) << 32) | static_cast<uint64_t>(0xffffffffu - idx);
}

// Cross-lane moves through DPP (a VALU operand modifier, no LDS round trip).
// CTRL is the gfx9 dpp_ctrl code, ROW_MASK selects the 16-lane rows written;
// rows left out keep their own value. All 64 lanes must be active.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL,
                                                           ROW_MASK, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xb1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over each aligned group of 8 lanes, returned to all 8 (all lanes active).
__device__ __forceinline__ float sum8_f32(float x) {
  x += __uint_as_float(dpp_u32<kDppQuadXor1>(__float_as_uint(x)));
  x += __uint_as_float(dpp_u32<kDppQuadXor2>(__float_as_uint(x)));
  x += __uint_as_float(dpp_u32<kDppRowHalfMirror>(__float_as_uint(x)));
  return x;
}
// Sum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ float sum16_f32(float x) {
  x = sum8_f32(x);
  x += __uint_as_float(dpp_u32<kDppRowMirror>(__float_as_uint(x)));
  return x;
}

// A selected group id as the attention and gather kernels use it: ids outside
// the history's groups [0, n_groups) count as empty slots, exactly like -1, so
// a bad selection can never address memory outside the history.
__device__ __forceinline__ int32_t valid_group(int32_t n, int64_t n_groups) {
  return n >= 0 && n < n_groups ? n : -1;
}

// Rows per KV head in k_hist / v_hist (and x64 / x8 in the chunk / group
// summaries): hist_stride when set, else hist_len.
inline int64_t hist_rows(const hga_shape& s) { return s.hist_stride ? s.hist_stride : s.hist_len; }
// Sink chunks actually present (the sink cannot exceed the history).
inline int sink_chunks(const hga_shape& s) {
  const int64_t n_c = s.hist_len / kChunk;
  return static_cast<int>(s.n_sink_chunks < n_c ? s.n_sink_chunks : n_c);
}
// Local window in tokens, clamped to the segment (0 means the whole segment).
inline int local_window(const hga_shape& s) {
  return s.local_window <= 0 || s.local_window > s.seg_len ? s.seg_len : s.local_window;
}

// Timing events of kernel `id` (hga_kernel) set by hga_set_kernel_events, or
// nullptr: which = 0 is stamped with the start of the entry point's first
// launch, which = 1 with the end of its last (hipExtLaunchKernelGGL records
// them from the dispatch itself, so timing adds no marker packets).
hipEvent_t timer_event(int id, int which);

// Kernel launchers (defined in the .hip files).
hipError_t launch_build_summaries(const hga_shape& s, const void* k_hist, int64_t tok_begin,
                                  int64_t tok_end, float* chunk_sum, float* group_sum,
                                  hipStream_t stream);
hipError_t launch_route(const hga_shape& s, const void* q, const float* chunk_sum,
                        const float* group_sum, int32_t* sel_chunks, int32_t* sel_groups,
                        void* ws, hipStream_t stream);

// Group-summary cache state, one caller buffer in 256-byte aligned parts:
// slot_of_chunk [n_kv][hist_rows/64] (-1: not cached), chunk_of_slot
// [n_kv][n_slots] (-1: empty), hand [n_kv] (clock position), data
// [n_kv][n_slots][8][head_dim] fp32 (the 8 group summaries of a chunk).
constexpr int kGcacheMaxSelected = 8192;  // seg_len/64 * top_k_chunks per call
constexpr int kGcacheMaxSlots = 16384;
constexpr int kGcacheMaxChunks = 131072;  // hist_rows/64 (8.4M history tokens)
struct GcacheLayout {
  int32_t* slot_of_chunk;
  int32_t* chunk_of_slot;
  int32_t* hand;
  float* data;
  int n_slots;
  size_t bytes;
};
GcacheLayout gcache_layout(const hga_shape& s, void* cache, int n_slots);
size_t route_workspace_bytes(const hga_shape& s);
size_t route_cached_workspace_bytes(const hga_shape& s);
hipError_t launch_gcache_reset(const hga_shape& s, const GcacheLayout& L, hipStream_t stream);
// chunk_sum_lo: bf16 copies of chunk_sum for the two-pass chunk route, or null
hipError_t launch_decode_route(const hga_shape& s, int batch, int n_new, const void* q,
                               const float* chunk_sum, const uint16_t* chunk_sum_lo, const float* group_sum,
                               const int32_t* hist_lens, int32_t* sel_chunks, int32_t* sel_groups, void* ws,
                               hipStream_t stream);
// n fp32 values (n % 8 == 0, 16-byte aligned) to bf16, round to nearest even
hipError_t launch_round_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t stream);
size_t decode_route_workspace_bytes(const hga_shape& s, int batch);
size_t decode_attn_workspace_bytes(const hga_shape& s, int batch, int n_new);
// History kept in host memory: rows per (sequence, KV head) of the device
// copies the decode attention reads instead, [batch][n_kv][sink rows + k_g*8]
// (the sink rows, then the 8 rows of each routed group slot by slot).
int64_t decode_stage_sink_rows(const hga_shape& s);
int64_t decode_stage_rows(const hga_shape& s);
// Copies every (sequence, KV head)'s sink rows and routed groups from the
// history (k_hist / v_hist, device addresses of page-locked host memory) into
// k_stage / v_stage.
hipError_t launch_decode_stage(const hga_shape& s, int batch, const void* k_hist, const void* v_hist,
                               const int32_t* sel_groups, void* k_stage, void* v_stage, hipStream_t stream);
// staged: k_hist / v_hist are the copies launch_decode_stage wrote.
hipError_t launch_decode_attn(const hga_shape& s, int batch, int n_new, const void* q, const void* k_hist,
                              const void* v_hist, const void* k_tail, const void* v_tail,
                              const int32_t* sel_groups, const int32_t* hist_lens, const int32_t* tail_lens,
                              void* o, float* lse, void* ws, hipStream_t stream, bool staged);
hipError_t launch_route_cached(const hga_shape& s, const void* q, const float* chunk_sum,
                               const GcacheLayout& L, const float* group_sum_dev, int32_t* sel_chunks,
                               int32_t* sel_groups, int32_t* stats, void* ws, hipStream_t stream);
hipError_t launch_gather(const hga_shape& s, const void* k_hist, const void* v_hist,
                         const int32_t* sel_groups, void* k_out, void* v_out,
                         int32_t block_begin, int32_t block_end, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop);
// staged != nullptr: history rows come from gathered buffers laid out as
// [n_blocks][n_kv][top_k_groups*8][head_dim] for blocks [block_begin, block_end).
// Sink rows (the first sink_chunks(s)*64 history tokens) come from k_sink /
// v_sink, [n_kv][sink_stride][head_dim].
hipError_t launch_attn_fwd(const hga_shape& s, const void* q, const void* k_hist,
                           const void* v_hist, const void* k_seg, const void* v_seg,
                           const int32_t* sel_groups, void* o, float* lse,
                           const void* k_staged, const void* v_staged, const void* k_sink,
                           const void* v_sink, int64_t sink_stride, int32_t block_begin,
                           int32_t block_end, hipStream_t stream, hipEvent_t ev_start,
                           hipEvent_t ev_stop);
// Device copies of the history rows the backward reads, for history kept in
// host memory: every block's routed groups, [n_blocks][n_kv][top_k_groups*8]
// [head_dim] (the layout launch_gather writes for blocks 0..n_blocks), and the
// sink rows, [n_kv][sink_stride][head_dim].
struct StagedHistory {
  const void* k_rows;
  const void* v_rows;
  const void* k_sink;
  const void* v_sink;
  int64_t sink_stride;
};
// staged == nullptr: k_hist / v_hist are the device-resident history.
hipError_t launch_attn_bwd(const hga_shape& s, const void* q, const void* k_hist,
                           const void* v_hist, const void* k_seg, const void* v_seg,
                           const int32_t* sel_groups, const void* o, const float* lse,
                           const void* d_o, void* dq, void* dk_seg, void* dv_seg, void* ws,
                           hipStream_t stream, const StagedHistory* staged);

}  // namespace hga
