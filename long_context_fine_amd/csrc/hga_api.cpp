// C ABI entry points: argument validation, workspace sizing and dispatch.
// Every check runs on the host before anything is enqueued; failures return a
// status code and record a message for hga_last_error().
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>

#include "hga.h"
#include "hga_common.hpp"

namespace hga {
size_t bwd_workspace_bytes(const hga_shape& s);
}  // namespace hga

// Workspace of hga_route_noalloc: a static device array, one copy per device,
// each held until the process ends. Host code never passes `scratch` itself
// (on the host the name is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current (scratch_address).
static __device__ __align__(256) unsigned char scratch[HGA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

hga_status fail(hga_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hga_status fail(hga_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hga_status ok() {
  g_last_error.clear();
  return HGA_OK;
}

hga_status hip_fail(hipError_t e, const char* what) {
  return fail(HGA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t elem_bytes(const hga_shape& s) { return s.dtype == HGA_BF16 ? 2 : 4; }

hga_status check_shape(const hga_shape* s) {
  if (!s) return fail(HGA_ERR_INVALID_ARG, "shape is NULL");
  if (s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(HGA_ERR_INVALID_ARG, "head counts must be positive (n_q=%d, n_kv=%d)", s->n_q_heads,
                s->n_kv_heads);
  if (s->n_q_heads % s->n_kv_heads)
    return fail(HGA_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                s->n_q_heads, s->n_kv_heads);
  if (s->dtype != HGA_F32 && s->dtype != HGA_BF16)
    return fail(HGA_ERR_INVALID_ARG, "unknown dtype %d", s->dtype);
  if (s->hist_loc != HGA_HIST_DEVICE && s->hist_loc != HGA_HIST_HOST_PINNED)
    return fail(HGA_ERR_INVALID_ARG, "unknown hist_loc %d", s->hist_loc);
  if (s->head_dim <= 0) return fail(HGA_ERR_INVALID_ARG, "head_dim must be positive");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(HGA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", s->head_dim);
  if (s->chunk <= 0 || s->group <= 0 || s->block_q <= 0)
    return fail(HGA_ERR_INVALID_ARG, "chunk, group and block_q must be positive");
  if (s->chunk != hga::kChunk || s->group != hga::kGroup || s->block_q != hga::kBlockQ)
    return fail(HGA_ERR_UNSUPPORTED, "chunk/group/block_q = %d/%d/%d (supported: 64/8/64)", s->chunk,
                s->group, s->block_q);
  if (s->top_k_chunks < 1 || s->top_k_groups < 1)
    return fail(HGA_ERR_INVALID_ARG, "top_k_chunks and top_k_groups must be >= 1");
  if (s->top_k_chunks > hga::kMaxTopKChunks || s->top_k_groups > hga::kMaxTopKGroups)
    return fail(HGA_ERR_UNSUPPORTED, "top_k_chunks %d / top_k_groups %d exceed 64 / 512",
                s->top_k_chunks, s->top_k_groups);
  if (s->hist_len < 0 || s->hist_len % hga::kChunk)
    return fail(HGA_ERR_INVALID_ARG, "hist_len %lld is not a non-negative multiple of 64",
                static_cast<long long>(s->hist_len));
  if (s->hist_len / hga::kGroup > INT32_MAX / 2)
    return fail(HGA_ERR_UNSUPPORTED, "hist_len %lld too large for int32 group ids",
                static_cast<long long>(s->hist_len));
  if (s->hist_stride != 0 &&
      (s->hist_stride < s->hist_len || s->hist_stride % hga::kChunk || s->hist_stride / hga::kGroup > INT32_MAX / 2))
    return fail(HGA_ERR_INVALID_ARG, "hist_stride %lld must be 0 or a multiple of 64 >= hist_len %lld",
                static_cast<long long>(s->hist_stride), static_cast<long long>(s->hist_len));
  if (s->n_sink_chunks < 0 || s->local_window < 0)
    return fail(HGA_ERR_INVALID_ARG, "n_sink_chunks %d and local_window %d must be >= 0", s->n_sink_chunks,
                s->local_window);
  if (s->seg_len <= 0 || s->seg_len % hga::kBlockQ)
    return fail(HGA_ERR_INVALID_ARG, "seg_len %d is not a positive multiple of 64", s->seg_len);
  if (!(std::isfinite(s->softmax_scale) && s->softmax_scale > 0.f))
    return fail(HGA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  return HGA_OK;
}

#define HGA_REQUIRE(cond, ...)                                   \
  do {                                                           \
    if (!(cond)) return fail(HGA_ERR_INVALID_ARG, __VA_ARGS__);  \
  } while (0)

#define HGA_TRY(stmt)                     \
  do {                                    \
    const hga_status st__ = (stmt);       \
    if (st__ != HGA_OK) return st__;      \
  } while (0)

// Device-side address of a page-locked host allocation.
hga_status host_to_device_ptr(const void* host, const void** dev, const char* name) {
  void* d = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&d, const_cast<void*>(host), 0);
  if (e != hipSuccess || !d) {
    (void)hipGetLastError();
    return fail(HGA_ERR_INVALID_ARG, "%s is not page-locked host memory from hipHostMalloc (%s)", name,
                hipGetErrorString(e));
  }
  *dev = d;
  return HGA_OK;
}

// The pinned-host tier gathers routed groups in phases of kPhaseBlocks query
// blocks, each into its own region of the staging buffers.
constexpr int kPhaseBlocks = 4;

// Routed rows of one query block, one tensor (K or V): [n_kv][k_g*8][d].
size_t block_rows_bytes(const hga_shape& s) {
  return static_cast<size_t>(s.n_kv_heads) * s.top_k_groups * hga::kGroup * s.head_dim * elem_bytes(s);
}

// Routed rows of every query block, one tensor (K or V): [n_blocks][n_kv][k_g*8][d].
size_t routed_rows_bytes(const hga_shape& s) {
  return static_cast<size_t>(s.seg_len / hga::kBlockQ) * block_rows_bytes(s);
}

// Sink rows staged once per call for the pinned-host tier: [n_kv][sink*64][D].
size_t sink_bytes(const hga_shape& s) {
  return static_cast<size_t>(s.n_kv_heads) * hga::sink_chunks(s) * hga::kChunk * s.head_dim * elem_bytes(s);
}

// Forward workspace with pinned-host history: K rows, V rows (every block's
// routed groups), K sink rows, V sink rows. After the call it still holds
// them, which hga_attn_bwd_staged reads.
struct FwdStaging {
  char* k_rows;
  char* v_rows;
  char* k_sink;
  char* v_sink;
};

FwdStaging fwd_staging(const hga_shape& s, void* ws) {
  char* base = static_cast<char*>(ws);
  const size_t rows = align256(routed_rows_bytes(s));
  return {base, base + rows, base + 2 * rows, base + 2 * rows + align256(sink_bytes(s))};
}

size_t fwd_workspace_bytes(const hga_shape& s) {
  if (s.hist_loc != HGA_HIST_HOST_PINNED) return 0;
  return 2 * align256(routed_rows_bytes(s)) + 2 * align256(sink_bytes(s));
}

bool bwd_stages_history(const hga_shape& s) { return s.hist_loc == HGA_HIST_HOST_PINNED && s.hist_len > 0; }

// The kernels' workspace, then (history in host memory) the K and V routed
// rows of every block and the K and V sink rows.
size_t bwd_total_workspace_bytes(const hga_shape& s) {
  const size_t base = align256(hga::bwd_workspace_bytes(s));
  if (!bwd_stages_history(s)) return base;
  return base + 2 * align256(routed_rows_bytes(s)) + 2 * align256(sink_bytes(s));
}

// The pinned-host tier's side stream and events, one set per device. A call
// holds `mu` for its whole enqueue sequence: calls from several threads on one
// device then record and wait on these events in turn, so every wait sees the
// record its own call made (the side stream is shared either way).
struct SideResources {
  std::mutex mu;
  hipStream_t side = nullptr;
  hipEvent_t start = nullptr;
  hipEvent_t gathered[2] = {nullptr, nullptr};
};

std::mutex g_side_mu;
std::unordered_map<int, std::unique_ptr<SideResources>> g_side;

hga_status side_resources(SideResources** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_side_mu);
  auto it = g_side.find(dev);
  if (it == g_side.end()) {
    std::unique_ptr<SideResources> r(new SideResources);
    hipEvent_t* evs[3] = {&r->start, &r->gathered[0], &r->gathered[1]};
    // on a failed creation, release what was created before reporting it
    auto release = [&]() {
      for (hipEvent_t* ev : evs)
        if (*ev) (void)hipEventDestroy(*ev);
      if (r->side) (void)hipStreamDestroy(r->side);
    };
    if ((e = hipStreamCreateWithFlags(&r->side, hipStreamNonBlocking)) != hipSuccess)
      return hip_fail(e, "hipStreamCreateWithFlags");
    for (hipEvent_t* ev : evs)
      if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) {
        release();
        return hip_fail(e, "hipEventCreateWithFlags");
      }
    it = g_side.emplace(dev, std::move(r)).first;
  }
  *out = it->second.get();
  return HGA_OK;
}

std::atomic<hipEvent_t> g_timer_ev[HGA_KERNEL_COUNT][2];

// Workspace of hga_route_noalloc: the file-scope array `scratch` below.
std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;

hga_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(HGA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    }
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return HGA_OK;
}

}  // namespace

namespace hga {
hipEvent_t timer_event(int id, int which) { return g_timer_ev[id][which].load(std::memory_order_relaxed); }
}  // namespace hga

extern "C" {

hga_status hga_set_kernel_events(int32_t kernel, void* ev_start, void* ev_stop) {
  if (kernel < 0 || kernel >= HGA_KERNEL_COUNT)
    return fail(HGA_ERR_INVALID_ARG, "unknown kernel id %d", kernel);
  if ((ev_start == nullptr) != (ev_stop == nullptr))
    return fail(HGA_ERR_INVALID_ARG, "give both events or neither");
  g_timer_ev[kernel][0].store(static_cast<hipEvent_t>(ev_start));
  g_timer_ev[kernel][1].store(static_cast<hipEvent_t>(ev_stop));
  return ok();
}

int32_t hga_abi_version(void) { return HGA_ABI_VERSION; }

const char* hga_status_string(int32_t status) {
  switch (status) {
    case HGA_OK: return "HGA_OK";
    case HGA_ERR_INVALID_ARG: return "HGA_ERR_INVALID_ARG";
    case HGA_ERR_UNSUPPORTED: return "HGA_ERR_UNSUPPORTED";
    case HGA_ERR_WORKSPACE: return "HGA_ERR_WORKSPACE";
    case HGA_ERR_HIP: return "HGA_ERR_HIP";
  }
  return "HGA_ERR_UNKNOWN";
}

const char* hga_last_error(void) { return g_last_error.c_str(); }

size_t hga_workspace_size(const hga_shape* shape, int32_t op) {
  const std::string saved = g_last_error;
  const hga_status st = check_shape(shape);
  g_last_error = saved;
  if (st != HGA_OK) return 0;
  switch (op) {
    case HGA_OP_ROUTE: return hga::route_workspace_bytes(*shape);
    case HGA_OP_ROUTE_CACHED: return hga::route_cached_workspace_bytes(*shape);
    case HGA_OP_ATTN_FWD: return fwd_workspace_bytes(*shape);
    case HGA_OP_ATTN_BWD: return bwd_total_workspace_bytes(*shape);
  }
  return 0;
}

hga_status hga_build_summaries(const hga_shape* shape, const void* k_hist, int64_t tok_begin,
                               int64_t tok_end, float* chunk_sum, float* group_sum, void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  HGA_REQUIRE(tok_begin >= 0 && tok_begin <= tok_end && tok_end <= s.hist_len,
              "token range [%lld, %lld) outside [0, %lld]", static_cast<long long>(tok_begin),
              static_cast<long long>(tok_end), static_cast<long long>(s.hist_len));
  HGA_REQUIRE(tok_begin % hga::kChunk == 0 && tok_end % hga::kChunk == 0,
              "token range bounds must be multiples of 64");
  if (tok_end == tok_begin) return ok();
  HGA_REQUIRE(k_hist && chunk_sum && group_sum, "k_hist, chunk_sum and group_sum must be non-NULL");
  HGA_REQUIRE(reinterpret_cast<uintptr_t>(chunk_sum) % 16 == 0 && reinterpret_cast<uintptr_t>(group_sum) % 16 == 0,
              "chunk_sum and group_sum must be 16-byte aligned");
  const void* kd = k_hist;
  if (s.hist_loc == HGA_HIST_HOST_PINNED) HGA_TRY(host_to_device_ptr(k_hist, &kd, "k_hist"));
  float* gd = group_sum;
  {
    // group summaries may live in page-locked host memory (the cached route)
    hipPointerAttribute_t attr;
    const hipError_t pe = hipPointerGetAttributes(&attr, group_sum);
    if (pe != hipSuccess) {
      (void)hipGetLastError();
      return fail(HGA_ERR_INVALID_ARG, "group_sum is neither device memory nor page-locked host memory");
    }
    if (attr.type == hipMemoryTypeHost) {
      const void* p = nullptr;
      HGA_TRY(host_to_device_ptr(group_sum, &p, "group_sum"));
      gd = static_cast<float*>(const_cast<void*>(p));
    }
  }
  const hipError_t e = hga::launch_build_summaries(s, kd, tok_begin, tok_end, chunk_sum, gd,
                                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "build_summaries launch");
  return ok();
}

hga_status hga_route(const hga_shape* shape, const void* q, const float* chunk_sum,
                     const float* group_sum, int32_t* sel_chunks, int32_t* sel_groups, void* ws,
                     size_t ws_bytes, void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  HGA_REQUIRE(q && sel_chunks && sel_groups, "q, sel_chunks and sel_groups must be non-NULL");
  HGA_REQUIRE(s.hist_len == 0 || (chunk_sum && group_sum),
              "chunk_sum and group_sum must be non-NULL when hist_len > 0");
  const size_t need = hga::route_workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "route needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(HGA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const hipError_t e = hga::launch_route(s, q, chunk_sum, group_sum, sel_chunks, sel_groups, ws,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "route launch");
  return ok();
}

hga_status hga_route_noalloc(const hga_shape* shape, const void* q, const float* chunk_sum,
                             const float* group_sum, int32_t* sel_chunks, int32_t* sel_groups,
                             void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  HGA_REQUIRE(q && sel_chunks && sel_groups, "q, sel_chunks and sel_groups must be non-NULL");
  HGA_REQUIRE(s.hist_len == 0 || (chunk_sum && group_sum),
              "chunk_sum and group_sum must be non-NULL when hist_len > 0");
  const size_t need = hga::route_workspace_bytes(s);
  if (need > HGA_NOALLOC_SCRATCH_BYTES)
    return fail(HGA_ERR_WORKSPACE, "route needs %zu workspace bytes, above the %zu-byte static scratch", need,
                static_cast<size_t>(HGA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  HGA_TRY(scratch_address(&ws));
  const hipError_t e = hga::launch_route(s, q, chunk_sum, group_sum, sel_chunks, sel_groups, ws,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "route launch");
  return ok();
}

// Validated cache size, or 0 with the error recorded.
size_t gcache_bytes_checked(const hga_shape& s, int32_t n_slots) {
  if (n_slots < 1 || n_slots > hga::kGcacheMaxSlots) {
    fail(HGA_ERR_INVALID_ARG, "n_slots %d outside [1, %d]", n_slots, hga::kGcacheMaxSlots);
    return 0;
  }
  return hga::gcache_layout(s, nullptr, n_slots).bytes;
}

size_t hga_gcache_bytes(const hga_shape* shape, int32_t n_slots) {
  if (check_shape(shape) != HGA_OK) return 0;
  return gcache_bytes_checked(*shape, n_slots);
}

hga_status hga_gcache_reset(const hga_shape* shape, void* cache, int32_t n_slots, void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  HGA_REQUIRE(cache, "cache must be non-NULL");
  if (gcache_bytes_checked(s, n_slots) == 0) return HGA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(cache) % 256) return fail(HGA_ERR_INVALID_ARG, "cache must be 256-byte aligned");
  const hipError_t e = hga::launch_gcache_reset(s, hga::gcache_layout(s, cache, n_slots),
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gcache reset launch");
  return ok();
}

hga_status hga_route_cached(const hga_shape* shape, const void* q, const float* chunk_sum,
                            const float* group_sum_host, void* cache, int32_t n_slots,
                            int32_t* sel_chunks, int32_t* sel_groups, int32_t* stats, void* ws,
                            size_t ws_bytes, void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  HGA_REQUIRE(q && sel_chunks && sel_groups && cache, "q, sel_chunks, sel_groups and cache must be non-NULL");
  HGA_REQUIRE(s.hist_len == 0 || (chunk_sum && group_sum_host),
              "chunk_sum and group_sum_host must be non-NULL when hist_len > 0");
  if (gcache_bytes_checked(s, n_slots) == 0) return HGA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(cache) % 256) return fail(HGA_ERR_INVALID_ARG, "cache must be 256-byte aligned");
  const int64_t per_call = static_cast<int64_t>(s.seg_len / hga::kBlockQ) * s.top_k_chunks;
  if (per_call > hga::kGcacheMaxSelected)
    return fail(HGA_ERR_UNSUPPORTED, "seg_len/64 * top_k_chunks = %lld exceeds %d", static_cast<long long>(per_call),
                hga::kGcacheMaxSelected);
  if (hga::hist_rows(s) / hga::kChunk > hga::kGcacheMaxChunks)
    return fail(HGA_ERR_UNSUPPORTED, "history of %lld rows exceeds the cached route's %d chunks",
                static_cast<long long>(hga::hist_rows(s)), hga::kGcacheMaxChunks);
  if (n_slots < per_call)
    return fail(HGA_ERR_INVALID_ARG, "n_slots %d below seg_len/64 * top_k_chunks = %lld (chunks kept per call)",
                n_slots, static_cast<long long>(per_call));
  const size_t need = hga::route_cached_workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "route_cached needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(HGA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const void* gd = nullptr;
  if (s.hist_len > 0) HGA_TRY(host_to_device_ptr(group_sum_host, &gd, "group_sum_host"));
  const hipError_t e = hga::launch_route_cached(s, q, chunk_sum, hga::gcache_layout(s, cache, n_slots),
                                                static_cast<const float*>(gd), sel_chunks, sel_groups, stats,
                                                ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "route_cached launch");
  return ok();
}

// Decode validation; 0 bytes (with the error recorded) when invalid.
hga_status decode_check(const hga_shape& s, int32_t batch, int32_t n_new) {
  if (batch < 1) return fail(HGA_ERR_INVALID_ARG, "batch %d must be >= 1", batch);
  if (n_new < 1 || n_new > s.seg_len)
    return fail(HGA_ERR_INVALID_ARG, "n_new %d outside [1, seg_len = %d]", n_new, s.seg_len);
  const int r = s.n_q_heads / s.n_kv_heads;
  if (r * n_new > 16)
    return fail(HGA_ERR_UNSUPPORTED, "r * n_new = %d query rows per KV head exceed 16", r * n_new);
  return HGA_OK;
}

bool decode_stages_history(const hga_shape& s) {
  return s.hist_loc == HGA_HIST_HOST_PINNED && hga::hist_rows(s) > 0;
}

// Route part, attention part, then (history in host memory) the K and V
// copies of every (sequence, KV head)'s sink rows and routed groups.
size_t decode_stage_bytes(const hga_shape& s, int32_t batch) {
  return align256(static_cast<size_t>(batch) * s.n_kv_heads * hga::decode_stage_rows(s) * s.head_dim *
                  elem_bytes(s));
}

size_t decode_ws_parts(const hga_shape& s, int32_t batch, int32_t n_new, size_t* route_part) {
  *route_part = align256(hga::decode_route_workspace_bytes(s, batch));
  const size_t attn = align256(hga::decode_attn_workspace_bytes(s, batch, n_new));
  return *route_part + attn + (decode_stages_history(s) ? 2 * decode_stage_bytes(s, batch) : 0);
}

size_t hga_decode_workspace_size(const hga_shape* shape, int32_t batch, int32_t n_new) {
  if (check_shape(shape) != HGA_OK || decode_check(*shape, batch, n_new) != HGA_OK) return 0;
  size_t route_part;
  return decode_ws_parts(*shape, batch, n_new, &route_part);
}

// hga_decode and hga_decode_twopass: chunk_sum_lo null for the one-pass route.
hga_status decode_impl(const hga_shape* shape, int32_t batch, int32_t n_new, const void* q,
                       const void* k_hist, const void* v_hist, const float* chunk_sum,
                       const uint16_t* chunk_sum_lo, const float* group_sum, const void* k_tail,
                       const void* v_tail, const int32_t* hist_lens, const int32_t* tail_lens,
                       int32_t* sel_chunks, int32_t* sel_groups, void* o, float* lse, void* ws,
                       size_t ws_bytes, void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  HGA_TRY(decode_check(s, batch, n_new));
  HGA_REQUIRE(q && k_tail && v_tail && hist_lens && tail_lens && sel_chunks && sel_groups && o && lse,
              "q, k_tail, v_tail, hist_lens, tail_lens, sel_chunks, sel_groups, o and lse must be non-NULL");
  HGA_REQUIRE(hga::hist_rows(s) == 0 || (k_hist && v_hist && chunk_sum && group_sum),
              "k_hist, v_hist, chunk_sum and group_sum must be non-NULL when the history capacity is > 0");
  size_t route_part;
  const size_t need = decode_ws_parts(s, batch, n_new, &route_part);
  if (!ws || ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(HGA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool staged = decode_stages_history(s);
  const void* kd = k_hist;
  const void* vd = v_hist;
  if (staged) {
    HGA_TRY(host_to_device_ptr(k_hist, &kd, "k_hist"));
    HGA_TRY(host_to_device_ptr(v_hist, &vd, "v_hist"));
  }
  hipError_t e = hga::launch_decode_route(s, batch, n_new, q, chunk_sum, chunk_sum_lo, group_sum, hist_lens,
                                          sel_chunks, sel_groups, ws, st);
  if (e != hipSuccess) return hip_fail(e, "decode route launch");
  char* attn_ws = static_cast<char*>(ws) + route_part;
  if (staged) {
    // history in page-locked host memory: bring each (sequence, KV head)'s
    // sink rows and routed groups over the host link, then attend to those
    char* stage = attn_ws + align256(hga::decode_attn_workspace_bytes(s, batch, n_new));
    void* ks = stage;
    void* vs = stage + decode_stage_bytes(s, batch);
    e = hga::launch_decode_stage(s, batch, kd, vd, sel_groups, ks, vs, st);
    if (e != hipSuccess) return hip_fail(e, "decode staging launch");
    kd = ks;
    vd = vs;
  }
  e = hga::launch_decode_attn(s, batch, n_new, q, kd, vd, k_tail, v_tail, sel_groups, hist_lens, tail_lens, o,
                              lse, attn_ws, st, staged);
  if (e != hipSuccess) return hip_fail(e, "decode attention launch");
  return ok();
}

hga_status hga_decode(const hga_shape* shape, int32_t batch, int32_t n_new, const void* q,
                      const void* k_hist, const void* v_hist, const float* chunk_sum,
                      const float* group_sum, const void* k_tail, const void* v_tail,
                      const int32_t* hist_lens, const int32_t* tail_lens, int32_t* sel_chunks,
                      int32_t* sel_groups, void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return decode_impl(shape, batch, n_new, q, k_hist, v_hist, chunk_sum, nullptr, group_sum, k_tail, v_tail,
                     hist_lens, tail_lens, sel_chunks, sel_groups, o, lse, ws, ws_bytes, stream);
}

hga_status hga_decode_twopass(const hga_shape* shape, int32_t batch, int32_t n_new, const void* q,
                              const void* k_hist, const void* v_hist, const float* chunk_sum,
                              const uint16_t* chunk_sum_bf16, const float* group_sum, const void* k_tail,
                              const void* v_tail, const int32_t* hist_lens, const int32_t* tail_lens,
                              int32_t* sel_chunks, int32_t* sel_groups, void* o, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
  HGA_TRY(check_shape(shape));
  if (hga::hist_rows(*shape) > 0) {
    HGA_REQUIRE(chunk_sum_bf16, "chunk_sum_bf16 must be non-NULL when the history capacity is > 0");
    if (reinterpret_cast<uintptr_t>(chunk_sum_bf16) % 16)
      return fail(HGA_ERR_INVALID_ARG, "chunk_sum_bf16 must be 16-byte aligned");
  }
  return decode_impl(shape, batch, n_new, q, k_hist, v_hist, chunk_sum, chunk_sum_bf16, group_sum, k_tail,
                     v_tail, hist_lens, tail_lens, sel_chunks, sel_groups, o, lse, ws, ws_bytes, stream);
}

hga_status hga_summaries_to_bf16(const float* src, uint16_t* dst, int64_t n, void* stream) {
  if (n < 0 || n % 8) return fail(HGA_ERR_INVALID_ARG, "n = %lld must be a non-negative multiple of 8",
                                  static_cast<long long>(n));
  if (n == 0) return ok();
  HGA_REQUIRE(src && dst, "src and dst must be non-NULL");
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
    return fail(HGA_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  const hipError_t e = hga::launch_round_bf16(src, dst, n, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bf16 rounding launch");
  return ok();
}

hga_status hga_gather_groups(const hga_shape* shape, const void* k_hist, const void* v_hist,
                             const int32_t* sel_groups, void* k_out, void* v_out, void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  HGA_REQUIRE(sel_groups && k_out && v_out, "sel_groups, k_out and v_out must be non-NULL");
  HGA_REQUIRE(s.hist_len == 0 || (k_hist && v_hist), "k_hist and v_hist must be non-NULL");
  const void* kd = k_hist;
  const void* vd = v_hist;
  if (s.hist_loc == HGA_HIST_HOST_PINNED && s.hist_len > 0) {
    HGA_TRY(host_to_device_ptr(k_hist, &kd, "k_hist"));
    HGA_TRY(host_to_device_ptr(v_hist, &vd, "v_hist"));
  }
  const hipError_t e = hga::launch_gather(s, kd, vd, sel_groups, k_out, v_out, 0,
                                          s.seg_len / hga::kBlockQ, static_cast<hipStream_t>(stream),
                                          hga::timer_event(HGA_KERNEL_GATHER, 0),
                                          hga::timer_event(HGA_KERNEL_GATHER, 1));
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return ok();
}

hga_status hga_attn_fwd(const hga_shape* shape, const void* q, const void* k_hist,
                        const void* v_hist, const void* k_seg, const void* v_seg,
                        const int32_t* sel_groups, void* o, float* lse, void* ws, size_t ws_bytes,
                        void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  HGA_REQUIRE(q && k_seg && v_seg && sel_groups && o && lse,
              "q, k_seg, v_seg, sel_groups, o and lse must be non-NULL");
  HGA_REQUIRE(s.hist_len == 0 || (k_hist && v_hist), "k_hist and v_hist must be non-NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int n_blocks = s.seg_len / hga::kBlockQ;
  if (s.hist_loc == HGA_HIST_DEVICE || s.hist_len == 0) {
    const hipError_t e = hga::launch_attn_fwd(s, q, k_hist, v_hist, k_seg, v_seg, sel_groups, o, lse,
                                              nullptr, nullptr, k_hist, v_hist, hga::hist_rows(s), 0,
                                              n_blocks, st,
                                              hga::timer_event(HGA_KERNEL_ATTN_FWD, 0),
                                              hga::timer_event(HGA_KERNEL_ATTN_FWD, 1));
    if (e != hipSuccess) return hip_fail(e, "attn_fwd launch");
    return ok();
  }

  // Pinned-host history: gather phase p (kPhaseBlocks query blocks) over the
  // host link on the side stream into its own region of the staging buffers,
  // while the main stream runs attention on phase p-1. The regions do not
  // overlap, so no gather waits for an attention phase, and after the call the
  // workspace holds every block's routed rows (read by hga_attn_bwd_staged).
  const size_t need = fwd_workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "attn_fwd (pinned-host history) needs %zu workspace bytes, got %zu",
                need, ws ? ws_bytes : 0);
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(HGA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const void* kd = nullptr;
  const void* vd = nullptr;
  HGA_TRY(host_to_device_ptr(k_hist, &kd, "k_hist"));
  HGA_TRY(host_to_device_ptr(v_hist, &vd, "v_hist"));
  SideResources* r = nullptr;
  HGA_TRY(side_resources(&r));
  std::lock_guard<std::mutex> call_lock(r->mu);
  const FwdStaging stg = fwd_staging(s, ws);
  const size_t block_bytes = block_rows_bytes(s);
  const int n_sink_rows = hga::sink_chunks(s) * hga::kChunk;
  void* ksink = stg.k_sink;
  void* vsink = stg.v_sink;
  hipError_t e;
  // the side stream must see everything already enqueued on `stream` (sel_groups)
  if ((e = hipEventRecord(r->start, st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if ((e = hipStreamWaitEvent(r->side, r->start, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  // sink rows: one strided copy per tensor, ahead of the first gather on the
  // side stream (the first attention phase waits for that gather)
  if (n_sink_rows > 0) {
    const size_t row = static_cast<size_t>(s.head_dim) * elem_bytes(s);
    const size_t pitch = static_cast<size_t>(hga::hist_rows(s)) * row;
    if ((e = hipMemcpy2DAsync(ksink, n_sink_rows * row, k_hist, pitch, n_sink_rows * row, s.n_kv_heads,
                              hipMemcpyHostToDevice, r->side)) != hipSuccess)
      return hip_fail(e, "sink copy");
    if ((e = hipMemcpy2DAsync(vsink, n_sink_rows * row, v_hist, pitch, n_sink_rows * row, s.n_kv_heads,
                              hipMemcpyHostToDevice, r->side)) != hipSuccess)
      return hip_fail(e, "sink copy");
  }
  // timers (hga_set_kernel_events) span the whole call: GATHER from the start
  // of the first gather to the end of the last, ATTN_FWD from the start of the
  // first attention phase to the end of the last (waits in between included)
  const int n_phases = (n_blocks + kPhaseBlocks - 1) / kPhaseBlocks;
  for (int ph = 0; ph < n_phases; ++ph) {
    const int b0 = ph * kPhaseBlocks;
    const int b1 = b0 + kPhaseBlocks < n_blocks ? b0 + kPhaseBlocks : n_blocks;
    const int x = ph % 2;
    void* kbuf = stg.k_rows + b0 * block_bytes;   // phase regions: blocks b0 .. b1-1
    void* vbuf = stg.v_rows + b0 * block_bytes;
    const bool first = ph == 0, last = ph == n_phases - 1;
    if ((e = hga::launch_gather(s, kd, vd, sel_groups, kbuf, vbuf, b0, b1, r->side,
                                first ? hga::timer_event(HGA_KERNEL_GATHER, 0) : nullptr,
                                last ? hga::timer_event(HGA_KERNEL_GATHER, 1) : nullptr)) != hipSuccess)
      return hip_fail(e, "gather launch");
    if ((e = hipEventRecord(r->gathered[x], r->side)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(st, r->gathered[x], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    if ((e = hga::launch_attn_fwd(s, q, kd, vd, k_seg, v_seg, sel_groups, o, lse, kbuf, vbuf,
                                  ksink, vsink, n_sink_rows, b0, b1, st, first ? hga::timer_event(HGA_KERNEL_ATTN_FWD, 0) : nullptr,
                                  last ? hga::timer_event(HGA_KERNEL_ATTN_FWD, 1) : nullptr)) != hipSuccess)
      return hip_fail(e, "attn_fwd launch");
  }
  return ok();
}

hga_status hga_attn_bwd(const hga_shape* shape, const void* q, const void* k_hist,
                        const void* v_hist, const void* k_seg, const void* v_seg,
                        const int32_t* sel_groups, const void* o, const float* lse, const void* d_o,
                        void* dq, void* dk_seg, void* dv_seg, void* ws, size_t ws_bytes,
                        void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  HGA_REQUIRE(q && k_seg && v_seg && sel_groups && o && lse && d_o && dq && dk_seg && dv_seg,
              "q, k_seg, v_seg, sel_groups, o, lse, d_o, dq, dk_seg and dv_seg must be non-NULL");
  HGA_REQUIRE(s.hist_len == 0 || (k_hist && v_hist), "k_hist and v_hist must be non-NULL");
  const size_t need = bwd_total_workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "attn_bwd needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(HGA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!bwd_stages_history(s)) {
    e = hga::launch_attn_bwd(s, q, k_hist, v_hist, k_seg, v_seg, sel_groups, o, lse, d_o, dq, dk_seg,
                             dv_seg, ws, st, nullptr);
    if (e != hipSuccess) return hip_fail(e, "attn_bwd launch");
    return ok();
  }

  // History in page-locked host memory: only dQ reads it (the history is
  // detached, so dK/dV cover segment keys only). Bring every block's routed
  // groups and the sink rows into the workspace over the host link, in
  // stream order, then run the kernels on those copies.
  const void* kd = nullptr;
  const void* vd = nullptr;
  HGA_TRY(host_to_device_ptr(k_hist, &kd, "k_hist"));
  HGA_TRY(host_to_device_ptr(v_hist, &vd, "v_hist"));
  char* base = static_cast<char*>(ws) + align256(hga::bwd_workspace_bytes(s));
  const size_t rows = align256(routed_rows_bytes(s));
  hga::StagedHistory sh;
  sh.k_rows = base;
  sh.v_rows = base + rows;
  sh.k_sink = base + 2 * rows;
  sh.v_sink = base + 2 * rows + align256(sink_bytes(s));
  const int n_sink_rows = hga::sink_chunks(s) * hga::kChunk;
  sh.sink_stride = n_sink_rows;
  if ((e = hga::launch_gather(s, kd, vd, sel_groups, const_cast<void*>(sh.k_rows), const_cast<void*>(sh.v_rows),
                              0, s.seg_len / hga::kBlockQ, st, hga::timer_event(HGA_KERNEL_GATHER, 0),
                              hga::timer_event(HGA_KERNEL_GATHER, 1))) != hipSuccess)
    return hip_fail(e, "gather launch");
  if (n_sink_rows > 0) {
    const size_t row = static_cast<size_t>(s.head_dim) * elem_bytes(s);
    const size_t pitch = static_cast<size_t>(hga::hist_rows(s)) * row;
    if ((e = hipMemcpy2DAsync(const_cast<void*>(sh.k_sink), n_sink_rows * row, k_hist, pitch, n_sink_rows * row,
                              s.n_kv_heads, hipMemcpyHostToDevice, st)) != hipSuccess)
      return hip_fail(e, "sink copy");
    if ((e = hipMemcpy2DAsync(const_cast<void*>(sh.v_sink), n_sink_rows * row, v_hist, pitch, n_sink_rows * row,
                              s.n_kv_heads, hipMemcpyHostToDevice, st)) != hipSuccess)
      return hip_fail(e, "sink copy");
  }
  e = hga::launch_attn_bwd(s, q, sh.k_rows, sh.v_rows, k_seg, v_seg, sel_groups, o, lse, d_o, dq, dk_seg,
                           dv_seg, ws, st, &sh);
  if (e != hipSuccess) return hip_fail(e, "attn_bwd launch");
  return ok();
}

hga_status hga_attn_bwd_staged(const hga_shape* shape, const void* q, const void* fwd_ws,
                               size_t fwd_ws_bytes, const void* k_seg, const void* v_seg,
                               const int32_t* sel_groups, const void* o, const float* lse,
                               const void* d_o, void* dq, void* dk_seg, void* dv_seg, void* ws,
                               size_t ws_bytes, void* stream) {
  HGA_TRY(check_shape(shape));
  const hga_shape& s = *shape;
  if (s.hist_loc != HGA_HIST_HOST_PINNED)
    return fail(HGA_ERR_INVALID_ARG, "attn_bwd_staged reads the staging of a pinned-host forward "
                                     "(hist_loc = HGA_HIST_HOST_PINNED)");
  HGA_REQUIRE(q && k_seg && v_seg && sel_groups && o && lse && d_o && dq && dk_seg && dv_seg,
              "q, k_seg, v_seg, sel_groups, o, lse, d_o, dq, dk_seg and dv_seg must be non-NULL");
  const size_t need_fwd = fwd_workspace_bytes(s);
  if (!fwd_ws || fwd_ws_bytes < need_fwd)
    return fail(HGA_ERR_WORKSPACE, "attn_bwd_staged needs the forward's %zu workspace bytes, got %zu", need_fwd,
                fwd_ws ? fwd_ws_bytes : 0);
  if (reinterpret_cast<uintptr_t>(fwd_ws) % 256)
    return fail(HGA_ERR_WORKSPACE, "the forward's workspace must be 256-byte aligned");
  const size_t need = align256(hga::bwd_workspace_bytes(s));
  if (!ws || ws_bytes < need)
    return fail(HGA_ERR_WORKSPACE, "attn_bwd_staged needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(HGA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (s.hist_len == 0) {  // no history: the forward staged nothing and nothing is read
    e = hga::launch_attn_bwd(s, q, nullptr, nullptr, k_seg, v_seg, sel_groups, o, lse, d_o, dq, dk_seg, dv_seg,
                             ws, st, nullptr);
  } else {
    const FwdStaging stg = fwd_staging(s, const_cast<void*>(fwd_ws));
    hga::StagedHistory sh;
    sh.k_rows = stg.k_rows;
    sh.v_rows = stg.v_rows;
    sh.k_sink = stg.k_sink;
    sh.v_sink = stg.v_sink;
    sh.sink_stride = hga::sink_chunks(s) * hga::kChunk;
    e = hga::launch_attn_bwd(s, q, sh.k_rows, sh.v_rows, k_seg, v_seg, sel_groups, o, lse, d_o, dq, dk_seg,
                             dv_seg, ws, st, &sh);
  }
  if (e != hipSuccess) return hip_fail(e, "attn_bwd launch");
  return ok();
}

}  // extern "C"
