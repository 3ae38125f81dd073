// Exact-token gather: copy the 8 rows of every selected group of K_hist and
// V_hist into a dense [block][kv head][k_g*8][d] staging buffer.
//
// The source is either HBM or page-locked host memory mapped into the GPU
// address space (the pinned-host history tier); in the latter case every load
// crosses the host link, so each workgroup keeps 8 independent 16-byte loads
// per thread in flight before storing. One workgroup moves 8 groups (64 rows)
// of K and of V; empty slots (-1, an id outside the history, or beyond k_g)
// are zero-filled.
#include "hga_common.hpp"

namespace hga {
namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint8_t* __restrict__ k_hist, const uint8_t* __restrict__ v_hist,
    const int32_t* __restrict__ sel, uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out,
    int elem_bytes, int64_t hist_rows, int64_t n_groups, int n_kv, int k_g, int block_begin) {
  const int row_bytes = D * elem_bytes;
  const int cpr = row_bytes / 16;            // 16-byte chunks per row
  const int rows_per_pass = kThreads / cpr;  // 16 or 8 (bf16) / 8 or 4 (fp32)
  const int n_tiles = (k_g + 7) / 8;
  int w = blockIdx.x;
  const int tile = w % n_tiles;
  w /= n_tiles;
  const int j = w % n_kv;
  const int bl = w / n_kv;  // block relative to block_begin
  const int b = block_begin + bl;
  const int32_t* sel_bj = sel + (static_cast<int64_t>(b) * n_kv + j) * k_g;
  const int c = threadIdx.x % cpr;
  const int r0 = threadIdx.x / cpr;
  const int64_t out_base = (static_cast<int64_t>(bl) * n_kv + j) * k_g * kGroup;

  for (int row0 = 0; row0 < 64; row0 += rows_per_pass * 4) {
    uint4 kv[4], vv[4];
    int64_t dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = row0 + r0 + u * rows_per_pass;  // 0..63 within the tile
      const int slot = tile * 8 + row / kGroup;
      kv[u] = make_uint4(0, 0, 0, 0);
      vv[u] = make_uint4(0, 0, 0, 0);
      dst[u] = -1;
      if (row < 64 && slot < k_g) {
        dst[u] = (out_base + static_cast<int64_t>(slot) * kGroup + row % kGroup) * row_bytes + c * 16;
        const int n = valid_group(sel_bj[slot], n_groups);
        if (n >= 0) {
          const int64_t src = (static_cast<int64_t>(j) * hist_rows + static_cast<int64_t>(n) * kGroup +
                               row % kGroup) * row_bytes + c * 16;
          kv[u] = *reinterpret_cast<const uint4*>(k_hist + src);
          vv[u] = *reinterpret_cast<const uint4*>(v_hist + src);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (dst[u] >= 0) {
        *reinterpret_cast<uint4*>(k_out + dst[u]) = kv[u];
        *reinterpret_cast<uint4*>(v_out + dst[u]) = vv[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_gather(const hga_shape& s, const void* k_hist, const void* v_hist,
                         const int32_t* sel_groups, void* k_out, void* v_out,
                         int32_t block_begin, int32_t block_end, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (block_end <= block_begin) return hipSuccess;
  const int elem = s.dtype == HGA_BF16 ? 2 : 4;
  const int n_tiles = (s.top_k_groups + 7) / 8;
  dim3 grid(static_cast<unsigned>((block_end - block_begin) * s.n_kv_heads * n_tiles));
  if (s.head_dim == 128)
    hipExtLaunchKernelGGL((gather_kernel<128>), grid, dim3(kThreads), 0, stream, ev_start, ev_stop, 0,
                       static_cast<const uint8_t*>(k_hist), static_cast<const uint8_t*>(v_hist),
                       sel_groups, static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out), elem,
                       hist_rows(s), s.hist_len / kGroup, s.n_kv_heads, s.top_k_groups, block_begin);
  else
    hipExtLaunchKernelGGL((gather_kernel<64>), grid, dim3(kThreads), 0, stream, ev_start, ev_stop, 0,
                       static_cast<const uint8_t*>(k_hist), static_cast<const uint8_t*>(v_hist),
                       sel_groups, static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out), elem,
                       hist_rows(s), s.hist_len / kGroup, s.n_kv_heads, s.top_k_groups, block_begin);
  return hipGetLastError();
}

}  // namespace hga
