// Chunk and group summaries: segmented means of the history keys.
//
// One workgroup summarises one 64-token chunk of one KV head: it streams the
// chunk's keys once (coalesced 16-byte loads, 256 B per token row), forms the
// eight 8-token group sums in LDS, and derives the chunk sum from them. HBM
// bound: per chunk it reads 64*d elements and writes 9*d floats.
#include "hga_common.hpp"

namespace hga {
namespace {

constexpr int kThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void build_summaries_kernel(
    const T* __restrict__ k_hist, int64_t hist_rows, int64_t chunk_begin,
    float* __restrict__ chunk_sum, float* __restrict__ group_sum) {
  constexpr int TPR = D / 8;                  // threads per token row
  constexpr int RG = kThreads / TPR;          // row groups
  constexpr int TOK_PER_RG = kChunk / RG;     // consecutive tokens per row group
  constexpr int RG_PER_GROUP = kGroup / TOK_PER_RG;
  static_assert(TOK_PER_RG * RG == kChunk && RG_PER_GROUP * TOK_PER_RG == kGroup, "tiling");

  __shared__ float part[RG][D + 1];
  __shared__ float gsum[kChunk / kGroup][D + 1];

  const int t = threadIdx.x;
  const int dc = t % TPR;
  const int rg = t / TPR;
  const int64_t m = chunk_begin + blockIdx.x;  // chunk index
  const int j = blockIdx.y;                    // KV head

  const T* src = k_hist + (static_cast<int64_t>(j) * hist_rows + m * kChunk + rg * TOK_PER_RG) * D + dc * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < TOK_PER_RG; ++u) {
    float v[8];
    Elem<T>::load8(src + static_cast<int64_t>(u) * D, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][dc * 8 + e] = acc[e];
  __syncthreads();

  const int64_t n_groups_total = hist_rows / kGroup;   // group rows per KV head
  for (int idx = t; idx < (kChunk / kGroup) * D; idx += kThreads) {
    const int g = idx / D, e = idx % D;
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < RG_PER_GROUP; ++q) s += part[g * RG_PER_GROUP + q][e];
    gsum[g][e] = s;
    group_sum[(static_cast<int64_t>(j) * n_groups_total + m * (kChunk / kGroup) + g) * D + e] =
        s * (1.0f / kGroup);
  }
  __syncthreads();
  if (t < D) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < kChunk / kGroup; ++g) s += gsum[g][t];
    chunk_sum[(static_cast<int64_t>(j) * (hist_rows / kChunk) + m) * D + t] = s * (1.0f / kChunk);
  }
}

template <typename T, int D>
hipError_t launch_t(const hga_shape& s, const void* k, int64_t c0, int64_t c1, float* cs,
                    float* gs, hipStream_t st) {
  dim3 grid(static_cast<unsigned>(c1 - c0), static_cast<unsigned>(s.n_kv_heads));
  hipExtLaunchKernelGGL((build_summaries_kernel<T, D>), grid, dim3(kThreads), 0, st,
                        timer_event(HGA_KERNEL_SUMMARIES, 0), timer_event(HGA_KERNEL_SUMMARIES, 1), 0,
                        static_cast<const T*>(k), hist_rows(s), c0, cs, gs);
  return hipGetLastError();
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet), overflow goes
// to infinity. Eight elements per thread: two 16-byte loads, one 16-byte store.
__device__ __forceinline__ uint32_t round_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kThreads) void round_bf16_kernel(const float* __restrict__ src,
                                                              uint16_t* __restrict__ dst, int64_t n8) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n8; i += stride) {
    const float4 a = reinterpret_cast<const float4*>(src)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(src)[2 * i + 1];
    uint4 o;
    o.x = round_bf16(a.x) | (round_bf16(a.y) << 16);
    o.y = round_bf16(a.z) | (round_bf16(a.w) << 16);
    o.z = round_bf16(b.x) | (round_bf16(b.y) << 16);
    o.w = round_bf16(b.z) | (round_bf16(b.w) << 16);
    reinterpret_cast<uint4*>(dst)[i] = o;
  }
}

}  // namespace

hipError_t launch_round_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t stream) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t wgs = (n8 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(round_bf16_kernel, dim3(static_cast<unsigned>(wgs < (1 << 20) ? wgs : (1 << 20))),
                     dim3(kThreads), 0, stream, src, dst, n8);
  return hipGetLastError();
}

hipError_t launch_build_summaries(const hga_shape& s, const void* k_hist, int64_t tok_begin,
                                  int64_t tok_end, float* chunk_sum, float* group_sum,
                                  hipStream_t stream) {
  const int64_t c0 = tok_begin / kChunk, c1 = tok_end / kChunk;
  if (c1 <= c0) return hipSuccess;
  const bool bf = s.dtype == HGA_BF16;
  if (s.head_dim == 128)
    return bf ? launch_t<uint16_t, 128>(s, k_hist, c0, c1, chunk_sum, group_sum, stream)
              : launch_t<float, 128>(s, k_hist, c0, c1, chunk_sum, group_sum, stream);
  return bf ? launch_t<uint16_t, 64>(s, k_hist, c0, c1, chunk_sum, group_sum, stream)
            : launch_t<float, 64>(s, k_hist, c0, c1, chunk_sum, group_sum, stream);
}

}  // namespace hga
