// Chunk and group summaries: segmented means of the history keys.
//
// One workgroup summarises one 64-token chunk of one KV head with D threads:
// thread (g, c) owns group g (8 tokens) and the 8 dims c*8..c*8+7, loads its
// eight 16-byte (bf16) pieces at once, sums them in registers and writes its
// part of the group mean straight to memory; the chunk sum then adds the
// eight group sums through LDS after one barrier. Every load of the chunk is
// in flight before any add, and only the chunk sums pass through LDS. HBM
// bound: per chunk it reads 64*d elements and writes 9*d floats.
// Summation order (bitwise the same for every launch shape): a group sum is
// (k0+k1+k2+k3) + (k4+k5+k6+k7); a chunk sum adds the group sums in order,
// each sum starting from +0.
#include "hga_common.hpp"

namespace hga {
namespace {

constexpr int kThreads = 256;   // round_bf16_kernel

template <typename T, int D>
__global__ __launch_bounds__(D) void build_summaries_kernel(
    const T* __restrict__ k_hist, int64_t hist_rows, int64_t chunk_begin,
    float* __restrict__ chunk_sum, float* __restrict__ group_sum) {
  constexpr int TPG = D / 8;                   // threads per group row
  constexpr int NG = kChunk / kGroup;          // groups per chunk
  static_assert(TPG * NG == D, "one thread per (group, 8 dims)");
  __shared__ __attribute__((aligned(16))) float gsum[NG][D];

  const int t = threadIdx.x;
  const int c = t % TPG;                       // 8-dim column
  const int g = t / TPG;                       // group within the chunk
  const int64_t m = chunk_begin + blockIdx.x;  // chunk index
  const int j = blockIdx.y;                    // KV head

  const T* src = k_hist + (static_cast<int64_t>(j) * hist_rows + m * kChunk + g * kGroup) * D + c * 8;
  float v[kGroup][8];
#pragma unroll
  for (int u = 0; u < kGroup; ++u) Elem<T>::load8(src + static_cast<int64_t>(u) * D, v[u]);
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float lo = (((0.f + v[0][e]) + v[1][e]) + v[2][e]) + v[3][e];
    const float hi = (((0.f + v[4][e]) + v[5][e]) + v[6][e]) + v[7][e];
    s[e] = (0.f + lo) + hi;
  }
  *reinterpret_cast<float4*>(&gsum[g][c * 8]) = make_float4(s[0], s[1], s[2], s[3]);
  *reinterpret_cast<float4*>(&gsum[g][c * 8 + 4]) = make_float4(s[4], s[5], s[6], s[7]);
  const int64_t n_groups_total = hist_rows / kGroup;   // group rows per KV head
  float* gdst = group_sum + (static_cast<int64_t>(j) * n_groups_total + m * NG + g) * D + c * 8;
  constexpr float kInvG = 1.0f / kGroup;
  *reinterpret_cast<float4*>(gdst) = make_float4(s[0] * kInvG, s[1] * kInvG, s[2] * kInvG, s[3] * kInvG);
  *reinterpret_cast<float4*>(gdst + 4) = make_float4(s[4] * kInvG, s[5] * kInvG, s[6] * kInvG, s[7] * kInvG);
  __syncthreads();
  if (t < D / 4) {                             // 4 chunk dims per thread
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const float4 b = *reinterpret_cast<const float4*>(&gsum[q][t * 4]);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    constexpr float kInvC = 1.0f / kChunk;
    *reinterpret_cast<float4*>(chunk_sum + (static_cast<int64_t>(j) * (hist_rows / kChunk) + m) * D + t * 4) =
        make_float4(a.x * kInvC, a.y * kInvC, a.z * kInvC, a.w * kInvC);
  }
}

template <typename T, int D>
hipError_t launch_t(const hga_shape& s, const void* k, int64_t c0, int64_t c1, float* cs,
                    float* gs, hipStream_t st) {
  dim3 grid(static_cast<unsigned>(c1 - c0), static_cast<unsigned>(s.n_kv_heads));
  hipExtLaunchKernelGGL((build_summaries_kernel<T, D>), grid, dim3(D), 0, st,
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
