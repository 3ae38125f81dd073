// Two-level content routing: block queries, chunk scores, chunk top-k, group
// scores inside the kept chunks, group top-k. Three launches:
//   block_query_kernel  (n_B x n_kv WGs)  Q -> qbar            reads Q once
//   chunk_score_kernel  (n_C/64 x n_kv)   qbar, C -> scores    reads C once
//   select_kernel       (n_B x n_kv)      scores, G -> lists   reads 8*k_c rows of G
// All three are HBM/latency bound. Ranking uses a 64-bit key (order-preserving
// fp32 bits, then the complemented index) so the max of keys is the best score
// with the lowest index on ties; the whole route is deterministic.
#include "hga_common.hpp"

namespace hga {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkTile = 64;  // chunks per chunk_score workgroup
constexpr int kBlockTile = 32;  // query blocks held in LDS at once

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// qbar[b][j][:] = mean of q[h][64b .. 64b+63][:] over h in [j*r, j*r + r).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void block_query_kernel(const T* __restrict__ q, int seg_len,
                                                               int n_kv, int r,
                                                               float* __restrict__ qbar) {
  constexpr int TPR = D / 8;
  constexpr int RG = kThreads / TPR;
  __shared__ float part[RG][D + 1];
  const int t = threadIdx.x, dc = t % TPR, rg = t / TPR;
  const int b = blockIdx.x, j = blockIdx.y;
  const int rows = kBlockQ * r;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 4
  for (int row = rg; row < rows; row += RG) {
    const int h = j * r + row / kBlockQ, i = b * kBlockQ + row % kBlockQ;
    float v[8];
    Elem<T>::load8(q + (static_cast<int64_t>(h) * seg_len + i) * D + dc * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][dc * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += part[g][t];
    qbar[(static_cast<int64_t>(b) * n_kv + j) * D + t] = s * (1.0f / static_cast<float>(rows));
  }
}

// scores[b][j][m] = qbar[b][j] . C[j][m] for a tile of 64 chunks, all blocks.
template <int D>
__global__ __launch_bounds__(kThreads) void chunk_score_kernel(const float* __restrict__ qbar,
                                                               const float* __restrict__ csum,
                                                               int n_blocks, int n_kv, int n_chunks,
                                                               float* __restrict__ scores) {
  __shared__ float ct[kChunkTile][D + 1];
  __shared__ float qb[kBlockTile][D];
  const int t = threadIdx.x;
  const int j = blockIdx.y;
  const int m0 = blockIdx.x * kChunkTile;
  const int n_here = min(kChunkTile, n_chunks - m0);
  for (int idx = t; idx < kChunkTile * D; idx += kThreads) {
    const int c = idx / D, e = idx % D;
    ct[c][e] = c < n_here ? csum[(static_cast<int64_t>(j) * n_chunks + m0 + c) * D + e] : 0.f;
  }
  const int c = t % kChunkTile;
  const int bq = t / kChunkTile;  // 0..3 (one per wave: broadcast reads of qb)
  for (int b0 = 0; b0 < n_blocks; b0 += kBlockTile) {
    const int nb = min(kBlockTile, n_blocks - b0);
    __syncthreads();
    for (int idx = t; idx < kBlockTile * D; idx += kThreads) {
      const int bb = idx / D, e = idx % D;
      qb[bb][e] = bb < nb ? qbar[(static_cast<int64_t>(b0 + bb) * n_kv + j) * D + e] : 0.f;
    }
    __syncthreads();
    float acc[kBlockTile / 4];
#pragma unroll
    for (int k = 0; k < kBlockTile / 4; ++k) acc[k] = 0.f;
    for (int e = 0; e < D; ++e) {
      const float cv = ct[c][e];
#pragma unroll
      for (int k = 0; k < kBlockTile / 4; ++k) acc[k] += qb[bq + 4 * k][e] * cv;
    }
    if (c < n_here) {
#pragma unroll
      for (int k = 0; k < kBlockTile / 4; ++k) {
        const int bb = bq + 4 * k;
        if (bb < nb)
          scores[(static_cast<int64_t>(b0 + bb) * n_kv + j) * n_chunks + m0 + c] = acc[k];
      }
    }
  }
}

__device__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
  v = wave_max_u64(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x % kWave) == 0) red[w] = v;
  __syncthreads();
  uint64_t best = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) best = red[i] > best ? red[i] : best;
  return best;
}

// Per (block, KV head): chunk top-k from the scores, then group scoring over the
// 8 groups of each kept chunk and group top-k. Outputs ascending, -1 padded.
template <int D>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ scores,
    const float* __restrict__ gsum, int n_kv, int n_chunks, int k_c, int k_g,
    int32_t* __restrict__ sel_chunks, int32_t* __restrict__ sel_groups) {
  constexpr int TPC = D / 8;  // threads per group candidate
  constexpr int kMaxCand = kMaxTopKChunks * (kChunk / kGroup);
  __shared__ uint64_t red[kThreads / kWave];
  __shared__ int32_t chosen[kMaxTopKChunks];
  __shared__ int32_t sorted[kMaxTopKChunks];
  __shared__ float qv[D];
  __shared__ float gsc[kMaxCand];
  __shared__ uint8_t flag[kMaxCand];

  const int t = threadIdx.x;
  const int b = blockIdx.x, j = blockIdx.y;
  const int64_t bj = static_cast<int64_t>(b) * n_kv + j;
  const float* sc = scores + bj * n_chunks;
  const int kc_eff = min(k_c, n_chunks);

  if (t < D) qv[t] = qbar[bj * D + t];

  // chunk top-k: each round takes the best key strictly below the previous one
  uint64_t prev = ~0ull;
  for (int round = 0; round < kc_eff; ++round) {
    uint64_t local = 0;
    for (int m = t; m < n_chunks; m += kThreads) {
      const uint64_t k = rank_key(sc[m], static_cast<uint32_t>(m));
      if (k < prev && k > local) local = k;
    }
    prev = block_max_u64(local, red);
    if (t == 0) chosen[round] = static_cast<int32_t>(rank_key_index(prev));
  }
  __syncthreads();
  if (t < kc_eff) {
    const int id = chosen[t];
    int pos = 0;
    for (int u = 0; u < kc_eff; ++u) pos += chosen[u] < id;
    sorted[pos] = id;
  }
  __syncthreads();
  if (t < k_c) sel_chunks[bj * k_c + t] = t < kc_eff ? sorted[t] : -1;

  // group scores for the 8 groups of every kept chunk
  const int n_cand = kc_eff * (kChunk / kGroup);
  const int64_t n_groups_total = static_cast<int64_t>(n_chunks) * (kChunk / kGroup);
  const int lane_in = t % TPC;
  for (int c0 = 0; c0 < n_cand; c0 += kThreads / TPC) {
    const int c = c0 + t / TPC;
    float part = 0.f;
    if (c < n_cand) {
      const int64_t gid = static_cast<int64_t>(sorted[c / 8]) * 8 + (c % 8);
      float g[8];
      Elem<float>::load8(gsum + (static_cast<int64_t>(j) * n_groups_total + gid) * D + lane_in * 8, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) part += g[e] * qv[lane_in * 8 + e];
    }
#pragma unroll
    for (int m = TPC / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, kWave);
    if (c < n_cand && lane_in == 0) gsc[c] = part;
  }
  __syncthreads();

  // group top-k by rank counting: selected iff fewer than k_g candidates beat it
  for (int c = t; c < n_cand; c += kThreads) {
    const uint32_t gid = static_cast<uint32_t>(sorted[c / 8] * 8 + (c % 8));
    const uint64_t kc = rank_key(gsc[c], gid);
    int beaten = 0;
    for (int o = 0; o < n_cand; ++o) {
      const uint32_t gido = static_cast<uint32_t>(sorted[o / 8] * 8 + (o % 8));
      beaten += rank_key(gsc[o], gido) > kc;
    }
    flag[c] = beaten < k_g;
  }
  __syncthreads();
  // candidates are enumerated in ascending group id, so the output position
  // of a selected candidate is the number of selected candidates before it
  for (int c = t; c < n_cand; c += kThreads) {
    if (flag[c]) {
      int pos = 0;
      for (int o = 0; o < c; ++o) pos += flag[o];
      sel_groups[bj * k_g + pos] = sorted[c / 8] * 8 + (c % 8);
    }
  }
  const int kg_eff = min(k_g, n_cand);
  for (int p = kg_eff + t; p < k_g; p += kThreads) sel_groups[bj * k_g + p] = -1;
}

template <typename T, int D>
hipError_t launch_t(const hga_shape& s, const void* q, const float* cs, const float* gs,
                    int32_t* sc_out, int32_t* sg_out, void* ws, hipStream_t st) {
  const int n_blocks = s.seg_len / kBlockQ;
  const int n_chunks = static_cast<int>(s.hist_len / kChunk);
  const int r = s.n_q_heads / s.n_kv_heads;
  float* qbar = static_cast<float*>(ws);
  float* scores = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                           align256(sizeof(float) * n_blocks * s.n_kv_heads * D));
  timer_begin(HGA_KERNEL_BLOCK_QUERY, st);
  hipLaunchKernelGGL((block_query_kernel<T, D>), dim3(n_blocks, s.n_kv_heads), dim3(kThreads), 0,
                     st, static_cast<const T*>(q), s.seg_len, s.n_kv_heads, r, qbar);
  timer_end(HGA_KERNEL_BLOCK_QUERY, st);
  if (n_chunks > 0) {
    timer_begin(HGA_KERNEL_CHUNK_SCORE, st);
    hipLaunchKernelGGL((chunk_score_kernel<D>),
                       dim3((n_chunks + kChunkTile - 1) / kChunkTile, s.n_kv_heads),
                       dim3(kThreads), 0, st, qbar, cs, n_blocks, s.n_kv_heads, n_chunks, scores);
    timer_end(HGA_KERNEL_CHUNK_SCORE, st);
  }
  timer_begin(HGA_KERNEL_SELECT, st);
  hipLaunchKernelGGL((select_kernel<D>), dim3(n_blocks, s.n_kv_heads), dim3(kThreads), 0, st,
                     qbar, scores, gs, s.n_kv_heads, n_chunks, s.top_k_chunks, s.top_k_groups,
                     sc_out, sg_out);
  timer_end(HGA_KERNEL_SELECT, st);
  return hipGetLastError();
}

}  // namespace

size_t route_workspace_bytes(const hga_shape& s) {
  const size_t n_blocks = s.seg_len / kBlockQ;
  const size_t n_chunks = static_cast<size_t>(s.hist_len / kChunk);
  return align256(sizeof(float) * n_blocks * s.n_kv_heads * s.head_dim) +
         align256(sizeof(float) * n_blocks * s.n_kv_heads * (n_chunks ? n_chunks : 1));
}

hipError_t launch_route(const hga_shape& s, const void* q, const float* chunk_sum,
                        const float* group_sum, int32_t* sel_chunks, int32_t* sel_groups,
                        void* ws, hipStream_t stream) {
  const bool bf = s.dtype == HGA_BF16;
  if (s.head_dim == 128)
    return bf ? launch_t<uint16_t, 128>(s, q, chunk_sum, group_sum, sel_chunks, sel_groups, ws, stream)
              : launch_t<float, 128>(s, q, chunk_sum, group_sum, sel_chunks, sel_groups, ws, stream);
  return bf ? launch_t<uint16_t, 64>(s, q, chunk_sum, group_sum, sel_chunks, sel_groups, ws, stream)
            : launch_t<float, 64>(s, q, chunk_sum, group_sum, sel_chunks, sel_groups, ws, stream);
}

}  // namespace hga
