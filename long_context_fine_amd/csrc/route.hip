// Two-level content routing, one workgroup per (query block b, KV head j):
//   1. block query qbar = mean of the block's 64 queries over the r heads of j
//      (reads its 64 KiB of Q once, 16-byte loads);
//   2. chunk scores qbar . C[j][m] for every history chunk (16 lanes per chunk,
//      coalesced 512-byte rows; C[j] stays in L2 across the 32 blocks);
//   3. chunk top-k: each wave takes the k_c best of its strided share in k_c
//      rounds of a wave-wide max over 64-bit keys strictly below the previous
//      one (key = order-preserving fp32 bits, then the complemented index, so
//      the maximum is the best score with the lowest index); the 4*k_c wave
//      candidates are merged by rank counting;
//   4. scores of the 8 groups of every kept chunk (reads 8*k_c rows of G);
//   5. group top-k by rank counting; candidates are enumerated in ascending
//      group id, so ballot prefix counts place the output in ascending order.
// HBM/latency bound. Deterministic.
#include "hga_common.hpp"

namespace hga {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsScores = 4096;  // chunk scores kept in LDS up to this many chunks

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Dot products of qv with `n` rows of `base` (row length D floats), 8 lanes per
// row, 8 rows per wave pass, UNROLL passes in flight; results to out[row].
template <int D, int UNROLL, class RowPtr>
__device__ __forceinline__ void score_rows(const float* qv, int n, RowPtr row_ptr, float* out) {
  constexpr int LPR = 8;                 // lanes per row
  constexpr int EPL = D / LPR;           // elements per lane (16 or 8)
  constexpr int RPP = kWave / LPR;       // rows per wave pass
  constexpr int NW = kThreads / kWave;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  static_assert(LPR == 8, "sum8_f32 reduces groups of 8 lanes");
  const int sub = lane % LPR;
  float qr[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qr[e] = qv[sub * EPL + e];
  for (int r0 = wave * RPP; r0 < n; r0 += NW * RPP * UNROLL) {
    float4 v[UNROLL][EPL / 4];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int row = r0 + u * NW * RPP + lane / LPR;
      const float* src = row < n ? row_ptr(row) + sub * EPL : nullptr;
#pragma unroll
      for (int c = 0; c < EPL / 4; ++c)
        v[u][c] = src ? reinterpret_cast<const float4*>(src)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < EPL / 4; ++c)
        s += v[u][c].x * qr[4 * c] + v[u][c].y * qr[4 * c + 1] + v[u][c].z * qr[4 * c + 2] +
             v[u][c].w * qr[4 * c + 3];
      s = sum8_f32(s);
      const int row = r0 + u * NW * RPP + lane / LPR;
      if (row < n && sub == 0) out[row] = s;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const T* __restrict__ q, const float* __restrict__ csum, const float* __restrict__ gsum,
    int seg_len, int n_kv, int r, int chunk0, int n_chunks, int chunk_rows, int k_c, int k_g,
    float* __restrict__ ws_scores,
    int32_t* __restrict__ sel_chunks, int32_t* __restrict__ sel_groups) {
  constexpr int TPR = D / 8;            // threads per Q row (8 elements each)
  constexpr int RG = kThreads / TPR;    // row groups
  constexpr int NW = kThreads / kWave;
  constexpr int kMaxCand = kMaxTopKChunks * (kChunk / kGroup);
  __shared__ float part[RG][D + 1];
  __shared__ float qv[D];
  __shared__ float sc_lds[kLdsScores];
  __shared__ __attribute__((aligned(16))) uint64_t wcand[NW][kMaxTopKChunks];
  __shared__ int32_t sorted[kMaxTopKChunks];
  __shared__ float gsc[kMaxCand];
  __shared__ __attribute__((aligned(16))) uint64_t gkey[kMaxCand];
  __shared__ uint64_t wmask[kMaxCand / kWave];
  __shared__ int32_t cnt_s[kThreads / 2];

  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int b = blockIdx.x, j = blockIdx.y;
  const int64_t bj = static_cast<int64_t>(b) * n_kv + j;

  // ---- 1. block query ----------------------------------------------------
  {
    const int dc = t % TPR, rg = t / TPR;
    const int rows = kBlockQ * r;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
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
      qv[t] = s * (1.0f / static_cast<float>(rows));
    }
    __syncthreads();
  }

  // ---- 2. chunk scores ----------------------------------------------------
  float* sc = n_chunks <= kLdsScores ? sc_lds : ws_scores + bj * n_chunks;
  // ranked chunks are chunk0 .. chunk0 + n_chunks - 1 (the sink is attended in full)
  const float* cbase = csum + (static_cast<int64_t>(j) * chunk_rows + chunk0) * D;
  score_rows<D, 8>(qv, n_chunks, [&](int m) { return cbase + static_cast<int64_t>(m) * D; }, sc);
  __syncthreads();

  // ---- 3. chunk top-k: per-wave top-k over strided elements, then merge ---
  const int kc_eff = min(k_c, n_chunks);
  {
    // keys of this lane's strided share kept in registers across the rounds
    // when the share is small (the common case), else re-read each round
    constexpr int kRegKeys = 8;
    uint64_t keys[kRegKeys];
#pragma unroll
    for (int e = 0; e < kRegKeys; ++e) {
      const int m = wave * kWave + lane + e * kThreads;
      keys[e] = m < n_chunks ? rank_key(sc[m], static_cast<uint32_t>(chunk0 + m)) : 0ull;
    }
    const bool in_regs = n_chunks <= kRegKeys * kThreads;
    uint64_t prev = ~0ull;
    for (int round = 0; round < kc_eff; ++round) {
      uint64_t local = 0;
      if (in_regs) {
#pragma unroll
        for (int e = 0; e < kRegKeys; ++e)
          if (keys[e] < prev && keys[e] > local) local = keys[e];
      } else {
        for (int m = wave * kWave + lane; m < n_chunks; m += kThreads) {
          const uint64_t k = rank_key(sc[m], static_cast<uint32_t>(chunk0 + m));
          if (k < prev && k > local) local = k;
        }
      }
      prev = wave_max_u64(local);      // 0 once this wave has no element left
      if (lane == 0) wcand[wave][round] = prev;
    }
  }
  __syncthreads();
  {
    // t < NW*kc_eff: candidate (wave t / kc_eff, round t % kc_eff)
    if (t < NW * kc_eff) {
      const uint64_t mine = wcand[t / kc_eff][t % kc_eff];
      // candidates are the first kc_eff slots of each wave's row, read two
      // keys at a time
      int rank = 0;
      for (int w2 = 0; w2 < NW; ++w2) {
        const ulonglong2* row = reinterpret_cast<const ulonglong2*>(wcand[w2]);
#pragma unroll 4
        for (int o2 = 0; o2 < (kc_eff + 1) / 2; ++o2) {
          const ulonglong2 c = row[o2];
          rank += c.x > mine;
          rank += (2 * o2 + 1 < kc_eff) && c.y > mine;
        }
      }
      // keys are unique (index in the low bits); the kc_eff best are all valid
      if (rank < kc_eff) part[0][rank] = __uint_as_float(rank_key_index(mine));
    }
    __syncthreads();
    if (t < kc_eff) {
      const int id = static_cast<int>(__float_as_uint(part[0][t]));
      int pos = 0;
      for (int u = 0; u < kc_eff; ++u) pos += static_cast<int>(__float_as_uint(part[0][u])) < id;
      sorted[pos] = id;
    }
    __syncthreads();
    if (t < k_c) sel_chunks[bj * k_c + t] = t < kc_eff ? sorted[t] : -1;
  }

  // ---- 4. group scores for the 8 groups of every kept chunk ----------------
  const int n_cand = kc_eff * (kChunk / kGroup);
  const float* gbase = gsum + static_cast<int64_t>(j) * chunk_rows * (kChunk / kGroup) * D;
  score_rows<D, 4>(qv, n_cand, [&](int c) {
    return gbase + (static_cast<int64_t>(sorted[c / 8]) * 8 + (c % 8)) * D;
  }, gsc);
  __syncthreads();
  for (int c = t; c < n_cand; c += kThreads)
    gkey[c] = rank_key(gsc[c], static_cast<uint32_t>(sorted[c / 8] * 8 + (c % 8)));
  __syncthreads();

  // ---- 5. group top-k by rank counting, ascending output via ballots ------
  // rank counts: with at most kThreads/2 candidates two threads share one
  // candidate, each counting half of the keys
  const ulonglong2* g2 = reinterpret_cast<const ulonglong2*>(gkey);
  const int n_pairs = n_cand / 2;           // n_cand = 8 * kc_eff is even
  if (n_cand <= kThreads / 2) {
    const int c = t % (kThreads / 2), hlf = t / (kThreads / 2);
    int beaten = 0;
    if (c < n_cand) {
      const uint64_t kc = gkey[c];
      const int o_end = hlf == 0 ? n_pairs / 2 : n_pairs;
#pragma unroll 4
      for (int o2 = hlf == 0 ? 0 : n_pairs / 2; o2 < o_end; ++o2) {
        const ulonglong2 x = g2[o2];
        beaten += (x.x > kc) + (x.y > kc);
      }
    }
    if (hlf == 1) cnt_s[c] = beaten;
    __syncthreads();
    if (hlf == 0) {
      const bool take = c < n_cand && beaten + cnt_s[c] < k_g;
      const uint64_t m = __ballot(take);
      if (lane == 0) wmask[wave] = m;
    }
  } else {
    for (int c0 = 0; c0 < n_cand; c0 += kThreads) {
      const int c = c0 + t;
      bool take = false;
      if (c < n_cand) {
        const uint64_t kc = gkey[c];
        int beaten = 0;
#pragma unroll 4
        for (int o2 = 0; o2 < n_pairs; ++o2) {
          const ulonglong2 x = g2[o2];
          beaten += (x.x > kc) + (x.y > kc);
        }
        take = beaten < k_g;
      }
      const uint64_t m = __ballot(take);
      if (lane == 0) wmask[(c0 / kWave) + wave] = m;
    }
  }
  __syncthreads();
  for (int c = t; c < n_cand; c += kThreads) {
    const uint64_t m = wmask[c / kWave];
    if ((m >> (c % kWave)) & 1ull) {
      int pos = __popcll(m & ((1ull << (c % kWave)) - 1ull));
      for (int w2 = 0; w2 < c / kWave; ++w2) pos += __popcll(wmask[w2]);
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
  const int chunk0 = sink_chunks(s);
  const int n_chunks = static_cast<int>(s.hist_len / kChunk) - chunk0;  // ranked chunks
  const int r = s.n_q_heads / s.n_kv_heads;
  float* scores = static_cast<float*>(ws);
  hipExtLaunchKernelGGL((route_kernel<T, D>), dim3(n_blocks, s.n_kv_heads), dim3(kThreads), 0, st,
                        timer_event(HGA_KERNEL_ROUTE, 0), timer_event(HGA_KERNEL_ROUTE, 1), 0,
                        static_cast<const T*>(q), cs, gs, s.seg_len, s.n_kv_heads, r, chunk0, n_chunks,
                        static_cast<int>(hist_rows(s) / kChunk),
                        s.top_k_chunks, s.top_k_groups, scores, sc_out, sg_out);
  return hipGetLastError();
}

}  // namespace

// Chunk scores spill to the workspace only when a KV head has more than
// kLdsScores history chunks; the size is reported for every shape anyway.
size_t route_workspace_bytes(const hga_shape& s) {
  const size_t n_blocks = s.seg_len / kBlockQ;
  const size_t n_chunks = static_cast<size_t>(s.hist_len / kChunk);
  return align256(sizeof(float) * n_blocks * s.n_kv_heads * (n_chunks ? n_chunks : 1));
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
