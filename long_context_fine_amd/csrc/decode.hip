// HGA decode step: the n_new newest tokens of every sequence in a batch
// attend the sink, the groups their query block routed to, and the causal
// window of the open (not yet summarised) segment that ends with them
// (gist.science Technical Summary §2.1 "Exact-Token Attention"; §3: the
// adapter runs with HGA for retrieval and generation).
//
// HBM-bound (each key row is read once for r * n_new query rows), so the
// kernel is VALU: D/8 lanes per key row (16-byte loads, one wave instruction
// covers 64/(D/8) whole rows), the virtual key list of a (sequence, KV head)
// [sink | routed groups | open-segment window] split into 256-key pieces, one
// workgroup each. A piece: scores of all its keys for all query rows to LDS,
// max and sum per row, then P.V; the unnormalised partial O with its (max,
// sum) goes to the workspace and decode_merge_kernel combines the pieces of
// each query row in a fixed order. Deterministic; no atomics.
#include "hga_common.hpp"

namespace hga {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecKeys = 256;  // keys per piece (one workgroup)
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeParams {
  const void* q;       // [batch][n_q][n_new][D]
  const void* k_hist;  // [batch][n_kv][P][D]
  const void* v_hist;
  const void* k_tail;  // [batch][n_kv][T][D]
  const void* v_tail;
  const int32_t* sel;  // [batch][n_kv][k_g]
  const int32_t* hist_lens;
  const int32_t* tail_lens;
  void* o;             // [batch][n_q][n_new][D]
  float* lse;          // [batch][n_q][n_new]
  float* part;         // [batch][n_q][n_new][n_piece][D]
  float* part_ml;      // [batch][n_q][n_new][n_piece][2]: max (log2 units), sum
  int n_q, n_kv, r, n_new;
  int64_t P;           // history rows per (sequence, KV head)
  int T;               // open-segment rows per (sequence, KV head)
  int k_g, n_sink, window, n_piece;
  float scale_log2;
};

// Lengths of sequence b, clamped to the buffers: history in whole chunks,
// open segment holding at least the new tokens. Key list [sink | routed |
// open-segment tokens t_lo .. tb-1 that some new token's window reaches].
struct SeqKeys {
  int hb, tb, sink, t_lo, n_keys;
};

__device__ __forceinline__ SeqKeys seq_keys(const DecodeParams& p, int b) {
  SeqKeys s;
  int hb = p.hist_lens[b];
  hb = hb < 0 ? 0 : (hb > p.P ? static_cast<int>(p.P) : hb);
  s.hb = hb - hb % kChunk;
  int tb = p.tail_lens[b];
  s.tb = tb < p.n_new ? p.n_new : (tb > p.T ? p.T : tb);
  s.sink = min(p.n_sink * kChunk, s.hb);
  s.t_lo = max(0, s.tb - p.n_new - p.window + 1);
  s.n_keys = s.sink + p.k_g * kGroup + (s.tb - s.t_lo);
  return s;
}

template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = 1; o < LPK; o <<= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

template <typename T, int D, int NQ>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(DecodeParams p) {
  constexpr int LPK = D / 8;              // lanes per key row
  constexpr int KPW = kWave / LPK;        // keys per wave and step
  constexpr int NW = kDecThreads / kWave;
  constexpr int KPS = NW * KPW;           // keys per workgroup and step
  __shared__ float s_lds[NQ][kDecKeys];
  __shared__ float o_lds[NW][NQ][D];
  const int piece = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int sub = lane % LPK, kin = lane / LPK;

  const SeqKeys sk = seq_keys(p, b);
  const int k0 = piece * kDecKeys;
  if (k0 >= sk.n_keys) return;            // whole workgroup: past this sequence's keys
  const int nk = min(kDecKeys, sk.n_keys - k0);
  const int R = p.r * p.n_new;            // query rows, <= NQ (checked on the host)
  const int n_routed = p.k_g * kGroup;
  const int64_t hrow0 = (static_cast<int64_t>(b) * p.n_kv + j) * p.P;
  const int64_t trow0 = (static_cast<int64_t>(b) * p.n_kv + j) * p.T;
  const int32_t* sel_bj = p.sel + (static_cast<int64_t>(b) * p.n_kv + j) * p.k_g;

  // row of virtual key v (nullptr: an empty routed slot); tail >= 0 is its
  // open-segment position
  auto key_row = [&](int v, const T* hist, const T* tail, int& tpos) -> const T* {
    tpos = -1;
    if (v < sk.sink) return hist + (hrow0 + v) * D;
    v -= sk.sink;
    if (v < n_routed) {
      const int g = sel_bj[v / kGroup];
      return g >= 0 ? hist + (hrow0 + static_cast<int64_t>(g) * kGroup + v % kGroup) * D : nullptr;
    }
    tpos = sk.t_lo + v - n_routed;
    return tail + (trow0 + tpos) * D;
  };

  float qr[NQ][8];
#pragma unroll
  for (int rq = 0; rq < NQ; ++rq) {
    if (rq < R) {
      const int64_t row = (static_cast<int64_t>(b) * p.n_q + j * p.r + rq / p.n_new) * p.n_new + rq % p.n_new;
      Elem<T>::load8(static_cast<const T*>(p.q) + row * D + sub * 8, qr[rq]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[rq][e] = 0.f;
    }
  }

  // ---- scores of every key of the piece, all query rows -------------------
  const T* kh = static_cast<const T*>(p.k_hist);
  const T* kt = static_cast<const T*>(p.k_tail);
  for (int base = wave * KPW; base < nk; base += KPS) {
    const int kk = base + kin;
    const bool live = kk < nk;
    int tpos = -1;
    const T* row = live ? key_row(k0 + kk, kh, kt, tpos) : nullptr;
    float kf[8];
    if (row) {
      Elem<T>::load8(row + sub * 8, kf);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = 0.f;
    }
#pragma unroll
    for (int rq = 0; rq < NQ; ++rq) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qr[rq][e], kf[e], d);
      d = group_sum<LPK>(d);
      if (live && sub == 0 && rq < R) {
        bool ok = row != nullptr;
        if (tpos >= 0) {
          const int qpos = sk.tb - p.n_new + rq % p.n_new;   // open-segment position of the row
          ok = tpos <= qpos && tpos > qpos - p.window;
        }
        s_lds[rq][kk] = ok ? d * p.scale_log2 : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- per row: max and sum over the piece; probabilities in place --------
  for (int rq = wave; rq < R; rq += NW) {
    float m = -INFINITY;
    for (int kk = lane; kk < nk; kk += kWave) m = fmaxf(m, s_lds[rq][kk]);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    float l = 0.f;
    for (int kk = lane; kk < nk; kk += kWave) {
      const float e = m == -INFINITY ? 0.f : exp2f(s_lds[rq][kk] - m);
      s_lds[rq][kk] = e;
      l += e;
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) l += __shfl_xor(l, o, kWave);
    if (lane == 0) {
      const int64_t row = (static_cast<int64_t>(b) * p.n_q + j * p.r + rq / p.n_new) * p.n_new + rq % p.n_new;
      float* ml = p.part_ml + (row * p.n_piece + piece) * 2;
      ml[0] = m;
      ml[1] = l;
    }
  }
  __syncthreads();

  // ---- P . V ---------------------------------------------------------------
  float acc[NQ][8];
#pragma unroll
  for (int rq = 0; rq < NQ; ++rq)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[rq][e] = 0.f;
  const T* vh = static_cast<const T*>(p.v_hist);
  const T* vt = static_cast<const T*>(p.v_tail);
  for (int base = wave * KPW; base < nk; base += KPS) {
    const int kk = base + kin;
    if (kk >= nk) continue;
    int tpos;
    const T* row = key_row(k0 + kk, vh, vt, tpos);
    if (!row) continue;
    float vf[8];
    Elem<T>::load8(row + sub * 8, vf);
#pragma unroll
    for (int rq = 0; rq < NQ; ++rq) {
      const float pr = rq < R ? s_lds[rq][kk] : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[rq][e] = fmaf(pr, vf[e], acc[rq][e]);
    }
  }
  // sum the wave's key groups (lanes with equal sub), then the waves in LDS
#pragma unroll
  for (int rq = 0; rq < NQ; ++rq)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = LPK; o < kWave; o <<= 1) acc[rq][e] += __shfl_xor(acc[rq][e], o, kWave);
  if (kin == 0) {
#pragma unroll
    for (int rq = 0; rq < NQ; ++rq)
#pragma unroll
      for (int e = 0; e < 8; ++e) o_lds[wave][rq][sub * 8 + e] = acc[rq][e];
  }
  __syncthreads();
  for (int x = t; x < R * D; x += kDecThreads) {
    const int rq = x / D, dd = x % D;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += o_lds[w][rq][dd];
    const int64_t row = (static_cast<int64_t>(b) * p.n_q + j * p.r + rq / p.n_new) * p.n_new + rq % p.n_new;
    p.part[(row * p.n_piece + piece) * D + dd] = v;
  }
}

// One workgroup of D threads per query row (sequence, head, new token):
// combines the row's pieces in piece order.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeParams p) {
  const int64_t row = blockIdx.x;                // (b * n_q + h) * n_new + i
  const int b = static_cast<int>(row / (static_cast<int64_t>(p.n_q) * p.n_new));
  const SeqKeys sk = seq_keys(p, b);
  const int n = (sk.n_keys + kDecKeys - 1) / kDecKeys;
  const float* ml = p.part_ml + row * p.n_piece * 2;
  float m = -INFINITY;
  for (int s = 0; s < n; ++s) m = fmaxf(m, ml[2 * s]);
  float l = 0.f, o = 0.f;
  const float* po = p.part + row * p.n_piece * D + threadIdx.x;
  for (int s = 0; s < n; ++s) {
    const float a = ml[2 * s] == -INFINITY ? 0.f : exp2f(ml[2 * s] - m);
    l += a * ml[2 * s + 1];
    o += a * po[static_cast<int64_t>(s) * D];
  }
  static_cast<T*>(p.o)[row * D + threadIdx.x] = Elem<T>::from_f32(o / l);
  if (threadIdx.x == 0) p.lse[row] = (m + log2f(l)) * kLn2;
}

template <typename T, int D>
hipError_t launch_td(const hga_shape& s, DecodeParams& p, int batch, hipStream_t st) {
  const dim3 grid(p.n_piece, s.n_kv_heads, batch);
  const int R = p.r * p.n_new;
  hipEvent_t e0 = timer_event(HGA_KERNEL_DECODE, 0), e1 = timer_event(HGA_KERNEL_DECODE, 1);
  if (R <= 4)
    hipExtLaunchKernelGGL((decode_attn_kernel<T, D, 4>), grid, dim3(kDecThreads), 0, st, e0, nullptr, 0, p);
  else if (R <= 8)
    hipExtLaunchKernelGGL((decode_attn_kernel<T, D, 8>), grid, dim3(kDecThreads), 0, st, e0, nullptr, 0, p);
  else
    hipExtLaunchKernelGGL((decode_attn_kernel<T, D, 16>), grid, dim3(kDecThreads), 0, st, e0, nullptr, 0, p);
  hipExtLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(static_cast<unsigned>(batch * p.n_q * p.n_new)),
                        dim3(D), 0, st, nullptr, e1, 0, p);
  return hipGetLastError();
}

}  // namespace

int decode_pieces(const hga_shape& s) {
  const int64_t P = hist_rows(s);
  const int64_t sink = static_cast<int64_t>(s.n_sink_chunks) * kChunk < P ? s.n_sink_chunks * kChunk : P;
  const int64_t keys = sink + static_cast<int64_t>(s.top_k_groups) * kGroup + s.seg_len;
  return static_cast<int>((keys + kDecKeys - 1) / kDecKeys);
}

size_t decode_attn_workspace_bytes(const hga_shape& s, int batch, int n_new) {
  const size_t rows = static_cast<size_t>(batch) * s.n_q_heads * n_new;
  const size_t n = decode_pieces(s);
  return ((rows * n * s.head_dim * sizeof(float) + 255) & ~size_t(255)) + rows * n * 2 * sizeof(float);
}

hipError_t launch_decode_attn(const hga_shape& s, int batch, int n_new, const void* q, const void* k_hist,
                              const void* v_hist, const void* k_tail, const void* v_tail,
                              const int32_t* sel_groups, const int32_t* hist_lens, const int32_t* tail_lens,
                              void* o, float* lse, void* ws, hipStream_t stream) {
  DecodeParams p;
  p.q = q; p.k_hist = k_hist; p.v_hist = v_hist; p.k_tail = k_tail; p.v_tail = v_tail;
  p.sel = sel_groups; p.hist_lens = hist_lens; p.tail_lens = tail_lens; p.o = o; p.lse = lse;
  p.n_q = s.n_q_heads; p.n_kv = s.n_kv_heads; p.r = s.n_q_heads / s.n_kv_heads; p.n_new = n_new;
  p.P = hist_rows(s); p.T = s.seg_len; p.k_g = s.top_k_groups; p.n_sink = s.n_sink_chunks;
  p.window = local_window(s); p.n_piece = decode_pieces(s);
  p.scale_log2 = s.softmax_scale * 1.4426950408889634f;
  const size_t rows = static_cast<size_t>(batch) * s.n_q_heads * n_new;
  p.part = static_cast<float*>(ws);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                       ((rows * p.n_piece * s.head_dim * sizeof(float) + 255) & ~size_t(255)));
  const bool bf = s.dtype == HGA_BF16;
  if (s.head_dim == 128) return bf ? launch_td<uint16_t, 128>(s, p, batch, stream) : launch_td<float, 128>(s, p, batch, stream);
  return bf ? launch_td<uint16_t, 64>(s, p, batch, stream) : launch_td<float, 64>(s, p, batch, stream);
}

}  // namespace hga
