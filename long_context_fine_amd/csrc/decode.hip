// HGA decode step: the n_new newest tokens of every sequence in a batch
// attend the sink, the groups their query block routed to, and the causal
// window of the open (not yet summarised) segment that ends with them
// (gist.science Technical Summary §2.1 "Exact-Token Attention"; §3: the
// adapter runs with HGA for retrieval and generation).
//
// HBM-bound: each key row is read once for r * n_new query rows. The virtual
// key list of a (sequence, KV head) [sink | routed groups | open-segment
// window] is split into 256-key pieces, one workgroup each. A piece: scores
// of all its keys for all query rows to LDS, max and sum per row, then P.V;
// the unnormalised partial O with its (max, sum) goes to the workspace and
// decode_merge_kernel combines the pieces of each query row in a fixed order.
// bf16: Q.K^T on MFMA (32 keys x the query rows as columns, K rows loaded
// straight from memory as A operands) and P.V on the VALU with each lane
// owning D/64 output dimensions (one coalesced row read per key, no
// cross-lane sums). fp32: VALU throughout, D/8 lanes per key row.
// Deterministic; no atomics.
#include "attn_tile.hpp"

namespace hga {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecKeys = 256;  // keys per piece (one workgroup); bf16 small batches: 128
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
  // rows per (sequence, KV head) of k_hist / v_hist as read by the attention:
  // P, or with staged copies (history in host memory) sink_rows + k_g*8, the
  // sink rows first and then the routed groups' rows slot by slot
  int64_t hrows;
  int staged;
  int sink_rows;
  int k_g, n_sink, window, n_piece;
  int piece_keys;      // keys per piece (kDecKeys, or 128 for small bf16 batches)
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

// Row, within its (sequence, KV head), of routed key u (slot u/8, valid group
// g): the group's own row in the history, or its slot's row in the copies.
__device__ __forceinline__ int64_t routed_row(const DecodeParams& p, int g, int u) {
  return p.staged ? static_cast<int64_t>(p.sink_rows) + u : static_cast<int64_t>(g) * kGroup + u % kGroup;
}

// Sum over the LPK lanes of a key row (in-row DPP adds).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPK == 8 || LPK == 16, "a key row spans 8 or 16 lanes");
  return LPK == 16 ? sum16_f32(x) : sum8_f32(x);
}

constexpr int kDecUnroll = 4;  // key steps whose loads are issued together

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
  const int64_t hrow0 = (static_cast<int64_t>(b) * p.n_kv + j) * p.hrows;
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
      return g >= 0 ? hist + (hrow0 + routed_row(p, g, v)) * D : nullptr;
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
  // (kDecUnroll key steps per pass: their loads are all in flight before
  // the first is used)
  const T* kh = static_cast<const T*>(p.k_hist);
  const T* kt = static_cast<const T*>(p.k_tail);
  for (int base = wave * KPW; base < nk; base += kDecUnroll * KPS) {
    const T* rowp[kDecUnroll];
    int tpos[kDecUnroll];
    float kf[kDecUnroll][8];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int kk = base + u * KPS + kin;
      tpos[u] = -1;
      rowp[u] = kk < nk ? key_row(k0 + kk, kh, kt, tpos[u]) : nullptr;
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      if (rowp[u]) {
        Elem<T>::load8(rowp[u] + sub * 8, kf[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kf[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int kk = base + u * KPS + kin;
#pragma unroll
      for (int rq = 0; rq < NQ; ++rq) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qr[rq][e], kf[u][e], d);
        d = group_sum<LPK>(d);
        if (kk < nk && sub == 0 && rq < R) {
          bool ok = rowp[u] != nullptr;
          if (tpos[u] >= 0) {
            const int qpos = sk.tb - p.n_new + rq % p.n_new;   // open-segment position of the row
            ok = tpos[u] <= qpos && tpos[u] > qpos - p.window;
          }
          s_lds[rq][kk] = ok ? d * p.scale_log2 : -INFINITY;
        }
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
  for (int base = wave * KPW; base < nk; base += kDecUnroll * KPS) {
    const T* rowp[kDecUnroll];
    float vf[kDecUnroll][8];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int kk = base + u * KPS + kin;
      int tpos;
      rowp[u] = kk < nk ? key_row(k0 + kk, vh, vt, tpos) : nullptr;
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      if (rowp[u]) {
        Elem<T>::load8(rowp[u] + sub * 8, vf[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int kk = base + u * KPS + kin;
      if (!rowp[u]) continue;
#pragma unroll
      for (int rq = 0; rq < NQ; ++rq) {
        const float pr = rq < R ? s_lds[rq][kk] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[rq][e] = fmaf(pr, vf[u][e], acc[rq][e]);
      }
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

// QR: query rows provisioned in LDS and registers (R = r * n_new <= QR); a
// smaller QR for the common R <= 4 or 8 frees LDS and registers for more
// resident workgroups, which hide the row loads. KEYS: keys per piece (128
// for small batches, so that more workgroups share the rows to load).
template <int D, int QR, int KEYS>
__global__ __launch_bounds__(kDecThreads) void decode_attn_bf16_kernel(DecodeParams p) {
  static_assert(QR <= 32, "query rows are the 32 columns of the score MFMA");
  static_assert(KEYS % (kDecThreads / kWave * 32) == 0, "whole 32-key tiles per wave");
  constexpr int NKS = D / 16;                   // MFMA k-steps over head_dim
  constexpr int NW = kDecThreads / kWave;
  constexpr int KT = 32;                        // keys per MFMA tile
  constexpr int TPW = KEYS / (NW * KT);     // tiles per wave
  constexpr int DPL = D / kWave;                // output dims per lane in P.V
  // 16 query rows: P.V on MFMA from a V tile staged in LDS (128-key pieces
  // keep the workgroup's LDS near 50 KiB); fewer rows: P.V on the VALU
  constexpr bool kMfmaPV = QR > 8;
  static_assert(!kMfmaPV || KEYS == 128, "the MFMA P.V path stages 128-key pieces");
  constexpr int NO = kMfmaPV ? 1 : NW;          // partial-O slots the epilogue sums
  // rows padded by 4 floats: the 32 query rows' 16-byte score stores spread over the banks
  __shared__ __attribute__((aligned(16))) float s_lds[QR][KEYS + 4];
  __shared__ int32_t kinfo[KEYS];           // -1 plain, -2 masked, >= 0 open-segment position
  // element offset of each key's row, one's complement for an open-segment
  // row: resolved once in the score phase, so that the V loads do not wait
  // for another read of the routed group ids
  __shared__ int64_t koff[KEYS];
  __shared__ float o_lds[NO][QR][D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kMfmaPV ? KEYS * D : 8];
  const int piece = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int l32 = lane % 32, hh = lane / 32;

  const SeqKeys sk = seq_keys(p, b);
  const int k0 = piece * KEYS;
  if (k0 >= sk.n_keys) return;
  const int nk = min(KEYS, sk.n_keys - k0);
  const int R = p.r * p.n_new;
  const int n_routed = p.k_g * kGroup;
  const int64_t hrow0 = (static_cast<int64_t>(b) * p.n_kv + j) * p.hrows;
  const int64_t trow0 = (static_cast<int64_t>(b) * p.n_kv + j) * p.T;
  const int32_t* sel_bj = p.sel + (static_cast<int64_t>(b) * p.n_kv + j) * p.k_g;
  const uint16_t* kh = static_cast<const uint16_t*>(p.k_hist);
  const uint16_t* vh = static_cast<const uint16_t*>(p.v_hist);
  const uint16_t* kt = static_cast<const uint16_t*>(p.k_tail);
  const uint16_t* vt = static_cast<const uint16_t*>(p.v_tail);

  // element offset of virtual key v's row and whether it is an open-segment
  // row; an empty routed slot (or v past the piece) reads the first attended
  // open-segment row, a finite row whose weight is zero
  auto resolve = [&](int v, bool& tail, int& info) -> int64_t {
    if (v < k0 + nk) {
      if (v < sk.sink) { tail = false; info = -1; return (hrow0 + v) * D; }
      const int u = v - sk.sink;
      if (u < n_routed) {
        const int g = sel_bj[u / kGroup];
        if (g >= 0) { tail = false; info = -1; return (hrow0 + routed_row(p, g, u)) * D; }
      } else {
        tail = true;
        info = sk.t_lo + u - n_routed;
        return (trow0 + info) * D;
      }
    }
    tail = true;
    info = -2;
    return (trow0 + sk.t_lo) * D;
  };

  // ---- scores: S^T = K . Q^T per 32-key tile ------------------------------
  bf16x8 qreg[NKS];
  {
    const bool live = l32 < R;
    // rows of KV head j: (j*r + rq / n_new) * n_new + rq % n_new = j*r*n_new + rq
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) +
                         ((static_cast<int64_t>(b) * p.n_q + j * p.r) * p.n_new + (live ? l32 : 0)) * D + hh * 8;
#pragma unroll
    for (int ss = 0; ss < NKS; ++ss) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + ss * 16);
      qreg[ss] = live ? v : bf16x8{};
    }
  }
  bf16x8 ka[TPW][NKS];
  int info[TPW];
  int64_t kcode[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int kk = (wave * TPW + tt) * KT + l32;
    bool tail;
    const int64_t off = resolve(k0 + kk, tail, info[tt]);
    kcode[tt] = tail ? ~off : off;
    const uint16_t* kp = (tail ? kt : kh) + off + hh * 8;
#pragma unroll
    for (int ss = 0; ss < NKS; ++ss) ka[tt][ss] = *reinterpret_cast<const bf16x8*>(kp + ss * 16);
  }
  // 16 query rows: this lane's half of its key's V row (16-byte chunks
  // 2i + hh), requested now so that the score MFMAs and the softmax hide its
  // latency; it goes to the LDS tile after them. A key past the piece reads
  // the finite filler row; its probability is zero.
  constexpr int NVE = kMfmaPV ? D / 16 : 1;
  bf16x8 vpre[NVE];
  if constexpr (kMfmaPV) {
    static_assert(TPW == 1, "one 32-key tile per wave");
    const uint16_t* vp = kcode[0] < 0 ? vt + ~kcode[0] : vh + kcode[0];
#pragma unroll
    for (int i = 0; i < NVE; ++i) vpre[i] = *reinterpret_cast<const bf16x8*>(vp + (2 * i + hh) * 8);
  }
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tile0 = (wave * TPW + tt) * KT;
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
    for (int ss = 0; ss < NKS; ++ss) acc = mfma32(ka[tt][ss], qreg[ss], acc);
    if (hh == 0) {
      kinfo[tile0 + l32] = info[tt];
      koff[tile0 + l32] = kcode[tt];
    }
    if (l32 < R) {
      // acc[v]: key tile0 + 8*(v/4) + 4*hh + v%4, query row l32
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        *reinterpret_cast<float4*>(&s_lds[l32][tile0 + 8 * v4 + 4 * hh]) =
            make_float4(acc[4 * v4] * p.scale_log2, acc[4 * v4 + 1] * p.scale_log2,
                        acc[4 * v4 + 2] * p.scale_log2, acc[4 * v4 + 3] * p.scale_log2);
    }
  }
  __syncthreads();

  // ---- per row: mask, max, probabilities in place, sum --------------------
  for (int rq = wave; rq < R; rq += NW) {
    const int qpos = sk.tb - p.n_new + rq % p.n_new;
    float m = -INFINITY;
    for (int kk = lane; kk < KEYS; kk += kWave) {
      const int inf = kinfo[kk];
      const bool ok = inf == -1 || (inf >= 0 && inf <= qpos && inf > qpos - p.window);
      const float sc = ok ? s_lds[rq][kk] : -INFINITY;
      s_lds[rq][kk] = sc;
      m = fmaxf(m, sc);
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    float l = 0.f;
    for (int kk = lane; kk < KEYS; kk += kWave) {
      const float e = m == -INFINITY ? 0.f : exp2f(s_lds[rq][kk] - m);
      s_lds[rq][kk] = e;
      l += e;
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) l += __shfl_xor(l, o, kWave);
    if (lane == 0) {
      float* ml = p.part_ml + ((static_cast<int64_t>(b) * p.n_q + j * p.r) * p.n_new + rq) * p.n_piece * 2 + piece * 2;
      ml[0] = m;
      ml[1] = l;
    }
  }
  __syncthreads();

  if constexpr (QR <= 8) {
    // ---- P . V: one V row per LPR lanes (16 bytes each), RPL rows per wave
    // load, all of a wave's rows requested before any is used; then the RPL
    // lane groups holding the same dims are summed across lanes. Keys past
    // the piece load nothing (their P is zero).
    constexpr int LPR = D / 8;            // lanes per V row
    constexpr int RPL = kWave / LPR;      // rows per wave load
    constexpr int KPW = KEYS / NW;        // keys per wave
    constexpr int NLD = KPW / RPL;        // row loads per lane
    const int sub = lane % LPR, rsub = lane / LPR;
    const int kq0 = wave * KPW;
    uint4 vr[NLD];
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int kk = kq0 + m * RPL + rsub;
      const int64_t c = koff[kk];
      const uint16_t* vp = c < 0 ? vt + ~c : vh + c;
      vr[m] = kk < nk ? *reinterpret_cast<const uint4*>(vp + sub * 8) : make_uint4(0, 0, 0, 0);
    }
    float acc[QR][8];
#pragma unroll
    for (int rq = 0; rq < QR; ++rq)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[rq][e] = 0.f;
#pragma unroll
    for (int m = 0; m < NLD; ++m) {
      const int kk = kq0 + m * RPL + rsub;
      const uint32_t w4[4] = {vr[m].x, vr[m].y, vr[m].z, vr[m].w};
      float vf[8];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        vf[2 * x] = __uint_as_float(w4[x] << 16);
        vf[2 * x + 1] = __uint_as_float(w4[x] & 0xffff0000u);
      }
#pragma unroll
      for (int rq = 0; rq < QR; ++rq) {
        if (rq < R) {
          const float pr = s_lds[rq][kk];  // zero past nk
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[rq][e] += pr * vf[e];
        }
      }
    }
#pragma unroll
    for (int rq = 0; rq < QR; ++rq)
      if (rq < R)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float x = acc[rq][e];
#pragma unroll
          for (int o = LPR; o < kWave; o <<= 1) x += __shfl_xor(x, o, kWave);
          acc[rq][e] = x;
        }
    if (rsub == 0) {
#pragma unroll
      for (int rq = 0; rq < QR; ++rq)
        if (rq < R)
#pragma unroll
          for (int e = 0; e < 8; ++e) o_lds[wave][rq][sub * 8 + e] = acc[rq][e];
    }
  } else {
    // ---- P . V on MFMA: O^T = V^T . P^T in 32 x 32 x 16 tiles. The piece's V
    // rows (requested in the score phase) go to a swizzled LDS tile; wave w
    // owns output dims [32w, 32w + 32) over all keys. V^T comes from transposed
    // LDS reads, whose contraction slots are keys k0 + 8*(i/4) + 4*hh + i%4;
    // the P^T operand takes the same keys from this lane's score row (query
    // row l32; rows R..31 are zero). P is rounded to bf16 for the MFMA, as in
    // the training forward.
    {
      const uint32_t kk = static_cast<uint32_t>(wave * KT + l32);   // this lane's key
#pragma unroll
      for (int i = 0; i < NVE; ++i)
        *reinterpret_cast<bf16x8*>(&v_lds[Swz<D>::off(kk, static_cast<uint32_t>((2 * i + hh) * 8))]) = vpre[i];
    }
    __syncthreads();
    if (wave < D / 32) {
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
      const bool live = l32 < R;
#pragma unroll
      for (int k0 = 0; k0 < KEYS; k0 += 16) {
        const bf16x8 a = lds_a_tr_swz<D>(v_lds, k0, wave * 32, lane);
        uint4 bu = make_uint4(0, 0, 0, 0);
        if (live) {
          const float4 p0 = *reinterpret_cast<const float4*>(&s_lds[l32][k0 + 4 * hh]);
          const float4 p1 = *reinterpret_cast<const float4*>(&s_lds[l32][k0 + 8 + 4 * hh]);
          bu = make_uint4(cvt_pk_bf16(p0.x, p0.y), cvt_pk_bf16(p0.z, p0.w), cvt_pk_bf16(p1.x, p1.y),
                          cvt_pk_bf16(p1.z, p1.w));
        }
        acc = mfma32(a, __builtin_bit_cast(bf16x8, bu), acc);
      }
      // acc[v]: O^T[dim 32*wave + 8*(v/4) + 4*hh + v%4][query row l32]
      if (live) {
#pragma unroll
        for (int v = 0; v < 16; ++v) o_lds[0][l32][wave * 32 + 8 * (v / 4) + 4 * hh + v % 4] = acc[v];
      }
    }
  }
  __syncthreads();
  for (int x = t; x < R * D; x += kDecThreads) {
    const int rq = x / D, dd = x % D;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NO; ++w) v += o_lds[w][rq][dd];
    const int64_t row = (static_cast<int64_t>(b) * p.n_q + j * p.r) * p.n_new + rq;
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
  const int n = (sk.n_keys + p.piece_keys - 1) / p.piece_keys;
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

// History in host memory: one workgroup per 64 staged rows of a (sequence,
// KV head) copies its sink rows and the rows of its routed groups, 16 bytes
// per lane, every load of a thread in flight before its stores. Rows of empty
// slots are not written; the attention never reads them.
constexpr int kStageRows = 64;

template <int CPR>  // 16-byte chunks per row
__global__ __launch_bounds__(256) void decode_stage_kernel(const uint4* __restrict__ k_hist,
                                                           const uint4* __restrict__ v_hist,
                                                           const int32_t* __restrict__ sel, int64_t P, int k_g,
                                                           int sink_rows, int64_t stage_rows,
                                                           uint4* __restrict__ k_st, uint4* __restrict__ v_st) {
  constexpr int PER = kStageRows * CPR / 256;  // chunks per thread
  static_assert(PER * 256 == kStageRows * CPR, "whole rows per workgroup");
  const int64_t bj = blockIdx.y;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kStageRows;
  // a native vector type: arrays of the HIP vector struct, loaded under a
  // branch, went to scratch, each store then waiting for its load
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 kv[PER], vv[PER];
  int64_t dst[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int x = static_cast<int>(threadIdx.x) + i * 256;
    const int64_t row = r0 + x / CPR;
    const int ch = x % CPR;
    int64_t src = -1;
    if (row < sink_rows) {
      src = row;
    } else if (row < stage_rows) {
      const int64_t u = row - sink_rows;
      const int g = sel[bj * k_g + u / kGroup];
      if (g >= 0) src = static_cast<int64_t>(g) * kGroup + u % kGroup;
    }
    dst[i] = -1;
    if (src >= 0) {
      const int64_t o = (bj * P + src) * CPR + ch;
      kv[i] = reinterpret_cast<const u32x4*>(k_hist)[o];
      vv[i] = reinterpret_cast<const u32x4*>(v_hist)[o];
      dst[i] = (bj * stage_rows + row) * CPR + ch;
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (dst[i] >= 0) {
      reinterpret_cast<u32x4*>(k_st)[dst[i]] = kv[i];
      reinterpret_cast<u32x4*>(v_st)[dst[i]] = vv[i];
    }
  }
}

template <typename T, int D>
hipError_t launch_td(const hga_shape& s, DecodeParams& p, int batch, hipStream_t st) {
  const dim3 grid(p.n_piece, s.n_kv_heads, batch);
  const int R = p.r * p.n_new;
  hipEvent_t e0 = timer_event(HGA_KERNEL_DECODE, 0), e1 = timer_event(HGA_KERNEL_DECODE, 1);
  if constexpr (sizeof(T) == 2) {
    if (R > 8) {  // decode_piece_keys gives 128-key pieces here
      hipExtLaunchKernelGGL((decode_attn_bf16_kernel<D, 16, 128>), grid, dim3(kDecThreads), 0, st, e0, nullptr, 0, p);
    } else if (p.piece_keys == 128) {
      if (R <= 4)
        hipExtLaunchKernelGGL((decode_attn_bf16_kernel<D, 4, 128>), grid, dim3(kDecThreads), 0, st, e0, nullptr, 0, p);
      else
        hipExtLaunchKernelGGL((decode_attn_bf16_kernel<D, 8, 128>), grid, dim3(kDecThreads), 0, st, e0, nullptr, 0, p);
    } else {
      if (R <= 4)
        hipExtLaunchKernelGGL((decode_attn_bf16_kernel<D, 4, kDecKeys>), grid, dim3(kDecThreads), 0, st, e0, nullptr, 0, p);
      else
        hipExtLaunchKernelGGL((decode_attn_bf16_kernel<D, 8, kDecKeys>), grid, dim3(kDecThreads), 0, st, e0, nullptr, 0, p);
    }
  } else if (R <= 4)
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

namespace {
// Keys attended per (sequence, KV head) at most: sink, routed groups, open segment.
int64_t decode_max_keys(const hga_shape& s) {
  const int64_t P = hist_rows(s);
  const int64_t sink = static_cast<int64_t>(s.n_sink_chunks) * kChunk < P ? s.n_sink_chunks * kChunk : P;
  return sink + static_cast<int64_t>(s.top_k_groups) * kGroup + s.seg_len;
}
}  // namespace

// Keys per piece: kDecKeys, or 128 for bf16 when 256-key pieces would give
// the attention launch fewer than 512 workgroups or the query rows per KV head
// (r * n_new) exceed 8 (the MFMA P.V path stages 128-key V tiles).
int decode_piece_keys(const hga_shape& s, int batch, int n_new) {
  if (s.dtype != HGA_BF16) return kDecKeys;
  if ((s.n_q_heads / s.n_kv_heads) * n_new > 8) return 128;
  const int64_t wgs = static_cast<int64_t>(batch) * s.n_kv_heads * ((decode_max_keys(s) + kDecKeys - 1) / kDecKeys);
  return wgs < 512 ? 128 : kDecKeys;
}

int decode_pieces(const hga_shape& s, int batch, int n_new) {
  const int pk = decode_piece_keys(s, batch, n_new);
  return static_cast<int>((decode_max_keys(s) + pk - 1) / pk);
}

int64_t decode_stage_sink_rows(const hga_shape& s) {
  const int64_t P = hist_rows(s);
  const int64_t sink = static_cast<int64_t>(s.n_sink_chunks) * kChunk;
  return sink < P ? sink : P;
}

int64_t decode_stage_rows(const hga_shape& s) {
  return decode_stage_sink_rows(s) + static_cast<int64_t>(s.top_k_groups) * kGroup;
}

hipError_t launch_decode_stage(const hga_shape& s, int batch, const void* k_hist, const void* v_hist,
                               const int32_t* sel_groups, void* k_stage, void* v_stage, hipStream_t stream) {
  const int64_t rows = decode_stage_rows(s);
  const int cpr = s.head_dim * (s.dtype == HGA_BF16 ? 2 : 4) / 16;
  const dim3 grid(static_cast<unsigned>((rows + kStageRows - 1) / kStageRows),
                  static_cast<unsigned>(batch * s.n_kv_heads));
  const uint4* kh = static_cast<const uint4*>(k_hist);
  const uint4* vh = static_cast<const uint4*>(v_hist);
  uint4* ko = static_cast<uint4*>(k_stage);
  uint4* vo = static_cast<uint4*>(v_stage);
  const int64_t P = hist_rows(s);
  const int sink = static_cast<int>(decode_stage_sink_rows(s));
  hipEvent_t e0 = timer_event(HGA_KERNEL_GATHER, 0), e1 = timer_event(HGA_KERNEL_GATHER, 1);
  if (cpr == 8)
    hipExtLaunchKernelGGL((decode_stage_kernel<8>), grid, dim3(256), 0, stream, e0, e1, 0, kh, vh, sel_groups, P,
                          s.top_k_groups, sink, rows, ko, vo);
  else if (cpr == 16)
    hipExtLaunchKernelGGL((decode_stage_kernel<16>), grid, dim3(256), 0, stream, e0, e1, 0, kh, vh, sel_groups, P,
                          s.top_k_groups, sink, rows, ko, vo);
  else
    hipExtLaunchKernelGGL((decode_stage_kernel<32>), grid, dim3(256), 0, stream, e0, e1, 0, kh, vh, sel_groups, P,
                          s.top_k_groups, sink, rows, ko, vo);
  return hipGetLastError();
}

size_t decode_attn_workspace_bytes(const hga_shape& s, int batch, int n_new) {
  const size_t rows = static_cast<size_t>(batch) * s.n_q_heads * n_new;
  const size_t n = decode_pieces(s, batch, n_new);
  return ((rows * n * s.head_dim * sizeof(float) + 255) & ~size_t(255)) + rows * n * 2 * sizeof(float);
}

hipError_t launch_decode_attn(const hga_shape& s, int batch, int n_new, const void* q, const void* k_hist,
                              const void* v_hist, const void* k_tail, const void* v_tail,
                              const int32_t* sel_groups, const int32_t* hist_lens, const int32_t* tail_lens,
                              void* o, float* lse, void* ws, hipStream_t stream, bool staged) {
  DecodeParams p;
  p.q = q; p.k_hist = k_hist; p.v_hist = v_hist; p.k_tail = k_tail; p.v_tail = v_tail;
  p.sel = sel_groups; p.hist_lens = hist_lens; p.tail_lens = tail_lens; p.o = o; p.lse = lse;
  p.n_q = s.n_q_heads; p.n_kv = s.n_kv_heads; p.r = s.n_q_heads / s.n_kv_heads; p.n_new = n_new;
  p.P = hist_rows(s); p.T = s.seg_len; p.k_g = s.top_k_groups; p.n_sink = s.n_sink_chunks;
  p.staged = staged ? 1 : 0;
  p.hrows = staged ? decode_stage_rows(s) : p.P;
  p.sink_rows = static_cast<int>(decode_stage_sink_rows(s));
  p.window = local_window(s); p.n_piece = decode_pieces(s, batch, n_new); p.piece_keys = decode_piece_keys(s, batch, n_new);
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
