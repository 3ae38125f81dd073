// Backward of exact-token attention with detached history.
//
//   Dvec[h][i] = dO[h][i] . O[h][i]                      (row_dot_kernel)
//   dQ[h][i]   = scale * sum_t P_t (dO.v_t - Dvec) k_t   over history + segment
//   dK_seg[j][t], dV_seg[j][t]                           over segment keys only
// with P_t = exp(scale q.k_t - LSE). The history K/V of the selected groups is
// read (it shapes P) but gets no gradient. dQ and dK/dV are separate kernels so
// every output element is written by exactly one workgroup: no atomics, bitwise
// repeatable results.
//
// bf16 path: MFMA 32x32x16. dQ uses the S^T = K.Q^T orientation (one query per
// lane column, as in the forward); dK/dV use S = Q.K^T (one key per lane
// column) so that P and dS feed the dV^T / dK^T products straight from the
// accumulators. Transposed copies of the streamed operand (K^T for dQ; Q^T and
// dO^T for dK/dV) are written to LDS while staging.
// fp32 path: plain VALU kernels.
#include "hga_common.hpp"

namespace hga {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTile = 64;

struct BwdParams {
  const void* q;
  const void* k_hist;
  const void* v_hist;
  const void* k_seg;
  const void* v_seg;
  const int32_t* sel;
  const void* o;
  const float* lse;
  const void* d_o;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;
  int n_q, n_kv, r;
  int seg_len;
  int64_t hist_len;
  int k_g;
  float scale;
  float scale_log2;
};

__device__ __forceinline__ int64_t hist_offset(const BwdParams& p, const int32_t* sel_s, int j,
                                               int ht, int kk, int D) {
  const int slot = ht * 8 + kk / kGroup;
  if (slot >= p.k_g) return -1;
  const int n = sel_s[slot];
  if (n < 0) return -1;
  return (static_cast<int64_t>(j) * p.hist_len + static_cast<int64_t>(n) * kGroup + kk % kGroup) * D;
}

// Dvec = rowsum(dO * O), fp32 accumulation; 16 threads per row (bf16 d=128).
template <typename T, int D>
__global__ __launch_bounds__(256) void row_dot_kernel(const T* __restrict__ o,
                                                      const T* __restrict__ d_o,
                                                      float* __restrict__ dvec, int64_t n_rows) {
  constexpr int TPR = D / 8;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (256 / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float s = 0.f;
  if (row < n_rows) {
    float a[8], g[8];
    Elem<T>::load8(o + row * D + c * 8, a);
    Elem<T>::load8(d_o + row * D + c * 8, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += a[e] * g[e];
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, kWave);
  if (row < n_rows && c == 0) dvec[row] = s;
}

// ---------------------------------------------------------------------------
// bf16: dQ
// ---------------------------------------------------------------------------
template <int D, int HPW>
__global__ __launch_bounds__(128 * HPW) void attn_bwd_dq_bf16_kernel(BwdParams p) {
  constexpr int NT = 128 * HPW;
  constexpr int KS = D + 8;
  constexpr int TS = kTile + 4;
  constexpr int NDT = D / 32;
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kTile * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * TS];
  __shared__ int32_t sel_s[kMaxTopKGroups];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int l32 = lane % 32, hh = lane / 32;
  const int n_hg = p.r / HPW;
  const int n_blocks = p.seg_len / kBlockQ;
  int w = blockIdx.x;
  const int j = w % p.n_kv;
  w /= p.n_kv;
  const int hg = w % n_hg;
  const int b = n_blocks - 1 - w / n_hg;
  const int head = j * p.r + hg * HPW + wave / 2;
  const int qrow0 = (wave % 2) * 32;
  const int q_tok = b * kBlockQ + qrow0 + l32;

  const uint16_t* kh = static_cast<const uint16_t*>(p.k_hist);
  const uint16_t* vh = static_cast<const uint16_t*>(p.v_hist);
  const uint16_t* ks_g = static_cast<const uint16_t*>(p.k_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const uint16_t* vs_g = static_cast<const uint16_t*>(p.v_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const int32_t* sel_bj = p.sel + (static_cast<int64_t>(b) * p.n_kv + j) * p.k_g;
  for (int i = tid; i < p.k_g; i += NT) sel_s[i] = sel_bj[i];

  const int64_t row_off = static_cast<int64_t>(head) * p.seg_len + q_tok;
  bf16x8 qreg[NKS], goreg[NKS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + row_off * D + hh * 8;
    const uint16_t* gp = static_cast<const uint16_t*>(p.d_o) + row_off * D + hh * 8;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qreg[s] = *reinterpret_cast<const bf16x8*>(qp + s * 16);
      goreg[s] = *reinterpret_cast<const bf16x8*>(gp + s * 16);
    }
  }
  const float lse2 = p.lse[row_off] * kLog2e;
  const float dq_row = p.dvec[row_off];

  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;

  const int n_hist_tiles = (p.k_g + 7) / 8;
  const int n_tiles = n_hist_tiles + b + 1;
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const bool is_hist = tile < n_hist_tiles;
    const int st = tile - n_hist_tiles;
    uint32_t gmask = 0xffu;
    if (is_hist) {
      gmask = 0;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int slot = tile * 8 + g;
        gmask |= (slot < p.k_g && sel_s[slot] >= 0) ? (1u << g) : 0u;
      }
      if (gmask == 0) continue;
    }
    {
      constexpr int CPR = D / 8;
      for (int idx = tid; idx < kTile * CPR; idx += NT) {
        const int kk = idx / CPR, c = idx % CPR;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (is_hist) {
          const int64_t off = hist_offset(p, sel_s, j, tile, kk, D);
          if (off >= 0) {
            kv = *reinterpret_cast<const uint4*>(kh + off + c * 8);
            vv = *reinterpret_cast<const uint4*>(vh + off + c * 8);
          }
        } else {
          const int64_t off = static_cast<int64_t>(st * kTile + kk) * D + c * 8;
          kv = *reinterpret_cast<const uint4*>(ks_g + off);
          vv = *reinterpret_cast<const uint4*>(vs_g + off);
        }
        *reinterpret_cast<uint4*>(&Ks[kk * KS + c * 8]) = kv;
        *reinterpret_cast<uint4*>(&Vs[kk * KS + c * 8]) = vv;
        const uint16_t* k16 = reinterpret_cast<const uint16_t*>(&kv);
#pragma unroll
        for (int e = 0; e < 8; ++e) Kt[(c * 8 + e) * TS + kk] = k16[e];
      }
    }
    __syncthreads();

    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[kt][v] = 0.f; pacc[kt][v] = 0.f; }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[(kt * 32 + l32) * KS + s * 16 + hh * 8]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s], sacc[kt], 0, 0, 0);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vs[(kt * 32 + l32) * KS + s * 16 + hh * 8]);
        pacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, goreg[s], pacc[kt], 0, 0, 0);
      }
    }
    const bool diag = !is_hist && st == b;
    bf16x8 dsb[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = kt * 32 + 8 * (v / 4) + 4 * hh + (v % 4);
        const bool masked = is_hist ? !((gmask >> (kk / 8)) & 1u) : (diag && kk > qrow0 + l32);
        const float pr = masked ? 0.f : exp2f(sacc[kt][v] * p.scale_log2 - lse2);
        const float ds = pr * (pacc[kt][v] - dq_row);
        dsb[kt][v / 8][v % 8] = static_cast<__bf16>(ds);
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint16_t* krow = &Kt[(dt * 32 + l32) * TS];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int ksi = 0; ksi < 2; ++ksi) {
          const int k0 = kt * 32 + ksi * 16 + 4 * hh;
          const uint2 lo = *reinterpret_cast<const uint2*>(krow + k0);
          const uint2 hi = *reinterpret_cast<const uint2*>(krow + k0 + 8);
          const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[kt][ksi], acc[dt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  uint16_t* dq = static_cast<uint16_t*>(p.dq) + row_off * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + 8 * g + 4 * hh;
      uint2 w2;
      w2.x = pack_bf16x2(acc[dt][4 * g + 0] * p.scale, acc[dt][4 * g + 1] * p.scale);
      w2.y = pack_bf16x2(acc[dt][4 * g + 2] * p.scale, acc[dt][4 * g + 3] * p.scale);
      *reinterpret_cast<uint2*>(dq + d0) = w2;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16: dK, dV for one 64-key segment tile of one KV head, over every query
// block at or after it and every query head of the group.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void attn_bwd_dkdv_bf16_kernel(BwdParams p) {
  constexpr int KS = D + 8;
  constexpr int TS = kTile + 4;
  constexpr int NDT = D / 32;
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[kTile * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[kTile * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t Gt[D * TS];
  __shared__ float lse_s[kTile];
  __shared__ float dvec_s[kTile];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int l32 = lane % 32, hh = lane / 32;
  const int n_blocks = p.seg_len / kBlockQ;
  const int j = blockIdx.x % p.n_kv;
  const int kt_blk = blockIdx.x / p.n_kv;  // key tile, heaviest (earliest) first
  const int key_local = wave * 32 + l32;   // key within the tile (lane column)
  const int key_tok = kt_blk * kTile + key_local;

  const uint16_t* kseg = static_cast<const uint16_t*>(p.k_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const uint16_t* vseg = static_cast<const uint16_t*>(p.v_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  bf16x8 kreg[NKS], vreg[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    kreg[s] = *reinterpret_cast<const bf16x8*>(kseg + static_cast<int64_t>(key_tok) * D + s * 16 + hh * 8);
    vreg[s] = *reinterpret_cast<const bf16x8*>(vseg + static_cast<int64_t>(key_tok) * D + s * 16 + hh * 8);
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) { dk[dt][v] = 0.f; dv[dt][v] = 0.f; }

  const uint16_t* qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* gg = static_cast<const uint16_t*>(p.d_o);
  for (int qb = kt_blk; qb < n_blocks; ++qb) {
    for (int hi = 0; hi < p.r; ++hi) {
      const int head = j * p.r + hi;
      const int64_t row0 = static_cast<int64_t>(head) * p.seg_len + qb * kBlockQ;
      __syncthreads();
      constexpr int CPR = D / 8;
      for (int idx = tid; idx < kTile * CPR; idx += 128) {
        const int qq = idx / CPR, c = idx % CPR;
        const uint4 qv = *reinterpret_cast<const uint4*>(qg + (row0 + qq) * D + c * 8);
        const uint4 gv = *reinterpret_cast<const uint4*>(gg + (row0 + qq) * D + c * 8);
        *reinterpret_cast<uint4*>(&Qs[qq * KS + c * 8]) = qv;
        *reinterpret_cast<uint4*>(&Gs[qq * KS + c * 8]) = gv;
        const uint16_t* q16 = reinterpret_cast<const uint16_t*>(&qv);
        const uint16_t* g16 = reinterpret_cast<const uint16_t*>(&gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          Qt[(c * 8 + e) * TS + qq] = q16[e];
          Gt[(c * 8 + e) * TS + qq] = g16[e];
        }
      }
      if (tid < kTile) {
        lse_s[tid] = p.lse[row0 + tid] * kLog2e;
        dvec_s[tid] = p.dvec[row0 + tid];
      }
      __syncthreads();

      const bool diag = qb == kt_blk;
      bf16x8 pb[2][2], dsb[2][2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; pacc[v] = 0.f; }
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[(qs * 32 + l32) * KS + s * 16 + hh * 8]);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kreg[s], sacc, 0, 0, 0);
          const bf16x8 ga = *reinterpret_cast<const bf16x8*>(&Gs[(qs * 32 + l32) * KS + s * 16 + hh * 8]);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vreg[s], pacc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int qi = qs * 32 + 8 * (v / 4) + 4 * hh + (v % 4);  // query row in block
          const bool masked = diag && key_local > qi;
          const float pr = masked ? 0.f : exp2f(sacc[v] * p.scale_log2 - lse_s[qi]);
          const float ds = pr * (pacc[v] - dvec_s[qi]);
          pb[qs][v / 8][v % 8] = static_cast<__bf16>(pr);
          dsb[qs][v / 8][v % 8] = static_cast<__bf16>(ds);
        }
      }
      // dV^T += dO^T . P ; dK^T += Q^T . dS   (contraction over the 64 queries)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint16_t* grow = &Gt[(dt * 32 + l32) * TS];
        const uint16_t* qrow = &Qt[(dt * 32 + l32) * TS];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
          for (int ksi = 0; ksi < 2; ++ksi) {
            const int k0 = qs * 32 + ksi * 16 + 4 * hh;
            const uint2 glo = *reinterpret_cast<const uint2*>(grow + k0);
            const uint2 ghi = *reinterpret_cast<const uint2*>(grow + k0 + 8);
            const bf16x8 ga = __builtin_bit_cast(bf16x8, make_uint4(glo.x, glo.y, ghi.x, ghi.y));
            dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, pb[qs][ksi], dv[dt], 0, 0, 0);
            const uint2 qlo = *reinterpret_cast<const uint2*>(qrow + k0);
            const uint2 qhi = *reinterpret_cast<const uint2*>(qrow + k0 + 8);
            const bf16x8 qa = __builtin_bit_cast(bf16x8, make_uint4(qlo.x, qlo.y, qhi.x, qhi.y));
            dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsb[qs][ksi], dk[dt], 0, 0, 0);
          }
        }
      }
    }
  }

  uint16_t* dkp = static_cast<uint16_t*>(p.dk) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D;
  uint16_t* dvp = static_cast<uint16_t*>(p.dv) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + 8 * g + 4 * hh;
      uint2 a, c;
      a.x = pack_bf16x2(dk[dt][4 * g + 0] * p.scale, dk[dt][4 * g + 1] * p.scale);
      a.y = pack_bf16x2(dk[dt][4 * g + 2] * p.scale, dk[dt][4 * g + 3] * p.scale);
      c.x = pack_bf16x2(dv[dt][4 * g + 0], dv[dt][4 * g + 1]);
      c.y = pack_bf16x2(dv[dt][4 * g + 2], dv[dt][4 * g + 3]);
      *reinterpret_cast<uint2*>(dkp + d0) = a;
      *reinterpret_cast<uint2*>(dvp + d0) = c;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU kernels
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kWave) void attn_bwd_dq_f32_kernel(BwdParams p) {
  __shared__ float Kt[kTile][D + 1];
  __shared__ float Vt[kTile][D + 1];
  __shared__ int32_t sel_s[kMaxTopKGroups];
  const int a = threadIdx.x;
  const int n_blocks = p.seg_len / kBlockQ;
  const int head = blockIdx.x % p.n_q;
  const int b = n_blocks - 1 - blockIdx.x / p.n_q;
  const int j = head / p.r;
  const int64_t row = static_cast<int64_t>(head) * p.seg_len + b * kBlockQ + a;
  const float* kh = static_cast<const float*>(p.k_hist);
  const float* vh = static_cast<const float*>(p.v_hist);
  const float* ks_g = static_cast<const float*>(p.k_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const float* vs_g = static_cast<const float*>(p.v_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const int32_t* sel_bj = p.sel + (static_cast<int64_t>(b) * p.n_kv + j) * p.k_g;
  for (int i = a; i < p.k_g; i += kWave) sel_s[i] = sel_bj[i];
  float qr[D], gr[D], acc[D];
  for (int e = 0; e < D; ++e) {
    qr[e] = static_cast<const float*>(p.q)[row * D + e];
    gr[e] = static_cast<const float*>(p.d_o)[row * D + e];
    acc[e] = 0.f;
  }
  const float lse2 = p.lse[row] * kLog2e;
  const float dr = p.dvec[row];
  const int n_hist_tiles = (p.k_g + 7) / 8;
  __syncthreads();
  for (int tile = 0; tile < n_hist_tiles + b + 1; ++tile) {
    const bool is_hist = tile < n_hist_tiles;
    const int st = tile - n_hist_tiles;
    for (int kk = 0; kk < kTile; ++kk) {
      int64_t off;
      if (is_hist) off = hist_offset(p, sel_s, j, tile, kk, D);
      else off = static_cast<int64_t>(st * kTile + kk) * D;
      const float* kb = is_hist ? kh : ks_g;
      const float* vb = is_hist ? vh : vs_g;
      for (int e = a; e < D; e += kWave) {
        Kt[kk][e] = off >= 0 ? kb[off + e] : 0.f;
        Vt[kk][e] = off >= 0 ? vb[off + e] : 0.f;
      }
    }
    __syncthreads();
    for (int kk = 0; kk < kTile; ++kk) {
      bool valid;
      if (is_hist) {
        const int slot = tile * 8 + kk / kGroup;
        valid = slot < p.k_g && sel_s[slot] >= 0;
      } else {
        valid = !(st == b && kk > a);
      }
      if (!valid) continue;
      float s = 0.f, dp = 0.f;
      for (int e = 0; e < D; ++e) {
        s += qr[e] * Kt[kk][e];
        dp += gr[e] * Vt[kk][e];
      }
      const float pr = exp2f(s * p.scale_log2 - lse2);
      const float ds = pr * (dp - dr);
      for (int e = 0; e < D; ++e) acc[e] += ds * Kt[kk][e];
    }
    __syncthreads();
  }
  float* dq = static_cast<float*>(p.dq) + row * D;
  for (int e = 0; e < D; ++e) dq[e] = acc[e] * p.scale;
}

template <int D>
__global__ __launch_bounds__(kWave) void attn_bwd_dkdv_f32_kernel(BwdParams p) {
  __shared__ float Qt[kTile][D + 1];
  __shared__ float Gt[kTile][D + 1];
  __shared__ float lse_s[kTile];
  __shared__ float dvec_s[kTile];
  const int a = threadIdx.x;  // key within the tile
  const int n_blocks = p.seg_len / kBlockQ;
  const int j = blockIdx.x % p.n_kv;
  const int kt_blk = blockIdx.x / p.n_kv;
  const int key_tok = kt_blk * kTile + a;
  const float* kseg = static_cast<const float*>(p.k_seg) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D;
  const float* vseg = static_cast<const float*>(p.v_seg) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D;
  float kr[D], vr[D], dk[D], dv[D];
  for (int e = 0; e < D; ++e) { kr[e] = kseg[e]; vr[e] = vseg[e]; dk[e] = 0.f; dv[e] = 0.f; }
  for (int qb = kt_blk; qb < n_blocks; ++qb) {
    for (int hi = 0; hi < p.r; ++hi) {
      const int64_t row0 = static_cast<int64_t>(j * p.r + hi) * p.seg_len + qb * kBlockQ;
      __syncthreads();
      for (int qq = 0; qq < kTile; ++qq)
        for (int e = a; e < D; e += kWave) {
          Qt[qq][e] = static_cast<const float*>(p.q)[(row0 + qq) * D + e];
          Gt[qq][e] = static_cast<const float*>(p.d_o)[(row0 + qq) * D + e];
        }
      lse_s[a] = p.lse[row0 + a] * kLog2e;
      dvec_s[a] = p.dvec[row0 + a];
      __syncthreads();
      for (int qq = 0; qq < kTile; ++qq) {
        if (qb == kt_blk && a > qq) continue;  // key after query: masked
        float s = 0.f, dp = 0.f;
        for (int e = 0; e < D; ++e) {
          s += Qt[qq][e] * kr[e];
          dp += Gt[qq][e] * vr[e];
        }
        const float pr = exp2f(s * p.scale_log2 - lse_s[qq]);
        const float ds = pr * (dp - dvec_s[qq]);
        for (int e = 0; e < D; ++e) {
          dv[e] += pr * Gt[qq][e];
          dk[e] += ds * Qt[qq][e];
        }
      }
    }
  }
  float* dkp = static_cast<float*>(p.dk) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D;
  float* dvp = static_cast<float*>(p.dv) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D;
  for (int e = 0; e < D; ++e) { dkp[e] = dk[e] * p.scale; dvp[e] = dv[e]; }
}

template <int D>
hipError_t launch_d(const hga_shape& s, BwdParams& p, hipStream_t st) {
  const int n_blocks = s.seg_len / kBlockQ;
  const int64_t n_rows = static_cast<int64_t>(s.n_q_heads) * s.seg_len;
  constexpr int RPB = 256 / (D / 8);
  const unsigned dot_grid = static_cast<unsigned>((n_rows + RPB - 1) / RPB);
  if (s.dtype == HGA_F32) {
    timer_begin(HGA_KERNEL_BWD_ROWDOT, st);
    hipLaunchKernelGGL((row_dot_kernel<float, D>), dim3(dot_grid), dim3(256), 0, st,
                       static_cast<const float*>(p.o), static_cast<const float*>(p.d_o), p.dvec, n_rows);
    timer_end(HGA_KERNEL_BWD_ROWDOT, st);
    timer_begin(HGA_KERNEL_BWD_DQ, st);
    hipLaunchKernelGGL((attn_bwd_dq_f32_kernel<D>), dim3(n_blocks * s.n_q_heads), dim3(kWave), 0, st, p);
    timer_end(HGA_KERNEL_BWD_DQ, st);
    timer_begin(HGA_KERNEL_BWD_DKDV, st);
    hipLaunchKernelGGL((attn_bwd_dkdv_f32_kernel<D>), dim3(n_blocks * s.n_kv_heads), dim3(kWave), 0, st, p);
    timer_end(HGA_KERNEL_BWD_DKDV, st);
  } else {
    timer_begin(HGA_KERNEL_BWD_ROWDOT, st);
    hipLaunchKernelGGL((row_dot_kernel<uint16_t, D>), dim3(dot_grid), dim3(256), 0, st,
                       static_cast<const uint16_t*>(p.o), static_cast<const uint16_t*>(p.d_o), p.dvec,
                       n_rows);
    timer_end(HGA_KERNEL_BWD_ROWDOT, st);
    timer_begin(HGA_KERNEL_BWD_DQ, st);
    if (p.r % 2 == 0)
      hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, 2>), dim3(n_blocks * s.n_kv_heads * (p.r / 2)),
                         dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, 1>), dim3(n_blocks * s.n_kv_heads * p.r),
                         dim3(128), 0, st, p);
    timer_end(HGA_KERNEL_BWD_DQ, st);
    timer_begin(HGA_KERNEL_BWD_DKDV, st);
    hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D>), dim3(n_blocks * s.n_kv_heads), dim3(128), 0, st, p);
    timer_end(HGA_KERNEL_BWD_DKDV, st);
  }
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(const hga_shape& s) {
  return ((sizeof(float) * static_cast<size_t>(s.n_q_heads) * s.seg_len) + 255) & ~size_t(255);
}

hipError_t launch_attn_bwd(const hga_shape& s, const void* q, const void* k_hist,
                           const void* v_hist, const void* k_seg, const void* v_seg,
                           const int32_t* sel_groups, const void* o, const float* lse,
                           const void* d_o, void* dq, void* dk_seg, void* dv_seg, void* ws,
                           hipStream_t stream) {
  BwdParams p;
  p.q = q; p.k_hist = k_hist; p.v_hist = v_hist; p.k_seg = k_seg; p.v_seg = v_seg;
  p.sel = sel_groups; p.o = o; p.lse = lse; p.d_o = d_o;
  p.dq = dq; p.dk = dk_seg; p.dv = dv_seg;
  p.dvec = static_cast<float*>(ws);
  p.n_q = s.n_q_heads; p.n_kv = s.n_kv_heads; p.r = s.n_q_heads / s.n_kv_heads;
  p.seg_len = s.seg_len; p.hist_len = s.hist_len; p.k_g = s.top_k_groups;
  p.scale = s.softmax_scale;
  p.scale_log2 = s.softmax_scale * kLog2e;
  return s.head_dim == 128 ? launch_d<128>(s, p, stream) : launch_d<64>(s, p, stream);
}

}  // namespace hga
