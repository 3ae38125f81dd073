// Exact-token attention forward over [selected history groups || causal segment].
//
// bf16 path (MFMA, gfx950 v_mfma_f32_32x32x16_bf16). One workgroup owns one
// query block b (64 queries) of HPW query heads that share KV head j, so every
// gathered K/V tile staged in LDS serves HPW*64 query rows (GQA reuse). Each
// wave owns 32 query rows of one head and keeps them in registers as the B
// operand of S^T = K . Q^T; the S^T accumulator layout (one query per lane
// column) then feeds O^T += V^T . P^T directly, with the online-softmax row
// statistics lane-local (plus one cross-half exchange for the max).
// Key tiles are 64 tokens: history tiles are 8 selected 8-token groups,
// gathered row by row from K_hist/V_hist (or from a staging buffer for the
// pinned-host tier); segment tiles 0..b follow, the last one causally masked.
//
// fp32 path: a plain VALU kernel, one thread per query row.
#include "hga_common.hpp"

namespace hga {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTile = 64;  // keys per tile

struct FwdParams {
  const void* q;
  const void* k_hist;
  const void* v_hist;
  const void* k_seg;
  const void* v_seg;
  const int32_t* sel;
  void* o;
  float* lse;
  const void* k_staged;
  const void* v_staged;
  int block_begin;
  int n_blocks_here;
  int n_q, n_kv, r;
  int seg_len;
  int64_t hist_len;
  int k_g;
  float scale_log2;  // softmax_scale * log2(e)
};

// Address of history key row `kk` (0..63) of history tile `ht` for (b, j),
// or nullptr when that group slot is empty (-1 or beyond k_g).
template <typename T>
__device__ __forceinline__ const T* hist_row(const FwdParams& p, const T* base, const T* staged,
                                             const int32_t* sel_bj, int b, int j, int ht, int kk,
                                             int D) {
  const int slot = ht * 8 + kk / kGroup;
  if (slot >= p.k_g) return nullptr;
  const int n = sel_bj[slot];
  if (n < 0) return nullptr;
  if (staged) {
    const int64_t bl = b - p.block_begin;
    return staged + ((bl * p.n_kv + j) * static_cast<int64_t>(p.k_g) * kGroup +
                     static_cast<int64_t>(slot) * kGroup + kk % kGroup) * D;
  }
  return base + (static_cast<int64_t>(j) * p.hist_len + static_cast<int64_t>(n) * kGroup +
                 kk % kGroup) * D;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
template <int D, int HPW>
__global__ __launch_bounds__(128 * HPW) void attn_fwd_bf16_kernel(FwdParams p) {
  constexpr int NT = 128 * HPW;       // threads
  constexpr int KS = D + 8;           // Ks row stride (elements)
  constexpr int VS = kTile + 4;       // Vt row stride (elements)
  constexpr int NDT = D / 32;         // 32-wide d tiles of O^T
  constexpr int NKS = D / 16;         // k-steps of S^T
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];
  __shared__ int32_t sel_s[kMaxTopKGroups];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int l32 = lane % 32;
  const int hh = lane / 32;  // lane half

  // workgroup -> (b, j, head group); KV head fastest so that with 8 KV heads
  // every workgroup of head j lands on the same XCD (round-robin dispatch);
  // heaviest (latest) query blocks first.
  const int n_hg = p.r / HPW;
  int w = blockIdx.x;
  const int j = w % p.n_kv;
  w /= p.n_kv;
  const int hg = w % n_hg;
  const int b = p.block_begin + p.n_blocks_here - 1 - w / n_hg;
  const int head = j * p.r + hg * HPW + wave / 2;
  const int qrow0 = (wave % 2) * 32;  // first query row (within the block) of this wave
  const int q_tok = b * kBlockQ + qrow0 + l32;

  const uint16_t* q = static_cast<const uint16_t*>(p.q);
  const uint16_t* kh = static_cast<const uint16_t*>(p.k_hist);
  const uint16_t* vh = static_cast<const uint16_t*>(p.v_hist);
  const uint16_t* ks_g = static_cast<const uint16_t*>(p.k_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const uint16_t* vs_g = static_cast<const uint16_t*>(p.v_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const uint16_t* kst = static_cast<const uint16_t*>(p.k_staged);
  const uint16_t* vst = static_cast<const uint16_t*>(p.v_staged);
  const int32_t* sel_bj = p.sel + (static_cast<int64_t>(b) * p.n_kv + j) * p.k_g;

  for (int i = tid; i < p.k_g; i += NT) sel_s[i] = sel_bj[i];

  // Q^T operand: lane column = query, slots = 8 consecutive d
  bf16x8 qreg[NKS];
  {
    const uint16_t* qp = q + (static_cast<int64_t>(head) * p.seg_len + q_tok) * D + hh * 8;
#pragma unroll
    for (int s = 0; s < NKS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + s * 16);
  }

  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
  float m_run = -INFINITY;  // running max (log2 domain), shared by both lane halves
  float l_run = 0.f;        // partial row sum over this lane's keys

  const int n_hist_tiles = (p.k_g + 7) / 8;
  const int n_tiles = n_hist_tiles + b + 1;
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const bool is_hist = tile < n_hist_tiles;
    const int st = tile - n_hist_tiles;  // segment tile index when !is_hist
    uint32_t gmask = 0xffu;              // valid 8-token groups of the tile
    if (is_hist) {
      gmask = 0;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int slot = tile * 8 + g;
        gmask |= (slot < p.k_g && sel_s[slot] >= 0) ? (1u << g) : 0u;
      }
      if (gmask == 0) continue;  // uniform across the workgroup
    }

    // ---- stage K (row-major) and V (transposed) tiles in LDS -------------
    {
      constexpr int CPR = D / 8;  // 16-byte chunks per row
      for (int idx = tid; idx < kTile * CPR; idx += NT) {
        const int kk = idx / CPR, c = idx % CPR;
        const uint16_t* src = is_hist ? hist_row(p, kh, kst, sel_s, b, j, tile, kk, D)
                                      : ks_g + static_cast<int64_t>(st * kTile + kk) * D;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (src) v = *reinterpret_cast<const uint4*>(src + c * 8);
        *reinterpret_cast<uint4*>(&Ks[kk * KS + c * 8]) = v;
      }
      for (int idx = tid; idx < (kTile / 4) * CPR; idx += NT) {
        const int kq = idx / CPR, c = idx % CPR;
        uint4 rows[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kk = kq * 4 + u;
          const uint16_t* src = is_hist ? hist_row(p, vh, vst, sel_s, b, j, tile, kk, D)
                                        : vs_g + static_cast<int64_t>(st * kTile + kk) * D;
          rows[u] = src ? *reinterpret_cast<const uint4*>(src + c * 8) : make_uint4(0, 0, 0, 0);
        }
        const uint16_t* r16[4] = {reinterpret_cast<const uint16_t*>(&rows[0]),
                                  reinterpret_cast<const uint16_t*>(&rows[1]),
                                  reinterpret_cast<const uint16_t*>(&rows[2]),
                                  reinterpret_cast<const uint16_t*>(&rows[3])};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint2 col;
          col.x = static_cast<uint32_t>(r16[0][e]) | (static_cast<uint32_t>(r16[1][e]) << 16);
          col.y = static_cast<uint32_t>(r16[2][e]) | (static_cast<uint32_t>(r16[3][e]) << 16);
          *reinterpret_cast<uint2*>(&Vt[(c * 8 + e) * VS + kq * 4]) = col;
        }
      }
    }
    __syncthreads();

    // ---- S^T = K . Q^T for two 32-key subtiles ---------------------------
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kt][v] = 0.f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(kt * 32 + l32) * KS + s * 16 + hh * 8]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[kt], 0, 0, 0);
      }
    }

    // ---- scale, mask, online softmax --------------------------------------
    const bool diag = !is_hist && st == b;
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = kt * 32 + 8 * (v / 4) + 4 * hh + (v % 4);
        float x = sacc[kt][v] * p.scale_log2;
        const bool masked = is_hist ? !((gmask >> (kk / 8)) & 1u) : (diag && kk > qrow0 + l32);
        x = masked ? -INFINITY : x;
        sacc[kt][v] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    const float m_base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_base);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = exp2f(sacc[kt][v] - m_base);
        psum += e;
        pb[kt][v / 8][v % 8] = static_cast<__bf16>(e);
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;

    // ---- O^T += V^T . P^T ------------------------------------------------
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint16_t* vrow = &Vt[(dt * 32 + l32) * VS];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int ksi = 0; ksi < 2; ++ksi) {
          const int k0 = kt * 32 + ksi * 16 + 4 * hh;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + k0);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + k0 + 8);
          const uint4 packed = make_uint4(lo.x, lo.y, hi.x, hi.y);
          const bf16x8 a = __builtin_bit_cast(bf16x8, packed);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][ksi], oacc[dt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---- normalise and write O (bf16) and LSE --------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = 1.0f / l_tot;
  uint16_t* o = static_cast<uint16_t*>(p.o) + (static_cast<int64_t>(head) * p.seg_len + q_tok) * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + 8 * g + 4 * hh;
      uint2 w2;
      w2.x = pack_bf16x2(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
      w2.y = pack_bf16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
      *reinterpret_cast<uint2*>(o + d0) = w2;
    }
  }
  if (hh == 0) p.lse[static_cast<int64_t>(head) * p.seg_len + q_tok] = (m_run + log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: one wave per (block, head), one thread per query row
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kWave) void attn_fwd_f32_kernel(FwdParams p) {
  __shared__ float Kt[kTile][D + 1];
  __shared__ float Vt[kTile][D + 1];
  __shared__ int32_t sel_s[kMaxTopKGroups];
  const int a = threadIdx.x;  // query row within the block
  int w = blockIdx.x;
  const int head = w % p.n_q;
  const int b = p.block_begin + p.n_blocks_here - 1 - w / p.n_q;
  const int j = head / p.r;
  const int q_tok = b * kBlockQ + a;
  const float* q = static_cast<const float*>(p.q);
  const float* kh = static_cast<const float*>(p.k_hist);
  const float* vh = static_cast<const float*>(p.v_hist);
  const float* kst = static_cast<const float*>(p.k_staged);
  const float* vst = static_cast<const float*>(p.v_staged);
  const float* ks_g = static_cast<const float*>(p.k_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const float* vs_g = static_cast<const float*>(p.v_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const int32_t* sel_bj = p.sel + (static_cast<int64_t>(b) * p.n_kv + j) * p.k_g;
  for (int i = a; i < p.k_g; i += kWave) sel_s[i] = sel_bj[i];

  float qr[D], acc[D];
  for (int e = 0; e < D; ++e) {
    qr[e] = q[(static_cast<int64_t>(head) * p.seg_len + q_tok) * D + e];
    acc[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const int n_hist_tiles = (p.k_g + 7) / 8;
  __syncthreads();
  for (int tile = 0; tile < n_hist_tiles + b + 1; ++tile) {
    const bool is_hist = tile < n_hist_tiles;
    const int st = tile - n_hist_tiles;
    for (int kk = 0; kk < kTile; ++kk) {
      const float* ksrc = is_hist ? hist_row(p, kh, kst, sel_s, b, j, tile, kk, D)
                                  : ks_g + static_cast<int64_t>(st * kTile + kk) * D;
      const float* vsrc = is_hist ? hist_row(p, vh, vst, sel_s, b, j, tile, kk, D)
                                  : vs_g + static_cast<int64_t>(st * kTile + kk) * D;
      for (int e = a; e < D; e += kWave) {
        Kt[kk][e] = ksrc ? ksrc[e] : 0.f;
        Vt[kk][e] = vsrc ? vsrc[e] : 0.f;
      }
    }
    __syncthreads();
    float sc[kTile];
    float tmax = -INFINITY;
    for (int kk = 0; kk < kTile; ++kk) {
      bool valid;
      if (is_hist) {
        const int slot = tile * 8 + kk / kGroup;
        valid = slot < p.k_g && sel_s[slot] >= 0;
      } else {
        valid = !(st == b && kk > a);
      }
      float s = 0.f;
      for (int e = 0; e < D; ++e) s += qr[e] * Kt[kk][e];
      sc[kk] = valid ? s * p.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sc[kk]);
    }
    const float m_new = fmaxf(m_run, tmax);
    const float m_base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_base);
    l_run *= alpha;
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
    for (int kk = 0; kk < kTile; ++kk) {
      const float e_ = exp2f(sc[kk] - m_base);
      l_run += e_;
      for (int e = 0; e < D; ++e) acc[e] += e_ * Vt[kk][e];
    }
    m_run = m_new;
    __syncthreads();
  }
  float* o = static_cast<float*>(p.o) + (static_cast<int64_t>(head) * p.seg_len + q_tok) * D;
  const float inv = 1.0f / l_run;
  for (int e = 0; e < D; ++e) o[e] = acc[e] * inv;
  p.lse[static_cast<int64_t>(head) * p.seg_len + q_tok] = (m_run + log2f(l_run)) * kLn2;
}

template <int D>
hipError_t launch_d(const hga_shape& s, FwdParams& p, hipStream_t st) {
  timer_begin(HGA_KERNEL_ATTN_FWD, st);
  if (s.dtype == HGA_F32) {
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3(p.n_blocks_here * s.n_q_heads), dim3(kWave),
                       0, st, p);
  } else if (p.r % 2 == 0) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 2>),
                       dim3(p.n_blocks_here * s.n_kv_heads * (p.r / 2)), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 1>), dim3(p.n_blocks_here * s.n_kv_heads * p.r),
                       dim3(128), 0, st, p);
  }
  timer_end(HGA_KERNEL_ATTN_FWD, st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const hga_shape& s, const void* q, const void* k_hist,
                           const void* v_hist, const void* k_seg, const void* v_seg,
                           const int32_t* sel_groups, void* o, float* lse,
                           const void* k_staged, const void* v_staged, int32_t block_begin,
                           int32_t block_end, hipStream_t stream) {
  if (block_end <= block_begin) return hipSuccess;
  FwdParams p;
  p.q = q; p.k_hist = k_hist; p.v_hist = v_hist; p.k_seg = k_seg; p.v_seg = v_seg;
  p.sel = sel_groups; p.o = o; p.lse = lse;
  p.k_staged = k_staged; p.v_staged = v_staged;
  p.block_begin = block_begin;
  p.n_blocks_here = block_end - block_begin;
  p.n_q = s.n_q_heads; p.n_kv = s.n_kv_heads; p.r = s.n_q_heads / s.n_kv_heads;
  p.seg_len = s.seg_len; p.hist_len = s.hist_len; p.k_g = s.top_k_groups;
  p.scale_log2 = s.softmax_scale * kLog2e;
  return s.head_dim == 128 ? launch_d<128>(s, p, stream) : launch_d<64>(s, p, stream);
}

}  // namespace hga
