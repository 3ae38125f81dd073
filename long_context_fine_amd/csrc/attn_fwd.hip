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
#include "attn_tile.hpp"

namespace hga {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;

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
  const void* k_sink;     // sink rows: [n_kv][sink_stride][D], first n_sink_tiles*64 used
  const void* v_sink;
  int64_t sink_stride;
  int n_sink_tiles;       // fixed sink, in 64-token tiles (chunks)
  int window;             // local window W in tokens (<= seg_len)
  int block_begin;
  int n_blocks_here;
  int n_q, n_kv, r;
  int seg_len;
  int64_t hist_len;
  int64_t hist_rows;  // rows per KV head in k_hist / v_hist
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
  return base + (static_cast<int64_t>(j) * p.hist_rows + static_cast<int64_t>(n) * kGroup +
                 kk % kGroup) * D;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
// Workgroup = (KV head j, group of HPW query heads, pair of query blocks). The
// pair is {b, n-1-b}: block b attends to b+1 segment tiles, so pairing the
// i-th latest with the i-th earliest block gives every workgroup the same
// amount of work. 4*HPW waves: wave (g, h, q) owns 32 query rows (half q) of
// head h for the key tiles of parity g, so two waves share each SIMD and one
// wave's softmax overlaps the other's MFMAs. The two parity groups keep their
// own online-softmax state; the states are merged exactly through LDS at the
// end of each block. Per iteration each group stages its next 64-key tile in
// registers while the current pair of tiles (double-buffered in LDS) is used.
// K and V both sit row-major in LDS; V^T reaches the MFMA through transposed
// LDS reads (ds_read_b64_tr_b16).
template <int D, int HPW, bool EXT>
__global__ __launch_bounds__(256 * HPW) void attn_fwd_bf16_kernel(FwdParams p) {
  constexpr int NT = 256 * HPW;       // threads
  constexpr int GT = NT / 2;          // threads per parity group
  constexpr int KS = D + 8;           // K row stride (elements): conflict-free row reads
  constexpr int VS = D + 32;          // V row stride: conflict-free transposed reads
  constexpr int NDT = D / 32;         // 32-wide d tiles of O^T
  constexpr int NKS = D / 16;         // k-steps of S^T
  constexpr int STAGE = kTile * (KS + VS);  // K + V of one tile (elements)
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][STAGE];  // [buffer][parity]
  __shared__ int32_t sel_s[kMaxTopKGroups];
  __shared__ int32_t hlist[kMaxTopKGroups / 8];
  __shared__ int32_t n_hist_s;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int l32 = lane % 32;
  const int hh = lane / 32;            // lane half
  const int grp = wave / (2 * HPW);    // tile parity group
  const int gw = wave % (2 * HPW);     // wave within the group
  const int gtid = tid % GT;           // thread within the group

  // KV head fastest: with 8 KV heads every workgroup of head j lands on the
  // same XCD under round-robin dispatch and shares that XCD's L2.
  const int n_hg = p.r / HPW;
  int w = blockIdx.x;
  const int j = w % p.n_kv;
  w /= p.n_kv;
  const int hg = w % n_hg;
  const int pair = w / n_hg;
  const int b_hi = p.block_begin + p.n_blocks_here - 1 - pair;
  const int b_lo = p.block_begin + pair;
  const int head = j * p.r + hg * HPW + gw / 2;
  const int qrow0 = (gw % 2) * 32;  // first query row (within the block) of this wave

  const uint16_t* q = static_cast<const uint16_t*>(p.q);
  const uint16_t* kh = static_cast<const uint16_t*>(p.k_hist);
  const uint16_t* vh = static_cast<const uint16_t*>(p.v_hist);
  const uint16_t* ks_g = static_cast<const uint16_t*>(p.k_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const uint16_t* vs_g = static_cast<const uint16_t*>(p.v_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const uint16_t* kst = static_cast<const uint16_t*>(p.k_staged);
  const uint16_t* vst = static_cast<const uint16_t*>(p.v_staged);
  const float c2 = p.scale_log2;

  for (int half = 0; half < 2; ++half) {
    const int b = half == 0 ? b_hi : b_lo;
    if (half == 1 && b_lo >= b_hi) break;  // odd count: the middle block runs once
    const int32_t* sel_bj = p.sel + (static_cast<int64_t>(b) * p.n_kv + j) * p.k_g;
    __syncthreads();
    for (int i = tid; i < p.k_g; i += NT) sel_s[i] = valid_group(sel_bj[i], p.hist_len / kGroup);
    __syncthreads();
    build_hist_tile_list(sel_s, p.k_g, hlist, &n_hist_s);
    __syncthreads();
    const int n_hist = n_hist_s;
    const int n_sink = EXT ? p.n_sink_tiles : 0;
    const int seg_t0 = seg_first_tile<EXT>(b, p.window);
    // tiles: sink (whole chunks), routed history (8 groups each), segment window
    const int n_pre = n_sink + n_hist;
    const int n_tiles = n_pre + b - seg_t0 + 1;
    const int n_iter = (n_tiles + 1) / 2;
    const int q_tok = b * kBlockQ + qrow0 + l32;
    const int64_t staged_row0 =
        (static_cast<int64_t>(b - p.block_begin) * p.n_kv + j) * static_cast<int64_t>(p.k_g) * kGroup;

    // rows 4kq..4kq+3 of tile t < n_tiles, for K (which=0) or V (which=1). A
    // history slot without a group (-1 or past k_g) reads the segment's first
    // rows instead: finite values whose scores are masked to -inf.
    auto rowptr = [&](int t, int kq, int which) -> const uint16_t* {
      const uint16_t* seg = which ? vs_g : ks_g;
      if (t < n_sink)
        return static_cast<const uint16_t*>(which ? p.v_sink : p.k_sink) +
               (static_cast<int64_t>(j) * p.sink_stride + t * kTile + kq * 4) * D;
      if (t < n_pre) {
        const int slot = hlist[t - n_sink] * 8 + kq / 2;
        const int n = slot < p.k_g ? sel_s[slot] : -1;
        if (n < 0) return seg + (kq % 2) * 4 * D;
        if (kst) return (which ? vst : kst) + (staged_row0 + slot * kGroup + (kq % 2) * 4) * D;
        return (which ? vh : kh) +
               (static_cast<int64_t>(j) * p.hist_rows + static_cast<int64_t>(n) * kGroup + (kq % 2) * 4) * D;
      }
      return seg + static_cast<int64_t>((seg_t0 + t - n_pre) * kTile + kq * 4) * D;
    };

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
    // running max (scaled, log2 domain), same in both lane halves; a finite
    // floor so a row whose first tiles are all masked (local window) keeps
    // exp2(-inf - m) = 0 instead of NaN
    float m_run = -1e30f;
    float l_run = 0.f;        // partial row sum over this lane's keys

    TileRegs<D, GT> kr, vr;
    if (grp < n_tiles) {
      kr.load(gtid, [&](int kq) { return rowptr(grp, kq, 0); });
      vr.load(gtid, [&](int kq) { return rowptr(grp, kq, 1); });
      kr.store_rows(gtid, smem[0][grp], KS);
      vr.store_rows(gtid, smem[0][grp] + kTile * KS, VS);
    }
    __syncthreads();

    for (int it = 0; it < n_iter; ++it) {
      const int cur = it & 1;
      const int t = 2 * it + grp;          // this group's tile
      const bool more = it + 1 < n_iter && t + 2 < n_tiles;
      if (more) {
        kr.load(gtid, [&](int kq) { return rowptr(t + 2, kq, 0); });
        vr.load(gtid, [&](int kq) { return rowptr(t + 2, kq, 1); });
      }
      if (t < n_tiles) {
        // keep: bit kt*16 + v set if accumulator element v of subtile kt (key
        // kt*32 + 8*(v/4) + 4*hh + v%4 of the tile) takes part; all ones
        // except on a history tile with empty slots or the diagonal tile
        uint32_t keep = 0xffffffffu;
        const int s_idx = seg_t0 + t - n_pre;
        const bool seg_edge = t >= n_pre && seg_tile_masked<EXT>(s_idx, b, p.window);
        if (t >= n_sink && t < n_pre) {
          const uint32_t gm = hist_group_mask(sel_s, p.k_g, hlist[t - n_sink]);
#pragma unroll
          for (int gi = 0; gi < 8; ++gi)
            if (!((gm >> gi) & 1u)) keep &= ~(0xfu << (4 * gi));
        } else if (seg_edge) {
          // causal diagonal and/or local-window start
          keep = window_keep<EXT>(q_tok, s_idx * kTile, p.window, hh);
        }
        const bool masked = seg_edge || __builtin_amdgcn_readfirstlane(keep == 0xffffffffu ? 0 : 1) != 0;
        const uint16_t* kbuf = smem[cur][grp];
        const uint16_t* vbuf = kbuf + kTile * KS;

        // ---- S^T = K . Q^T for two 32-key subtiles -----------------------
        f32x16 sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) sacc[kt][v] = 0.f;
        // raised wave priority over each MFMA cluster: of the two waves on a
        // SIMD, the one with MFMAs ready issues first while the other one's
        // softmax and LDS work fills the gaps
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kbuf[(kt * 32 + l32) * KS + s * 16 + hh * 8]);
            sacc[kt] = mfma32(a, qreg[s], sacc[kt]);
          }
        }
        __builtin_amdgcn_s_setprio(0);

        // ---- mask, online softmax (raw scores; scale folded into exp2) ------
        if (masked) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              sacc[kt][v] = (keep >> (kt * 16 + v)) & 1u ? sacc[kt][v] : -INFINITY;
        }
        float tmax = sacc[0][0];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sacc[kt][v]);
        tmax = max_xor32(tmax);
        // lazy rescale: the reference max only moves when some row's max
        // exceeds it by more than kRescaleSlack (log2 units), so most tiles
        // skip rescaling O; probabilities relative to a stale max stay below
        // 2^kRescaleSlack and the final division by the row sum is exact
        const float mt = tmax * c2;
        if (__any(mt > m_run + kRescaleSlack)) {
          const float m_new = fmaxf(m_run, mt);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
        }
        const float m_new = m_run;
        float psum = 0.f;
        bf16x8 pb[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float e = fast_exp2(fmaf(sacc[kt][v], c2, -m_new));
            psum += e;
            sacc[kt][v] = e;
          }
          pb[kt][0] = acc_to_bf16x8(sacc[kt], 0);
          pb[kt][1] = acc_to_bf16x8(sacc[kt], 8);
        }
        l_run += psum;

        // ---- O^T += V^T . P^T --------------------------------------------
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ksi = 0; ksi < 2; ++ksi)
              oacc[dt] = mfma32(lds_a_tr(vbuf, VS, kt * 32 + ksi * 16, dt * 32, lane), pb[kt][ksi], oacc[dt]);
        __builtin_amdgcn_s_setprio(0);
      }
      if (more) {
        kr.store_rows(gtid, smem[cur ^ 1][grp], KS);
        vr.store_rows(gtid, smem[cur ^ 1][grp] + kTile * KS, VS);
      }
      __syncthreads();
    }

    // ---- merge the two parity states, normalise, write O (bf16) and LSE -----
    // exchange layout [wave][4-float column][lane][4] (b128 accesses of a wave
    // cover 1 KiB contiguously, no bank conflicts), then m and l per lane
    float* xch = reinterpret_cast<float*>(&smem[0][0][0]);  // free after the last barrier
    constexpr int XW = NDT * 16;
    auto xaddr = [&](int idx) -> float* {
      return xch + ((static_cast<int64_t>(gw) * (XW / 4) + idx / 4) * kWave + lane) * 4;
    };
    float* xml = xch + static_cast<int64_t>(2 * HPW) * XW * kWave + (gw * kWave + lane) * 2;
    if (grp == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; v += 4)
          *reinterpret_cast<float4*>(xaddr(dt * 16 + v)) =
              make_float4(oacc[dt][v], oacc[dt][v + 1], oacc[dt][v + 2], oacc[dt][v + 3]);
      *reinterpret_cast<float2*>(xml) = make_float2(m_run, l_run);
    }
    __syncthreads();
    if (grp == 0) {
      const float2 ml = *reinterpret_cast<const float2*>(xml);
      const float m1 = ml.x, l1 = ml.y;
      const float m = fmaxf(m_run, m1);
      const float a0 = fast_exp2(m_run - m), a1 = fast_exp2(m1 - m);
      const float l_lane = l_run * a0 + l1 * a1;
      const float l_tot = l_lane + __shfl_xor(l_lane, 32, kWave);
      const float inv = 1.0f / l_tot;
      const float s0 = a0 * inv, s1 = a1 * inv;
      uint16_t* o = static_cast<uint16_t*>(p.o) + (static_cast<int64_t>(head) * p.seg_len + q_tok) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = dt * 32 + 8 * g + 4 * hh;
          const float4 x1 = *reinterpret_cast<const float4*>(xaddr(dt * 16 + 4 * g));
          const float x[4] = {oacc[dt][4 * g] * s0 + x1.x * s1, oacc[dt][4 * g + 1] * s0 + x1.y * s1,
                              oacc[dt][4 * g + 2] * s0 + x1.z * s1, oacc[dt][4 * g + 3] * s0 + x1.w * s1};
          uint2 w2;
          w2.x = cvt_pk_bf16(x[0], x[1]);
          w2.y = cvt_pk_bf16(x[2], x[3]);
          *reinterpret_cast<uint2*>(o + d0) = w2;
        }
      }
      if (hh == 0) p.lse[static_cast<int64_t>(head) * p.seg_len + q_tok] = (m + __log2f(l_tot)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: one wave per (block, head), one thread per query row.
// The query rows and the tile's scores live in LDS (each thread's row or
// column, padded so the wave's accesses fall in distinct banks); only the
// output accumulator stays in registers.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kWave) void attn_fwd_f32_kernel(FwdParams p) {
  __shared__ float Kt[kTile][D + 1];
  __shared__ float Vt[kTile][D + 1];
  __shared__ float Qs[kWave][D + 1];        // query row of thread a
  __shared__ float Ps[kTile][kWave + 1];    // scaled scores of the tile, column a
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
  for (int i = a; i < p.k_g; i += kWave) sel_s[i] = valid_group(sel_bj[i], p.hist_len / kGroup);

  {
    const float* qb = q + (static_cast<int64_t>(head) * p.seg_len + b * kBlockQ) * D;
    for (int x = a; x < kWave * D; x += kWave) Qs[x / D][x % D] = qb[x];
  }
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int n_hist_tiles = (p.k_g + 7) / 8;
  const int n_sink = p.n_sink_tiles;
  const int seg_t0 = seg_first_tile<true>(b, p.window);
  const float* k_sink = static_cast<const float*>(p.k_sink) + static_cast<int64_t>(j) * p.sink_stride * D;
  const float* v_sink = static_cast<const float*>(p.v_sink) + static_cast<int64_t>(j) * p.sink_stride * D;
  __syncthreads();
  for (int tile = 0; tile < n_sink + n_hist_tiles + b - seg_t0 + 1; ++tile) {
    const bool is_sink = tile < n_sink;
    const bool is_hist = !is_sink && tile < n_sink + n_hist_tiles;
    const int ht = tile - n_sink;
    const int st = seg_t0 + tile - n_sink - n_hist_tiles;
    for (int kk = 0; kk < kTile; ++kk) {
      const int64_t sink_off = static_cast<int64_t>(tile * kTile + kk) * D;
      const float* ksrc = is_sink ? k_sink + sink_off
                          : is_hist ? hist_row(p, kh, kst, sel_s, b, j, ht, kk, D)
                                    : ks_g + static_cast<int64_t>(st * kTile + kk) * D;
      const float* vsrc = is_sink ? v_sink + sink_off
                          : is_hist ? hist_row(p, vh, vst, sel_s, b, j, ht, kk, D)
                                    : vs_g + static_cast<int64_t>(st * kTile + kk) * D;
      for (int e = a; e < D; e += kWave) {
        Kt[kk][e] = ksrc ? ksrc[e] : 0.f;
        Vt[kk][e] = vsrc ? vsrc[e] : 0.f;
      }
    }
    __syncthreads();
    float tmax = -INFINITY;
    for (int kk = 0; kk < kTile; ++kk) {
      bool valid;
      if (is_sink) {
        valid = true;
      } else if (is_hist) {
        const int slot = ht * 8 + kk / kGroup;
        valid = slot < p.k_g && sel_s[slot] >= 0;
      } else {
        const int key = st * kTile + kk;
        valid = key <= q_tok && key > q_tok - p.window;
      }
      float s = 0.f;
      for (int e = 0; e < D; ++e) s += Qs[a][e] * Kt[kk][e];
      const float sc = valid ? s * p.scale_log2 : -INFINITY;
      Ps[kk][a] = sc;
      tmax = fmaxf(tmax, sc);
    }
    const float m_new = fmaxf(m_run, tmax);
    const float m_base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_base);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
    for (int kk = 0; kk < kTile; ++kk) {
      const float e_ = exp2f(Ps[kk][a] - m_base);
      l_run += e_;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] += e_ * Vt[kk][e];
    }
    m_run = m_new;
    __syncthreads();
  }
  float* o = static_cast<float*>(p.o) + (static_cast<int64_t>(head) * p.seg_len + q_tok) * D;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int e = 0; e < D; ++e) o[e] = acc[e] * inv;
  p.lse[static_cast<int64_t>(head) * p.seg_len + q_tok] = (m_run + log2f(l_run)) * kLn2;
}

template <int D>
hipError_t launch_d(const hga_shape& s, FwdParams& p, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (s.dtype == HGA_F32) {
    hipExtLaunchKernelGGL((attn_fwd_f32_kernel<D>), dim3(p.n_blocks_here * s.n_q_heads), dim3(kWave), 0,
                          st, ev0, ev1, 0, p);
  } else {
    const int n_pairs = (p.n_blocks_here + 1) / 2;
    // sink or local window: the extended kernels; otherwise the plain ones
    const bool ext = p.window < s.seg_len || p.n_sink_tiles > 0;
    if (p.r % 2 == 0) {
      const dim3 grid(n_pairs * s.n_kv_heads * (p.r / 2));
      if (ext) hipExtLaunchKernelGGL((attn_fwd_bf16_kernel<D, 2, true>), grid, dim3(512), 0, st, ev0, ev1, 0, p);
      else hipExtLaunchKernelGGL((attn_fwd_bf16_kernel<D, 2, false>), grid, dim3(512), 0, st, ev0, ev1, 0, p);
    } else {
      const dim3 grid(n_pairs * s.n_kv_heads * p.r);
      if (ext) hipExtLaunchKernelGGL((attn_fwd_bf16_kernel<D, 1, true>), grid, dim3(256), 0, st, ev0, ev1, 0, p);
      else hipExtLaunchKernelGGL((attn_fwd_bf16_kernel<D, 1, false>), grid, dim3(256), 0, st, ev0, ev1, 0, p);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const hga_shape& s, const void* q, const void* k_hist,
                           const void* v_hist, const void* k_seg, const void* v_seg,
                           const int32_t* sel_groups, void* o, float* lse,
                           const void* k_staged, const void* v_staged, const void* k_sink,
                           const void* v_sink, int64_t sink_stride, int32_t block_begin,
                           int32_t block_end, hipStream_t stream, hipEvent_t ev_start,
                           hipEvent_t ev_stop) {
  if (block_end <= block_begin) return hipSuccess;
  FwdParams p;
  p.q = q; p.k_hist = k_hist; p.v_hist = v_hist; p.k_seg = k_seg; p.v_seg = v_seg;
  p.sel = sel_groups; p.o = o; p.lse = lse;
  p.k_staged = k_staged; p.v_staged = v_staged;
  p.k_sink = k_sink; p.v_sink = v_sink; p.sink_stride = sink_stride;
  p.n_sink_tiles = sink_chunks(s);
  p.window = local_window(s);
  p.block_begin = block_begin;
  p.n_blocks_here = block_end - block_begin;
  p.n_q = s.n_q_heads; p.n_kv = s.n_kv_heads; p.r = s.n_q_heads / s.n_kv_heads;
  p.seg_len = s.seg_len; p.hist_len = s.hist_len; p.hist_rows = hist_rows(s); p.k_g = s.top_k_groups;
  p.scale_log2 = s.softmax_scale * kLog2e;
  return s.head_dim == 128 ? launch_d<128>(s, p, stream, ev_start, ev_stop) : launch_d<64>(s, p, stream, ev_start, ev_stop);
}

}  // namespace hga
