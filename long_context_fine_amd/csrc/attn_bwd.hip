// Backward of exact-token attention with detached history.
//
//   Dvec[h][i] = dO[h][i] . O[h][i]                      (in the dQ kernel)
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
#include "attn_tile.hpp"

namespace hga {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

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
  float* lse2;       // [n_q][S] LSE * log2(e), written by the bf16 dQ kernel for dK/dV
  float* dkdv_part;  // [n_hg][2][n_kv][S][D] fp32 partials (dK, dV) when n_hg > 1
  int n_q, n_kv, r;
  int seg_len;
  int64_t hist_len;
  int64_t hist_rows;  // rows per KV head in k_hist / v_hist
  // Staged routed rows (history in host memory): k_hist / v_hist then point
  // at [n_blocks][n_kv][k_g*8][D] copies of each block's routed groups, with
  // hist_rows = k_g*8, and the kernels keep group b*n_kv*k_g + slot in place
  // of the valid group of slot `slot` of block b (see staged_group), which
  // addresses exactly that copy.
  int staged;
  const void* k_sink;  // sink rows [n_kv][sink_stride][D] (the history itself when not staged)
  const void* v_sink;
  int64_t sink_stride;
  int k_g;
  int n_sink_tiles;   // fixed sink: the first n_sink_tiles*64 history rows
  int window;         // local window W in tokens (<= seg_len)
  float scale;
  float scale_log2;
};

// Group whose rows the kernels read for slot `slot` of block b: the validated
// id (-1 for an empty slot), or with staged rows the block's copy of it.
__device__ __forceinline__ int32_t staged_group(const BwdParams& p, int b, int slot, int32_t id) {
  const int32_t n = valid_group(id, p.hist_len / kGroup);
  return n >= 0 && p.staged ? b * p.n_kv * p.k_g + slot : n;
}

__device__ __forceinline__ int64_t hist_offset(const BwdParams& p, const int32_t* sel_s, int j,
                                               int ht, int kk, int D) {
  const int slot = ht * 8 + kk / kGroup;
  if (slot >= p.k_g) return -1;
  const int n = sel_s[slot];
  if (n < 0) return -1;
  return (static_cast<int64_t>(j) * p.hist_rows + static_cast<int64_t>(n) * kGroup + kk % kGroup) * D;
}

// Dvec = rowsum(dO * O), fp32 accumulation (fp32 path; the bf16 dQ kernel
// computes it for its own rows).
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
// Same decomposition as the forward: workgroup = (KV head j, HPW query heads,
// pair of query blocks {b, n-1-b}); 4*HPW waves in two tile-parity groups,
// each wave owning 32 query rows of one head (Q^T and dO^T stay in registers
// as B operands). Per 64-key tile: S^T = K.Q^T, dP^T = V.dO^T, dS^T = P^T o
// (dP^T - Dvec), dQ^T += K^T.dS^T with K^T read transposed from the K tile.
// Each parity group loads its K/V tiles straight from global memory into a
// double-buffered, XOR-swizzled LDS stage (global_load_lds; history tiles are
// runs of whole selected groups) while it works on the current one; LDS
// operands are read one k-step ahead of their MFMAs. The two parity groups'
// dQ partials are summed in a fixed order.
template <int D, int HPW, bool EXT>
__global__ __launch_bounds__(256 * HPW) void attn_bwd_dq_bf16_kernel(BwdParams p) {
  constexpr int NT = 256 * HPW;
  constexpr int GT = NT / 2;
  constexpr int NDT = D / 32;
  constexpr int NKS = D / 16;
  constexpr int TILE = kTile * D;
  constexpr uint32_t RPI = kWave / (D / 8);  // rows per global_load_lds run
  constexpr int IPT = tile_lds_instrs<D, GT>();
  constexpr int NDMA = 2 * IPT;          // copy instructions per K/V tile pair
  static_assert(NDMA <= 2 * (D / 16), "one copy per S/dP k-step");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][2][TILE];  // [buffer][parity][K, V]
  __shared__ int32_t sel_s[kMaxTopKGroups];
  __shared__ int32_t hlist[kMaxTopKGroups / 8];
  __shared__ int32_t n_hist_s;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int l32 = lane % 32, hh = lane / 32;
  const int grp = wave / (2 * HPW);
  const int gw = wave % (2 * HPW);
  const int gtid = tid % GT;
  const uint32_t gwave = static_cast<uint32_t>(wave % (2 * HPW));  // wave within the group
  const int n_blocks = p.seg_len / kBlockQ;
  const int n_hg = p.r / HPW;
  int w = blockIdx.x;
  const int j = w % p.n_kv;
  w /= p.n_kv;
  const int hg = w % n_hg;
  const int pair = w / n_hg;
  const int b_hi = n_blocks - 1 - pair;
  const int b_lo = pair;
  const int head = j * p.r + hg * HPW + gw / 2;
  const int qrow0 = (gw % 2) * 32;

  const uint16_t* kh = static_cast<const uint16_t*>(p.k_hist) + static_cast<int64_t>(j) * p.hist_rows * D;
  const uint16_t* vh = static_cast<const uint16_t*>(p.v_hist) + static_cast<int64_t>(j) * p.hist_rows * D;
  const uint16_t* ksk = static_cast<const uint16_t*>(p.k_sink) + static_cast<int64_t>(j) * p.sink_stride * D;
  const uint16_t* vsk = static_cast<const uint16_t*>(p.v_sink) + static_cast<int64_t>(j) * p.sink_stride * D;
  const uint16_t* ks_g = static_cast<const uint16_t*>(p.k_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const uint16_t* vs_g = static_cast<const uint16_t*>(p.v_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const float c2 = p.scale_log2;

  for (int half = 0; half < 2; ++half) {
    const int b = half == 0 ? b_hi : b_lo;
    if (half == 1 && b_lo >= b_hi) break;
    const int32_t* sel_bj = p.sel + (static_cast<int64_t>(b) * p.n_kv + j) * p.k_g;
    __syncthreads();
    for (int i = tid; i < p.k_g; i += NT) sel_s[i] = staged_group(p, b, i, sel_bj[i]);
    __syncthreads();
    build_hist_tile_list(sel_s, p.k_g, hlist, &n_hist_s);
    __syncthreads();
    const int n_hist = n_hist_s;
    const int n_sink = EXT ? p.n_sink_tiles : 0;
    const int seg_t0 = seg_first_tile<EXT>(b, p.window);
    const int n_pre = n_sink + n_hist;
    const int n_tiles = n_pre + b - seg_t0 + 1;
    const int n_iter = (n_tiles + 1) / 2;
    const int q_tok = b * kBlockQ + qrow0 + l32;
    const int64_t row_off = static_cast<int64_t>(head) * p.seg_len + q_tok;

    // K and V of tile t (sink tiles, routed history tiles, then segment tiles
    // seg_t0..b of the local window) into
    // LDS buffer buf of this parity group, as NDMA single wave instructions
    // (copy k: instruction k % IPT of the K (k < IPT) or V tile). A history
    // slot without a group (-1 or past k_g) loads the segment's first rows
    // instead: finite values whose probabilities are forced to zero.
    auto issue_copy = [&](int t, int buf, int k) {
      const int which = k / IPT, part = k % IPT;
      const uint16_t* seg = which ? vs_g : ks_g;
      if (t < n_sink) {
        tile_copy_rows_part<D, GT>(smem[buf][grp][which], gwave, lane,
                                   (which ? vsk : ksk) + static_cast<int64_t>(t) * kTile * D, part);
      } else if (t < n_pre) {
        const int ht = __builtin_amdgcn_readfirstlane(hlist[t - n_sink]);
        const uint16_t* base = which ? vh : kh;
        tile_copy_part<D, GT>(smem[buf][grp][which], gwave, lane, [&](uint32_t kq) -> const uint16_t* {
          const uint32_t slot = static_cast<uint32_t>(ht) * 8u + (kq * RPI) / kGroup;
          const int n = slot < static_cast<uint32_t>(p.k_g) ? __builtin_amdgcn_readfirstlane(sel_s[slot]) : -1;
          const uint32_t sub = (kq * RPI) % kGroup;
          return n >= 0 ? base + (static_cast<int64_t>(n) * kGroup + sub) * D : seg + sub * D;
        }, part);
      } else {
        tile_copy_rows_part<D, GT>(smem[buf][grp][which], gwave, lane,
                                   seg + static_cast<int64_t>(seg_t0 + t - n_pre) * kTile * D, part);
      }
    };
    auto issue_tile = [&](int t, int buf) {
      if (t >= n_tiles) return;
#pragma unroll
      for (int k = 0; k < NDMA; ++k) issue_copy(t, buf, k);
    };

    issue_tile(grp, 0);

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
    // Dvec = dO . O for this row (O is the forward's bf16 output); the dK/dV
    // kernel, launched next on the same stream, reads it back.
    float drow = 0.f;
    {
      const uint16_t* op = static_cast<const uint16_t*>(p.o) + row_off * D + hh * 8;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 ov = *reinterpret_cast<const bf16x8*>(op + s * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) drow += static_cast<float>(goreg[s][e]) * static_cast<float>(ov[e]);
      }
      drow += __shfl_xor(drow, 32, kWave);
      if (grp == 0 && hh == 0) {
        p.dvec[row_off] = drow;
        p.lse2[row_off] = lse2;
      }
    }
    f32x16 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;

    wait_vmem();
    __syncthreads();

    for (int it = 0; it < n_iter; ++it) {
      const int cur = it & 1;
      const int t = 2 * it + grp;
      const bool more = it + 1 < n_iter && t + 2 < n_tiles;
      if (t < n_tiles) {
        // keep: bit kt*16 + v set if accumulator element v of subtile kt (key
        // kt*32 + 8*(v/4) + 4*hh + v%4 of the tile) takes part; all ones
        // except on a history tile with empty slots or a segment tile on the
        // causal diagonal or the local-window start
        uint32_t keep = 0xffffffffu;
        const int s_idx = seg_t0 + t - n_pre;
        const bool seg_edge = t >= n_pre && seg_tile_masked<EXT>(s_idx, b, p.window);
        if (t >= n_sink && t < n_pre) {
          const uint32_t gm = hist_group_mask(sel_s, p.k_g, hlist[t - n_sink]);
#pragma unroll
          for (int gi = 0; gi < 8; ++gi)
            if (!((gm >> gi) & 1u)) keep &= ~(0xfu << (4 * gi));
        } else if (seg_edge) {
          keep = window_keep<EXT>(q_tok, s_idx * kTile, p.window, hh);
        }
        const bool masked = seg_edge || __builtin_amdgcn_readfirstlane(keep == 0xffffffffu ? 0 : 1) != 0;
        const uint16_t* kbuf = smem[cur][grp][0];
        const uint16_t* vbuf = smem[cur][grp][1];
        // the swizzled LDS offsets derive from the lane id; an opaque copy per
        // tile keeps the compiler from hoisting all of them into live registers
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {   // one 32-key subtile at a time
          f32x16 sacc, pacc;
#pragma unroll
          for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; pacc[v] = 0.f; }
          bf16x8 ka = lds_a_row_swz<D>(kbuf, kt * 32, 0, ln);
          bf16x8 va = lds_a_row_swz<D>(vbuf, kt * 32, 0, ln);
          // raised wave priority over each MFMA cluster (two waves per SIMD:
          // the one with MFMAs ready issues first)
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int s = 0; s < NKS; ++s) {
            bf16x8 kn = ka, vn = va;
            if (s + 1 < NKS) {
              kn = lds_a_row_swz<D>(kbuf, kt * 32, (s + 1) * 16, ln);
              vn = lds_a_row_swz<D>(vbuf, kt * 32, (s + 1) * 16, ln);
            }
            {  // NDMA copies spread evenly over the 2*NKS k-steps, at most one each
              const int st = kt * NKS + s;
              const int k_lo = st * NDMA / (2 * NKS), k_hi = (st + 1) * NDMA / (2 * NKS);
              if (more && k_hi > k_lo) issue_copy(t + 2, cur ^ 1, k_lo);
            }
            sacc = mfma32(ka, qreg[s], sacc);
            pacc = mfma32(va, goreg[s], pacc);
            ka = kn;
            va = vn;
            __builtin_amdgcn_sched_barrier(0);
          }
          __builtin_amdgcn_s_setprio(0);
          bf16x8 a0 = lds_a_tr_swz<D>(kbuf, kt * 32, 0, ln);
          bf16x8 a1 = lds_a_tr_swz<D>(kbuf, kt * 32 + 16, 0, ln);
          if (masked) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float pr = fast_exp2(fmaf(sacc[v], c2, -lse2));
              pr = (keep >> (kt * 16 + v)) & 1u ? pr : 0.f;
              sacc[v] = pr * (pacc[v] - drow);
            }
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) sacc[v] = fast_exp2(fmaf(sacc[v], c2, -lse2)) * (pacc[v] - drow);
          }
          const bf16x8 ds0 = acc_to_bf16x8(sacc, 0);
          const bf16x8 ds1 = acc_to_bf16x8(sacc, 8);
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            bf16x8 n0 = a0, n1 = a1;
            if (dt + 1 < NDT) {
              n0 = lds_a_tr_swz<D>(kbuf, kt * 32, (dt + 1) * 32, ln);
              n1 = lds_a_tr_swz<D>(kbuf, kt * 32 + 16, (dt + 1) * 32, ln);
            }
            acc[dt] = mfma32(a0, ds0, acc[dt]);
            acc[dt] = mfma32(a1, ds1, acc[dt]);
            a0 = n0;
            a1 = n1;
            __builtin_amdgcn_sched_barrier(0);
          }
          __builtin_amdgcn_s_setprio(0);
        }
      }
      wait_vmem();
      __syncthreads();
    }

    // ---- sum the two parity partials (group 0 + group 1), write dQ ----------
    // exchange layout [wave][4-float column][lane][4]: a wave's b128 accesses
    // cover 1 KiB contiguously (no bank conflicts)
    float* xch = reinterpret_cast<float*>(&smem[0][0][0][0]);
    constexpr int XW = NDT * 16;
    auto xaddr = [&](int idx) -> float* {
      return xch + ((static_cast<int64_t>(gw) * (XW / 4) + idx / 4) * kWave + lane) * 4;
    };
    if (grp == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; v += 4)
          *reinterpret_cast<float4*>(xaddr(dt * 16 + v)) =
              make_float4(acc[dt][v], acc[dt][v + 1], acc[dt][v + 2], acc[dt][v + 3]);
    }
    __syncthreads();
    if (grp == 0) {
      uint16_t* dq = static_cast<uint16_t*>(p.dq) + row_off * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = dt * 32 + 8 * g + 4 * hh;
          const float4 o = *reinterpret_cast<const float4*>(xaddr(dt * 16 + 4 * g));
          const float x[4] = {(acc[dt][4 * g] + o.x) * p.scale, (acc[dt][4 * g + 1] + o.y) * p.scale,
                              (acc[dt][4 * g + 2] + o.z) * p.scale, (acc[dt][4 * g + 3] + o.w) * p.scale};
          uint2 w2;
          w2.x = cvt_pk_bf16(x[0], x[1]);
          w2.y = cvt_pk_bf16(x[2], x[3]);
          *reinterpret_cast<uint2*>(dq + d0) = w2;
        }
      }
    }
  }
}

// bf16: dK, dV of the active segment
// ---------------------------------------------------------------------------
// Workgroup = (KV head j, pair of 64-key segment tiles {kt, n-1-kt}, group of
// HPW query heads). Key tile kt receives gradient from query blocks kt..n-1,
// so the pair gives every workgroup the same work. 2*HPW waves: wave (g, ks)
// keeps K^T and V^T of its 32 keys (subtile ks) in registers as B operands and
// streams the 64-query tiles of head g: S = Q.K^T, dP = dO.V^T, then
// dV^T += dO^T.P and dK^T += Q^T.dS with Q^T / dO^T read transposed
// (ds_read_b64_tr_b16). Q/dO tiles (XOR-swizzled, so row reads and transposed
// reads are both conflict-free) and LSE/Dvec go straight from global memory
// into the other half of a double-buffered LDS stage (global_load_lds) while
// the current one is used, one copy instruction per S/dP k-step; LDS operands
// are read one k-step ahead of their MFMAs. Head partials are summed in LDS; with more than one head group per
// KV head each workgroup writes an fp32 partial that dkdv_reduce_kernel sums
// in a fixed order.
template <int D, int HPW, bool EXT>
__global__ __launch_bounds__(128 * HPW) void attn_bwd_dkdv_bf16_kernel(BwdParams p) {
  constexpr int NT = 128 * HPW;
  constexpr int NDT = D / 32;
  constexpr int NKS = D / 16;
  constexpr int TILE = kTile * D;     // swizzled Q / dO tile (Swz<D>)
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][HPW][2][TILE];  // [buf][head][Q, dO]
  __shared__ __attribute__((aligned(16))) float lse_s[2][HPW][kTile];       // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float dvec_s[2][HPW][kTile];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int l32 = lane % 32, hh = lane / 32;
  const int ks = wave % 2;       // 32-key subtile
  const uint32_t wave_u = static_cast<uint32_t>(wave);
  const int g = wave / 2;        // head within the group
  const int n_blocks = p.seg_len / kBlockQ;
  const int n_hg = p.r / HPW;
  int w = blockIdx.x;
  const int j = w % p.n_kv;
  w /= p.n_kv;
  const int hg = w % n_hg;
  const int pair = w / n_hg;
  const float c2 = p.scale_log2;

  const uint16_t* kseg = static_cast<const uint16_t*>(p.k_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const uint16_t* vseg = static_cast<const uint16_t*>(p.v_seg) + static_cast<int64_t>(j) * p.seg_len * D;
  const uint16_t* qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* gg = static_cast<const uint16_t*>(p.d_o);

  // Copies of query block qb (Q and dO tiles of the HPW heads, LSE, Dvec) into
  // LDS stage buf, as NDMA single wave instructions: copy k (0 <= k < NDMA)
  // is instruction k % IPT of tile k / IPT (tile = head * 2 + {Q, dO}); LSE
  // and Dvec ride with copy 0.
  constexpr int IPT = tile_lds_instrs<D, NT>();
  constexpr int NDMA = 2 * HPW * IPT;
  static_assert(NDMA <= 2 * NKS, "one copy per S/dP k-step");
  auto issue_copy = [&](int qb, int buf, int k) {
    const int tile = k / IPT, h = tile / 2;
    const int64_t row0 = static_cast<int64_t>(j * p.r + hg * HPW + h) * p.seg_len + qb * kBlockQ;
    tile_copy_rows_part<D, NT>(smem[buf][h][tile % 2], wave_u, lane, (tile % 2 ? gg : qg) + row0 * D, k % IPT);
    if (k == 0) {
#pragma unroll
      for (int hh2 = 0; hh2 < HPW; ++hh2) {
        const int64_t r0 = static_cast<int64_t>(j * p.r + hg * HPW + hh2) * p.seg_len + qb * kBlockQ;
        if (wave == 0) row64_load_lds(lse_s[buf][hh2], p.lse2 + r0, lane);
        if (wave == 1) row64_load_lds(dvec_s[buf][hh2], p.dvec + r0, lane);
      }
    }
  };
  auto issue_block = [&](int qb, int buf) {
#pragma unroll
    for (int k = 0; k < NDMA; ++k) issue_copy(qb, buf, k);
  };

  for (int half = 0; half < 2; ++half) {
    const int kt = half == 0 ? pair : n_blocks - 1 - pair;
    if (half == 1 && kt <= pair) break;  // odd count: the middle tile runs once
    const int key_local = ks * 32 + l32;
    const int key_tok = kt * kTile + key_local;
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

    // query blocks that attend this key tile: kt .. q_end-1 (a key k is seen
    // by queries k .. k+W-1)
    const int q_last = (kt * kTile + kTile - 2 + p.window) / kBlockQ;
    const int q_end = EXT && q_last + 1 < n_blocks ? q_last + 1 : n_blocks;
    __syncthreads();  // previous key tile's readers of smem are done
    issue_block(kt, 0);
    wait_vmem();
    __syncthreads();
    for (int qb = kt; qb < q_end; ++qb) {
      const int cur = (qb - kt) & 1;
      const bool more = qb + 1 < q_end;
      const uint16_t* Qs = smem[cur][g][0];
      const uint16_t* Gs = smem[cur][g][1];
      const float* lse_b = lse_s[cur][g];
      const float* dvec_b = dvec_s[cur][g];
      // causal diagonal or keys that fall out of some query's local window
      const bool edge = qb == kt || (EXT && (qb - kt) * kBlockQ + kBlockQ - 1 >= p.window);
      const int qk0 = (qb - kt) * kBlockQ - key_local;  // query - key offset, plus the row
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {  // 32-query halves of the tile
        f32x16 sacc, pacc;
#pragma unroll
        for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; pacc[v] = 0.f; }
        bf16x8 qa = lds_a_row_swz<D>(Qs, qs * 32, 0, lane);
        bf16x8 ga = lds_a_row_swz<D>(Gs, qs * 32, 0, lane);
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          bf16x8 qn = qa, gn = ga;
          if (s + 1 < NKS) {
            qn = lds_a_row_swz<D>(Qs, qs * 32, (s + 1) * 16, lane);
            gn = lds_a_row_swz<D>(Gs, qs * 32, (s + 1) * 16, lane);
          }
          if (more && qs * NKS + s < NDMA) issue_copy(qb + 1, cur ^ 1, qs * NKS + s);
          sacc = mfma32(qa, kreg[s], sacc);
          pacc = mfma32(ga, vreg[s], pacc);
          qa = qn;
          ga = gn;
          __builtin_amdgcn_sched_barrier(0);
        }
        // rows of the accumulators: queries qs*32 + 8*(v/4) + 4*hh + v%4
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int q0 = qs * 32 + 8 * r4 + 4 * hh;
          const float4 l4 = *reinterpret_cast<const float4*>(&lse_b[q0]);
          const float4 d4 = *reinterpret_cast<const float4*>(&dvec_b[q0]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
          if (edge) {  // keep 0 <= query - key < W
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 4 * r4 + e;
              const int dqk = qk0 + q0 + e;
              const float pr = dqk < 0 || (EXT && dqk >= p.window) ? 0.f : fast_exp2(fmaf(sacc[v], c2, -lv[e]));
              sacc[v] = pr;
              pacc[v] = pr * (pacc[v] - dvv[e]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 4 * r4 + e;
              const float pr = fast_exp2(fmaf(sacc[v], c2, -lv[e]));
              sacc[v] = pr;
              pacc[v] = pr * (pacc[v] - dvv[e]);
            }
          }
        }
        const bf16x8 p0 = acc_to_bf16x8(sacc, 0), p1 = acc_to_bf16x8(sacc, 8);
        const bf16x8 d0 = acc_to_bf16x8(pacc, 0), d1 = acc_to_bf16x8(pacc, 8);
        bf16x8 a[4], an[4];
        a[0] = lds_a_tr_swz<D>(Gs, qs * 32, 0, lane);
        a[1] = lds_a_tr_swz<D>(Gs, qs * 32 + 16, 0, lane);
        a[2] = lds_a_tr_swz<D>(Qs, qs * 32, 0, lane);
        a[3] = lds_a_tr_swz<D>(Qs, qs * 32 + 16, 0, lane);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          if (dt + 1 < NDT) {
            an[0] = lds_a_tr_swz<D>(Gs, qs * 32, (dt + 1) * 32, lane);
            an[1] = lds_a_tr_swz<D>(Gs, qs * 32 + 16, (dt + 1) * 32, lane);
            an[2] = lds_a_tr_swz<D>(Qs, qs * 32, (dt + 1) * 32, lane);
            an[3] = lds_a_tr_swz<D>(Qs, qs * 32 + 16, (dt + 1) * 32, lane);
          }
          dv[dt] = mfma32(a[0], p0, dv[dt]);
          dv[dt] = mfma32(a[1], p1, dv[dt]);
          dk[dt] = mfma32(a[2], d0, dk[dt]);
          dk[dt] = mfma32(a[3], d1, dk[dt]);
          if (dt + 1 < NDT) {
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = an[u];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_vmem();
      __syncthreads();
    }

    // ---- sum over the heads of the group (fixed order), then write ----------
    // exchange layout [slot][4-float column][lane][4]: b128 accesses of a wave
    // cover 1 KiB contiguously (no bank conflicts)
    float* xch = reinterpret_cast<float*>(&smem[0][0][0][0]);  // free after the last barrier
    constexpr int XW = NDT * 32;            // floats per lane: dK then dV
    auto xaddr = [&](int slot, int idx) -> float* {
      return xch + ((static_cast<int64_t>(slot) * (XW / 4) + idx / 4) * kWave + lane) * 4;
    };
    if (HPW > 1) {
      if (g > 0) {
        const int slot = (g - 1) * 2 + ks;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int v = 0; v < 16; v += 4) {
            *reinterpret_cast<float4*>(xaddr(slot, dt * 32 + v)) =
                make_float4(dk[dt][v], dk[dt][v + 1], dk[dt][v + 2], dk[dt][v + 3]);
            *reinterpret_cast<float4*>(xaddr(slot, dt * 32 + 16 + v)) =
                make_float4(dv[dt][v], dv[dt][v + 1], dv[dt][v + 2], dv[dt][v + 3]);
          }
      }
      __syncthreads();
      if (g == 0) {
        for (int h = 1; h < HPW; ++h) {
          const int slot = (h - 1) * 2 + ks;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int v = 0; v < 16; v += 4) {
              const float4 a = *reinterpret_cast<const float4*>(xaddr(slot, dt * 32 + v));
              const float4 c = *reinterpret_cast<const float4*>(xaddr(slot, dt * 32 + 16 + v));
              dk[dt][v] += a.x; dk[dt][v + 1] += a.y; dk[dt][v + 2] += a.z; dk[dt][v + 3] += a.w;
              dv[dt][v] += c.x; dv[dt][v + 1] += c.y; dv[dt][v + 2] += c.z; dv[dt][v + 3] += c.w;
            }
        }
      }
    }
    if (g == 0) {
      // accumulator rows: d = dt*32 + 8*(v/4) + 4*hh + v%4 ; column: this lane's key
      if (n_hg == 1) {
        uint16_t* dkp = static_cast<uint16_t*>(p.dk) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D;
        uint16_t* dvp = static_cast<uint16_t*>(p.dv) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = dt * 32 + 8 * r4 + 4 * hh;
            uint2 a, c;
            a.x = cvt_pk_bf16(dk[dt][4 * r4 + 0] * p.scale, dk[dt][4 * r4 + 1] * p.scale);
            a.y = cvt_pk_bf16(dk[dt][4 * r4 + 2] * p.scale, dk[dt][4 * r4 + 3] * p.scale);
            c.x = cvt_pk_bf16(dv[dt][4 * r4 + 0], dv[dt][4 * r4 + 1]);
            c.y = cvt_pk_bf16(dv[dt][4 * r4 + 2], dv[dt][4 * r4 + 3]);
            *reinterpret_cast<uint2*>(dkp + d0) = a;
            *reinterpret_cast<uint2*>(dvp + d0) = c;
          }
        }
      } else {
        const int64_t slot = static_cast<int64_t>(p.n_kv) * p.seg_len * D;
        float* pk = p.dkdv_part + (static_cast<int64_t>(hg) * 2) * slot +
                    (static_cast<int64_t>(j) * p.seg_len + key_tok) * D;
        float* pv = pk + slot;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = dt * 32 + 8 * r4 + 4 * hh;
            *reinterpret_cast<float4*>(pk + d0) =
                make_float4(dk[dt][4 * r4], dk[dt][4 * r4 + 1], dk[dt][4 * r4 + 2], dk[dt][4 * r4 + 3]);
            *reinterpret_cast<float4*>(pv + d0) =
                make_float4(dv[dt][4 * r4], dv[dt][4 * r4 + 1], dv[dt][4 * r4 + 2], dv[dt][4 * r4 + 3]);
          }
        }
      }
    }
  }
}

// dK = scale * sum_h partial_h, dV = sum_h partial_h, summed in head-group order.
// Eight elements per thread: every partial's two 16-byte loads are issued
// before the adds.
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* __restrict__ part, int n_hg,
                                                          int64_t n_elem, float scale,
                                                          uint16_t* __restrict__ dk,
                                                          uint16_t* __restrict__ dv) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= n_elem) return;
  float4 sk0 = *reinterpret_cast<const float4*>(part + i);
  float4 sk1 = *reinterpret_cast<const float4*>(part + i + 4);
  float4 sv0 = *reinterpret_cast<const float4*>(part + n_elem + i);
  float4 sv1 = *reinterpret_cast<const float4*>(part + n_elem + i + 4);
  for (int h = 1; h < n_hg; ++h) {
    const float* pk = part + (2 * h) * n_elem + i;
    const float* pv = part + (2 * h + 1) * n_elem + i;
    const float4 a0 = *reinterpret_cast<const float4*>(pk), a1 = *reinterpret_cast<const float4*>(pk + 4);
    const float4 b0 = *reinterpret_cast<const float4*>(pv), b1 = *reinterpret_cast<const float4*>(pv + 4);
    sk0.x += a0.x; sk0.y += a0.y; sk0.z += a0.z; sk0.w += a0.w;
    sk1.x += a1.x; sk1.y += a1.y; sk1.z += a1.z; sk1.w += a1.w;
    sv0.x += b0.x; sv0.y += b0.y; sv0.z += b0.z; sv0.w += b0.w;
    sv1.x += b1.x; sv1.y += b1.y; sv1.z += b1.z; sv1.w += b1.w;
  }
  uint2* ok = reinterpret_cast<uint2*>(dk + i);   // 8-byte stores: dK/dV need 8-byte alignment only
  uint2* ov = reinterpret_cast<uint2*>(dv + i);
  ok[0] = make_uint2(cvt_pk_bf16(sk0.x * scale, sk0.y * scale), cvt_pk_bf16(sk0.z * scale, sk0.w * scale));
  ok[1] = make_uint2(cvt_pk_bf16(sk1.x * scale, sk1.y * scale), cvt_pk_bf16(sk1.z * scale, sk1.w * scale));
  ov[0] = make_uint2(cvt_pk_bf16(sv0.x, sv0.y), cvt_pk_bf16(sv0.z, sv0.w));
  ov[1] = make_uint2(cvt_pk_bf16(sv1.x, sv1.y), cvt_pk_bf16(sv1.z, sv1.w));
}

// ---------------------------------------------------------------------------
// fp32 VALU kernels
// ---------------------------------------------------------------------------
// fp32 dQ: one wave per (block, head), one thread per query row; the query
// and dO rows live in LDS (each thread's own padded row), dQ in registers.
template <int D>
__global__ __launch_bounds__(kWave) void attn_bwd_dq_f32_kernel(BwdParams p) {
  __shared__ float Kt[kTile][D + 1];
  __shared__ float Vt[kTile][D + 1];
  __shared__ float Qs[kWave][D + 1];
  __shared__ float Gs[kWave][D + 1];
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
  for (int i = a; i < p.k_g; i += kWave) sel_s[i] = staged_group(p, b, i, sel_bj[i]);
  {
    const int64_t row0 = row - a;
    const float* qb = static_cast<const float*>(p.q) + row0 * D;
    const float* gb = static_cast<const float*>(p.d_o) + row0 * D;
    for (int x = a; x < kWave * D; x += kWave) {
      Qs[x / D][x % D] = qb[x];
      Gs[x / D][x % D] = gb[x];
    }
  }
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  const float lse2 = p.lse[row] * kLog2e;
  const float dr = p.dvec[row];
  const int n_hist_tiles = (p.k_g + 7) / 8;
  const int n_sink = p.n_sink_tiles;
  const int seg_t0 = seg_first_tile<true>(b, p.window);
  const int q_tok = b * kBlockQ + a;
  __syncthreads();
  for (int tile = 0; tile < n_sink + n_hist_tiles + b - seg_t0 + 1; ++tile) {
    const bool is_sink = tile < n_sink;
    const bool is_hist = !is_sink && tile < n_sink + n_hist_tiles;
    const int ht = tile - n_sink;
    const int st = seg_t0 + tile - n_sink - n_hist_tiles;
    for (int kk = 0; kk < kTile; ++kk) {
      int64_t off;
      if (is_sink) off = (static_cast<int64_t>(j) * p.sink_stride + tile * kTile + kk) * D;
      else if (is_hist) off = hist_offset(p, sel_s, j, ht, kk, D);
      else off = static_cast<int64_t>(st * kTile + kk) * D;
      const float* kb = is_sink ? static_cast<const float*>(p.k_sink) : is_hist ? kh : ks_g;
      const float* vb = is_sink ? static_cast<const float*>(p.v_sink) : is_hist ? vh : vs_g;
      for (int e = a; e < D; e += kWave) {
        Kt[kk][e] = off >= 0 ? kb[off + e] : 0.f;
        Vt[kk][e] = off >= 0 ? vb[off + e] : 0.f;
      }
    }
    __syncthreads();
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
      if (!valid) continue;
      float s = 0.f, dp = 0.f;
      for (int e = 0; e < D; ++e) {
        s += Qs[a][e] * Kt[kk][e];
        dp += Gs[a][e] * Vt[kk][e];
      }
      const float pr = exp2f(s * p.scale_log2 - lse2);
      const float ds = pr * (dp - dr);
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] += ds * Kt[kk][e];
    }
    __syncthreads();
  }
  float* dq = static_cast<float*>(p.dq) + row * D;
#pragma unroll
  for (int e = 0; e < D; ++e) dq[e] = acc[e] * p.scale;
}

// fp32 dK/dV: one workgroup of two waves per (64-key segment tile, KV head),
// one key per lane; wave h accumulates dimensions [h*D/2, (h+1)*D/2) of dK and
// dV (both waves form the full scores). The keys' K and V rows live in LDS
// (each lane's own padded row).
template <int D>
__global__ __launch_bounds__(2 * kWave) void attn_bwd_dkdv_f32_kernel(BwdParams p) {
  constexpr int DH = D / 2;
  __shared__ float Qt[kTile][D + 1];
  __shared__ float Gt[kTile][D + 1];
  __shared__ float Ks[kTile][D + 1];
  __shared__ float Vs[kTile][D + 1];
  __shared__ float lse_s[kTile];
  __shared__ float dvec_s[kTile];
  const int t = threadIdx.x, a = t % kWave, h = t / kWave;  // key within the tile, dimension half
  const int n_blocks = p.seg_len / kBlockQ;
  const int j = blockIdx.x % p.n_kv;
  const int kt_blk = blockIdx.x / p.n_kv;
  const int key_tok = kt_blk * kTile + a;
  {
    const float* kb = static_cast<const float*>(p.k_seg) + (static_cast<int64_t>(j) * p.seg_len + kt_blk * kTile) * D;
    const float* vb = static_cast<const float*>(p.v_seg) + (static_cast<int64_t>(j) * p.seg_len + kt_blk * kTile) * D;
    for (int x = t; x < kTile * D; x += 2 * kWave) {
      Ks[x / D][x % D] = kb[x];
      Vs[x / D][x % D] = vb[x];
    }
  }
  float dk[DH], dv[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) { dk[e] = 0.f; dv[e] = 0.f; }
  const int q_last = (kt_blk * kTile + kTile - 2 + p.window) / kBlockQ;
  const int q_end = q_last + 1 < n_blocks ? q_last + 1 : n_blocks;
  for (int qb = kt_blk; qb < q_end; ++qb) {
    for (int hi = 0; hi < p.r; ++hi) {
      const int64_t row0 = static_cast<int64_t>(j * p.r + hi) * p.seg_len + qb * kBlockQ;
      __syncthreads();
      for (int x = t; x < kTile * D; x += 2 * kWave) {
        Qt[x / D][x % D] = static_cast<const float*>(p.q)[row0 * D + x];
        Gt[x / D][x % D] = static_cast<const float*>(p.d_o)[row0 * D + x];
      }
      if (h == 0) {
        lse_s[a] = p.lse[row0 + a] * kLog2e;
        dvec_s[a] = p.dvec[row0 + a];
      }
      __syncthreads();
      for (int qq = 0; qq < kTile; ++qq) {
        const int dqk = qb * kBlockQ + qq - key_tok;
        if (dqk < 0 || dqk >= p.window) continue;  // key after the query or out of its window
        float s = 0.f, dp = 0.f;
        for (int e = 0; e < D; ++e) {
          s += Qt[qq][e] * Ks[a][e];
          dp += Gt[qq][e] * Vs[a][e];
        }
        const float pr = exp2f(s * p.scale_log2 - lse_s[qq]);
        const float ds = pr * (dp - dvec_s[qq]);
#pragma unroll
        for (int e = 0; e < DH; ++e) {
          dv[e] += pr * Gt[qq][h * DH + e];
          dk[e] += ds * Qt[qq][h * DH + e];
        }
      }
    }
  }
  float* dkp = static_cast<float*>(p.dk) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D + h * DH;
  float* dvp = static_cast<float*>(p.dv) + (static_cast<int64_t>(j) * p.seg_len + key_tok) * D + h * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) { dkp[e] = dk[e] * p.scale; dvp[e] = dv[e]; }
}

template <int D>
hipError_t launch_d(const hga_shape& s, BwdParams& p, hipStream_t st) {
  const int n_blocks = s.seg_len / kBlockQ;
  const int64_t n_rows = static_cast<int64_t>(s.n_q_heads) * s.seg_len;
  constexpr int RPB = 256 / (D / 8);
  const unsigned dot_grid = static_cast<unsigned>((n_rows + RPB - 1) / RPB);
  hipEvent_t dq0 = timer_event(HGA_KERNEL_BWD_DQ, 0), dq1 = timer_event(HGA_KERNEL_BWD_DQ, 1);
  hipEvent_t kv0 = timer_event(HGA_KERNEL_BWD_DKDV, 0), kv1 = timer_event(HGA_KERNEL_BWD_DKDV, 1);
  if (s.dtype == HGA_F32) {
    hipExtLaunchKernelGGL((row_dot_kernel<float, D>), dim3(dot_grid), dim3(256), 0, st, dq0, nullptr, 0,
                          static_cast<const float*>(p.o), static_cast<const float*>(p.d_o), p.dvec, n_rows);
    hipExtLaunchKernelGGL((attn_bwd_dq_f32_kernel<D>), dim3(n_blocks * s.n_q_heads), dim3(kWave), 0, st,
                          nullptr, dq1, 0, p);
    hipExtLaunchKernelGGL((attn_bwd_dkdv_f32_kernel<D>), dim3(n_blocks * s.n_kv_heads), dim3(2 * kWave), 0, st,
                          kv0, kv1, 0, p);
  } else {
    const int n_pairs = (n_blocks + 1) / 2;
    // sink or local window: the extended kernels; otherwise the plain ones
    const bool ext = p.window < s.seg_len || p.n_sink_tiles > 0;
    if (p.r % 2 == 0) {
      const dim3 g2(n_pairs * s.n_kv_heads * (p.r / 2));
      if (ext) hipExtLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, 2, true>), g2, dim3(512), 0, st, dq0, dq1, 0, p);
      else hipExtLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, 2, false>), g2, dim3(512), 0, st, dq0, dq1, 0, p);
    } else {
      const dim3 g1(n_pairs * s.n_kv_heads * p.r);
      if (ext) hipExtLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, 1, true>), g1, dim3(256), 0, st, dq0, dq1, 0, p);
      else hipExtLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, 1, false>), g1, dim3(256), 0, st, dq0, dq1, 0, p);
    }
    const int hpw = p.r % 2 == 0 ? 2 : 1;
    const int n_hg = p.r / hpw;
    const unsigned grid = static_cast<unsigned>(n_pairs * s.n_kv_heads * n_hg);
    // the fixed-order partial sum, when there is one, ends the dK/dV span
    hipEvent_t kv_end = n_hg > 1 ? nullptr : kv1;
    if (hpw == 2) {
      if (ext) hipExtLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, 2, true>), dim3(grid), dim3(256), 0, st, kv0, kv_end, 0, p);
      else hipExtLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, 2, false>), dim3(grid), dim3(256), 0, st, kv0, kv_end, 0, p);
    } else {
      if (ext) hipExtLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, 1, true>), dim3(grid), dim3(128), 0, st, kv0, kv_end, 0, p);
      else hipExtLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, 1, false>), dim3(grid), dim3(128), 0, st, kv0, kv_end, 0, p);
    }
    if (n_hg > 1) {
      const int64_t n_elem = static_cast<int64_t>(s.n_kv_heads) * s.seg_len * D;
      hipExtLaunchKernelGGL(dkdv_reduce_kernel, dim3(static_cast<unsigned>((n_elem / 8 + 255) / 256)),
                            dim3(256), 0, st, nullptr, kv1, 0, p.dkdv_part, n_hg, n_elem, p.scale,
                            static_cast<uint16_t*>(p.dk), static_cast<uint16_t*>(p.dv));
    }
  }
  return hipGetLastError();
}

}  // namespace

// Dvec [n_q][S] fp32, LSE*log2(e) [n_q][S] fp32, then (bf16, more than one
// head group per KV head) the dK/dV partials [n_hg][2][n_kv][S][D] fp32.
size_t bwd_workspace_bytes(const hga_shape& s) {
  const size_t row = ((sizeof(float) * static_cast<size_t>(s.n_q_heads) * s.seg_len) + 255) & ~size_t(255);
  const int r = s.n_q_heads / s.n_kv_heads;
  const int n_hg = r / (r % 2 == 0 ? 2 : 1);
  if (s.dtype != HGA_BF16 || n_hg <= 1) return 2 * row;
  return 2 * row + sizeof(float) * static_cast<size_t>(n_hg) * 2 * s.n_kv_heads * s.seg_len * s.head_dim;
}

hipError_t launch_attn_bwd(const hga_shape& s, const void* q, const void* k_hist,
                           const void* v_hist, const void* k_seg, const void* v_seg,
                           const int32_t* sel_groups, const void* o, const float* lse,
                           const void* d_o, void* dq, void* dk_seg, void* dv_seg, void* ws,
                           hipStream_t stream, const StagedHistory* staged) {
  BwdParams p;
  p.q = q; p.k_hist = k_hist; p.v_hist = v_hist; p.k_seg = k_seg; p.v_seg = v_seg;
  p.sel = sel_groups; p.o = o; p.lse = lse; p.d_o = d_o;
  p.dq = dq; p.dk = dk_seg; p.dv = dv_seg;
  const size_t row = ((sizeof(float) * static_cast<size_t>(s.n_q_heads) * s.seg_len) + 255) & ~size_t(255);
  p.dvec = static_cast<float*>(ws);
  p.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + row);
  p.dkdv_part = reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * row);
  p.n_q = s.n_q_heads; p.n_kv = s.n_kv_heads; p.r = s.n_q_heads / s.n_kv_heads;
  p.seg_len = s.seg_len; p.hist_len = s.hist_len; p.hist_rows = hist_rows(s); p.k_g = s.top_k_groups;
  p.staged = 0;
  p.k_sink = k_hist; p.v_sink = v_hist; p.sink_stride = hist_rows(s);
  if (staged) {
    p.staged = 1;
    p.k_hist = staged->k_rows; p.v_hist = staged->v_rows;
    p.hist_rows = static_cast<int64_t>(s.top_k_groups) * kGroup;
    p.k_sink = staged->k_sink; p.v_sink = staged->v_sink; p.sink_stride = staged->sink_stride;
  }
  p.n_sink_tiles = sink_chunks(s);
  p.window = local_window(s);
  p.scale = s.softmax_scale;
  p.scale_log2 = s.softmax_scale * kLog2e;
  return s.head_dim == 128 ? launch_d<128>(s, p, stream) : launch_d<64>(s, p, stream);
}

}  // namespace hga
