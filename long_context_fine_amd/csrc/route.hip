// Two-level content routing, one workgroup per (query block b, KV head j),
// the KV head the fastest grid index (a head's workgroups share one XCD's L2):
//   1. block query qbar = mean of the block's 64 queries over the r heads of j
//      (reads its 64 KiB of Q once, 16-byte loads);
//   2. chunk scores qbar . C[j][m] for every ranked history chunk (8 lanes per
//      512-byte row, whole 128-byte lines per load instruction, the next rows
//      in flight while the current ones are reduced);
//   3. chunk top-k by exact radix select over order-preserving 32-bit score
//      keys (8-bit digit histograms in LDS, most significant digit first),
//      ties at the threshold key going to the lowest index, then the kept
//      chunks in ascending order;
//   4. scores of the 8 groups of every kept chunk (reads 8*k_c rows of G);
//   5. group top-k by rank counting over 64-bit keys (score key, then the
//      complemented index, so larger means better and lower index); the
//      candidates are enumerated in ascending group id, so ballot prefix
//      counts place the output in ascending order.
// HBM/latency bound. Deterministic: the only atomics are integer adds into
// LDS histograms and counters, whose results do not depend on their order.
//
// With group summaries in host memory (the group-summary cache) the same
// kernel runs in two halves around gcache_update_kernel: phases 1-3 (and q-bar
// kept in the workspace), then the cache update for all blocks of a KV head,
// then phases 4-5 reading group rows from the cache slots. For a decode batch
// it runs with one sequence per workgroup row (decode mode).
#include "hga_common.hpp"

namespace hga {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsScores = 4096;  // chunk scores kept in LDS up to this many chunks

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Dot products of qv with `n` rows (row length D floats, row_ptr(i) gives row
// i), 8 lanes per row, 8 rows per wave pass; results to out[row]. Load c of
// lane sub reads floats [32c + 4 sub, 32c + 4 sub + 4): the 8 lanes of a row
// read one whole 128-byte line per instruction. Software-pipelined: the loads
// of the next UNROLL passes are in flight while the current ones are reduced;
// rows past n re-read row n-1 (branch-free) and are not written.
template <int D, int UNROLL, class RowPtr>
__device__ __forceinline__ void score_rows(const float* qv, int n, RowPtr row_ptr, float* out) {
  constexpr int LPR = 8;                 // lanes per row
  constexpr int EPL = D / LPR;           // elements per lane (16 or 8)
  constexpr int RPP = kWave / LPR;       // rows per wave pass
  constexpr int NW = kThreads / kWave;
  constexpr int STEP = NW * RPP * UNROLL;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  static_assert(LPR == 8, "sum8_f32 reduces groups of 8 lanes");
  const int sub = lane % LPR;
  float qr[EPL];
#pragma unroll
  for (int c = 0; c < EPL / 4; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) qr[4 * c + e] = qv[c * 4 * LPR + sub * 4 + e];
  using Buf = float4[UNROLL][EPL / 4];
  auto load = [&](int r0, Buf& v) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int row = min(r0 + u * NW * RPP + lane / LPR, n - 1);
      const float4* src = reinterpret_cast<const float4*>(row_ptr(row) + sub * 4);
#pragma unroll
      for (int c = 0; c < EPL / 4; ++c) v[u][c] = src[c * LPR];
    }
  };
  auto reduce = [&](int r0, const Buf& v) {
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
  };
  Buf va, vb;
  int r0 = wave * RPP;
  if (r0 < n) load(r0, va);
  while (r0 < n) {
    if (r0 + STEP < n) load(r0 + STEP, vb);
    reduce(r0, va);
    r0 += STEP;
    if (r0 >= n) break;
    if (r0 + STEP < n) load(r0 + STEP, va);
    reduce(r0, vb);
    r0 += STEP;
  }
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

// Exclusive prefix sum of v over a workgroup of NT threads in thread order;
// *total gets the sum. wsum: NT/64 + 1 ints of LDS. Contains barriers: every
// thread must call it. Without the trailing barrier the caller must pass
// another barrier before wsum is written again.
template <int NT, bool kTrailingBarrier = true>
__device__ int block_scan_excl(int v, int* total, int32_t* wsum) {
  constexpr int NWV = NT / kWave;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int inc = wave_incl_scan(v, lane);
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < NWV ? wsum[lane] : 0;
    const int wi = wave_incl_scan(w, lane);
    if (lane < NWV) wsum[lane] = wi - w;
    if (lane == NWV - 1) wsum[NWV] = wi;
  }
  __syncthreads();
  const int r = wsum[wave] + inc - v;
  *total = wsum[NWV];
  if (kTrailingBarrier) __syncthreads();
  return r;
}

// Radix select of the need-th largest order-preserving key among sc[0, n)
// (1 <= need <= n; need = 0 selects nothing): 8-bit digits, most significant
// first, one LDS histogram (256 bins, one per thread) per pass. Histograms and
// selections alternate between two buffers by pass, so a pass needs four
// barriers: counts done, two in the scan, selection. The digits below bit
// last_shift are left open. Every thread returns the same result:
//   whole:  the keys k with (k & pmask) >= prefix are exactly the need
//           largest (the threshold bin is taken whole);
//   exact:  the need-th largest key equals prefix (all 32 bits fixed) and
//           `need` of the keys equal to prefix are still to be taken;
//   neither (last_shift > 0): the need-th largest key has prefix under pmask,
//           so it lies in [prefix, prefix | ~pmask].
struct RadixSel {
  uint32_t prefix, pmask;
  int need;
  bool exact, whole;
};

__device__ RadixSel radix_select(const float* sc, int n, int need, int32_t (*hist_s)[kThreads],
                                 int32_t (*rsel)[3], int32_t* scan_ws, int last_shift = 0) {
  static_assert(kThreads == 256, "one histogram bin per thread");
  const int t = threadIdx.x;
  RadixSel rs{0u, 0u, need, false, false};
  hist_s[0][t] = 0;
  __syncthreads();
  int hb = 0;
  for (int shift = 24; shift >= last_shift && need > 0; shift -= 8, hb ^= 1) {
    for (int m = t; m < n; m += kThreads) {
      const uint32_t k = score_key(sc[m]);
      if ((k & rs.pmask) == rs.prefix) atomicAdd(&hist_s[hb][(k >> shift) & 255u], 1);
    }
    __syncthreads();
    const int bin = kThreads - 1 - t;           // thread order = bins descending
    const int h = hist_s[hb][bin];
    hist_s[hb ^ 1][t] = 0;                      // the next pass's histogram
    int total;
    const int at_or_above = block_scan_excl<kThreads, false>(h, &total, scan_ws) + h;
    if (at_or_above >= rs.need && at_or_above - h < rs.need) {
      rsel[hb][0] = bin;
      rsel[hb][1] = at_or_above - h;
      rsel[hb][2] = h;
    }
    __syncthreads();
    rs.prefix |= static_cast<uint32_t>(rsel[hb][0]) << shift;
    rs.pmask |= 255u << shift;
    rs.need -= rsel[hb][1];
    if (rsel[hb][2] == rs.need) {               // the whole bin is kept
      rs.whole = true;
      break;
    }
    if (shift == 0) rs.exact = true;
  }
  return rs;
}

// Top-k of n 64-bit rank keys gkey[0, n) by rank counting (0 marks an empty
// slot; gkey[n] must be readable and 0): candidate c is taken when fewer than
// k keys exceed its own. One ballot word per 64 candidates into wmask, so the
// taken candidates keep their order (ordered_pos). Every thread must call it;
// the caller passes a barrier before reading wmask.
__device__ __forceinline__ void rank_take_mask(const uint64_t* gkey, int n, int k, uint64_t* wmask) {
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(gkey);
  for (int cb = 0; cb < n; cb += kThreads) {
    const int c = cb + t;
    bool take = false;
    if (c < n) {
      const uint64_t mine = gkey[c];
      if (mine != 0ull) {
        int beaten = 0;
#pragma unroll 4
        for (int o2 = 0; o2 < (n + 1) / 2; ++o2) {
          const ulonglong2 x = k2[o2];
          beaten += (x.x > mine) + (x.y > mine);
        }
        take = beaten < k;
      }
    }
    const uint64_t m = __ballot(take);
    if (lane == 0) wmask[cb / kWave + wave] = m;
  }
}

__device__ __forceinline__ bool mask_taken(const uint64_t* wmask, int c) {
  return (wmask[c / kWave] >> (c % kWave)) & 1ull;
}
// Output position of taken candidate c: the taken candidates before it.
__device__ __forceinline__ int ordered_pos(const uint64_t* wmask, int c) {
  int pos = __popcll(wmask[c / kWave] & ((1ull << (c % kWave)) - 1ull));
  for (int w2 = 0; w2 < c / kWave; ++w2) pos += __popcll(wmask[w2]);
  return pos;
}

// score_rows for rows of D bf16 values (row_ptr(i): the row's first element),
// loads of 16 bytes (lane sub reads elements [8(8c + sub), 8(8c + sub) + 8)),
// 8*UNROLL rows per wave in flight. Also returns, per thread, the largest
// sum over a row of |qv[e]| * |row[e]| among the rows it reduced, as raw bits
// with the sign cleared (a NaN compares above every number), and in *q1 the
// sum of |qv[e]| (the same bits in every lane).
template <int D, int UNROLL, class RowPtr>
__device__ __forceinline__ uint32_t score_rows_bf16(const float* qv, int n, RowPtr row_ptr, float* out,
                                                    float* q1) {
  constexpr int LPR = 8;                 // lanes per row
  constexpr int EPL = D / LPR;           // elements per lane (16 or 8)
  constexpr int VPL = EPL / 8;           // 16-byte loads per lane and row
  constexpr int RPP = kWave / LPR;       // rows per wave pass
  constexpr int NW = kThreads / kWave;
  constexpr int STEP = NW * RPP * UNROLL;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int sub = lane % LPR;
  float qr[EPL];
#pragma unroll
  for (int c = 0; c < VPL; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[8 * c + e] = qv[(c * LPR + sub) * 8 + e];
  {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a += fabsf(qr[e]);
    *q1 = sum8_f32(a);               // the 8 lanes of a row hold all of qv
  }
  using Buf = uint4[UNROLL][VPL];
  auto load = [&](int r0, Buf& v) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int row = min(r0 + u * NW * RPP + lane / LPR, n - 1);
      const uint4* src = reinterpret_cast<const uint4*>(row_ptr(row));
#pragma unroll
      for (int c = 0; c < VPL; ++c) v[u][c] = src[c * LPR + sub];
    }
  };
  uint32_t amax = 0u;
  auto reduce = [&](int r0, const Buf& v) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float s = 0.f, a = 0.f;
#pragma unroll
      for (int c = 0; c < VPL; ++c) {
        const uint32_t w[4] = {v[u][c].x, v[u][c].y, v[u][c].z, v[u][c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
          s += lo * qr[8 * c + 2 * i] + hi * qr[8 * c + 2 * i + 1];
          a += fabsf(lo) * fabsf(qr[8 * c + 2 * i]) + fabsf(hi) * fabsf(qr[8 * c + 2 * i + 1]);
        }
      }
      s = sum8_f32(s);
      a = sum8_f32(a);
      const int row = r0 + u * NW * RPP + lane / LPR;
      if (row < n && sub == 0) {
        out[row] = s;
        amax = max(amax, __float_as_uint(a) & 0x7fffffffu);
      }
    }
  };
  Buf va, vb;
  int r0 = wave * RPP;
  if (r0 < n) load(r0, va);
  while (r0 < n) {
    if (r0 + STEP < n) load(r0 + STEP, vb);
    reduce(r0, va);
    r0 += STEP;
    if (r0 >= n) break;
    if (r0 + STEP < n) load(r0 + STEP, va);
    reduce(r0, vb);
    r0 += STEP;
  }
  return amax;
}

// Inverse of score_key for the keys of finite scores.
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

enum RouteMode {
  kRouteFull = 0, kRouteChunks = 1, kRouteGroups = 2, kRouteDecode = 3,
  // decode with the chunk scan split over n_part workgroups per (sequence,
  // KV head): each ranks one contiguous part of the chunks and keeps its own
  // top k_c (with scores); a merge then keeps the top k_c of those candidates
  // and runs the group steps. Exact: every chunk of the overall top k_c is in
  // the top k_c of its part, under the same (score, lower index) order.
  kRouteDecodePart = 4, kRouteDecodeMerge = 5
};

// Decode: blockIdx.y is a sequence of the batch, the query block is its
// seg_len newest tokens (q [batch][n_q][seg_len][D]); summaries are
// [batch][n_kv][chunk_rows][D] and [batch][n_kv][8*chunk_rows][D]; the
// sequence's history length comes from hist_lens (clamped to the capacity,
// whole chunks).
struct DecodeView {
  const int32_t* hist_lens;
  int n_sink;
  int n_q;
  int n_part = 1;              // split decode: parts per (sequence, KV head)
  int32_t* cand_id = nullptr;  // [batch][n_kv][n_part][k_c] kept chunk ids (-1: none)
  float* cand_sc = nullptr;    // their scores
  // bf16 copies of the chunk summaries (layout of csum) for the two-pass
  // chunk route of the unsplit decode mode, or null: scores from these bound
  // the fp32 scores, and only the chunks that can reach the top k_c are
  // re-scored from csum
  const uint16_t* csum_lo = nullptr;
};

// Group rows of the cache: [n_kv][n_slots][8][D] fp32, slot of each chunk in
// slot_of_chunk[n_kv][chunk_rows] (-1: not cached).
struct CacheView {
  const int32_t* slot_of_chunk;
  const float* data;
  int n_slots;
};

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const T* __restrict__ q, const float* __restrict__ csum, const float* __restrict__ gsum,
    int seg_len, int n_kv, int r, int chunk0, int n_chunks, int chunk_rows, int k_c, int k_g,
    float* __restrict__ ws_scores,
    int32_t* __restrict__ sel_chunks, int32_t* __restrict__ sel_groups,
    float* __restrict__ ws_qbar, CacheView cache, DecodeView dec) {
  constexpr int TPR = D / 8;            // threads per Q row (8 elements each)
  constexpr int RG = kThreads / TPR;    // row groups
  constexpr int NW = kThreads / kWave;
  constexpr int kMaxCand = kMaxTopKChunks * (kChunk / kGroup);
  __shared__ float part[RG][D + 1];
  __shared__ float qv[D];
  __shared__ float sc_lds[kLdsScores];
  __shared__ int32_t hist_s[2][kThreads];    // radix-select digit histograms (256 bins), by pass parity
  __shared__ int32_t rsel[2][3];
  __shared__ int32_t scan_ws[NW + 1];
  __shared__ int32_t gtmp_s[kMaxTopKChunks];  // kept chunk ids before ordering
  __shared__ int32_t n_app;
  __shared__ int32_t sorted[kMaxTopKChunks];
  __shared__ float gsc[kMaxCand];
  __shared__ __attribute__((aligned(16))) uint64_t gkey[kMaxCand];
  __shared__ uint64_t wmask[kMaxCand / kWave];
  __shared__ int32_t cnt_s[kThreads / 2];
  __shared__ int32_t slot_s[kMaxTopKChunks];
  constexpr bool kTwoPass = MODE == kRouteDecode;
  __shared__ int32_t cidx_s[kTwoPass ? kMaxCand : 1];      // two-pass candidates (ascending)
  __shared__ uint32_t red_s[2];                             // two-pass: max |q||C~| bits, threshold key

  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  // KV head fastest: with 8 KV heads all workgroups of head j run on one XCD
  // (round-robin dispatch), whose L2 then holds that head's chunk summaries
  const int j = blockIdx.x, b = blockIdx.y;
  const int64_t bj = static_cast<int64_t>(b) * n_kv + j;
  constexpr bool kDec = MODE == kRouteDecode || MODE == kRouteDecodePart || MODE == kRouteDecodeMerge;
  if constexpr (kDec) {
    int hb = dec.hist_lens[b];
    hb = hb < 0 ? 0 : (hb > chunk_rows * kChunk ? chunk_rows * kChunk : hb);
    const int nc = hb / kChunk;
    chunk0 = dec.n_sink < nc ? dec.n_sink : nc;
    n_chunks = nc - chunk0;
    csum += static_cast<int64_t>(b) * n_kv * chunk_rows * D;
    gsum += static_cast<int64_t>(b) * n_kv * chunk_rows * (kChunk / kGroup) * D;
    if (dec.csum_lo != nullptr) dec.csum_lo += static_cast<int64_t>(b) * n_kv * chunk_rows * D;
    if constexpr (MODE == kRouteDecodePart) {  // this workgroup's part of the ranked chunks
      const int per = (n_chunks + dec.n_part - 1) / dec.n_part;
      const int lo = min(n_chunks, static_cast<int>(blockIdx.z) * per);
      chunk0 += lo;
      n_chunks = min(n_chunks - lo, per);
    }
  }

  // ---- 1. block query ----------------------------------------------------
  if constexpr (MODE == kRouteGroups || MODE == kRouteDecodeMerge) {
    if (t < D) qv[t] = ws_qbar[bj * D + t];
    __syncthreads();
  } else {
    const int dc = t % TPR, rg = t / TPR;
    const int rows = (kDec ? seg_len : kBlockQ) * r;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
    for (int row = rg; row < rows; row += RG) {
      int64_t qrow;
      if constexpr (kDec) {
        qrow = (static_cast<int64_t>(b) * dec.n_q + j * r + row / seg_len) * seg_len + row % seg_len;
      } else {
        const int h = j * r + row / kBlockQ, i = b * kBlockQ + row % kBlockQ;
        qrow = static_cast<int64_t>(h) * seg_len + i;
      }
      float v[8];
      Elem<T>::load8(q + qrow * D + dc * 8, v);
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
      if constexpr (MODE == kRouteChunks) ws_qbar[bj * D + t] = qv[t];
      if constexpr (MODE == kRouteDecodePart) {
        if (blockIdx.z == 0) ws_qbar[bj * D + t] = qv[t];
      }
    }
    __syncthreads();
  }

  int kc_eff;
  if constexpr (MODE == kRouteGroups) {
    // kept chunks (ascending, -1 padded) from the first half, with their slots
    const int c = t < k_c ? sel_chunks[bj * k_c + t] : -1;
    if (c >= 0) {
      sorted[t] = c;
      slot_s[t] = cache.slot_of_chunk[static_cast<int64_t>(j) * chunk_rows + c];
    }
    kc_eff = __syncthreads_count(c >= 0);
  } else if constexpr (MODE == kRouteDecodeMerge) {
    // ---- 3'. top k_c of the parts' candidates (ids ascending within a part,
    // parts in chunk order, so candidate order is chunk order): rank count
    // over 64-bit keys (score key, complemented id; 0 marks an empty slot)
    const int ncc = dec.n_part * k_c;          // host-checked: ncc < kMaxCand
    const int64_t c0 = bj * ncc;
    for (int c = t; c <= ncc; c += kThreads) {
      const int id = c < ncc ? dec.cand_id[c0 + c] : -1;
      gkey[c] = id >= 0 ? rank_key(dec.cand_sc[c0 + c], static_cast<uint32_t>(id)) : 0ull;
    }
    __syncthreads();
    rank_take_mask(gkey, ncc, k_c, wmask);
    __syncthreads();
    int total = 0;
    for (int w2 = 0; w2 < (ncc + kWave - 1) / kWave; ++w2) total += __popcll(wmask[w2]);
    kc_eff = total;
    for (int c = t; c < ncc; c += kThreads)
      if (mask_taken(wmask, c)) sorted[ordered_pos(wmask, c)] = dec.cand_id[c0 + c];
    __syncthreads();
    if (t < k_c) sel_chunks[bj * k_c + t] = t < kc_eff ? sorted[t] : -1;
  } else {
    float* sc = n_chunks <= kLdsScores ? sc_lds
                                       : ws_scores + bj * (kDec ? chunk_rows : n_chunks);
    // ranked chunks are chunk0 .. chunk0 + n_chunks - 1 (the sink is attended in full)
    const float* cbase = csum + (static_cast<int64_t>(j) * chunk_rows + chunk0) * D;
    bool done = false;
    if constexpr (kTwoPass) {
      // ---- 2-3 in two passes. Scores s~ from the bf16 copies C~ differ from
      // the fp32 scores s by at most e = 0.0045 * max_m sum|qbar||C~_m| (plus
      // 1e-30 * (1 + sum|qbar|) for subnormals): 2^-8 relative rounding of C~,
      // 128 * 2^-24 for either fp32 dot product, with room to spare. Every
      // chunk of the fp32 top k_c then has s~ >= tau - 2e, tau the k_c-th
      // largest s~; those candidates are re-scored from the fp32 summaries
      // (the same arithmetic as the one-pass scan) and their top k_c under
      // (score, lower index) is the one-pass selection. Non-finite or huge
      // values, or more candidates than fit, fall back to the one-pass scan.
      if (dec.csum_lo != nullptr && n_chunks > k_c) {
        if (t == 0) {
          red_s[0] = 0u;
          red_s[1] = 0xffffffffu;
        }
        __syncthreads();
        const uint16_t* lbase = dec.csum_lo + (static_cast<int64_t>(j) * chunk_rows + chunk0) * D;
        float q1;
        uint32_t am = score_rows_bf16<D, 4>(
            qv, n_chunks, [&](int m) { return lbase + static_cast<int64_t>(m) * D; }, sc, &q1);
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1)
          am = max(am, static_cast<uint32_t>(__shfl_xor(static_cast<int>(am), o, kWave)));
        if (lane == 0) atomicMax(&red_s[0], am);
        __syncthreads();
        const float amax = __uint_as_float(red_s[0]);
        if (amax <= 1e30f) {                    // the same for every thread; false for NaN
          // tau only bounds the candidates from below: two digits (sign,
          // exponent, 7 mantissa bits) leave it within 2^-7 of the k_c-th
          // largest s~, well inside the 2e band
          const RadixSel rs = radix_select(sc, n_chunks, k_c, hist_s, rsel, scan_ws, 16);
          if (rs.whole) {
            // the threshold bin was taken whole: tau is its smallest key
            uint32_t kmin = 0xffffffffu;
            for (int m = t; m < n_chunks; m += kThreads) {
              const uint32_t k = score_key(sc[m]);
              if ((k & rs.pmask) == rs.prefix) kmin = min(kmin, k);
            }
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1)
              kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o, kWave)));
            if (lane == 0) atomicMin(&red_s[1], kmin);
          }
          __syncthreads();
          // the same value in every thread: tau is the bin's smallest key, or
          // the k_c-th largest key's lower bound with the open digits 0
          const float bound = 0.0045f * amax + 1e-30f * (1.f + q1);
          const float thr = key_score(rs.whole ? red_s[1] : rs.prefix) - 2.f * bound;
          // candidates in ascending chunk order: thread t owns [t*E, t*E + E)
          const int E = (n_chunks + kThreads - 1) / kThreads;
          const int m0 = min(t * E, n_chunks), m1 = min(m0 + E, n_chunks);
          int n_here = 0;
          for (int m = m0; m < m1; ++m) n_here += sc[m] >= thr;
          int n_cand;
          int pos = block_scan_excl<kThreads>(n_here, &n_cand, scan_ws);
          if (n_cand < kMaxCand) {              // the same for every thread
            for (int m = m0; m < m1; ++m)
              if (sc[m] >= thr) cidx_s[pos++] = m;
            __syncthreads();
            score_rows<D, 4>(qv, n_cand, [&](int c) { return cbase + static_cast<int64_t>(cidx_s[c]) * D; }, gsc);
            __syncthreads();
            for (int c = t; c <= n_cand; c += kThreads)
              gkey[c] = c < n_cand ? rank_key(gsc[c], static_cast<uint32_t>(chunk0 + cidx_s[c])) : 0ull;
            __syncthreads();
            rank_take_mask(gkey, n_cand, k_c, wmask);
            __syncthreads();
            for (int c = t; c < n_cand; c += kThreads)
              if (mask_taken(wmask, c)) sorted[ordered_pos(wmask, c)] = chunk0 + cidx_s[c];
            // k_c taken (n_cand >= k_c: the k_c largest s~ are candidates), counted anyway
            int taken = 0;
            for (int w2 = 0; w2 < (n_cand + kWave - 1) / kWave; ++w2) taken += __popcll(wmask[w2]);
            __syncthreads();
            kc_eff = taken;
            done = true;
            if (t < k_c) sel_chunks[bj * k_c + t] = t < kc_eff ? sorted[t] : -1;
          }
        }
      }
    }
    if (!done) {
      // ---- 2. chunk scores --------------------------------------------------
      score_rows<D, 4>(qv, n_chunks, [&](int m) { return cbase + static_cast<int64_t>(m) * D; }, sc);
      __syncthreads();

      // ---- 3. chunk top-k: exact radix select over the order-preserving
      // score keys until the threshold bin is taken whole or the key is fixed
      // in all 32 bits; equal keys at the threshold go to the lowest indices.
      // The kept chunks are then written in ascending index order.
      kc_eff = min(k_c, n_chunks);
      const RadixSel rs = radix_select(sc, n_chunks, kc_eff, hist_s, rsel, scan_ws);
      const uint32_t prefix = rs.prefix, pmask = rs.pmask;
      const int need = rs.need;
      if (!rs.exact) {
        // every key with the prefix under the mask, or above it, is kept: the
        // kc_eff chunk ids are appended in any order, then placed by rank
        // (ids are unique, so the result is fixed)
        if (t == 0) n_app = 0;
        __syncthreads();
        for (int m = t; m < n_chunks && kc_eff > 0; m += kThreads)
          if ((score_key(sc[m]) & pmask) >= prefix) gtmp_s[atomicAdd(&n_app, 1)] = chunk0 + m;
        __syncthreads();
        if (t < kc_eff) {
          const int id = gtmp_s[t];
          int pos = 0;
          for (int u = 0; u < kc_eff; ++u) pos += gtmp_s[u] < id;
          sorted[pos] = id;
        }
      } else {
        // equal keys at the threshold: the need lowest indices among them.
        // Ordered compaction, thread t owns chunks [t*E, t*E + E)
        const int E = (n_chunks + kThreads - 1) / kThreads;
        const int m0 = min(t * E, n_chunks), m1 = min(m0 + E, n_chunks);
        int total, ties = 0;
        for (int m = m0; m < m1; ++m) ties += score_key(sc[m]) == prefix;
        const int tie_rank = block_scan_excl<kThreads>(ties, &total, scan_ws);
        auto taken = [&](uint32_t k, int& tr) { return k > prefix || (k == prefix && tr++ < need); };
        int n_here = 0;
        {
          int tr = tie_rank;
          for (int m = m0; m < m1; ++m) n_here += taken(score_key(sc[m]), tr);
        }
        int pos = block_scan_excl<kThreads>(n_here, &total, scan_ws);
        int tr = tie_rank;
        for (int m = m0; m < m1; ++m)
          if (taken(score_key(sc[m]), tr)) sorted[pos++] = chunk0 + m;
      }
      __syncthreads();
      if constexpr (MODE == kRouteDecodePart) {
        // this part's kept chunks and their scores, for the merge
        if (t < k_c) {
          const int64_t o = (bj * dec.n_part + blockIdx.z) * k_c + t;
          const bool v = t < kc_eff;
          dec.cand_id[o] = v ? sorted[t] : -1;
          dec.cand_sc[o] = v ? sc[sorted[t] - chunk0] : 0.f;
        }
      } else {
        if (t < k_c) sel_chunks[bj * k_c + t] = t < kc_eff ? sorted[t] : -1;
      }
    }
  }
  if constexpr (MODE == kRouteChunks || MODE == kRouteDecodePart) return;

  // ---- 4. group scores for the 8 groups of every kept chunk ----------------
  const int n_cand = kc_eff * (kChunk / kGroup);
  if constexpr (MODE == kRouteGroups) {
    const float* cbase = cache.data + static_cast<int64_t>(j) * cache.n_slots * (kChunk / kGroup) * D;
    score_rows<D, 4>(qv, n_cand, [&](int c) {
      return cbase + (static_cast<int64_t>(slot_s[c / 8]) * 8 + (c % 8)) * D;
    }, gsc);
  } else {
    const float* gbase = gsum + static_cast<int64_t>(j) * chunk_rows * (kChunk / kGroup) * D;
    score_rows<D, 4>(qv, n_cand, [&](int c) {
      return gbase + (static_cast<int64_t>(sorted[c / 8]) * 8 + (c % 8)) * D;
    }, gsc);
  }
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


// ---------------------------------------------------------------------------
// Group-summary cache update, one workgroup per KV head, between the two
// halves of the route: the chunks kept by all query blocks of head j are
// de-duplicated through an LDS bitmap over chunk ids; cached ones are hits and
// pin their slots; each miss (ascending chunk id) takes the next unpinned slot
// in clock order from the head's hand, evicting whatever chunk held it, and
// its 8 group rows are copied from host memory over the host link.
// Deterministic (the only atomics are bitwise ORs into the bitmap).
// ---------------------------------------------------------------------------
constexpr int kUpdThreads = 1024;
constexpr int kUpdWaves = kUpdThreads / kWave;

template <int D>
__global__ __launch_bounds__(kUpdThreads) void gcache_update_kernel(
    const int32_t* __restrict__ sel_chunks, int n_blocks, int n_kv, int k_c,
    const float* __restrict__ g_src, int chunk_rows, int32_t* __restrict__ slot_of_chunk,
    int32_t* __restrict__ chunk_of_slot, int32_t* __restrict__ hand, float* __restrict__ data,
    int n_slots, int32_t* __restrict__ stats) {
  __shared__ uint32_t bits[kGcacheMaxChunks / 32];  // chunks kept by some block
  __shared__ int32_t miss[kGcacheMaxSelected];      // missed chunks, ascending
  __shared__ int32_t assign[kGcacheMaxSelected];    // their slots
  __shared__ uint8_t pinned[kGcacheMaxSlots];
  __shared__ int32_t wsum[kUpdWaves + 1];
  const int t = threadIdx.x, j = blockIdx.x;
  const int64_t soc0 = static_cast<int64_t>(j) * chunk_rows;
  const int64_t cos0 = static_cast<int64_t>(j) * n_slots;
  const int n_words = (chunk_rows + 31) / 32;

  for (int i = t; i < n_words; i += kUpdThreads) bits[i] = 0u;
  for (int i = t; i < n_slots; i += kUpdThreads) pinned[i] = 0;
  __syncthreads();
  const int n = n_blocks * k_c;
  for (int i = t; i < n; i += kUpdThreads) {
    const int c = sel_chunks[(static_cast<int64_t>(i / k_c) * n_kv + j) * k_c + i % k_c];
    if (c >= 0) atomicOr(&bits[c >> 5], 1u << (c & 31));
  }
  __syncthreads();

  // each thread owns WPT consecutive bitmap words, i.e. an ascending run of
  // chunk ids: look the chunks up, pin the hits, count hits and misses
  const int WPT = (n_words + kUpdThreads - 1) / kUpdThreads;
  const int w0 = t * WPT, w1 = min(w0 + WPT, n_words);
  int hits_here = 0, misses_here = 0;
  for (int w = w0; w < w1; ++w) {
    for (uint32_t m = bits[w]; m; m &= m - 1) {
      const int c = w * 32 + __builtin_ctz(m);
      const int sl = slot_of_chunk[soc0 + c];
      if (sl >= 0) {
        pinned[sl] = 1;
        ++hits_here;
      } else {
        ++misses_here;
      }
    }
  }
  int packed_total;
  const int base = block_scan_excl<kUpdThreads>(hits_here | (misses_here << 16), &packed_total, wsum);
  const int n_hit = packed_total & 0xffff, n_miss = packed_total >> 16;
  int k = base >> 16;
  for (int w = w0; w < w1; ++w)
    for (uint32_t m = bits[w]; m; m &= m - 1) {
      const int c = w * 32 + __builtin_ctz(m);
      if (slot_of_chunk[soc0 + c] < 0) miss[k++] = c;
    }

  // the k-th unpinned slot in clock order from the hand serves miss k (the
  // host guarantees n_slots >= n_blocks * k_c, so there are enough)
  const int h0 = hand[j];
  const int F = (n_slots + kUpdThreads - 1) / kUpdThreads;
  int free_here = 0;
  for (int f = 0; f < F; ++f) {
    const int i = t * F + f;
    if (i < n_slots && !pinned[(h0 + i) % n_slots]) ++free_here;
  }
  int n_free;
  int rk = block_scan_excl<kUpdThreads>(free_here, &n_free, wsum);
  for (int f = 0; f < F; ++f) {
    const int i = t * F + f;
    if (i >= n_slots) break;
    const int p = (h0 + i) % n_slots;
    if (pinned[p]) continue;
    if (rk < n_miss) {
      assign[rk] = p;
      if (rk == n_miss - 1) hand[j] = (p + 1) % n_slots;
    }
    ++rk;
  }
  __syncthreads();

  // tables: an evicted chunk is never one of this call's misses
  for (int q = t; q < n_miss; q += kUpdThreads) {
    const int p = assign[q];
    const int old = chunk_of_slot[cos0 + p];
    if (old >= 0) slot_of_chunk[soc0 + old] = -1;
    slot_of_chunk[soc0 + miss[q]] = p;
    chunk_of_slot[cos0 + p] = miss[q];
  }
  // rows: 8 group summaries (8*D floats) per missed chunk, 4 loads in flight
  // per thread across the host link
  constexpr int V4 = kGroup * D / 4;
  const int64_t total = static_cast<int64_t>(n_miss) * V4;
  const float4* src = reinterpret_cast<const float4*>(g_src + soc0 * (kChunk / kGroup) * D);
  float4* dst = reinterpret_cast<float4*>(data + cos0 * (kChunk / kGroup) * D);
  for (int64_t x0 = t; x0 < total; x0 += 4 * kUpdThreads) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t x = x0 + u * kUpdThreads;
      v[u] = x < total ? src[static_cast<int64_t>(miss[x / V4]) * V4 + x % V4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t x = x0 + u * kUpdThreads;
      if (x < total) dst[static_cast<int64_t>(assign[x / V4]) * V4 + x % V4] = v[u];
    }
  }
  if (t == 0 && stats) {
    stats[2 * j] = n_hit;
    stats[2 * j + 1] = n_miss;
  }
}

__global__ void gcache_reset_kernel(int32_t* __restrict__ slot_of_chunk, int64_t n_soc,
                                    int32_t* __restrict__ chunk_of_slot, int64_t n_cos,
                                    int32_t* __restrict__ hand, int n_kv) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n_soc) slot_of_chunk[i] = -1;
  if (i < n_cos) chunk_of_slot[i] = -1;
  if (i < n_kv) hand[i] = 0;
}

template <typename T, int D>
hipError_t launch_t(const hga_shape& s, const void* q, const float* cs, const float* gs,
                    int32_t* sc_out, int32_t* sg_out, void* ws, hipStream_t st) {
  const int n_blocks = s.seg_len / kBlockQ;
  const int chunk0 = sink_chunks(s);
  const int n_chunks = static_cast<int>(s.hist_len / kChunk) - chunk0;  // ranked chunks
  const int r = s.n_q_heads / s.n_kv_heads;
  float* scores = static_cast<float*>(ws);
  hipExtLaunchKernelGGL((route_kernel<T, D, kRouteFull>), dim3(s.n_kv_heads, n_blocks), dim3(kThreads), 0, st,
                        timer_event(HGA_KERNEL_ROUTE, 0), timer_event(HGA_KERNEL_ROUTE, 1), 0,
                        static_cast<const T*>(q), cs, gs, s.seg_len, s.n_kv_heads, r, chunk0, n_chunks,
                        static_cast<int>(hist_rows(s) / kChunk),
                        s.top_k_chunks, s.top_k_groups, scores, sc_out, sg_out, nullptr, CacheView{}, DecodeView{});
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_cached_t(const hga_shape& s, const void* q, const float* cs, const GcacheLayout& L,
                           const float* g_src, int32_t* sc_out, int32_t* sg_out, int32_t* stats,
                           void* ws, hipStream_t st) {
  const int n_blocks = s.seg_len / kBlockQ;
  const int chunk0 = sink_chunks(s);
  const int n_chunks = static_cast<int>(s.hist_len / kChunk) - chunk0;
  const int chunk_rows = static_cast<int>(hist_rows(s) / kChunk);
  const int r = s.n_q_heads / s.n_kv_heads;
  float* scores = static_cast<float*>(ws);
  float* qbar = reinterpret_cast<float*>(static_cast<char*>(ws) + route_workspace_bytes(s));
  const dim3 grid(s.n_kv_heads, n_blocks);
  const CacheView view{L.slot_of_chunk, L.data, L.n_slots};
  // ROUTE spans both halves and the update between them; GCACHE the update
  hipExtLaunchKernelGGL((route_kernel<T, D, kRouteChunks>), grid, dim3(kThreads), 0, st,
                        timer_event(HGA_KERNEL_ROUTE, 0), nullptr, 0,
                        static_cast<const T*>(q), cs, nullptr, s.seg_len, s.n_kv_heads, r, chunk0, n_chunks,
                        chunk_rows, s.top_k_chunks, s.top_k_groups, scores, sc_out, sg_out, qbar, view, DecodeView{});
  hipExtLaunchKernelGGL((gcache_update_kernel<D>), dim3(s.n_kv_heads), dim3(kUpdThreads), 0, st,
                        timer_event(HGA_KERNEL_GCACHE, 0), timer_event(HGA_KERNEL_GCACHE, 1), 0,
                        static_cast<const int32_t*>(sc_out), n_blocks, s.n_kv_heads, s.top_k_chunks, g_src,
                        chunk_rows, L.slot_of_chunk, L.chunk_of_slot, L.hand, L.data, L.n_slots, stats);
  hipExtLaunchKernelGGL((route_kernel<T, D, kRouteGroups>), grid, dim3(kThreads), 0, st,
                        nullptr, timer_event(HGA_KERNEL_ROUTE, 1), 0,
                        static_cast<const T*>(q), cs, nullptr, s.seg_len, s.n_kv_heads, r, chunk0, n_chunks,
                        chunk_rows, s.top_k_chunks, s.top_k_groups, scores, sc_out, sg_out, qbar, view, DecodeView{});
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

GcacheLayout gcache_layout(const hga_shape& s, void* cache, int n_slots) {
  const size_t n_soc = static_cast<size_t>(s.n_kv_heads) * (hist_rows(s) / kChunk);
  const size_t n_cos = static_cast<size_t>(s.n_kv_heads) * n_slots;
  const size_t o_cos = align256(sizeof(int32_t) * n_soc);
  const size_t o_hand = o_cos + align256(sizeof(int32_t) * n_cos);
  const size_t o_data = o_hand + align256(sizeof(int32_t) * s.n_kv_heads);
  char* base = static_cast<char*>(cache);
  GcacheLayout L;
  L.slot_of_chunk = base ? reinterpret_cast<int32_t*>(base) : nullptr;
  L.chunk_of_slot = base ? reinterpret_cast<int32_t*>(base + o_cos) : nullptr;
  L.hand = base ? reinterpret_cast<int32_t*>(base + o_hand) : nullptr;
  L.data = base ? reinterpret_cast<float*>(base + o_data) : nullptr;
  L.n_slots = n_slots;
  L.bytes = o_data + align256(sizeof(float) * n_cos * (kChunk / kGroup) * s.head_dim);
  return L;
}

size_t route_cached_workspace_bytes(const hga_shape& s) {
  const size_t n_blocks = s.seg_len / kBlockQ;
  return route_workspace_bytes(s) + align256(sizeof(float) * n_blocks * s.n_kv_heads * s.head_dim);
}

hipError_t launch_gcache_reset(const hga_shape& s, const GcacheLayout& L, hipStream_t stream) {
  const int64_t n_soc = static_cast<int64_t>(s.n_kv_heads) * (hist_rows(s) / kChunk);
  const int64_t n_cos = static_cast<int64_t>(s.n_kv_heads) * L.n_slots;
  int64_t n = n_soc > n_cos ? n_soc : n_cos;
  if (n < s.n_kv_heads) n = s.n_kv_heads;
  hipLaunchKernelGGL(gcache_reset_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                     L.slot_of_chunk, n_soc, L.chunk_of_slot, n_cos, L.hand, s.n_kv_heads);
  return hipGetLastError();
}

hipError_t launch_route_cached(const hga_shape& s, const void* q, const float* chunk_sum,
                               const GcacheLayout& L, const float* group_sum_dev, int32_t* sel_chunks,
                               int32_t* sel_groups, int32_t* stats, void* ws, hipStream_t stream) {
  const bool bf = s.dtype == HGA_BF16;
  if (s.head_dim == 128)
    return bf ? launch_cached_t<uint16_t, 128>(s, q, chunk_sum, L, group_sum_dev, sel_chunks, sel_groups, stats, ws, stream)
              : launch_cached_t<float, 128>(s, q, chunk_sum, L, group_sum_dev, sel_chunks, sel_groups, stats, ws, stream);
  return bf ? launch_cached_t<uint16_t, 64>(s, q, chunk_sum, L, group_sum_dev, sel_chunks, sel_groups, stats, ws, stream)
            : launch_cached_t<float, 64>(s, q, chunk_sum, L, group_sum_dev, sel_chunks, sel_groups, stats, ws, stream);
}

// Parts per (sequence, KV head) for the decode route: split the chunk scan
// only when the batch leaves most CUs idle (at most 32 (sequence, KV head)
// pairs; from 64 pairs on the two launches and the merge cost what the split
// saves), each part fits the LDS scores and the merge's candidates fit its
// key array.
int decode_route_parts(const hga_shape& s, int batch) {
  const int64_t rows = hist_rows(s) / kChunk;
  const int64_t wgs = static_cast<int64_t>(batch) * s.n_kv_heads;
  if (wgs > 64 || rows < 2 * kThreads) return 1;
  // up to 32 pairs: about two workgroups per CU; 33 to 64 pairs: about one per
  // CU (four to seven parts). Fewer parts over more pairs measured slower
  // than one workgroup per pair.
  const int64_t want = wgs <= 32 ? (2 * kThreads + wgs - 1) / wgs : kThreads / wgs;
  int P = static_cast<int>(want < 8 ? want : 8);
  while (P > 1 && P * s.top_k_chunks >= kMaxTopKChunks * (kChunk / kGroup)) --P;
  if (P <= 1 || (rows + P - 1) / P > kLdsScores) return 1;
  return P;
}

struct DecodeRouteWs {
  size_t scores, qbar, cand;  // byte offsets
  size_t bytes;
};

// [chunk scores, above 4,096 chunks per (sequence, KV head), unsplit only]
// [q-bar [batch][n_kv][D] fp32] [candidate ids] [candidate scores]
DecodeRouteWs decode_route_ws(const hga_shape& s, int batch) {
  DecodeRouteWs w{};
  const int P = decode_route_parts(s, batch);
  w.scores = 0;
  size_t off = align256(sizeof(float) * batch * s.n_kv_heads * (hist_rows(s) / kChunk + 1));
  if (P > 1) {
    const size_t nc = static_cast<size_t>(batch) * s.n_kv_heads * P * s.top_k_chunks;
    w.qbar = off;
    off += align256(sizeof(float) * batch * s.n_kv_heads * s.head_dim);
    w.cand = off;
    off += 2 * align256(sizeof(int32_t) * nc);
  }
  w.bytes = off;
  return w;
}

template <typename T, int D>
hipError_t launch_decode_t(const hga_shape& s, int batch, int n_new, const void* q, const float* cs,
                           const uint16_t* cs_lo, const float* gs, const int32_t* hist_lens, int32_t* sc_out,
                           int32_t* sg_out, void* ws, hipStream_t st) {
  const int r = s.n_q_heads / s.n_kv_heads;
  const int chunk_rows = static_cast<int>(hist_rows(s) / kChunk);
  const int P = decode_route_parts(s, batch);
  if (P == 1) {
    DecodeView dv{hist_lens, s.n_sink_chunks, s.n_q_heads};
    dv.csum_lo = cs_lo;
    hipExtLaunchKernelGGL((route_kernel<T, D, kRouteDecode>), dim3(s.n_kv_heads, batch), dim3(kThreads), 0, st,
                          timer_event(HGA_KERNEL_ROUTE, 0), timer_event(HGA_KERNEL_ROUTE, 1), 0,
                          static_cast<const T*>(q), cs, gs, n_new, s.n_kv_heads, r, 0, 0, chunk_rows,
                          s.top_k_chunks, s.top_k_groups, static_cast<float*>(ws), sc_out, sg_out, nullptr,
                          CacheView{}, dv);
    return hipGetLastError();
  }
  const DecodeRouteWs w = decode_route_ws(s, batch);
  char* base = static_cast<char*>(ws);
  float* qbar = reinterpret_cast<float*>(base + w.qbar);
  const size_t nc = static_cast<size_t>(batch) * s.n_kv_heads * P * s.top_k_chunks;
  DecodeView dv{hist_lens, s.n_sink_chunks, s.n_q_heads};
  dv.n_part = P;  // parts of a split scan are short and latency bound: fp32 scan
  dv.cand_id = reinterpret_cast<int32_t*>(base + w.cand);
  dv.cand_sc = reinterpret_cast<float*>(base + w.cand + align256(sizeof(int32_t) * nc));
  hipExtLaunchKernelGGL((route_kernel<T, D, kRouteDecodePart>), dim3(s.n_kv_heads, batch, P), dim3(kThreads), 0,
                        st, timer_event(HGA_KERNEL_ROUTE, 0), nullptr, 0, static_cast<const T*>(q), cs, gs, n_new,
                        s.n_kv_heads, r, 0, 0, chunk_rows, s.top_k_chunks, s.top_k_groups,
                        static_cast<float*>(ws), sc_out, sg_out, qbar, CacheView{}, dv);
  hipExtLaunchKernelGGL((route_kernel<T, D, kRouteDecodeMerge>), dim3(s.n_kv_heads, batch), dim3(kThreads), 0, st,
                        nullptr, timer_event(HGA_KERNEL_ROUTE, 1), 0, static_cast<const T*>(q), cs, gs, n_new,
                        s.n_kv_heads, r, 0, 0, chunk_rows, s.top_k_chunks, s.top_k_groups,
                        static_cast<float*>(ws), sc_out, sg_out, qbar, CacheView{}, dv);
  return hipGetLastError();
}

// Chunk scores of every (sequence, KV head) when a history exceeds the LDS,
// or (small batches) the split route's q-bar and candidates.
size_t decode_route_workspace_bytes(const hga_shape& s, int batch) { return decode_route_ws(s, batch).bytes; }

hipError_t launch_decode_route(const hga_shape& s, int batch, int n_new, const void* q,
                               const float* chunk_sum, const uint16_t* chunk_sum_lo, const float* group_sum,
                               const int32_t* hist_lens, int32_t* sel_chunks, int32_t* sel_groups, void* ws,
                               hipStream_t stream) {
  const bool bf = s.dtype == HGA_BF16;
#define HGA_DECODE_ROUTE(T, D)                                                                              \
  launch_decode_t<T, D>(s, batch, n_new, q, chunk_sum, chunk_sum_lo, group_sum, hist_lens, sel_chunks, \
                        sel_groups, ws, stream)
  if (s.head_dim == 128) return bf ? HGA_DECODE_ROUTE(uint16_t, 128) : HGA_DECODE_ROUTE(float, 128);
  return bf ? HGA_DECODE_ROUTE(uint16_t, 64) : HGA_DECODE_ROUTE(float, 64);
#undef HGA_DECODE_ROUTE
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
