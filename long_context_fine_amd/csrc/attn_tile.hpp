// Shared pieces of the MFMA attention kernels: register-staged 64-key tiles and
// small MFMA / softmax helpers (gfx950, wave64, v_mfma_f32_32x32x16_bf16).
//
// MFMA 32x32x16 operand layout used throughout: A[i][k] comes from lane
// (i % 32) + 32*h with k = 8h .. 8h+7 in its 8 slots; B[k][j] from lane
// (j % 32) + 32*h likewise; the 16 accumulator registers v of lane l hold
// D[8*(v/4) + 4*(l/32) + v%4][l % 32]. The k <-> (lane half, slot) pairing only
// has to agree between A and B, which lets an accumulator tile be fed back as a
// B operand with the contraction index permuted the same way on the A side.
#pragma once

#include "hga_common.hpp"

namespace hga {

constexpr int kTile = 64;  // keys (or queries) per tile

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 8 accumulator registers [v0, v0+8) of a 32x32 tile as a bf16 B operand
// (contraction slots = rows 8*(v/4) + 4*half + v%4 of the tile).
__device__ __forceinline__ bf16x8 acc_to_bf16x8(const f32x16& acc, int v0) {
  uint4 u;
  u.x = cvt_pk_bf16(acc[v0 + 0], acc[v0 + 1]);
  u.y = cvt_pk_bf16(acc[v0 + 2], acc[v0 + 3]);
  u.z = cvt_pk_bf16(acc[v0 + 4], acc[v0 + 5]);
  u.w = cvt_pk_bf16(acc[v0 + 6], acc[v0 + 7]);
  return __builtin_bit_cast(bf16x8, u);
}

// A operand from a transposed LDS tile T[row][col] (row stride `ts` elements):
// row = this lane's row, columns {c0..c0+3} and {c0+8..c0+11} -- the column
// permutation that matches acc_to_bf16x8 on the B side when c0 = base + 4*half.
__device__ __forceinline__ bf16x8 lds_a_permuted(const uint16_t* row, int c0) {
  const uint2 lo = *reinterpret_cast<const uint2*>(row + c0);
  const uint2 hi = *reinterpret_cast<const uint2*>(row + c0 + 8);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// gfx950 ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives
// element (i % 4) of the 8-byte chunks read by lanes 4k + i/4, k = 0..3.
__device__ __forceinline__ i16x4 ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(reinterpret_cast<uintptr_t>(p)));
}

// A operand read transposed from a row-major LDS tile T[row][col] (row stride
// `stride` elements): the lane's M index is column cbase + lane % 32, and its 8
// contraction slots are rows rbase + 8*(i/4) + 4*(lane/32) + i%4 -- the row
// permutation acc_to_bf16x8 produces on the B side. Each 16-lane group reads 4
// rows x 16 columns per instruction.
__device__ __forceinline__ bf16x8 lds_a_tr(const uint16_t* T, int stride, int rbase, int cbase,
                                           int lane) {
  const int g16 = lane >> 4, gl = lane & 15;
  const int col = cbase + 16 * (g16 & 1) + 4 * (gl & 3);
  const int row = rbase + 4 * (g16 >> 1) + (gl >> 2);
  const i16x4 lo = ds_read_tr16(T + row * stride + col);
  const i16x4 hi = ds_read_tr16(T + (row + 8) * stride + col);
  const uint2 l2 = __builtin_bit_cast(uint2, lo);
  const uint2 h2 = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
}

// Unpadded 64 x D bf16 LDS tile whose 16-byte chunks are XOR-permuted by row,
// so that both row reads (b128, 16 lanes on 16 rows at one column) and
// transposed reads (ds_read_b64_tr_b16, 4 rows x 16 columns per 16 lanes) hit
// 64 distinct banks (checked with a bank model of both access patterns).
template <int D>
struct Swz {
  static constexpr uint32_t NCH = D / 8;  // chunks per row
  __device__ __forceinline__ static uint32_t f(uint32_t row) {
    return NCH == 16 ? (((row & 3u) << 2) | ((row >> 2) & 3u)) : (((row & 3u) << 1) | ((row >> 2) & 1u));
  }
  __device__ __forceinline__ static uint32_t off(uint32_t row, uint32_t col) {
    return row * D + ((((col >> 3) ^ f(row)) & (NCH - 1)) << 3) + (col & 7u);
  }
};

// A operand (rows of the tile = M index) from a swizzled tile: lane row
// rbase + lane % 32, slots = 8 columns starting at k0 + 8 * (lane / 32).
template <int D>
__device__ __forceinline__ bf16x8 lds_a_row_swz(const uint16_t* T, int rbase, int k0, int lane) {
  const uint32_t l = static_cast<uint32_t>(lane);
  return *reinterpret_cast<const bf16x8*>(
      T + Swz<D>::off(static_cast<uint32_t>(rbase) + (l & 31u), static_cast<uint32_t>(k0) + 8u * (l >> 5)));
}

// lds_a_tr for a swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 lds_a_tr_swz(const uint16_t* T, int rbase, int cbase, int lane) {
  const uint32_t g16 = static_cast<uint32_t>(lane) >> 4, gl = static_cast<uint32_t>(lane) & 15u;
  const uint32_t col = static_cast<uint32_t>(cbase) + 16u * (g16 & 1u) + 4u * (gl & 3u);
  const uint32_t row = static_cast<uint32_t>(rbase) + 4u * (g16 >> 1) + (gl >> 2);
  const i16x4 lo = ds_read_tr16(T + Swz<D>::off(row, col));
  const i16x4 hi = ds_read_tr16(T + Swz<D>::off(row + 8, col));
  const uint2 l2 = __builtin_bit_cast(uint2, lo);
  const uint2 h2 = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x[i], x[i ^ 32]) on every lane i: v_permlane32_swap exchanges the upper
// 32 lanes of its first operand with the lower 32 lanes of its second, so with
// both operands x the two results hold x's lower and upper halves.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One 64-row x D tile held in registers between its global load and its LDS
// store. A task is 4 consecutive rows x 8 columns (one 16-byte chunk per row);
// the 4 rows are contiguous in memory for every tile kind used here.
template <int D, int NT>
struct TileRegs {
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int NTASK = (kTile / 4) * CPR;
  static constexpr int TPT = (NTASK + NT - 1) / NT;
  uint4 a[TPT][4];

  // rowptr(kq) -> pointer to row 4*kq of the tile (nullptr: rows are zero)
  template <class F>
  __device__ __forceinline__ void load(int tid, F rowptr) {
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      const int task = tid + t * NT;
      if (NTASK % NT == 0 || task < NTASK) {
        const int kq = task / CPR, c = task % CPR;
        const uint16_t* src = rowptr(kq);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          a[t][u] = src ? *reinterpret_cast<const uint4*>(src + u * D + c * 8) : make_uint4(0, 0, 0, 0);
      }
    }
  }
  // row-major: dst[row * stride + col]
  __device__ __forceinline__ void store_rows(int tid, uint16_t* dst, int stride) const {
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      const int task = tid + t * NT;
      if (NTASK % NT == 0 || task < NTASK) {
        const int kq = task / CPR, c = task % CPR;
#pragma unroll
        for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(dst + (kq * 4 + u) * stride + c * 8) = a[t][u];
      }
    }
  }
  // swizzled row-major (Swz<D>)
  __device__ __forceinline__ void store_swz(int tid, uint16_t* dst) const {
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      const int task = tid + t * NT;
      if (NTASK % NT == 0 || task < NTASK) {
        const int kq = task / CPR, c = task % CPR;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          *reinterpret_cast<uint4*>(dst + Swz<D>::off(kq * 4 + u, c * 8)) = a[t][u];
      }
    }
  }
  // transposed: dst[col * stride + row], 4 rows packed per 8-byte store
  __device__ __forceinline__ void store_transposed(int tid, uint16_t* dst, int stride) const {
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      const int task = tid + t * NT;
      if (NTASK % NT == 0 || task < NTASK) {
        const int kq = task / CPR, c = task % CPR;
        const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&a[t][0]);
        const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&a[t][1]);
        const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&a[t][2]);
        const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&a[t][3]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // column pair (2w, 2w+1) of the chunk
          uint2 lo, hi;
          lo.x = (r0[w] & 0xffffu) | (r1[w] << 16);
          lo.y = (r2[w] & 0xffffu) | (r3[w] << 16);
          hi.x = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
          hi.y = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
          *reinterpret_cast<uint2*>(dst + (c * 8 + 2 * w) * stride + kq * 4) = lo;
          *reinterpret_cast<uint2*>(dst + (c * 8 + 2 * w + 1) * stride + kq * 4) = hi;
        }
      }
    }
  }
};

// Global-to-LDS copies (global_load_lds): lane i of the wave copies `size`
// bytes from sbase + voff to LDS address M0 + size * i. They are issued from
// inline asm because the compiler, when it sees such a copy pending, waits for
// every outstanding LDS read (lgkmcnt(0)) and for the copy itself (vmcnt(0))
// before later LDS reads it cannot prove disjoint, which serializes the
// pipeline. The instructions have no register outputs; M0 is used by nothing
// else in these kernels; one wait state separates the M0 write from the copy
// that reads it. Callers wait with wait_vmem() and a workgroup
// barrier before any wave reads the LDS they fill, and issue them only into a
// buffer no wave is reading.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
// The base address must be the same on every lane; it is moved to SGPRs.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ void dma_b128(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(sbase)),
               "s"(__builtin_amdgcn_readfirstlane(m0))
               : "memory");
}
__device__ __forceinline__ void dma_b32(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(uniform_ptr(sbase)),
               "s"(__builtin_amdgcn_readfirstlane(m0))
               : "memory");
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


// Number of wave instructions a group of NT threads needs to copy one 64 x D
// bf16 tile (16 bytes per lane per instruction).
template <int D, int NT>
constexpr int tile_lds_instrs() { return (kTile * (D / 8) + NT - 1) / NT; }

// One wave instruction (`part`, 0 .. tile_lds_instrs - 1) of a copy of a
// 64 x D bf16 tile straight from global memory into the swizzled LDS layout
// of Swz<D>, 16 bytes per lane, no registers held. Copies are issued one
// instruction at a time so they can be spread between MFMAs: a wave that
// issues many back to back stalls once the memory pipeline's queue fills.
// The tile is made of runs of RPI = 64 / (D / 8) rows that are contiguous in
// global memory, one run per instruction; run(kq) returns the first row of
// rows RPI*kq .. RPI*kq + RPI - 1. `wave` (index within the NT threads) and
// everything run() returns must be wave-uniform: the source base and LDS
// address go to SGPRs, only the lane offset (4 distinct values) is per lane.
template <int D, int NT, class RunPtr>
__device__ __forceinline__ void tile_copy_part(uint16_t* lds_tile, uint32_t wave, uint32_t lane, RunPtr run,
                                               int part) {
  constexpr uint32_t CPR = D / 8;
  constexpr uint32_t RPI = kWave / CPR;
  constexpr uint32_t CHUNKS = kTile * CPR;
  const uint32_t i = static_cast<uint32_t>(part) * NT + wave * kWave;  // first chunk of the instruction
  if (CHUNKS % NT == 0 || i < CHUNKS) {
    const uint32_t kq = i / kWave;
    const uint32_t lrow = lane / CPR, pc = lane % CPR;
    const uint32_t lc = (pc ^ Swz<D>::f(kq * RPI + lrow)) & (CPR - 1);
    dma_b128((lrow * D + lc * 8) * 2, run(kq), lds_addr(lds_tile) + i * 16);
  }
}

// tile_copy_part for a tile whose 64 rows are contiguous (row stride D).
template <int D, int NT>
__device__ __forceinline__ void tile_copy_rows_part(uint16_t* lds_tile, uint32_t wave, uint32_t lane,
                                                    const uint16_t* src, int part) {
  constexpr uint32_t RPI = kWave / (D / 8);
  tile_copy_part<D, NT>(lds_tile, wave, lane, [&](uint32_t kq) { return src + kq * RPI * D; }, part);
}

// 64 consecutive floats from global memory into LDS (one wave instruction).
__device__ __forceinline__ void row64_load_lds(float* lds_dst, const float* src, int lane) {
  dma_b32(static_cast<uint32_t>(lane * 4), src, lds_addr(lds_dst));
}

// Builds, in LDS, the list of history tiles (8 selected groups each) that hold
// at least one valid group; returns nothing, the count lands in *n_out.
__device__ __forceinline__ void build_hist_tile_list(const int32_t* sel_s, int k_g, int32_t* list,
                                                     int32_t* n_out) {
  if (threadIdx.x == 0) {
    int n = 0;
    for (int ht = 0; ht < (k_g + 7) / 8; ++ht) {
      bool any = false;
      for (int g = 0; g < 8; ++g) {
        const int slot = ht * 8 + g;
        any |= slot < k_g && sel_s[slot] >= 0;
      }
      if (any) list[n++] = ht;
    }
    *n_out = n;
  }
}

// Keep bitmask of a segment tile whose first key is key0, for the lane's query
// row i and local window W: bit kt*16 + v is set iff key
// key0 + kt*32 + 8*(v/4) + 4*hh + v%4 satisfies i - W < key <= i. Within a
// subtile and lane half the keys rise with v, so the kept slots lie between
// two prefix counts: n(x) = sum_g clamp(x - 8g + 1, 0, 4). WIN = false: no
// window (W >= the segment), only the causal bound.
template <bool WIN>
__device__ __forceinline__ uint32_t window_keep(int i, int key0, int W, int hh) {
  uint32_t keep = 0u;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int x = i - (key0 + kt * 32 + 4 * hh);
    int n_hi = 0, n_lo = 0;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      n_hi += min(max(x - 8 * gi + 1, 0), 4);
      if (WIN) n_lo += min(max(x - W - 8 * gi + 1, 0), 4);
    }
    keep |= static_cast<uint32_t>(((1ull << n_hi) - 1ull) & ~((1ull << n_lo) - 1ull)) << (16 * kt);
  }
  return keep;
}

// Whether segment tile s_idx (<= b) needs masking for query block b: it holds
// keys after some query of the block (the diagonal) or at or before some
// query's window start.
template <bool WIN>
__device__ __forceinline__ bool seg_tile_masked(int s_idx, int b, int W) {
  return s_idx >= b || (WIN && s_idx * kTile <= b * kBlockQ + kBlockQ - 1 - W);
}

// First segment tile any query of block b attends with local window W.
template <bool WIN>
__device__ __forceinline__ int seg_first_tile(int b, int W) {
  const int k = b * kBlockQ - W + 1;
  return WIN && k > 0 ? k / kTile : 0;
}

__device__ __forceinline__ uint32_t hist_group_mask(const int32_t* sel_s, int k_g, int ht) {
  uint32_t m = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const int slot = ht * 8 + g;
    m |= (slot < k_g && sel_s[slot] >= 0) ? (1u << g) : 0u;
  }
  return m;
}

}  // namespace hga
