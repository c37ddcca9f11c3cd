// sla_tiles.hpp - 64-token tile staging shared by the gfx950 kernels of libsla.
//
// A tile is 64 consecutive tokens x D channels of one (batch, head).  It travels HBM ->
// registers (16-byte coalesced loads, issued ahead of use) -> LDS as row-major bf16 (see
// TileLayout).  fp32 inputs are rounded to bf16 (nearest even) on the way into LDS.
#pragma once

#include "sla_device.hpp"

namespace sla {

constexpr int kPad = 8;  // bf16 elements of padding per LDS row (d = 64 tiles)

// Where element (row, col) of a 64-row tile lives in LDS (bf16 elements from the tile base).
// d = 128: 256-byte rows without padding, the 16-byte chunk c of row r stored at chunk
// c ^ f(r) with f(r) = 4 (r & 3) + ((r >> 2) & 3).  Then 16 consecutive rows reading one chunk
// (row-wise 16-byte MFMA operand reads) and 4 consecutive rows x 4 consecutive chunks (the
// transposed ds_read_b64_tr_b16 reads of two 16-lane groups) each touch 16 distinct 16-byte
// bank groups.  d = 64: rows padded by kPad elements.
template <int D>
struct TileLayout {
  static constexpr int PITCH = D == 128 ? D : D + kPad;
  static constexpr int ELEMS = kBlock * PITCH;
  static __device__ __forceinline__ int off(int row, int col) {
    if constexpr (D == 128) {
      const int f = 4 * (row & 3) + ((row >> 2) & 3);
      return row * PITCH + (((col >> 3) ^ f) << 3) + (col & 7);
    } else {
      return row * PITCH + col;
    }
  }
};

template <class T>
struct Vec16;  // elements of one 16-byte global load
template <>
struct Vec16<__bf16> {
  static constexpr int n = 8;
};
template <>
struct Vec16<float> {
  static constexpr int n = 4;
};

// Registers holding one tile of a [rows][D] tensor for THREADS cooperating threads; rows at or
// beyond `valid` read as zero.
template <class T, int D, int THREADS>
struct TileLoader {
  static constexpr int VEC = Vec16<T>::n;
  static constexpr int CPR = D / VEC;                 // 16-byte chunks per row
  static constexpr int PER = kBlock * CPR / THREADS;  // chunks per thread
  static_assert(PER * THREADS == kBlock * CPR, "tile must split evenly over the threads");
  i32x4 r[PER];
  __device__ __forceinline__ void load(const T* base, int valid, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * THREADS;
      const int row = q / CPR, ch = q % CPR;
      r[u] = row < valid ? ld16(base + (size_t)row * D + ch * VEC) : i32x4{0, 0, 0, 0};
    }
  }
  // fp32 inputs only: store the bf16 rounding (hi) and the bf16 rounding of the remainder (lo)
  __device__ __forceinline__ void store_split(__bf16* hi, __bf16* lo, int tid) const {
    static_assert(sizeof(T) == 4, "split staging is for fp32 inputs");
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * THREADS;
      const int row = q / CPR, ch = q % CPR;
      const f32x4 f = __builtin_bit_cast(f32x4, r[u]);
      bf16x4 h, l;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = f2bf(f[e]);
        l[e] = f2bf(f[e] - bf2f(h[e]));
      }
      *reinterpret_cast<bf16x4*>(hi + TileLayout<D>::off(row, ch * VEC)) = h;
      *reinterpret_cast<bf16x4*>(lo + TileLayout<D>::off(row, ch * VEC)) = l;
    }
  }
  __device__ __forceinline__ void store(__bf16* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = tid + u * THREADS;
      const int row = q / CPR, ch = q % CPR;
      __bf16* dst = lds + TileLayout<D>::off(row, ch * VEC);
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<i32x4*>(dst) = r[u];
      } else {
        const f32x4 f = __builtin_bit_cast(f32x4, r[u]);
        bf16x4 b = {f2bf(f[0]), f2bf(f[1]), f2bf(f[2]), f2bf(f[3])};
        *reinterpret_cast<bf16x4*>(dst) = b;
      }
    }
  }
};

// Direct (register-free) copy of a full 64-row bf16 tile with D = 128 into the swizzled
// TileLayout by THREADS/64 wavefronts: wavefront w fills rows 4(NW u + w) .. +3 for u < 16/NW,
// 1 KB per load, lane i taking physical chunk i % 16 of row i / 16, i.e. logical chunk
// (i % 16) ^ f(row) of the source row.  With NW = 4 the swizzle of those rows is
// 4 (i / 16) + w for every u, so each lane's source offset is one register and the per-load
// part is wavefront-uniform.  Only for tiles with all 64 rows valid.
template <int THREADS>
__device__ __forceinline__ void load_tile_direct(const __bf16* src, __bf16* tile, int tid) {
  constexpr int NW = THREADS / 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
#pragma unroll
  for (int u = 0; u < 16 / NW; ++u) {
    const int r0 = 4 * (NW * u + w);
    const int f = 4 * (lane / 16) + ((NW * u + w) & 3);
    const int lane_off = (lane / 16) * 128 + ((lane % 16) ^ f) * 8;
    load_lds16(src + r0 * 128 + lane_off, tile + r0 * 128);
  }
}

// load_tile_direct through a buffer resource: the tile starts `toff` bytes into the resource
// (wavefront-uniform), each lane's offset inside it is lane_voff(tid).  The buffer range check
// covers the vector and immediate offsets only, not the scalar one: a full tile (every row
// inside the resource) takes the tile and row-group offsets as scalars, no per-lane
// arithmetic; a tile that crosses the resource's end (`crosses`, wavefront-uniform: the short
// last block of a sequence) puts them in the vector offset, so its rows past the end read as
// zero and no read leaves the resource.
template <int THREADS>
__device__ __forceinline__ uint32_t tile_lane_voff(int tid) {
  constexpr int NW = THREADS / 64;
  static_assert(NW == 4, "the per-lane offset is load-invariant for four wavefronts");
  const int w = tid / 64, lane = tid % 64;
  const int f = 4 * (lane / 16) + (w & 3);
  return (uint32_t)(((lane / 16) * 128 + ((lane % 16) ^ f) * 8) * 2);
}
template <int THREADS>
__device__ __forceinline__ void load_tile_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t toff,
                                              __bf16* tile, int tid, bool crosses) {
  constexpr int NW = THREADS / 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  if (crosses) {
#pragma unroll
    for (int u = 0; u < 16 / NW; ++u) {
      const int r0 = 4 * (NW * u + w);
      load_lds16_buf(rsrc, voff + toff + (uint32_t)r0 * 256u, 0u, tile + r0 * 128);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 16 / NW; ++u) {
      const int r0 = 4 * (NW * u + w);
      load_lds16_buf(rsrc, voff, toff + (uint32_t)r0 * 256u, tile + r0 * 128);
    }
  }
}

// load_tile_direct for a tile of `valid` < 64 rows: rows at or past `valid` re-read the last
// valid row (every address stays inside the source tensor); the caller zeroes them with
// zero_tile_rows once the loads have landed.
template <int THREADS>
__device__ __forceinline__ void load_tile_direct_clamped(const __bf16* src, __bf16* tile, int tid,
                                                         int valid) {
  constexpr int NW = THREADS / 64;
  const int w = tid / 64, lane = tid % 64;
#pragma unroll
  for (int u = 0; u < 16 / NW; ++u) {
    const int r0 = 4 * (NW * u + w);
    const int row = r0 + lane / 16;
    const int f = 4 * (row & 3) + ((row >> 2) & 3);
    const int chunk = (lane % 16) ^ f;
    load_lds16(src + min(row, valid - 1) * 128 + chunk * 8, tile + r0 * 128);
  }
}

// Zero rows valid .. 63 of a D = 128 tile in TileLayout (the swizzle only permutes chunks
// within a row, so whole rows are contiguous).
template <int THREADS>
__device__ __forceinline__ void zero_tile_rows(__bf16* tile, int tid, int valid) {
  for (int q = valid * 16 + tid; q < kBlock * 16; q += THREADS)
    *reinterpret_cast<i32x4*>(tile + q * 8) = i32x4{0, 0, 0, 0};
}

__device__ __forceinline__ bf16x8 join_tr(i16x4 a, i16x4 b) {
  i32x4 v = {(int)((u32)(uint16_t)a[0] | ((u32)(uint16_t)a[1] << 16)),
             (int)((u32)(uint16_t)a[2] | ((u32)(uint16_t)a[3] << 16)),
             (int)((u32)(uint16_t)b[0] | ((u32)(uint16_t)b[1] << 16)),
             (int)((u32)(uint16_t)b[2] | ((u32)(uint16_t)b[3] << 16))};
  return __builtin_bit_cast(bf16x8, v);
}

// Transposed MFMA operand from a 64-row LDS tile (TileLayout): lane l (g = l/32) receives
// column col0 + l%32 at the rows row0 + r_off + e and row0 + r_off + gap + e (e = 0..3) where
// r_off = step * g.  step = 8, gap = 4 gives rows row0 + 8g + 0..7; step = 4, gap = 8 gives
// rows row0 + 4g + {0..3, 8..11} (the key order of a 32x32 MFMA accumulator).
template <int D, int STEP, int GAP>
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* tile, int row0, int col0, int lane) {
  const int h = lane / 16, L = lane % 16;
  const int g = h / 2, cs = h % 2;
  const int r = row0 + STEP * g + L / 4;
  const int c = col0 + 16 * cs + 4 * (L % 4);
  return join_tr(lds_read_tr16(tile + TileLayout<D>::off(r, c)),
                 lds_read_tr16(tile + TileLayout<D>::off(r + GAP, c)));
}

// Byte addressing of a D = 128 TileLayout tile split as (per-lane part) XOR (block part) plus
// an immediate: with f = swz(r), the 16-byte chunk c of row r sits at chunk c ^ f, and f depends
// on r & 15 only, so for row offsets that are multiples of 16 and column blocks of 32 channels:
//   row-wise read of row R0 + lane%32 (R0 % 32 == 0), channels 16k + 8g .. + 7:
//     R0 * 256 + (row_part(lane) ^ 32k)
//   transposed read (tr_operand) of rows row0 + STEP g + L/4 [+ GAP], channels
//   32J + 16cs + 4(L%4) (row0 % 16 == 0):   row0 * 256 + (tr_part<STEP, GAP?>(lane) ^ 64J)
// The XOR only touches bits 5..7, disjoint from the row part (bits >= 8) and the in-chunk
// offset (bit 3), which is what makes the split exact.
__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ int row_part(int lane) {
  const int g = lane / 32;
  return (lane % 32) * 256 + 16 * (swz(lane % 16) ^ g);
}
template <int STEP>
__device__ __forceinline__ int tr_part(int lane, int gap) {
  const int h = lane / 16, L = lane % 16;
  const int g = h / 2, cs = h % 2;
  const int r = STEP * g + L / 4 + gap;  // < 16
  const int cl = 2 * cs + (L % 4) / 2;
  return r * 256 + 16 * (cl ^ swz(r)) + 8 * (L % 2);
}
__device__ __forceinline__ bf16x8 lds_row16(const __bf16* base, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(base) + byte_off);
}
__device__ __forceinline__ i16x4 lds_tr_at(const __bf16* base, int byte_off) {
  return lds_read_tr16(reinterpret_cast<const __bf16*>(reinterpret_cast<const char*>(base) + byte_off));
}

// Map a workgroup id to a logical work item so that each of the 8 XCDs (which receive
// workgroups round-robin) processes one contiguous range of items: neighbouring query blocks
// of a head share their XCD's L2.  A bijection on [0, total).
__host__ __device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int q = total / 8, r = total % 8;
  const int xcd = wg % 8, k = wg / 8;
  return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

// Workgroup -> (head, item within the head) for work grouped by head, when heads may carry
// unequal work (a dropped branch): each XCD takes the same eighth of every head, chunk x of a
// head being its items x * per_head / 8 ..  (sizes differ by at most one), so no XCD idles while
// others finish; consecutive workgroups of an XCD walk consecutive items of one head (they share
// L2).  The grid has 8 * heads * ceil(per_head / 8) workgroups (xcd_chunk_grid): XCD x (the
// workgroups wg % 8 == x) runs k = wg / 8 -> head k / ceil(per_head / 8), item chunk_start(x) +
// k % ceil(per_head / 8); the few workgroups past a short chunk get false and exit at once.
__host__ __device__ __forceinline__ int xcd_chunk_grid(int heads, int per_head) {
  return 8 * heads * ((per_head + 7) / 8);
}
__host__ __device__ __forceinline__ bool xcd_chunk_map(int wg, int per_head, int* head, int* item) {
  const int q = per_head / 8, r = per_head % 8;
  const int smax = q + (r > 0 ? 1 : 0);
  const int x = wg % 8, k = wg / 8;
  const int off = k % smax;
  *head = k / smax;
  *item = x * q + (x < r ? x : r) + off;
  return off < q + (x < r ? 1 : 0);
}
// The inverse of xcd_chunk_map: the workgroup id that runs item `item` of head `head`.
__host__ __device__ __forceinline__ int xcd_chunk_id(int head, int item, int per_head) {
  const int q = per_head / 8, r = per_head % 8;
  const int smax = q + (r > 0 ? 1 : 0);
  const int big = r * (q + 1);  // the items of the r XCDs that take q + 1
  const int x = item < big ? item / (q + 1) : r + (item - big) / q;
  const int off = item - (x * q + (x < r ? x : r));
  return 8 * (head * smax + off) + x;
}

// The same with the heads split among 8 / XG groups of XG XCDs (XG = 8, 4, 2 or 1): head h runs
// on the XCDs of group h % (8 / XG), each of them taking 1 / XG of the head's items, so each XCD
// works through a larger, contiguous share of fewer heads at a time (XG = 8 is the map above).
// XCD x = wg % 8 is position x % XG of group x / XG; its k-th workgroup (k = wg / 8) runs item
// chunk_start(x % XG) + k % smax of head (k / smax) (8 / XG) + x / XG, smax = ceil(per_head / XG).
template <int XG>
__host__ __device__ __forceinline__ int xcd_group_grid(int heads, int per_head) {
  constexpr int G = 8 / XG;
  return 8 * ((heads + G - 1) / G) * ((per_head + XG - 1) / XG);
}
template <int XG>
__host__ __device__ __forceinline__ bool xcd_group_map(int wg, int heads, int per_head, int* head, int* item) {
  static_assert(XG == 1 || XG == 2 || XG == 4 || XG == 8, "XCDs per head group");
  constexpr int G = 8 / XG;
  const int q = per_head / XG, r = per_head % XG;
  const int smax = q + (r > 0 ? 1 : 0);
  const int x = wg % 8, k = wg / 8, px = x % XG;
  const int off = k % smax;
  *head = (k / smax) * G + x / XG;
  *item = px * q + (px < r ? px : r) + off;
  return *head < heads && off < q + (px < r ? 1 : 0);
}
template <int XG>
__host__ __device__ __forceinline__ int xcd_group_id(int head, int item, int per_head) {
  constexpr int G = 8 / XG;
  const int q = per_head / XG, r = per_head % XG;
  const int smax = q + (r > 0 ? 1 : 0);
  const int big = r * (q + 1);
  const int px = item < big ? item / (q + 1) : r + (item - big) / q;
  const int off = item - (px * q + (px < r ? px : r));
  return 8 * ((head / G) * smax + off) + (head % G) * XG + px;
}

}  // namespace sla
