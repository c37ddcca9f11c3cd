// sla_quant.hpp - the per-block quantiser of the low-bit sparse branch (SLA2 Italian summary
// section 2.C and Arabic summary section 2.jim: the forward quantises Q, K, P and V), shared by
// the stand-alone quantiser (fp8.hip) and the state kernel that quantises K and V on the way
// (linear_state.hip), so that both produce the same bytes.
//
// Reading: one absmax scale per (batch, head, 64-token block): inv = Q_max / a, s = a / Q_max
// (fp32, IEEE division; s = 1 for an all-zero block), code = round-to-nearest-even of x * inv,
// saturated to +-Q_max (Q_max = 448 for OCP e4m3, 127 for symmetric int8).  A 64 x 128 bf16 tile
// is held by 256 threads as 16-byte chunks: thread t holds chunk t % 16 (channels 8 (t % 16) ..
// + 7) of rows t / 16 + 16 u, u = 0..3 (the TileLoader layout); rows past the sequence are zero.
// K codes are row-major like the input; V codes are stored per block transposed, [channel][64]
// bytes with the keys in the order the PV MFMA reads them (v8_pos).
#pragma once

#include "sla_device.hpp"

namespace sla {

constexpr float kE4M3Max = 448.f;
constexpr float kInt8Max = 127.f;
enum { kFmtE4M3 = 0, kFmtInt8 = 1 };
template <int FMT>
constexpr float fmt_max() { return FMT == kFmtInt8 ? kInt8Max : kE4M3Max; }

// int8 codes of 4 floats (round to nearest even, saturating at +-127)
__device__ __forceinline__ u32 cvt4_i8(float a, float b, float c, float d) {
  auto q = [](float v) { return (u32)(uint8_t)(int8_t)(int)rintf(fminf(fmaxf(v, -kInt8Max), kInt8Max)); };
  return q(a) | (q(b) << 8) | (q(c) << 16) | (q(d) << 24);
}

// e4m3 codes of 4 floats (round to nearest even; the caller keeps |x| <= 448)
__device__ __forceinline__ u32 cvt4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (u32)w;
}
__device__ __forceinline__ float sat(float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); }

// key position inside a transposed V8 row: lane group g of the PV MFMA reads bytes
// 32g .. 32g + 31, k-slot 16kt + 4q + e <-> key 32kt + 8q + 4g + e
__host__ __device__ __forceinline__ int v8_pos(int n) {
  const int kt = n / 32, q = (n % 32) / 8, g = (n % 8) / 4, e = n % 4;
  return 32 * g + 16 * kt + 4 * q + e;
}

template <int FMT>
__device__ __forceinline__ u32 qz_cvt4(float a, float b, float c, float d) {
  if constexpr (FMT == kFmtInt8)
    return cvt4_i8(a, b, c, d);
  else
    return cvt4_e4m3(sat(a), sat(b), sat(c), sat(d));
}

// this thread's largest |x| over its chunks
template <int PER>
__device__ __forceinline__ float qz_local_amax(const i32x4 (&r)[PER]) {
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, r[u]);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(bf2f(v[e])));
  }
  return amax;
}
template <int FMT>
__device__ __forceinline__ float qz_inv(float amax) { return amax > 0.f ? fmt_max<FMT>() / amax : 0.f; }
template <int FMT>
__device__ __forceinline__ float qz_scale(float amax) { return amax > 0.f ? amax / fmt_max<FMT>() : 1.f; }

// the 8 codes of one chunk, row-major
template <int FMT>
__device__ __forceinline__ uint2 qz_row_codes(i32x4 chunk, float inv) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, chunk);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = bf2f(v[e]) * inv;
  return make_uint2(qz_cvt4<FMT>(y[0], y[1], y[2], y[3]), qz_cvt4<FMT>(y[4], y[5], y[6], y[7]));
}

// The transposed [D][64] byte tile in LDS: byte pos of channel row c sits at word
// (pos / 4) ^ (c / 8) of the row (the words of a row permuted by the row's 8-channel group), so
// that the 16 lanes writing one byte position of 16 channel groups at once hit 16 different
// words (unpermuted, every row's byte pos falls in the same bank).
__host__ __device__ __forceinline__ int qz_tr_word(int c, int w) { return ((w ^ (c >> 3)) & 15); }
__host__ __device__ __forceinline__ int qz_tr_at(int c, int pos) { return c * kBlock + (qz_tr_word(c, pos >> 2) << 2) + (pos & 3); }

// the 8 codes of the chunk (row r, channels 8 ch .. + 7) into the transposed tile
template <int FMT>
__device__ __forceinline__ void qz_tr_codes(i32x4 chunk, float inv, uint8_t* tl, int r, int ch) {
  const uint2 c = qz_row_codes<FMT>(chunk, inv);
  const int pos = v8_pos(r);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    tl[qz_tr_at(ch * 8 + e, pos)] = (uint8_t)(c.x >> (8 * e));
    tl[qz_tr_at(ch * 8 + 4 + e, pos)] = (uint8_t)(c.y >> (8 * e));
  }
}

// the transposed tile from LDS to its block's place in memory ([D][64] bytes, keys in v8_pos
// order), 16 bytes per store
template <int D, int THREADS>
__device__ __forceinline__ void qz_tr_flush(const uint8_t* tl, uint8_t* dst, int tid) {
  for (int q = tid; q < D * kBlock / 16; q += THREADS) {
    const int c = q / 4, k = q % 4;
    const u32* row = reinterpret_cast<const u32*>(tl + c * kBlock);
    i32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (int)row[qz_tr_word(c, 4 * k + i)];
    *reinterpret_cast<i32x4*>(dst + q * 16) = v;
  }
}

}  // namespace sla
