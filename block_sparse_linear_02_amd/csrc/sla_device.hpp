// sla_device.hpp - device-side types and helpers shared by the gfx950 kernels of libsla.
//
// MFMA operand layouts used throughout (64-lane wavefronts, verified on gfx950):
//   v_mfma_f32_32x32x16_bf16: A[32][16]  lane l holds A[l%32][8*(l/32) + 0..7]
//                             B[16][32]  lane l holds B[8*(l/32) + 0..7][l%32]
//                             C[32][32]  lane l, reg i holds C[8*(i/4) + 4*(l/32) + i%4][l%32]
//   v_mfma_f32_16x16x32_bf16: A[16][32]  lane l holds A[l%16][8*(l/16) + 0..7]
//                             B[32][16]  lane l holds B[8*(l/16) + 0..7][l%16]
//                             C[16][16]  lane l, reg i holds C[4*(l/16) + i][l%16]
// The order of the k-slots inside a lane is free as long as A and B use the same order.
//   ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element (i%4) of the
//   64-bit words read by lanes 4e + i/4, e = 0..3.  With lane L of the group addressing row
//   r0 + L/4, columns c0 + 4*(L%4) .. +3 of a row-major bf16 tile, lane i receives
//   T[r0 + e][c0 + i], e = 0..3: four consecutive rows of one column.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32;

constexpr int kBlock = 64;   // tokens per block (the compiled block size)
constexpr int kWave = 64;    // gfx950 wavefront size

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 <-> float (round to nearest even; the gfx950 conversion instruction)
__device__ __forceinline__ __bf16 f2bf(float x) { return (__bf16)x; }
__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }

// relu of 8 packed bf16 values with a packed 16-bit integer max: a bf16 with the sign bit set
// is a negative int16, so max(x, 0) as int16 is relu(x) (and maps -0 to +0).
typedef short i16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 relu8(bf16x8 x) {
  const i16x8 v = __builtin_bit_cast(i16x8, x);
  return __builtin_bit_cast(bf16x8, __builtin_elementwise_max(v, i16x8{}));
}

// 2^x on the hardware transcendental unit (v_exp_f32): about 1 ulp; results below 2^-126 may
// flush to zero, which only drops probabilities under 2^-126 of the row maximum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposing LDS read (see the header comment); `p` must point into LDS.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// max / sum of a value and its copy in lane l ^ 32, in every lane (v_permlane32_swap: with
// both operands equal, the two results hold the lower and the upper half-wave values)
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Asynchronous 16-byte global -> LDS copy (gfx950 global_load_lds_dwordx4): lane i's 16 bytes
// land at lds_wave_base + 16 i, the 64 lanes of a wavefront fill 1 KB contiguously.  Completion
// is tracked by vmcnt (wait_vmem() before the barrier that publishes the data).
__device__ __forceinline__ void load_lds16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x3f70); }  // vmcnt(0)

// Buffer resource over `bytes` bytes at `base` (raw buffer: stride 0, the offset is a byte
// offset; reads at or past `bytes` return zero).  Word 3 = 0x00020000 (32-bit data format, no
// swizzle) for gfx9-class buffer instructions.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Asynchronous 16-byte buffer -> LDS copy (gfx950 buffer_load_dwordx4 ... lds): lane i's 16
// bytes from rsrc + voff + soff land at lds_wave_base + 16 i.  voff is per lane (a VGPR), soff
// wavefront-uniform (an SGPR), so a tile walk adds no per-lane address arithmetic.
__device__ __forceinline__ void load_lds16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                               void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           voff, soff, 0, 0);
}

// Wave-wide reductions over all 64 lanes.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Maximum of an int over all 64 lanes, in every lane (all lanes active): DPP inside each row of
// 16 lanes (swap within pairs, then within quads, then the half-row and row mirrors), then the
// four rows' maxima read into scalars.
__device__ __forceinline__ int wave_max_int(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));  // row_mirror
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Order-preserving map of a float to uint32 (larger float -> larger key); -0 and +0 map to
// the same key.
__device__ __forceinline__ u32 float_key(float f) {
  u32 u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16-byte global load/store helpers (addresses must be 16-byte aligned).
template <class T>
__device__ __forceinline__ i32x4 ld16(const T* p) { return *reinterpret_cast<const i32x4*>(p); }
template <class T>
__device__ __forceinline__ void st16(T* p, i32x4 v) { *reinterpret_cast<i32x4*>(p) = v; }

}  // namespace sla
