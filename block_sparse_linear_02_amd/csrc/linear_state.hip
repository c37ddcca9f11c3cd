// linear_state.hip - per-key-block states of the ReLU linear branch on gfx950.
//
// The linear branch ("SALAD: Achieve High-Sparsity Attention via Efficient Linear Attention
// Tuning for Video Diffusion Transformer", section 2: ReLU kernel function; SLA2 Italian summary
// section 1: it covers what the sparse branch leaves out) needs, per key block j,
//   h_j = relu(K_j)^T V_j  [d x d]   and   z_j = relu(K_j)^T 1  [d],
// and their totals H = sum_j h_j, Z = sum_j z_j per (batch, head).
//
//   state_kernel   one workgroup per (chunk of key blocks, head).  Each 64-token tile of K and
//                  V is streamed from HBM with 16-byte coalesced loads (the next tile's loads
//                  are in flight while the current one is used) into row-major LDS tiles; the
//                  4 wavefronts read them back transposed (ds_read_b64_tr_b16) as MFMA operands
//                  and accumulate H^T = V^T relu(K) (bf16 MFMA, fp32 accumulation) for the
//                  chunk, z_j by fp32 sums.  Literal mode also stores every h_j (fp32); the
//                  mask-product mode stores every h_j^T rounded to bf16.  With a low-bit
//                  sparse branch it also writes each block's K and V codes and scales from the
//                  tiles' registers (SLA2 Italian summary section 2.C: the forward quantises K
//                  and V), so the quantiser does not read K and V again.
//   reduce_kernel  sums the chunk partials in a fixed order (deterministic), splits H^T into
//                  bf16 hi + lo parts (the sparse kernel's MFMA operand) and writes Z.
#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"
#include "sla_quant.hpp"

namespace sla {

namespace {

constexpr int kStateThreads = 256;

// MODE: 0 totals only, 1 also every h_j in fp32 in the natural layout h_j[c'][c] (K channel
// major), 2 also every h_j^T[c][c'] (V channel major) rounded to bf16, stored in slices of 64
// entries, slice-major, so that one slice of all blocks is contiguous.
// QF (bf16 inputs, d = 128): -1 nothing more; kFmtE4M3 or kFmtInt8: also the low-bit sparse
// branch's per-block codes and scales of K (row-major) and V (transposed per block), from the
// tiles' registers on their way to LDS, the same bytes as the stand-alone quantiser (the
// quantisation helpers are shared), so K and V are read once for both
template <class T, int D, int MODE, int QF = -1>
__global__ __launch_bounds__(kStateThreads, QF >= 0 ? 2 : 1) void state_kernel(
    const T* __restrict__ K, const T* __restrict__ V, int N, int nb, int cb,
    float* __restrict__ zb, float* __restrict__ h_part, float* __restrict__ z_part,
    void* __restrict__ hj, const uint32_t* __restrict__ flags,
    uint8_t* __restrict__ k8 = nullptr, uint8_t* __restrict__ v8t = nullptr,
    float* __restrict__ sk = nullptr, float* __restrict__ sv = nullptr) {
  constexpr bool QUANT = QF >= 0;
  static_assert(!QUANT || (sizeof(T) == 2 && D == 128), "the quantised branch takes bf16, d = 128");
  constexpr bool LITERAL = MODE != 0;
  // MODE 2 computes h_j = relu(K_j)^T V_j (rows: K channels) so that a lane's four consecutive
  // accumulator rows are four consecutive entries of a row of h_j^T; the others V^T relu(K)
  constexpr bool SWAP = MODE == 2;
  constexpr int NT = D / 64;  // 32x32 output tiles per wave per dimension (D=128: 2, D=64: 1)
  __shared__ __attribute__((aligned(16))) __bf16 Ks[TileLayout<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[TileLayout<D>::ELEMS];
  __shared__ float zred[kStateThreads / D][D];
  __shared__ float qmax[2][kStateThreads / kWave];  // per-wavefront absmax of the K and V tiles
  __shared__ __attribute__((aligned(16))) uint8_t tl[QUANT ? D * kBlock : 16];  // V codes, transposed

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int nchunk = gridDim.x;
  if (flags && (flags[bh] & kDropLinear)) return;  // the head's linear branch is dropped
  const int j0 = chunk * cb;
  const int j1 = min(nb, j0 + cb);
  const T* Kb = K + (size_t)bh * N * D;
  const T* Vb = V + (size_t)bh * N * D;

  // wave -> (rows c of H^T = V channels, cols c' = K channels)
  const int r0 = (wave / 2) * 32 * NT;
  const int c0 = (wave % 2) * 32 * NT;

  // MODE 2 needs no totals of h (its linear branch sums the unselected h_j directly)
  constexpr bool TOT = MODE == 1;
  f32x16 acc[NT][NT];
  f32x16 tot[TOT ? NT : 1][TOT ? NT : 1];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f32x16{};
  if constexpr (TOT) {
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int b = 0; b < NT; ++b) tot[a][b] = f32x16{};
  }
  float zsum = 0.f;  // thread tid < D: running chunk z for channel tid

  TileLoader<T, D, kStateThreads> lk, lv;
  lk.load(Kb + (size_t)j0 * kBlock * D, min(kBlock, N - j0 * kBlock), tid);
  lv.load(Vb + (size_t)j0 * kBlock * D, min(kBlock, N - j0 * kBlock), tid);

  for (int j = j0; j < j1; ++j) {
    __syncthreads();  // previous tile fully consumed
    if constexpr (QUANT) {
      // the previous block's V codes, staged below in its iteration
      if (j > j0) qz_tr_flush<D, kStateThreads>(tl, v8t + ((size_t)bh * nb + j - 1) * D * kBlock, tid);
      const float ak = wave_max(qz_local_amax(lk.r)), av = wave_max(qz_local_amax(lv.r));
      if (lane == 0) {
        qmax[0][wave] = ak;
        qmax[1][wave] = av;
      }
    }
    lk.store(Ks, tid);
    lv.store(Vs, tid);
    __syncthreads();
    if constexpr (QUANT) {
      // block j's scales and codes from the registers, before they take the next tile's loads
      float ak = qmax[0][0], av = qmax[1][0];
#pragma unroll
      for (int w = 1; w < kStateThreads / kWave; ++w) {
        ak = fmaxf(ak, qmax[0][w]);
        av = fmaxf(av, qmax[1][w]);
      }
      const float ik = qz_inv<QF>(ak), iv = qz_inv<QF>(av);
      if (tid == 0) {
        sk[(size_t)bh * nb + j] = qz_scale<QF>(ak);
        sv[(size_t)bh * nb + j] = qz_scale<QF>(av);
      }
      const int cnt = min(kBlock, N - j * kBlock);
      constexpr int CPR = D / 8;
#pragma unroll
      for (int u = 0; u < kBlock * CPR / kStateThreads; ++u) {
        const int q = tid + u * kStateThreads, r = q / CPR, ch = q % CPR;
        if (r < cnt)
          *reinterpret_cast<uint2*>(k8 + ((size_t)bh * N + (size_t)j * kBlock + r) * D + ch * 8) =
              qz_row_codes<QF>(lk.r[u], ik);
        qz_tr_codes<QF>(lv.r[u], iv, tl, r, ch);
      }
    }
    if (j + 1 < j1) {
      const int nv = min(kBlock, N - (j + 1) * kBlock);
      lk.load(Kb + (size_t)(j + 1) * kBlock * D, nv, tid);
      lv.load(Vb + (size_t)(j + 1) * kBlock * D, nv, tid);
    }
#pragma unroll
    for (int ks = 0; ks < kBlock / 16; ++ks) {
      bf16x8 av[NT], bk[NT];
#pragma unroll
      for (int a = 0; a < NT; ++a) av[a] = tr_operand<D, 8, 4>(Vs, 16 * ks, r0 + 32 * a, lane);
#pragma unroll
      for (int b = 0; b < NT; ++b) bk[b] = relu8(tr_operand<D, 8, 4>(Ks, 16 * ks, c0 + 32 * b, lane));
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b)
          acc[a][b] = SWAP ? mfma32(bk[b], av[a], acc[a][b]) : mfma32(av[a], bk[b], acc[a][b]);
    }
    // z_j = sum over the tile's rows of relu(K)
    {
      constexpr int PARTS = kStateThreads / D;
      const int c = tid % D, part = tid / D;
      float s = 0.f;
#pragma unroll 8
      for (int n = part * (kBlock / PARTS); n < (part + 1) * (kBlock / PARTS); ++n)
        s += fmaxf(bf2f(Ks[TileLayout<D>::off(n, c)]), 0.f);
      zred[part][c] = s;
    }
    if constexpr (MODE == 1) {
      // store h_j in natural layout h_j[c'][c]; lane holds c' = col, c = rows 8(i/4)+4g+i%4
      const size_t hoff = ((size_t)bh * nb + j) * D * D;
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b) {
          const int cp = c0 + 32 * b + lane % 32;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = r0 + 32 * a + 8 * q + 4 * (lane / 32);
            f32x4 v = {acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                       acc[a][b][4 * q + 3]};
            *reinterpret_cast<f32x4*>(static_cast<float*>(hj) + hoff + (size_t)cp * D + c) = v;
          }
          tot[a][b] += acc[a][b];
          acc[a][b] = f32x16{};
        }
    }
    if constexpr (MODE == 2) {
      // h_j^T[c][c'] in bf16, in 64-entry slices, slice-major ([bh][n / 64][j][n % 64] with
      // n = c D + c').  The wave's quadrant (c = r0 + 0..32NT-1, c' = c0 + 0..32NT-1) is staged
      // in LDS, where the K and V tiles are no longer needed, as rows of c' (16-byte chunks
      // XOR-swizzled by row), then stored with 16-byte writes.
      constexpr int RL = 32 * NT;          // entries per staged row
      constexpr int CH = RL / 8;           // 16-byte chunks per row
      constexpr int RPL = 128 / RL;        // rows per 256-byte line of banks
      auto soff = [&](int row, int chunk) { return row * RL + ((chunk ^ ((row / RPL) & (CH - 1))) << 3); };
      __syncthreads();  // every wave is done reading Ks and Vs
      __bf16* stg = (wave < 2 ? Ks : Vs) + (wave % 2) * RL * RL;
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // rows c' = c0 + 32 b + 8 q + 4 g + e, column c = r0 + 32 a + lane % 32
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = f2bf(acc[a][b][4 * q + e]);
            const int row = 32 * a + lane % 32, col = 32 * b + 8 * q + 4 * (lane / 32);
            *reinterpret_cast<bf16x4*>(stg + soff(row, col / 8) + (col & 4)) = v;
          }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __bf16* dst = static_cast<__bf16*>(hj);
#pragma unroll
      for (int u = 0; u < RL * CH / kWave; ++u) {
        const int k = lane + kWave * u;
        const int row = k / CH, chunk = k % CH;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + soff(row, chunk));
        const int n = (r0 + row) * D + c0 + 8 * chunk;
        *reinterpret_cast<bf16x8*>(dst + (((size_t)bh * (D * D / 64) + n / 64) * nb + j) * 64 + n % 64) = v;
      }
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b) acc[a][b] = f32x16{};
    }
    __syncthreads();
    if (tid < D) {
      float z = 0.f;
#pragma unroll
      for (int p = 0; p < kStateThreads / D; ++p) z += zred[p][tid];
      zb[((size_t)bh * nb + j) * D + tid] = z;
      zsum += z;
    }
  }

  // the last block's V codes (staged before the loop's last barrier)
  if constexpr (QUANT) {
    if (j1 > j0) qz_tr_flush<D, kStateThreads>(tl, v8t + ((size_t)bh * nb + j1 - 1) * D * kBlock, tid);
  }

  // chunk partial of H^T [c][c'] (not in MODE 2) and Z
  if constexpr (MODE != 2) {
    float* hp = h_part + ((size_t)bh * nchunk + chunk) * D * D;
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int b = 0; b < NT; ++b) {
        const f32x16 v = TOT ? tot[TOT ? a : 0][TOT ? b : 0] : acc[a][b];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = r0 + 32 * a + 8 * (i / 4) + 4 * (lane / 32) + i % 4;
          const int cp = c0 + 32 * b + lane % 32;
          hp[(size_t)c * D + cp] = v[i];
        }
      }
  }
  if (tid < D) z_part[((size_t)bh * nchunk + chunk) * D + tid] = zsum;
}

// One workgroup per 256 consecutive elements of H^T (64 float4 columns): thread t sums every
// fourth chunk partial starting at chunk t / 64 for the float4 column t % 64, then the four
// partial sums are added in a fixed order through LDS (deterministic).  Without chunk partials of
// H (h_part null, mask-product mode) only Z is reduced; without z_part only H.
template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ h_part,
                                                     const float* __restrict__ z_part,
                                                     int nchunk, __bf16* __restrict__ ht_hi,
                                                     __bf16* __restrict__ ht_lo,
                                                     float* __restrict__ Z,
                                                     float* __restrict__ h_full) {
  __shared__ f32x4 part[4][64];
  const int bh = blockIdx.y;
  const int col = threadIdx.x % 64, grp = threadIdx.x / 64;
  if (h_part) {
    const int e4 = blockIdx.x * 64 + col;  // float4 index into H^T
    const f32x4* hp = reinterpret_cast<const f32x4*>(h_part + (size_t)bh * nchunk * D * D);
    constexpr int ROW4 = D * D / 4;  // float4s per chunk partial
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    int k = grp;
    for (; k + 12 < nchunk; k += 16) {  // four loads in flight
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = hp[(size_t)(k + 4 * u) * ROW4 + e4];
#pragma unroll
      for (int u = 0; u < 4; ++u) s += v[u];
    }
    for (; k < nchunk; k += 4) s += hp[(size_t)k * ROW4 + e4];
    part[grp][col] = s;
    __syncthreads();
    if (grp == 0) {
      const f32x4 t = ((part[0][col] + part[1][col]) + part[2][col]) + part[3][col];
      bf16x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = f2bf(t[e]);
        lo[e] = f2bf(t[e] - bf2f(hi[e]));
      }
      const size_t o = (size_t)bh * D * D + 4 * (size_t)e4;
      *reinterpret_cast<bf16x4*>(ht_hi + o) = hi;
      if (ht_lo) *reinterpret_cast<bf16x4*>(ht_lo + o) = lo;
      if (h_full) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int el = 4 * e4 + e;  // element of H^T: c = el / D, c' = el % D
          h_full[(size_t)bh * D * D + (size_t)(el % D) * D + el / D] = t[e];
        }
      }
    }
  }
  if (z_part && blockIdx.x == 0 && threadIdx.x < D) {
    // in chunk order (deterministic), sixteen loads in flight
    const float* zp = z_part + (size_t)bh * nchunk * D + threadIdx.x;
    float z = 0.f;
    int c = 0;
    for (; c + 16 <= nchunk; c += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = zp[(size_t)(c + u) * D];
#pragma unroll
      for (int u = 0; u < 16; ++u) z += v[u];
    }
    for (; c < nchunk; ++c) z += zp[(size_t)c * D];
    Z[(size_t)bh * D + threadIdx.x] = z;
  }
}

template <class T, int D>
hipError_t launch_states_t(const Dims& p, const void* K, const void* V, float* zb,
                           float* h_part, float* z_part, float* hj, __bf16* hj_bf,
                           hipStream_t stream, const uint32_t* flags, const StateQuant* q) {
  const int cb = state_chunk_blocks(p, hj != nullptr || hj_bf == nullptr);
  dim3 grid((p.nb + cb - 1) / cb, p.B * p.H);
  if constexpr (sizeof(T) == 2 && D == 128) {
    if (q) {  // the low-bit branch's K and V codes on the way (no literal mode, no dropped heads)
      auto go = [&](auto kern, void* out) {
        kern<<<grid, kStateThreads, 0, stream>>>((const T*)K, (const T*)V, p.N, p.nb, cb, zb, h_part,
                                                 z_part, out, nullptr, q->k8, q->v8t, q->sk, q->sv);
        return hipGetLastError();
      };
      if (hj_bf)
        return q->int8 ? go(state_kernel<T, D, 2, kFmtInt8>, hj_bf) : go(state_kernel<T, D, 2, kFmtE4M3>, hj_bf);
      return q->int8 ? go(state_kernel<T, D, 0, kFmtInt8>, nullptr) : go(state_kernel<T, D, 0, kFmtE4M3>, nullptr);
    }
  }
  if (hj)
    state_kernel<T, D, 1><<<grid, kStateThreads, 0, stream>>>(
        (const T*)K, (const T*)V, p.N, p.nb, cb, zb, h_part, z_part, hj, flags);
  else if (hj_bf)
    state_kernel<T, D, 2><<<grid, kStateThreads, 0, stream>>>(
        (const T*)K, (const T*)V, p.N, p.nb, cb, zb, h_part, z_part, hj_bf, flags);
  else
    state_kernel<T, D, 0><<<grid, kStateThreads, 0, stream>>>(
        (const T*)K, (const T*)V, p.N, p.nb, cb, zb, h_part, z_part, nullptr, flags);
  return hipGetLastError();
}

}  // namespace

int state_chunk_blocks(const Dims& p, bool h_partials) {
  // about >= 512 workgroups (two per CU) while keeping the partials of h (64 KB per chunk at
  // d = 128) small next to the K/V stream (32 KB per block); a launch without them (the
  // mask-product mode, whose chunk partials are z alone) takes about >= 1024, which keeps more
  // tile loads in flight
  const long work = (long)p.nb * p.B * p.H;
  long cb = work / (h_partials ? 512 : 1024);
  if (cb < 1) cb = 1;
  if (cb > 64) cb = 64;
  return (int)cb;
}

hipError_t launch_states(const Dims& p, const void* K, const void* V, float* zb, float* h_part,
                         float* z_part, float* hj, __bf16* hj_bf,
                         hipStream_t stream, const uint32_t* flags, const StateQuant* q) {
  if (q && (hj || flags || p.dtype != kBF16 || p.d != 128)) return hipErrorInvalidValue;
  if (p.dtype == kBF16 && p.d == 128)
    return launch_states_t<__bf16, 128>(p, K, V, zb, h_part, z_part, hj, hj_bf, stream, flags, q);
  if (p.dtype == kBF16 && p.d == 64)
    return launch_states_t<__bf16, 64>(p, K, V, zb, h_part, z_part, hj, hj_bf, stream, flags, q);
  if (p.dtype == kF32 && p.d == 128)
    return launch_states_t<float, 128>(p, K, V, zb, h_part, z_part, hj, hj_bf, stream, flags, q);
  return launch_states_t<float, 64>(p, K, V, zb, h_part, z_part, hj, hj_bf, stream, flags, q);
}

hipError_t launch_state_reduce(const Dims& p, const float* h_part, const float* z_part,
                               __bf16* ht_hi, __bf16* ht_lo, float* Z, float* h_full,
                               hipStream_t stream) {
  const int cb = state_chunk_blocks(p, h_part != nullptr);
  const int nchunk = (p.nb + cb - 1) / cb;
  // 256 elements (64 float4 columns) of H^T per workgroup; Z alone without chunk partials of H
  dim3 grid(h_part ? p.d * p.d / 256 : 1, p.B * p.H);
  if (p.d == 128)
    reduce_kernel<128><<<grid, 256, 0, stream>>>(h_part, z_part, nchunk, ht_hi, ht_lo, Z, h_full);
  else
    reduce_kernel<64><<<grid, 256, 0, stream>>>(h_part, z_part, nchunk, ht_hi, ht_lo, Z, h_full);
  return hipGetLastError();
}

}  // namespace sla
