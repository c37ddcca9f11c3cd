// linear_gemm.hip - the linear branch's per-query-block states for all query blocks at once.
//
// The linear branch of query block i uses the states of the key blocks the router did not keep
// (SLA2 Italian summary section 1 and Arabic summary section 1: the linear part covers what the
// sparse branch leaves; SALAD section 2: ReLU features), A_i = H - sum_{j in sel(i)} h_j with
// h_j = relu(K_j)^T V_j and H = sum_j h_j.  Written as a product over the 0/1 mask M of the
// router (M[i][j] = 1 iff j in sel(i)):
//     S_sel = M h,   h = [n_b][d*d] (every block's state, flattened),   A = H - S_sel,
// one dense GEMM of 2 n_b^2 d^2 flops per head.  That is far less work than rebuilding
// sum_sel h_j for every query block from K and V (2 * 64 * d^2 flops per kept pair), because
// each h_j is formed once and the n_b / k factor of the mask replaces the 64 rows of a block.
//
//   mask_bits_kernel  per (b, h, query block): the ascending index list -> a bit row of n_b
//                     bits (32-bit words), the GEMM's B operand source.
//   tsel_kernel       C^T = h^T M^T on v_mfma_f32_32x32x16_bf16: rows = 64 columns of h (a slice
//                     of the d*d state entries), columns = 512 query blocks, k = key blocks in
//                     stages of 64.  h is stored as bf16 hi + lo (about fp32 precision, the two
//                     halves accumulated into the same fp32 accumulator); the h stage goes
//                     HBM -> LDS by direct loads into rows of 128 bytes whose 16-byte chunks are
//                     XOR-swizzled (chunk c of row j at c ^ 4((j >> 1) & 1)) so that the
//                     transposed operand reads (ds_read_b64_tr_b16) hit distinct banks; the mask
//                     operand is 8 bits per lane turned into eight bf16 0/1 values through a
//                     256-entry LDS table.  Epilogue: A = H - S_sel as bf16 hi + lo, in the
//                     transposed state layout [c][c'] (V channel major) per query block.
#include <type_traits>

#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kGemmN = 64;    // state entries (rows of C^T) per workgroup
constexpr int kGemmM = 512;   // query blocks (columns of C^T) per workgroup
constexpr int kGemmCT = kGemmM / 4 / 32;  // 32-column tiles per wavefront
constexpr int kGemmK = 64;    // key blocks per LDS stage

__global__ __launch_bounds__(256) void mask_bits_kernel(const int32_t* __restrict__ idx, int nb,
                                                        int topk, int nw,
                                                        uint32_t* __restrict__ bits) {
  // one thread per (query block, 32-bit word): the word's bits are the contiguous run of the
  // ascending list that falls in [32 w, 32 w + 32), found by binary search
  const int bh = blockIdx.y;
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= nb * nw) return;
  const int i = q / nw, w = q % nw;
  uint32_t word = 0;
  if (topk > 0) {
    const int32_t* sel = idx + ((size_t)bh * nb + i) * topk;
    int lo = 0, hi = topk;  // first entry >= 32 w
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (sel[mid] < 32 * w) lo = mid + 1; else hi = mid;
    }
    for (int p = lo; p < topk && sel[p] < 32 * (w + 1); ++p) word |= 1u << (sel[p] - 32 * w);
  }
  bits[((size_t)bh * nb + i) * nw + w] = word;
}

// byte offset of element (row j, column c) of an h stage tile [kGemmK][kGemmN] bf16
__device__ __forceinline__ int hs_off(int j, int c) {
  return j * 128 + ((((c >> 3) ^ (4 * ((j >> 1) & 1)))) << 4) + (c & 7) * 2;
}

template <int D>
__global__ __launch_bounds__(kGemmThreads, 2) void tsel_kernel(
    const __bf16* __restrict__ hj_hi, const __bf16* __restrict__ hj_lo,
    const uint32_t* __restrict__ bits, const __bf16* __restrict__ ht_hi,
    const __bf16* __restrict__ ht_lo, int nb, int nw, int tiles_m, int tiles_n,
    __bf16* __restrict__ t_hi, __bf16* __restrict__ t_lo) {
  constexpr int DD = D * D;
  constexpr int STAGE = kGemmK * kGemmN;  // bf16 elements of one h stage (hi or lo)
  __shared__ __attribute__((aligned(16))) __bf16 sb0[2 * STAGE];  // buffer 0: hi, lo
  __shared__ __attribute__((aligned(16))) __bf16 sb1[2 * STAGE];  // buffer 1: hi, lo
  __shared__ __attribute__((aligned(16))) bf16x8 lut[256];         // 8 bits -> eight bf16 0/1
  auto buf = [&](auto B) -> __bf16* { return decltype(B)::value ? sb1 : sb0; };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave, g = lane / 32;
  // workgroup -> (query-block tile, state slice, head) with the query-block tiles fastest, so
  // that the workgroups reading the same slice of h run next to each other on one XCD
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = item % tiles_m;
  const int nt = (item / tiles_m) % tiles_n;
  const int bh = item / (tiles_m * tiles_n);
  const int n0 = nt * kGemmN;
  const int i0 = mt * kGemmM + 32 * kGemmCT * w;  // this wavefront's query blocks

  {
    const int b = tid;  // 256 threads, 256 entries
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ((b >> e) & 1) ? f2bf(1.f) : f2bf(0.f);
    lut[b] = v;
  }

  // this workgroup's slice of every block's state: [j][64] contiguous (slice-major layout)
  const __bf16* hh = hj_hi + ((size_t)bh * (DD / kGemmN) + nt) * nb * kGemmN;
  const __bf16* hl = hj_lo + ((size_t)bh * (DD / kGemmN) + nt) * nb * kGemmN;
  const uint32_t* brow = bits + (size_t)bh * nb * nw;
  const int nstage = (nb + kGemmK - 1) / kGemmK;

  // stage s: rows j = 64 s .. 64 s + 63 (clamped to n_b - 1: their mask bits are 0), 128 bytes
  // each, hi then lo; wavefront w loads rows 16 w .. 16 w + 15 of both (8 rows per 1 KB load)
  auto stage = [&](int s, auto BUFC) {
    __bf16* dst = buf(BUFC);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r0 = 16 * w + 8 * u;
      const int r = r0 + lane / 8;
      const int j = min(kGemmK * s + r, nb - 1);
      const int chunk = (lane % 8) ^ (4 * ((r >> 1) & 1));
      load_lds16(hh + (size_t)j * kGemmN + chunk * 8, dst + r0 * kGemmN);
      load_lds16(hl + (size_t)j * kGemmN + chunk * 8, dst + STAGE + r0 * kGemmN);
    }
  };
  // mask words of this lane's query-block columns (i0 + 32 ct + lane % 32) for stage s
  uint32_t mw[kGemmCT][2];
  auto mask_words = [&](int s) {
#pragma unroll
    for (int ct = 0; ct < kGemmCT; ++ct) {
      const int i = min(i0 + 32 * ct + lane % 32, nb - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int word = 2 * s + h;
        mw[ct][h] = word < nw ? brow[(size_t)i * nw + word] : 0u;
      }
    }
  };

  f32x16 acc[2][kGemmCT];  // [state row tile][query-block column tile]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < kGemmCT; ++b) acc[a][b] = f32x16{};

  auto tr_a = [&](const __bf16* tile, int row0, int col0) -> bf16x8 {
    // A operand (h^T): lane gets column col0 + lane%32 at rows row0 + 8g + {0..3} and {4..7}
    const int hq = lane / 16, L = lane % 16;
    const int gg = hq / 2, cs = hq % 2;
    const int r = row0 + 8 * gg + L / 4;
    const int c = col0 + 16 * cs + 4 * (L % 4);
    const char* base = reinterpret_cast<const char*>(tile);
    return join_tr(lds_read_tr16(reinterpret_cast<const __bf16*>(base + hs_off(r, c))),
                   lds_read_tr16(reinterpret_cast<const __bf16*>(base + hs_off(r + 4, c))));
  };

  stage(0, B0{});
  mask_words(0);
  wait_vmem();
  __syncthreads();
  auto step = [&](int s, auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    uint32_t cur[kGemmCT][2];
#pragma unroll
    for (int ct = 0; ct < kGemmCT; ++ct)
#pragma unroll
      for (int h = 0; h < 2; ++h) cur[ct][h] = mw[ct][h];
    if (s + 1 < nstage) {
      stage(s + 1, std::integral_constant<int, 1 - BUF>{});
      mask_words(s + 1);
    }
    const __bf16* tile = buf(BUFC);
#pragma unroll
    for (int ks = 0; ks < kGemmK / 16; ++ks) {
      // mask operand: bits 16 ks + 8 g .. + 7 of the stage, i.e. of word ks / 2
      bf16x8 bm[kGemmCT];
#pragma unroll
      for (int ct = 0; ct < kGemmCT; ++ct) bm[ct] = lut[(cur[ct][ks / 2] >> (16 * (ks % 2) + 8 * g)) & 0xff];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const bf16x8 ah = tr_a(tile, 16 * ks, 32 * a);
        const bf16x8 al = tr_a(tile + STAGE, 16 * ks, 32 * a);
#pragma unroll
        for (int ct = 0; ct < kGemmCT; ++ct) {
          acc[a][ct] = mfma32(al, bm[ct], acc[a][ct]);
          acc[a][ct] = mfma32(ah, bm[ct], acc[a][ct]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  for (int s = 0; s < nstage; s += 2) {
    step(s, B0{});
    if (s + 1 < nstage) step(s + 1, B1{});
  }

  // T = H - S_sel for this wavefront's query blocks: lane holds query block i0 + 32 ct + lane%32
  // and state entries n0 + 32 a + 8 q + 4 g + {0..3}; H from its bf16 hi + lo parts
  const __bf16* hh1 = ht_hi + (size_t)bh * DD + n0;
  const __bf16* hh0 = ht_lo + (size_t)bh * DD + n0;
#pragma unroll
  for (int ct = 0; ct < kGemmCT; ++ct) {
    const int i = i0 + 32 * ct + lane % 32;
    if (i >= nb) continue;
    __bf16* oh = t_hi + ((size_t)bh * nb + i) * DD + n0;
    __bf16* ol = t_lo + ((size_t)bh * nb + i) * DD + n0;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = 32 * a + 8 * q + 4 * g;
        const bf16x4 h1 = *reinterpret_cast<const bf16x4*>(hh1 + n);
        const bf16x4 h0 = *reinterpret_cast<const bf16x4*>(hh0 + n);
        bf16x4 vh, vl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float tv = (bf2f(h1[e]) + bf2f(h0[e])) - acc[a][ct][4 * q + e];
          vh[e] = f2bf(tv);
          vl[e] = f2bf(tv - bf2f(vh[e]));
        }
        *reinterpret_cast<bf16x4*>(oh + n) = vh;
        *reinterpret_cast<bf16x4*>(ol + n) = vl;
      }
  }
}

}  // namespace

int mask_words(int nb) { return (nb + 31) / 32; }

hipError_t launch_mask_bits(const Dims& p, const int32_t* idx, uint32_t* bits,
                            hipStream_t stream) {
  const int nw = mask_words(p.nb);
  dim3 grid((p.nb * nw + 255) / 256, p.B * p.H);
  mask_bits_kernel<<<grid, 256, 0, stream>>>(idx, p.nb, p.topk, nw, bits);
  return hipGetLastError();
}

hipError_t launch_tsel(const Dims& p, const __bf16* hj_hi, const __bf16* hj_lo,
                       const uint32_t* bits, const __bf16* ht_hi, const __bf16* ht_lo,
                       __bf16* t_hi, __bf16* t_lo, hipStream_t stream) {
  const int tiles_m = (p.nb + kGemmM - 1) / kGemmM;
  const int tiles_n = p.d * p.d / kGemmN;
  const int total = tiles_m * tiles_n * p.B * p.H;
  if (p.d == 128)
    tsel_kernel<128><<<total, kGemmThreads, 0, stream>>>(hj_hi, hj_lo, bits, ht_hi, ht_lo, p.nb,
                                                         mask_words(p.nb), tiles_m, tiles_n,
                                                         t_hi, t_lo);
  else
    tsel_kernel<64><<<total, kGemmThreads, 0, stream>>>(hj_hi, hj_lo, bits, ht_hi, ht_lo, p.nb,
                                                        mask_words(p.nb), tiles_m, tiles_n,
                                                        t_hi, t_lo);
  return hipGetLastError();
}

}  // namespace sla
