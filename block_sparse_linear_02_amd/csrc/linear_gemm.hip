// linear_gemm.hip - the linear branch's per-query-block states for all query blocks at once.
//
// The linear branch of query block i uses the states of the key blocks the router did not keep
// (SLA2 Italian summary section 1 and Arabic summary section 1: the linear part covers what the
// sparse branch leaves; SALAD section 2: ReLU features), T_i = sum_{j not in sel(i)} h_j with
// h_j = relu(K_j)^T V_j.  Written as a product over the 0/1 complement mask U of the router
// (U[i][j] = 1 iff j < n_b is not in sel(i)):
//     T = U h,   h = [n_b][d*d] (every block's state, flattened),
// one dense GEMM of 2 n_b^2 d^2 flops per head.  That is far less work than summing states per
// query block from K and V (2 * 64 * d^2 flops per block pair), because each h_j is formed once
// and the n_b factor of the mask replaces the 64 rows of a block.  Summing the unselected states
// directly (rather than subtracting the kept ones from the total) keeps the bf16 rounding of h_j
// relative to T_i itself, even when almost every block is kept.
//
//   mask_bits_kernel  per (b, h, query block): the ascending index list -> a bit row of the
//                     unselected blocks (n_b bits in 32-bit words), the GEMM's B operand source.
//   tsel_kernel       T^T = h^T U^T on v_mfma_f32_32x32x16_bf16: rows = 128 columns of h (two
//                     slices of the d*d state entries), columns = 256 query blocks, k = key
//                     blocks in stages of kGemmK; each wavefront takes all 128 rows and 64
//                     columns, so every decoded mask operand feeds four MFMAs.  h is stored in
//                     bf16, the sum is accumulated in fp32 and T is rounded to bf16 once (a
//                     relative error of about 2^-9 on the linear branch's state); the h stage
//                     goes HBM -> LDS by direct loads into rows of 256 bytes whose 16-byte chunks
//                     are XOR-swizzled (chunk c of row j at c ^ 4 (j & 3)) so that the transposed
//                     operand reads (ds_read_b64_tr_b16) of four consecutive rows hit distinct
//                     banks; the mask operand is 8 bits per lane turned into eight bf16 0/1
//                     values by two lookups in a 16-entry LDS table.  Epilogue:
//                     T_i in bf16, in the transposed state layout [c][c'] (V channel major) per
//                     query block, staged through LDS so that every lane stores 16 contiguous
//                     bytes.
#include <type_traits>

#include "sla_device.hpp"
#include "sla_launch.hpp"
#include "sla_tiles.hpp"

namespace sla {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kGemmN = 128;   // state entries (rows of T^T) per workgroup
constexpr int kGemmRT = kGemmN / 32;      // 32-row tiles per wavefront (all of them)
constexpr int kGemmM = 256;   // query blocks (columns of T^T) per workgroup
constexpr int kGemmCT = kGemmM / 4 / 32;  // 32-column tiles per wavefront
constexpr int kGemmK = 128;   // key blocks per LDS stage
constexpr int kGemmKW = kGemmK / 32;      // mask words per stage
constexpr int kSlice = 64;    // entries per slice of the stored h_j^T

__global__ __launch_bounds__(256) void mask_bits_kernel(const int32_t* __restrict__ idx, int nb,
                                                        int topk, int nw,
                                                        uint32_t* __restrict__ bits) {
  // one thread per (query block, 32-bit word): the kept blocks of the word are the contiguous
  // run of the ascending list that falls in [32 w, 32 w + 32), found by binary search; the word
  // is their complement within the blocks j < n_b
  const int bh = blockIdx.y;
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= nb * nw) return;
  const int i = q / nw, w = q % nw;
  const int valid = min(32, nb - 32 * w);
  const uint32_t all = valid == 32 ? 0xffffffffu : (1u << valid) - 1u;
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
  bits[((size_t)bh * nb + i) * nw + w] = all & ~word;
}

// byte offset of element (row j, column c) of an h stage [kGemmK][kGemmN] bf16: rows of 256
// bytes, 16-byte chunk c of row j at c ^ 4 (j & 3)
__device__ __forceinline__ int hs_off(int j, int c) {
  return j * (2 * kGemmN) + (((c >> 3) ^ (4 * (j & 3))) << 4) + (c & 7) * 2;
}

// WT (the SoftTop-k training path): the B operand comes from a bf16 weight matrix wt
// [BH][nb][wpitch] (row i: the weights of the key blocks j for query block i, zero past n_b)
// instead of the complement bits: T_i = sum_j wt[i][j] h_j.
template <int D, bool WT = false>
__global__ __launch_bounds__(kGemmThreads, 2) void tsel_kernel(
    const __bf16* __restrict__ hj, const uint32_t* __restrict__ bits, int nb, int nw,
    int tiles_m, int tiles_n, __bf16* __restrict__ t_out, const uint32_t* __restrict__ flags,
    const __bf16* __restrict__ wt = nullptr, int wpitch = 0) {
  constexpr int DD = D * D;
  constexpr int STAGE = kGemmK * kGemmN;  // bf16 elements of one h stage
  __shared__ __attribute__((aligned(16))) __bf16 sb0[STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 sb1[STAGE];
  // four mask bits -> four bf16 0/1 values: 16 entries of 8 bytes, so the 64 lanes of a lookup
  // touch at most 16 distinct addresses in distinct bank pairs (no conflict; equal addresses
  // are broadcast)
  __shared__ __attribute__((aligned(16))) bf16x4 nib[16];
  auto buf = [&](auto B) -> __bf16* { return decltype(B)::value ? sb1 : sb0; };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave, g = lane / 32;
  if (tid < 16) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = ((tid >> e) & 1) ? f2bf(1.f) : f2bf(0.f);
    nib[tid] = v;
  }
  // workgroup -> (head, query-block tile, state rows) with the query-block tiles fastest, so
  // that the workgroups reading the same rows of h run next to each other on one XCD; every XCD
  // takes the same eighth of every head (a head whose linear branch is dropped does no work)
  int bh, item;
  if (!xcd_chunk_map(blockIdx.x, tiles_m * tiles_n, &bh, &item)) return;
  const int mt = item % tiles_m;
  const int nt = item / tiles_m;
  if (flags && (flags[bh] & kDropLinear)) return;  // the head's linear branch is dropped
  const int n0 = nt * kGemmN;
  const int i0 = mt * kGemmM + 32 * kGemmCT * w;  // this wavefront's query blocks

  // this workgroup's two slices of every block's state (slice-major: [j][64] contiguous each)
  const __bf16* hh = hj + ((size_t)bh * (DD / kSlice) + n0 / kSlice) * nb * kSlice;
  const uint32_t* brow = bits + (size_t)bh * nb * nw;
  const int nstage = (nb + kGemmK - 1) / kGemmK;

  // stage s: rows j = kGemmK s + 0 .. kGemmK - 1, 256 bytes each (chunks 0..7 from the first
  // slice, 8..15 from the second); each 1 KB direct load covers 4 rows, wavefront w loads rows
  // 32 w .. 32 w + 31.  The loads go through a buffer resource over the two slices: the lane's
  // offset is row 32 w + lane / 16 of its chunk's slice (the swizzle depends on the row mod 4
  // only) plus the stage's rows, the 4-row step an immediate offset; the whole offset is in the
  // vector and immediate parts, which the range check covers (the scalar offset is not
  // checked).  Rows past n_b read the second slice's first rows or, past its end, zero: finite
  // values whose mask bits are 0.
  const __amdgpu_buffer_rsrc_t hrs = make_rsrc(hh, (uint32_t)(2 * nb * kSlice * sizeof(__bf16)));
  uint32_t hvoff;
  {
    const int r = (kGemmK / 4) * w + lane / 16;
    const int chunk = (lane % 16) ^ (4 * (r & 3));
    hvoff = (uint32_t)((((chunk / 8) * nb + r) * kSlice + (chunk % 8) * 8) * sizeof(__bf16));
  }
  auto stage = [&](int s, auto BUFC) {
    __bf16* dst = buf(BUFC);
    const uint32_t vs = hvoff + (uint32_t)(kGemmK * s * kSlice * sizeof(__bf16));
#pragma unroll
    for (int u = 0; u < kGemmK / 16; ++u)
      load_lds16_buf(hrs, vs + (uint32_t)(4 * u * kSlice * sizeof(__bf16)), 0u,
                     dst + ((kGemmK / 4) * w + 4 * u) * kGemmN);
  };
  // mask words of this lane's query-block columns (i0 + 32 ct + lane % 32, clamped to n_b - 1)
  // for stage s, through a buffer resource over the head's bit rows (the stage's word offset in
  // the range-checked vector offset): words past a row read the next row's (or, past the last,
  // zero) and are zeroed when used (no branch around the loads
  // and no use right after them: either makes the compiler wait for every outstanding load, the
  // stage prefetch included, on the spot)
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(brow, (uint32_t)((size_t)nb * nw * sizeof(uint32_t)));
  uint32_t mvoff[kGemmCT];
#pragma unroll
  for (int ct = 0; ct < kGemmCT; ++ct)
    mvoff[ct] = (uint32_t)(min(i0 + 32 * ct + lane % 32, nb - 1) * nw * sizeof(uint32_t));
  uint32_t mw[kGemmCT][kGemmKW];
  auto mask_words = [&](int s) {
#pragma unroll
    for (int ct = 0; ct < kGemmCT; ++ct)
#pragma unroll
      for (int h = 0; h < kGemmKW; ++h)
        mw[ct][h] = __builtin_amdgcn_raw_buffer_load_b32(
            brs, (int)(mvoff[ct] + (kGemmKW * s + h) * sizeof(uint32_t)), 0, 0);
  };
  // this wavefront's column tiles with a query block < n_b (wavefront-uniform): the others
  // issue no MFMA
  const int ncv = min(kGemmCT, max(0, (nb - i0 + 31) / 32));

  f32x16 acc[kGemmRT][kGemmCT];  // [state row tile][query-block column tile]
#pragma unroll
  for (int a = 0; a < kGemmRT; ++a)
#pragma unroll
    for (int b = 0; b < kGemmCT; ++b) acc[a][b] = f32x16{};

  // A operand (h^T) of k step ks and row tile a: lane gets column 32 a + lane%32 at rows
  // 16 ks + 8 gg + {0..3} and {4..7}, byte offsets hs_off(16 ks + 8 gg + L/4, 32 a + 16 cs +
  // 4 (L%4)) and 1024 past it, i.e. pa[a] + 4096 ks with pa[a] depending on the lane only (the
  // swizzle depends on j & 3).  The lane parts are laundered through an empty asm so that every
  // read address stays one offset from the stage array: the compiler then keeps track of which
  // array each read touches and does not make the reads of one stage wait for the direct loads
  // into the other.
  int pa[kGemmRT];
  {
    const int hq = lane / 16, L = lane % 16;
    const int gg = hq / 2, cs = hq % 2;
#pragma unroll
    for (int a = 0; a < kGemmRT; ++a) pa[a] = hs_off(8 * gg + L / 4, 32 * a + 16 * cs + 4 * (L % 4));
    asm volatile("" : "+v"(pa[0]), "+v"(pa[1]), "+v"(pa[2]), "+v"(pa[3]));
  }
  auto tr_a = [&](const __bf16* tile, int ks, int a) -> bf16x8 {
    const char* p = reinterpret_cast<const char*>(tile) + pa[a] + 16 * ks * (2 * kGemmN);
    return join_tr(lds_read_tr16(reinterpret_cast<const __bf16*>(p)),
                   lds_read_tr16(reinterpret_cast<const __bf16*>(p + 4 * (2 * kGemmN))));
  };

  stage(0, B0{});
  if constexpr (!WT) mask_words(0);
  wait_vmem();
  __syncthreads();
  auto step = [&](int s, auto BUFC) {
    constexpr int BUF = decltype(BUFC)::value;
    uint32_t cur[kGemmCT][kGemmKW];
#pragma unroll
    for (int ct = 0; ct < kGemmCT; ++ct)
#pragma unroll
      for (int h = 0; h < kGemmKW; ++h) cur[ct][h] = (!WT && kGemmKW * s + h < nw) ? mw[ct][h] : 0u;
    if (s + 1 < nstage) {
      stage(s + 1, std::integral_constant<int, 1 - BUF>{});
      if constexpr (!WT) mask_words(s + 1);
    }
    const __bf16* tile = buf(BUFC);
    // KEDGE: the stage holds fewer than kGemmK key blocks (steps of 16 past n_b are skipped);
    // NCT: the wavefront's column tiles with a query block < n_b (the others issue no MFMA)
    auto compute = [&](auto KEDGEC, auto NCTC) {
      constexpr bool KEDGE = decltype(KEDGEC)::value;
      constexpr int NCT = decltype(NCTC)::value;
      const int rem = nb - kGemmK * s;
#pragma unroll
      for (int ks = 0; ks < kGemmK / 16; ++ks) {
        if (KEDGE && 16 * ks >= rem) break;
        // mask operand: bits 16 ks + 8 g .. + 7 of the stage, i.e. of word ks / 2 (or, WT, the
        // weights of key blocks kGemmK s + 16 ks + 8 g .. + 7)
        bf16x8 bm[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          if constexpr (WT) {
            const int i = min(i0 + 32 * ct + lane % 32, nb - 1);
            bm[ct] = *reinterpret_cast<const bf16x8*>(wt + ((size_t)bh * nb + i) * wpitch + kGemmK * s + 16 * ks + 8 * g);
          } else {
            const u32 byte = (cur[ct][ks / 2] >> (16 * (ks % 2) + 8 * g)) & 0xffu;
            const bf16x4 lo = nib[byte & 15u], hi = nib[byte >> 4];
            bm[ct] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
        bf16x8 ah[kGemmRT];
#pragma unroll
        for (int a = 0; a < kGemmRT; ++a) ah[a] = tr_a(tile, ks, a);
#pragma unroll
        for (int a = 0; a < kGemmRT; ++a)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) acc[a][ct] = mfma32(ah[a], bm[ct], acc[a][ct]);
      }
    };
    static_assert(kGemmCT == 2, "column-tile dispatch below");
    const bool kfull = kGemmK * (s + 1) <= nb;
    if (ncv == kGemmCT && kfull)
      compute(std::false_type{}, std::integral_constant<int, 2>{});
    else if (ncv == kGemmCT)
      compute(std::true_type{}, std::integral_constant<int, 2>{});
    else if (ncv == 1)
      compute(std::true_type{}, std::integral_constant<int, 1>{});
    wait_vmem();
    __syncthreads();
  };
  for (int s = 0; s < nstage; s += 2) {
    step(s, B0{});
    if (s + 1 < nstage) step(s + 1, B1{});
  }

  // T for this wavefront's query blocks: lane holds query block i0 + 32 ct + lane%32 and state
  // entries n0 + 32 a + 8 q + 4 g + {0..3}.  Each 32-query-block tile goes through this
  // wavefront's own 8 KB of buffer 0 (32 rows of 256 bytes, 16-byte chunk c of row r at
  // c ^ (r & 15)) and leaves as 16-byte stores, sixteen lanes per row.  The stage buffers are
  // free: the last step ended with a barrier after every wavefront's reads.
  static_assert(STAGE >= 4 * 32 * kGemmN, "epilogue staging fits stage buffer 0");
  __bf16* stg = sb0 + w * 32 * kGemmN;
  auto eoff = [](int r, int chunk) { return r * kGemmN + ((chunk ^ (r & 15)) << 3); };
#pragma unroll
  for (int ct = 0; ct < kGemmCT; ++ct) {
#pragma unroll
    for (int a = 0; a < kGemmRT; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = f2bf(acc[a][ct][4 * q + e]);
        *reinterpret_cast<bf16x4*>(stg + eoff(lane % 32, 4 * a + q) + 4 * g) = v;
      }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < 32 * (kGemmN / 8) / kWave; ++u) {
      const int k = lane + kWave * u;
      const int r = k / (kGemmN / 8), ch = k % (kGemmN / 8);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + eoff(r, ch));
      const int i = i0 + 32 * ct + r;
      if (i < nb) *reinterpret_cast<bf16x8*>(t_out + ((size_t)bh * nb + i) * DD + n0 + 8 * ch) = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

int mask_words(int nb) { return (nb + 31) / 32; }

int tsel_weight_pitch(int nb) { return (nb + kGemmK - 1) / kGemmK * kGemmK; }

hipError_t launch_tsel_weighted(const Dims& p, const __bf16* hj_bf, const __bf16* wt, __bf16* t_bf,
                                hipStream_t stream) {
  const int tiles_m = (p.nb + kGemmM - 1) / kGemmM;
  const int tiles_n = p.d * p.d / kGemmN;
  const int total = xcd_chunk_grid(p.B * p.H, tiles_m * tiles_n);
  const int wpitch = tsel_weight_pitch(p.nb);
  if (p.d == 128)
    tsel_kernel<128, true><<<total, kGemmThreads, 0, stream>>>(hj_bf, nullptr, p.nb, 0, tiles_m, tiles_n,
                                                               t_bf, nullptr, wt, wpitch);
  else
    tsel_kernel<64, true><<<total, kGemmThreads, 0, stream>>>(hj_bf, nullptr, p.nb, 0, tiles_m, tiles_n,
                                                              t_bf, nullptr, wt, wpitch);
  return hipGetLastError();
}

hipError_t launch_mask_bits(const Dims& p, const int32_t* idx, uint32_t* bits,
                            hipStream_t stream) {
  const int nw = mask_words(p.nb);
  dim3 grid((p.nb * nw + 255) / 256, p.B * p.H);
  mask_bits_kernel<<<grid, 256, 0, stream>>>(idx, p.nb, p.topk, nw, bits);
  return hipGetLastError();
}

hipError_t launch_tsel(const Dims& p, const __bf16* hj_bf, const uint32_t* bits, __bf16* t_bf,
                       hipStream_t stream, const uint32_t* flags) {
  const int tiles_m = (p.nb + kGemmM - 1) / kGemmM;
  const int tiles_n = p.d * p.d / kGemmN;
  const int total = xcd_chunk_grid(p.B * p.H, tiles_m * tiles_n);
  if (p.d == 128)
    tsel_kernel<128><<<total, kGemmThreads, 0, stream>>>(hj_bf, bits, p.nb, mask_words(p.nb),
                                                         tiles_m, tiles_n, t_bf, flags);
  else
    tsel_kernel<64><<<total, kGemmThreads, 0, stream>>>(hj_bf, bits, p.nb, mask_words(p.nb),
                                                        tiles_m, tiles_n, t_bf, flags);
  return hipGetLastError();
}

}  // namespace sla
