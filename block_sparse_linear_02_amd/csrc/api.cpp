// api.cpp - the C ABI of libsla (declared in include/sla.h): argument checks, workspace
// carving and the launch sequence on the caller's stream.
#include "sla.h"
#include "sla_pisa.h"
#include "sla_svoo.h"
#include "sla_soft.h"

#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstdint>
#include <mutex>

#include "sla_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over the caller's workspace (sizes only when base == nullptr).
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

// Host-side checks shared by every entry point; fills dims on success.
int check_problem(const sla_problem* p, sla::Dims* dims) {
  if (!p) return SLA_ERR_INVALID;
  if (p->B < 1 || p->H < 1 || p->N < 1 || p->d < 1 || p->block < 1) return SLA_ERR_INVALID;
  const int64_t nb = ((int64_t)p->N + p->block - 1) / p->block;
  if (p->topk < 0 || p->topk > nb) return SLA_ERR_INVALID;
  const int64_t elems = (int64_t)p->B * p->H;
  if (elems > (int64_t)INT_MAX / nb) return SLA_ERR_INVALID;  // (b, h, block) ids fit an int
  if ((__int128)elems * p->N * p->d > ((__int128)1 << 62)) return SLA_ERR_INVALID;
  if (p->dtype != SLA_F32 && p->dtype != SLA_BF16) return SLA_ERR_UNSUPPORTED;
  if (p->block != 64) return SLA_ERR_UNSUPPORTED;
  if (p->d != 64 && p->d != 128) return SLA_ERR_UNSUPPORTED;
  if (nb > sla::route_max_blocks()) return SLA_ERR_UNSUPPORTED;
  dims->B = p->B;
  dims->H = p->H;
  dims->N = p->N;
  dims->d = p->d;
  dims->nb = (int)nb;
  dims->topk = p->topk;
  dims->dtype = p->dtype == SLA_BF16 ? sla::kBF16 : sla::kF32;
  return SLA_OK;
}

struct RouteWs {
  __bf16 *q_hi, *q_lo, *k_hi, *k_lo;
};
size_t carve_route(const sla::Dims& d, void* ws, RouteWs* out) {
  Carve c(ws);
  const size_t n = (size_t)d.B * d.H * d.nb * d.d;
  RouteWs r;
  r.q_hi = c.take<__bf16>(n);
  r.q_lo = c.take<__bf16>(n);
  r.k_hi = c.take<__bf16>(n);
  r.k_lo = c.take<__bf16>(n);
  if (out) *out = r;
  return c.off;
}

struct FwdWs {
  float *zb, *h_part, *z_part, *Z, *hj, *h_full;
  __bf16 *ht_hi, *ht_lo;
  __bf16 *hj_bf, *t_bf;
  uint32_t *bits, *flags;
  int32_t *psize, *porder, *pairs;  // the pair kernel's block pairs and dispatch order
  uint8_t *q8, *k8, *v8;
  float *sq, *sk, *sv;
};
// variant: 0 fused, 1 fp8 (fused), 2 literal, 3 mask product, 4 fp8 (mask product),
// 5 int8 (mask product)
size_t carve_forward(const sla::Dims& d, int variant, void* ws, FwdWs* out) {
  Carve c(ws);
  const size_t BH = (size_t)d.B * d.H;
  const size_t dd = (size_t)d.d * d.d;
  const bool mp = variant == 3 || variant == 4 || variant == 5;
  const int cb = sla::state_chunk_blocks(d, !mp);  // the mask-product mode has no h partials
  const size_t nchunk = (d.nb + cb - 1) / cb;
  const bool f8 = variant == 1 || variant == 4 || variant == 5;  // low-bit codes and scales
  FwdWs f = {};
  f.zb = c.take<float>(BH * d.nb * d.d);
  if (!mp) f.h_part = c.take<float>(BH * nchunk * dd);
  f.z_part = c.take<float>(BH * nchunk * d.d);
  f.Z = c.take<float>(BH * d.d);
  f.ht_hi = c.take<__bf16>(BH * dd);
  f.ht_lo = c.take<__bf16>(BH * dd);
  if (variant == 2) {
    f.hj = c.take<float>(BH * d.nb * dd);
    f.h_full = c.take<float>(BH * dd);
  }
  if (mp) {
    f.hj_bf = c.take<__bf16>(BH * d.nb * dd);
    f.t_bf = c.take<__bf16>(BH * d.nb * dd);
    f.bits = c.take<uint32_t>(BH * d.nb * sla::mask_words(d.nb));
    f.flags = c.take<uint32_t>(BH);
  }
  if (variant == 3) {
    f.psize = c.take<int32_t>(sla::pair_order_ints(d));
    f.porder = c.take<int32_t>(sla::pair_order_ints(d));
  }
  if (mp) f.pairs = c.take<int32_t>(sla::pair_match_ints(d));
  if (f8) {
    const size_t n = BH * d.N * d.d;
    f.q8 = c.take<uint8_t>(n);
    f.k8 = c.take<uint8_t>(n);
    f.v8 = c.take<uint8_t>(BH * d.nb * 64 * d.d);  // per-block transposed, padded to 64 keys
    f.sq = c.take<float>(BH * d.nb);
    f.sk = c.take<float>(BH * d.nb);
    f.sv = c.take<float>(BH * d.nb);
  }
  if (out) *out = f;
  return c.off;
}

// PISA statistics buffer (caller-owned, written by sla_pisa_stats, read by route and forward)
struct PisaStats {
  __bf16 *kbar_hi, *kbar_lo, *vsum, *hbar_t;
  float *hbar, *M, *lnM;
};
size_t carve_pisa_stats(const sla::Dims& d, void* base, PisaStats* out, size_t* offsets) {
  Carve c(base);
  const size_t BH = (size_t)d.B * d.H;
  const size_t n = BH * d.nb * d.d, dd = BH * d.d * d.d;
  PisaStats s;
  size_t o[7];
  o[0] = c.off; s.kbar_hi = c.take<__bf16>(n);
  o[1] = c.off; s.kbar_lo = c.take<__bf16>(n);
  o[2] = c.off; s.vsum = c.take<__bf16>(n);
  o[3] = c.off; s.hbar_t = c.take<__bf16>(dd);
  o[4] = c.off; s.hbar = c.take<float>(dd);
  o[5] = c.off; s.M = c.take<float>(BH * d.nb);
  o[6] = c.off; s.lnM = c.take<float>(BH * d.nb);
  if (out) *out = s;
  if (offsets)
    for (int i = 0; i < 7; ++i) offsets[i] = o[i];
  return c.off;
}
// PISA scratch: chunk partials of Hbar (sla_pisa_stats), pooled queries (sla_pisa_route)
struct PisaWs {
  float* h_part;
  __bf16 *q_hi, *q_lo;
};
size_t carve_pisa_ws(const sla::Dims& d, void* base, PisaWs* out) {
  Carve c(base);
  const size_t BH = (size_t)d.B * d.H;
  const int cb = sla::state_chunk_blocks(d);
  const size_t nchunk = (d.nb + cb - 1) / cb;
  PisaWs w;
  w.h_part = c.take<float>(BH * nchunk * d.d * d.d);
  w.q_hi = c.take<__bf16>(BH * d.nb * d.d);
  w.q_lo = c.take<__bf16>(BH * d.nb * d.d);
  if (out) *out = w;
  return c.off;
}

// Backward scratch
struct BwdWs {
  float *zb, *z_part, *Z, *O, *Os, *Ol, *lse2, *rden, *Dr, *e, *dzeta, *dz, *zb2, *z_part2, *dzt;
  __bf16 *hj_bf, *t_bf, *dh_bf, *dOs, *G;
  uint32_t *bits, *kept_t, *unsel_t;
};
size_t carve_backward(const sla::Dims& d, void* ws, BwdWs* out) {
  Carve c(ws);
  const size_t BH = (size_t)d.B * d.H;
  const size_t dd = (size_t)d.d * d.d;
  const size_t rows = BH * d.N, elems = rows * d.d, blocks = BH * d.nb;
  const int cb = sla::state_chunk_blocks(d, false);  // mask-product states: z partials only
  const size_t nchunk = (d.nb + cb - 1) / cb;
  const size_t words = blocks * sla::mask_words(d.nb);
  BwdWs w = {};
  w.zb = c.take<float>(blocks * d.d);
  w.z_part = c.take<float>(BH * nchunk * d.d);
  w.Z = c.take<float>(BH * d.d);
  w.hj_bf = c.take<__bf16>(blocks * dd);  // h_j^T of the forward, then dA_i^T
  w.t_bf = c.take<__bf16>(blocks * dd);
  w.dh_bf = c.take<__bf16>(blocks * dd);
  w.bits = c.take<uint32_t>(words);
  w.kept_t = c.take<uint32_t>(words);
  w.unsel_t = c.take<uint32_t>(words);
  w.O = c.take<float>(elems);
  w.Os = c.take<float>(elems);
  w.Ol = c.take<float>(elems);
  w.lse2 = c.take<float>(rows);
  w.rden = c.take<float>(rows);
  w.dOs = c.take<__bf16>(elems);
  w.G = c.take<__bf16>(elems);
  w.Dr = c.take<float>(rows);
  w.e = c.take<float>(rows);
  w.dzeta = c.take<float>(blocks * d.d);
  w.dz = c.take<float>(blocks * d.d);
  w.zb2 = c.take<float>(blocks * d.d);
  w.z_part2 = c.take<float>(BH * nchunk * d.d);
  w.dzt = c.take<float>(BH * d.d);
  if (out) *out = w;
  return c.off;
}

inline int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return SLA_ERR_HIP;
}

bool validate_requested();
int validate_idx_impl(const sla::Dims& d, const int32_t* idx, hipStream_t stream);

// lowbit: 0 none, 1 e4m3, 2 int8 (int8 exists in the mask-product mode only, its default)
int forward_impl(const sla_problem* p, const void* Q, const void* K, const void* V,
                 const int32_t* idx, const float* alpha, float* O, void* ws, size_t ws_bytes,
                 hipStream_t stream, const sla_forward_opts* opts, int lowbit) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  const bool fp8 = lowbit != 0, int8 = lowbit == 2;
  const int mode = opts ? opts->linear_mode : (int8 ? SLA_LINEAR_MASK_PRODUCT : SLA_LINEAR_FUSED);
  if (mode != SLA_LINEAR_FUSED && mode != SLA_LINEAR_LITERAL && mode != SLA_LINEAR_MASK_PRODUCT)
    return SLA_ERR_INVALID;
  if (fp8 && mode == SLA_LINEAR_LITERAL) return SLA_ERR_INVALID;
  if (int8 && mode != SLA_LINEAR_MASK_PRODUCT) return SLA_ERR_UNSUPPORTED;
  const bool drop = opts && opts->branch_drop;
  if (drop && !(opts->drop_tau >= 0.f && opts->drop_tau < 0.5f)) return SLA_ERR_INVALID;
  if (drop && (fp8 || mode != SLA_LINEAR_MASK_PRODUCT)) return SLA_ERR_UNSUPPORTED;
  const int32_t* out_rows = opts ? opts->out_rows : nullptr;
  if (out_rows && (fp8 || mode != SLA_LINEAR_MASK_PRODUCT)) return SLA_ERR_UNSUPPORTED;
  if (fp8 && (d.dtype != sla::kBF16 || d.d != 128)) return SLA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !alpha || !O || (d.topk > 0 && !idx)) return SLA_ERR_INVALID;
  const int variant = int8  ? 5
                      : fp8 ? (mode == SLA_LINEAR_MASK_PRODUCT ? 4 : 1)
                            : (mode == SLA_LINEAR_LITERAL ? 2 : (mode == SLA_LINEAR_MASK_PRODUCT ? 3 : 0));
  const size_t need = carve_forward(d, variant, nullptr, nullptr);
  if (!ws) return SLA_ERR_INVALID;
  if (ws_bytes < need) return SLA_ERR_WORKSPACE;
  FwdWs w;
  carve_forward(d, variant, ws, &w);

  hipError_t e = hipSuccess;
  if (validate_requested()) {
    if (opts && opts->idx_ready) {
      e = hipStreamWaitEvent(stream, opts->idx_ready, 0);
      if (e != hipSuccess) return hip_fail(e);
    }
    st = validate_idx_impl(d, idx, stream);
    if (st != SLA_OK) return st;
  }
  const uint32_t* flags = nullptr;
  if (drop) {
    e = sla::launch_branch_flags(d, alpha, opts->drop_tau, w.flags, stream);
    if (e != hipSuccess) return hip_fail(e);
    flags = w.flags;
  }
  if (opts && opts->states_begin) {
    e = hipEventRecord(opts->states_begin, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  // the low-bit branch's K and V codes come out of the state kernel, which reads K and V anyway
  // (heads with a dropped linear branch skip that kernel, so then they are quantised apart)
  const sla::StateQuant sq{w.k8, w.v8, w.sk, w.sv, int8};
  const char* sep = getenv("SLA_SEPARATE_QUANT");
  const bool kv_codes = fp8 && !flags && !w.hj && !(sep && sep[0] == '1' && sep[1] == '\0');
  e = sla::launch_states(d, K, V, w.zb, w.h_part, w.z_part, w.hj, w.hj_bf, stream, flags,
                         kv_codes ? &sq : nullptr);
  if (e != hipSuccess) return hip_fail(e);
  e = sla::launch_state_reduce(d, w.h_part, w.z_part, w.ht_hi, w.ht_lo, w.Z, w.h_full, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (opts && opts->idx_ready) {  // nothing above reads idx
    e = hipStreamWaitEvent(stream, opts->idx_ready, 0);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (mode == SLA_LINEAR_MASK_PRODUCT) {
    // every block unselected when topk == 0; the query blocks are paired on the way (the fp8
    // kernel takes no dispatch order, so no sizes)
    e = sla::launch_pair_match(d, idx, w.bits, w.pairs, fp8 ? nullptr : w.psize, flags != nullptr, stream);
    if (e == hipSuccess) e = sla::launch_tsel(d, w.hj_bf, w.bits, w.t_bf, stream, flags);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (opts && opts->states_end) {
    e = hipEventRecord(opts->states_end, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  // the mask-product low-bit kernel quantises its own query blocks (each is read by one
  // workgroup) unless the codes are made apart
  const bool q_in_kernel = kv_codes && mode == SLA_LINEAR_MASK_PRODUCT;
  if (fp8) {
    if (!q_in_kernel) e = sla::launch_quantize(d, Q, w.q8, w.sq, stream, int8);
    if (e == hipSuccess && !kv_codes) e = sla::launch_quantize(d, K, w.k8, w.sk, stream, int8);
    if (e == hipSuccess && !kv_codes) e = sla::launch_quantize_v8t(d, V, w.v8, w.sv, stream, int8);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (opts && opts->sparse_begin) {
    e = hipEventRecord(opts->sparse_begin, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (fp8 && mode == SLA_LINEAR_MASK_PRODUCT)
    e = sla::launch_sparse_pair8(d, Q, q_in_kernel ? nullptr : w.q8, w.k8, w.v8, w.sq, w.sk, w.sv,
                                 idx, alpha, w.t_bf, w.Z, w.zb, O, stream, int8, w.pairs);
  else if (fp8)
    e = sla::launch_sparse_fp8(d, Q, K, V, w.q8, w.k8, w.v8, w.sq, w.sk, w.sv, idx, alpha,
                               w.ht_hi, w.ht_lo, w.Z, w.zb, O, stream);
  else if (mode == SLA_LINEAR_MASK_PRODUCT) {
    e = sla::launch_pair_order(d, w.psize, w.porder, flags != nullptr, stream);
    if (e == hipSuccess)
      e = sla::launch_sparse_pair(d, Q, K, V, idx, alpha, w.t_bf, w.Z, w.zb, O, stream, flags,
                                  nullptr, out_rows, w.porder, w.pairs);
  }
  else
    e = sla::launch_sparse(d, Q, K, V, idx, alpha, w.ht_hi, w.ht_lo, w.Z, w.zb, O,
                           mode == SLA_LINEAR_FUSED ? 1 : 0, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (opts && opts->sparse_end) {
    e = hipEventRecord(opts->sparse_end, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (mode == SLA_LINEAR_LITERAL) {
    e = sla::launch_linear_literal(d, Q, idx, alpha, w.h_full, w.Z, w.hj, w.zb, O, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return SLA_OK;
}

// SVOO co-clustering workspace
struct SvooWs {
  __bf16 *q_hi, *q_lo, *k_hi, *k_lo;
  int32_t *qa, *ka, *hist, *start;
};
size_t carve_svoo(const sla::Dims& d, void* ws, SvooWs* out) {
  Carve c(ws);
  const size_t BH = (size_t)d.B * d.H;
  const size_t n = BH * d.nb * d.d;
  SvooWs w;
  w.q_hi = c.take<__bf16>(n);
  w.q_lo = c.take<__bf16>(n);
  w.k_hi = c.take<__bf16>(n);
  w.k_lo = c.take<__bf16>(n);
  w.qa = c.take<int32_t>(BH * d.N);
  w.ka = c.take<int32_t>(BH * d.N);
  w.hist = c.take<int32_t>(BH * sla::svoo_segments(d.N) * d.nb);
  w.start = c.take<int32_t>(BH * (d.nb + 1));
  if (out) *out = w;
  return c.off;
}

int check_svoo(const sla_problem* p, sla::Dims* d) {
  int st = check_problem(p, d);
  if (st != SLA_OK) return st;
  if (d->dtype != sla::kBF16 || d->d != 128) return SLA_ERR_UNSUPPORTED;
  return SLA_OK;
}

int permute_impl(const sla_problem* p, const void* X, int32_t row_bytes, const int32_t* perm,
                 void* Y, int scatter, hipStream_t stream) {
  if (!p || p->B < 1 || p->H < 1 || p->N < 1) return SLA_ERR_INVALID;
  if (!X || !Y || !perm || row_bytes < 4 || row_bytes > 4096 || row_bytes % 4) return SLA_ERR_INVALID;
  if ((int64_t)p->B * p->H > 65535) return SLA_ERR_UNSUPPORTED;  // grid y
  sla::Dims d = {};
  d.B = p->B;
  d.H = p->H;
  d.N = p->N;
  const hipError_t e = sla::launch_permute_rows(d, X, row_bytes, perm, Y, scatter, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

// SoftTop-k training path workspace
struct SoftWs {
  float *qbar, *kbar, *qt, *kt, *dqt, *dkt;
  __bf16* wt;
  float *zb, *z_part, *Z;
  __bf16 *hj_bf, *t_bf, *dA_bf;
  float *O, *Os, *Ol, *lse2, *rden;
  __bf16 *dOs, *G, *dO;
  float *Dr, *e, *dzeta, *zb2, *z_part2;
  float *dmsp, *dmlin, *ds, *Mw, *dWq, *dWk, *dalpha, *parts, *pg;
};
size_t carve_soft(const sla::Dims& d, void* ws, SoftWs* out) {
  Carve c(ws);
  const size_t BH = (size_t)d.B * d.H;
  const size_t dd = (size_t)d.d * d.d;
  const size_t rows = BH * d.N, elems = rows * d.d, blocks = BH * d.nb, pairs = blocks * d.nb;
  const int cb = sla::state_chunk_blocks(d, false);
  const size_t nchunk = (d.nb + cb - 1) / cb;
  SoftWs w = {};
  w.qbar = c.take<float>(blocks * d.d);
  w.kbar = c.take<float>(blocks * d.d);
  w.qt = c.take<float>(blocks * d.d);
  w.kt = c.take<float>(blocks * d.d);
  w.dqt = c.take<float>(blocks * d.d);
  w.dkt = c.take<float>(blocks * d.d);
  w.wt = c.take<__bf16>(blocks * sla::tsel_weight_pitch(d.nb));
  w.zb = c.take<float>(blocks * d.d);
  w.z_part = c.take<float>(BH * nchunk * d.d);
  w.Z = c.take<float>(BH * d.d);
  w.hj_bf = c.take<__bf16>(blocks * dd);
  w.t_bf = c.take<__bf16>(blocks * dd);
  w.dA_bf = c.take<__bf16>(blocks * dd);
  w.O = c.take<float>(elems);
  w.Os = c.take<float>(elems);
  w.Ol = c.take<float>(elems);
  w.lse2 = c.take<float>(rows);
  w.rden = c.take<float>(rows);
  w.dOs = c.take<__bf16>(elems);
  w.G = c.take<__bf16>(elems);
  w.dO = c.take<__bf16>(elems);
  w.Dr = c.take<float>(rows);
  w.e = c.take<float>(rows);
  w.dzeta = c.take<float>(blocks * d.d);
  w.zb2 = c.take<float>(blocks * d.d);
  w.z_part2 = c.take<float>(BH * nchunk * d.d);
  w.dmsp = c.take<float>(pairs * 4);
  w.dmlin = c.take<float>(pairs);
  w.ds = c.take<float>(pairs);
  w.Mw = c.take<float>(pairs);
  w.dWq = c.take<float>(dd);
  w.dWk = c.take<float>(dd);
  w.dalpha = c.take<float>(rows);
  w.parts = c.take<float>(sla::soft_loss_parts(d));
  w.pg = c.take<float>(sla::router_bwd_part_floats());
  if (out) *out = w;
  return c.off;
}
int check_soft(const sla_problem* p, sla::Dims* d) {
  const int st = check_problem(p, d);
  if (st != SLA_OK) return st;
  if (d->dtype != sla::kBF16 || d->d != 128) return SLA_ERR_UNSUPPORTED;
  return SLA_OK;
}
// the soft forward: states, the weighted mask GEMM, the weighted sparse branch (+ its rows)
hipError_t soft_forward_impl(const sla::Dims& d, const void* Q, const void* K, const void* V,
                             const float* M, const float* alpha, float* O, const SoftWs& w,
                             hipStream_t stream) {
  hipError_t e = sla::launch_states(d, K, V, w.zb, nullptr, w.z_part, nullptr, w.hj_bf, stream);
  if (e == hipSuccess)
    e = sla::launch_state_reduce(d, nullptr, w.z_part, nullptr, nullptr, w.Z, nullptr, stream);
  if (e == hipSuccess) e = sla::launch_soft_weights(d, M, w.wt, stream);
  if (e == hipSuccess) e = sla::launch_tsel_weighted(d, w.hj_bf, w.wt, w.t_bf, stream);
  const sla::TrainRows tr = {w.Os, w.Ol, w.lse2, w.rden};
  if (e == hipSuccess) e = sla::launch_sparse_soft(d, Q, K, V, M, alpha, w.t_bf, w.Z, w.zb, O, stream, &tr);
  return e;
}
// the soft backward after soft_forward_impl: dalpha, dM (parts), ds, the router gradients
hipError_t soft_backward_impl(const sla::Dims& d, const void* Q, const void* K, const void* V,
                              const float* Wq, const float* Wk, float temp, const float* M,
                              const float* alpha, const void* dO, float* dWq, float* dWk,
                              float* dalpha, float* dM, const SoftWs& w, hipStream_t stream) {
  const sla::TrainRows tr = {w.Os, w.Ol, w.lse2, w.rden};
  hipError_t e = sla::launch_bwd_prep(d, Q, dO, alpha, tr, dalpha, w.dOs, w.Dr, w.G, w.e, w.dzeta, stream);
  if (e == hipSuccess) e = sla::launch_states(d, Q, w.G, w.zb2, nullptr, w.z_part2, nullptr, w.dA_bf, stream);
  if (e == hipSuccess) e = sla::launch_soft_dm_sparse(d, Q, K, V, w.dOs, w.lse2, w.Dr, w.dmsp, stream);
  if (e == hipSuccess) e = sla::launch_soft_dm_linear(d, w.dA_bf, w.hj_bf, w.dzeta, w.zb, w.dmlin, stream);
  if (e == hipSuccess) e = sla::launch_soft_topk_bwd(d, M, w.dmsp, w.dmlin, temp, w.ds, dM, stream);
  if (e == hipSuccess) e = sla::launch_soft_pool(d, Q, K, Wq, Wk, w.qbar, w.kbar, w.qt, w.kt, stream);
  if (e == hipSuccess)
    e = sla::launch_router_bwd(d, w.ds, w.qbar, w.kbar, w.qt, w.kt, w.dqt, w.dkt, dWq, dWk, w.pg, stream);
  return e;
}

// Static workspace of sla_route_noalloc: one copy per GPU, alive until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: only the address that
// hipGetSymbolAddress returns (kept per device below) is handed to kernels.
static __device__ __align__(256) unsigned char scratch[SLA_ROUTE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of a file-scope __device__ symbol on the current device, looked up on the
// first call with that device current and kept in cache[device].
int symbol_of_current_device(const void* symbol, std::atomic<void*>* cache, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return SLA_ERR_UNSUPPORTED;
  void* ptr = cache[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = cache[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, symbol);
      if (e != hipSuccess) return hip_fail(e);
      if (!ptr) return hip_fail(hipErrorInvalidSymbol);
      cache[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return SLA_OK;
}

// Device address of this device's `scratch`.
int scratch_of_current_device(void** out) {
  return symbol_of_current_device(HIP_SYMBOL(scratch), g_scratch_ptr, out);
}

// Result word of the debug idx check: one per GPU, alive until the process ends; checks that
// overlap on one GPU race on it (a debug path).
static __device__ int validate_bad[1];
std::atomic<void*> g_validate_ptr[kMaxDevices];

// SLA_VALIDATE=1 in the environment: the entry points that read idx check it first.
bool validate_requested() {
  const char* e = getenv("SLA_VALIDATE");
  return e && e[0] == '1' && e[1] == '\0';
}

// Check idx on the device (entries in [0, n_b), rows strictly ascending), synchronise the
// stream and read the verdict: SLA_OK or SLA_ERR_INVALID.
int validate_idx_impl(const sla::Dims& d, const int32_t* idx, hipStream_t stream) {
  if (d.topk == 0) return SLA_OK;
  void* flag = nullptr;
  int st = symbol_of_current_device(HIP_SYMBOL(validate_bad), g_validate_ptr, &flag);
  if (st != SLA_OK) return st;
  int bad = 0;
  hipError_t e = sla::launch_validate_idx(d, idx, static_cast<int*>(flag), stream);
  if (e == hipSuccess) e = hipMemcpyAsync(&bad, flag, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e);
  return bad == 0 ? SLA_OK : SLA_ERR_INVALID;
}

}  // namespace

extern "C" {

size_t sla_route_workspace_bytes(const sla_problem* p) {
  sla::Dims d;
  if (check_problem(p, &d) != SLA_OK) return 0;
  return carve_route(d, nullptr, nullptr);
}

size_t sla_forward_workspace_bytes(const sla_problem* p, int variant) {
  sla::Dims d;
  if (check_problem(p, &d) != SLA_OK || variant < 0 || variant > 5) return 0;
  return carve_forward(d, variant, nullptr, nullptr);
}

int sla_route(const sla_problem* p, const void* Q, const void* K, const float* proj_q,
              const float* proj_k, int32_t* idx, uint8_t* mask, float* scores, void* ws,
              size_t ws_bytes, hipStream_t stream) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  if (!Q || !K || !proj_q || !proj_k || (d.topk > 0 && !idx) || !ws) return SLA_ERR_INVALID;
  if (ws_bytes < carve_route(d, nullptr, nullptr)) return SLA_ERR_WORKSPACE;
  RouteWs w;
  carve_route(d, ws, &w);
  hipError_t e = sla::launch_route(d, Q, K, proj_q, proj_k, w.q_hi, w.q_lo, w.k_hi, w.k_lo, idx,
                                   mask, scores, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

size_t sla_soft_workspace_bytes(const sla_problem* p) {
  sla::Dims d;
  if (check_soft(p, &d) != SLA_OK) return 0;
  return carve_soft(d, nullptr, nullptr);
}

int sla_soft_route(const sla_problem* p, const void* Q, const void* K, const float* proj_q,
                   const float* proj_k, float temperature, float* M, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  sla::Dims d;
  int st = check_soft(p, &d);
  if (st != SLA_OK) return st;
  if (!Q || !K || !proj_q || !proj_k || !M || !ws) return SLA_ERR_INVALID;
  if (!(temperature > 0.f) || !(temperature < 1e30f)) return SLA_ERR_INVALID;
  if (ws_bytes < carve_soft(d, nullptr, nullptr)) return SLA_ERR_WORKSPACE;
  SoftWs w;
  carve_soft(d, ws, &w);
  hipError_t e = sla::launch_soft_pool(d, Q, K, proj_q, proj_k, w.qbar, w.kbar, w.qt, w.kt, stream);
  if (e == hipSuccess) e = sla::launch_soft_topk(d, w.qt, w.kt, temperature, M, w.wt, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

int sla_soft_forward(const sla_problem* p, const void* Q, const void* K, const void* V,
                     const float* M, const float* alpha, float* O, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  sla::Dims d;
  int st = check_soft(p, &d);
  if (st != SLA_OK) return st;
  if (!Q || !K || !V || !M || !alpha || !O || !ws) return SLA_ERR_INVALID;
  if (ws_bytes < carve_soft(d, nullptr, nullptr)) return SLA_ERR_WORKSPACE;
  SoftWs w;
  carve_soft(d, ws, &w);
  const hipError_t e = soft_forward_impl(d, Q, K, V, M, alpha, O, w, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

int sla_soft_backward(const sla_problem* p, const void* Q, const void* K, const void* V,
                      const float* proj_q, const float* proj_k, float temperature, const float* M,
                      const float* alpha, const void* dO, float* dproj_q, float* dproj_k,
                      float* dalpha, float* dM, float* O, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  sla::Dims d;
  int st = check_soft(p, &d);
  if (st != SLA_OK) return st;
  if (!Q || !K || !V || !proj_q || !proj_k || !M || !alpha || !dO || !dproj_q || !dproj_k || !dalpha || !ws)
    return SLA_ERR_INVALID;
  if (!(temperature > 0.f) || !(temperature < 1e30f)) return SLA_ERR_INVALID;
  if (ws_bytes < carve_soft(d, nullptr, nullptr)) return SLA_ERR_WORKSPACE;
  SoftWs w;
  carve_soft(d, ws, &w);
  hipError_t e = soft_forward_impl(d, Q, K, V, M, alpha, O ? O : w.O, w, stream);
  if (e == hipSuccess)
    e = soft_backward_impl(d, Q, K, V, proj_q, proj_k, temperature, M, alpha, dO, dproj_q, dproj_k,
                           dalpha, dM, w, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

int sla_stage1_step(const sla_problem* p, const void* Q, const void* K, const void* V,
                    const float* O_full, float* proj_q, float* proj_k, float* alpha,
                    float temperature, float lr_proj, float lr_alpha, float* loss, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  sla::Dims d;
  int st = check_soft(p, &d);
  if (st != SLA_OK) return st;
  if (!Q || !K || !V || !O_full || !proj_q || !proj_k || !alpha || !loss || !ws) return SLA_ERR_INVALID;
  if (!(temperature > 0.f) || !(temperature < 1e30f)) return SLA_ERR_INVALID;
  if (ws_bytes < carve_soft(d, nullptr, nullptr)) return SLA_ERR_WORKSPACE;
  SoftWs w;
  carve_soft(d, ws, &w);
  hipError_t e = sla::launch_soft_pool(d, Q, K, proj_q, proj_k, w.qbar, w.kbar, w.qt, w.kt, stream);
  if (e == hipSuccess) e = sla::launch_soft_topk(d, w.qt, w.kt, temperature, w.Mw, w.wt, stream);
  if (e == hipSuccess) e = soft_forward_impl(d, Q, K, V, w.Mw, alpha, w.O, w, stream);
  if (e == hipSuccess) e = sla::launch_soft_loss(d, w.O, O_full, w.dO, w.parts, loss, stream);
  if (e == hipSuccess)
    e = soft_backward_impl(d, Q, K, V, proj_q, proj_k, temperature, w.Mw, alpha, w.dO, w.dWq, w.dWk,
                           w.dalpha, nullptr, w, stream);
  if (e == hipSuccess)
    e = sla::launch_soft_update(d, proj_q, proj_k, alpha, w.dWq, w.dWk, w.dalpha, lr_proj, lr_alpha, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

int sla_route_noalloc(const sla_problem* p, const void* Q, const void* K, const float* proj_q,
                      const float* proj_k, int32_t* idx, uint8_t* mask, float* scores,
                      hipStream_t stream) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  if (!Q || !K || !proj_q || !proj_k || (d.topk > 0 && !idx)) return SLA_ERR_INVALID;
  if (carve_route(d, nullptr, nullptr) > SLA_ROUTE_NOALLOC_SCRATCH_BYTES) return SLA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != SLA_OK) return st;
  RouteWs w;
  carve_route(d, ws, &w);
  hipError_t e = sla::launch_route(d, Q, K, proj_q, proj_k, w.q_hi, w.q_lo, w.k_hi, w.k_lo, idx,
                                   mask, scores, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

int sla_forward(const sla_problem* p, const void* Q, const void* K, const void* V,
                const int32_t* idx, const float* alpha, float* O, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  return forward_impl(p, Q, K, V, idx, alpha, O, ws, ws_bytes, stream, nullptr, 0);
}

int sla_forward_ex(const sla_problem* p, const void* Q, const void* K, const void* V,
                   const int32_t* idx, const float* alpha, float* O, void* ws, size_t ws_bytes,
                   hipStream_t stream, const sla_forward_opts* opts) {
  return forward_impl(p, Q, K, V, idx, alpha, O, ws, ws_bytes, stream, opts, 0);
}

int sla_forward_fp8(const sla_problem* p, const void* Q, const void* K, const void* V,
                    const int32_t* idx, const float* alpha, float* O, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  return forward_impl(p, Q, K, V, idx, alpha, O, ws, ws_bytes, stream, nullptr, 1);
}

int sla_forward_fp8_ex(const sla_problem* p, const void* Q, const void* K, const void* V,
                       const int32_t* idx, const float* alpha, float* O, void* ws,
                       size_t ws_bytes, hipStream_t stream, const sla_forward_opts* opts) {
  return forward_impl(p, Q, K, V, idx, alpha, O, ws, ws_bytes, stream, opts, 1);
}

int sla_forward_int8(const sla_problem* p, const void* Q, const void* K, const void* V,
                     const int32_t* idx, const float* alpha, float* O, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  return forward_impl(p, Q, K, V, idx, alpha, O, ws, ws_bytes, stream, nullptr, 2);
}

int sla_forward_int8_ex(const sla_problem* p, const void* Q, const void* K, const void* V,
                        const int32_t* idx, const float* alpha, float* O, void* ws,
                        size_t ws_bytes, hipStream_t stream, const sla_forward_opts* opts) {
  return forward_impl(p, Q, K, V, idx, alpha, O, ws, ws_bytes, stream, opts, 2);
}

int quantize_impl(const sla_problem* p, const void* X, uint8_t* codes, float* scales,
                  hipStream_t stream, int int8) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  if (d.dtype != sla::kBF16 || d.d != 128) return SLA_ERR_UNSUPPORTED;
  if (!X || !codes || !scales) return SLA_ERR_INVALID;
  hipError_t e = sla::launch_quantize(d, X, codes, scales, stream, int8);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

int sla_quantize_e4m3(const sla_problem* p, const void* X, uint8_t* codes, float* scales,
                      hipStream_t stream) {
  return quantize_impl(p, X, codes, scales, stream, 0);
}

int sla_quantize_int8(const sla_problem* p, const void* X, int8_t* codes, float* scales,
                      hipStream_t stream) {
  return quantize_impl(p, X, reinterpret_cast<uint8_t*>(codes), scales, stream, 1);
}

size_t sla_pisa_stats_bytes(const sla_problem* p) {
  sla::Dims d;
  if (check_problem(p, &d) != SLA_OK) return 0;
  return carve_pisa_stats(d, nullptr, nullptr, nullptr);
}

int sla_pisa_stats_offsets(const sla_problem* p, size_t offsets[7]) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  if (!offsets) return SLA_ERR_INVALID;
  carve_pisa_stats(d, nullptr, nullptr, offsets);
  return SLA_OK;
}

size_t sla_pisa_workspace_bytes(const sla_problem* p) {
  sla::Dims d;
  if (check_problem(p, &d) != SLA_OK) return 0;
  return carve_pisa_ws(d, nullptr, nullptr);
}

int sla_pisa_stats(const sla_problem* p, const void* K, const void* V, void* stats,
                   size_t stats_bytes, void* ws, size_t ws_bytes, hipStream_t stream) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  if (!K || !V || !stats || !ws) return SLA_ERR_INVALID;
  if (stats_bytes < carve_pisa_stats(d, nullptr, nullptr, nullptr) ||
      ws_bytes < carve_pisa_ws(d, nullptr, nullptr))
    return SLA_ERR_WORKSPACE;
  PisaStats s;
  carve_pisa_stats(d, stats, &s, nullptr);
  PisaWs w;
  carve_pisa_ws(d, ws, &w);
  hipError_t e = sla::launch_pisa_stats(d, K, V, s.kbar_hi, s.kbar_lo, s.vsum, w.h_part, s.hbar_t,
                                        s.hbar, s.M, s.lnM, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

int sla_pisa_route(const sla_problem* p, const void* Q, const void* stats, size_t stats_bytes,
                   int covariance, int32_t* idx, uint8_t* mask, float* scores, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  if (!Q || !stats || (d.topk > 0 && !idx) || !ws) return SLA_ERR_INVALID;
  if (covariance != 0 && covariance != 1) return SLA_ERR_INVALID;
  if (stats_bytes < carve_pisa_stats(d, nullptr, nullptr, nullptr) ||
      ws_bytes < carve_pisa_ws(d, nullptr, nullptr))
    return SLA_ERR_WORKSPACE;
  PisaStats s;
  carve_pisa_stats(d, const_cast<void*>(stats), &s, nullptr);
  PisaWs w;
  carve_pisa_ws(d, ws, &w);
  hipError_t e = sla::launch_pisa_route(d, Q, w.q_hi, w.q_lo, s.kbar_hi, s.kbar_lo,
                                        covariance ? s.lnM : nullptr, idx, mask, scores, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

int sla_pisa_forward(const sla_problem* p, const void* Q, const void* K, const void* V,
                     const void* stats, size_t stats_bytes, const int32_t* idx, float* O,
                     hipStream_t stream) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  if (!Q || !K || !V || !stats || !O || (d.topk > 0 && !idx)) return SLA_ERR_INVALID;
  if (d.nb > sla::pisa_max_blocks()) return SLA_ERR_UNSUPPORTED;
  if (stats_bytes < carve_pisa_stats(d, nullptr, nullptr, nullptr)) return SLA_ERR_WORKSPACE;
  if (validate_requested()) {
    st = validate_idx_impl(d, idx, stream);
    if (st != SLA_OK) return st;
  }
  PisaStats s;
  carve_pisa_stats(d, const_cast<void*>(stats), &s, nullptr);
  hipError_t e = sla::launch_pisa(d, Q, K, V, idx, s.kbar_hi, s.kbar_lo, s.vsum, s.hbar_t, O, stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

size_t sla_backward_workspace_bytes(const sla_problem* p) {
  sla::Dims d;
  if (check_problem(p, &d) != SLA_OK) return 0;
  return carve_backward(d, nullptr, nullptr);
}

int sla_backward(const sla_problem* p, const void* Q, const void* K, const void* V,
                 const int32_t* idx, const float* alpha, const void* dO, float* dQ, float* dK,
                 float* dV, float* dalpha, float* O, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  if (d.dtype != sla::kBF16 || d.d != 128) return SLA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !alpha || !dO || !dQ || !dK || !dV || !dalpha || (d.topk > 0 && !idx) || !ws)
    return SLA_ERR_INVALID;
  if (ws_bytes < carve_backward(d, nullptr, nullptr)) return SLA_ERR_WORKSPACE;
  if (validate_requested()) {
    st = validate_idx_impl(d, idx, stream);
    if (st != SLA_OK) return st;
  }
  BwdWs w;
  carve_backward(d, ws, &w);
  hipError_t e;
  // the forward in the mask-product mode, keeping what the backward reads
  e = sla::launch_states(d, K, V, w.zb, nullptr, w.z_part, nullptr, w.hj_bf, stream);
  if (e == hipSuccess)
    e = sla::launch_state_reduce(d, nullptr, w.z_part, nullptr, nullptr, w.Z, nullptr, stream);
  if (e == hipSuccess) e = sla::launch_mask_bits(d, idx, w.bits, stream);
  if (e == hipSuccess) e = sla::launch_tsel(d, w.hj_bf, w.bits, w.t_bf, stream);
  const sla::TrainRows tr = {w.Os, w.Ol, w.lse2, w.rden};
  if (e == hipSuccess)
    e = sla::launch_sparse_pair(d, Q, K, V, idx, alpha, w.t_bf, w.Z, w.zb, O ? O : w.O, stream,
                                nullptr, &tr);
  // per-row terms, the transposed kept sets, the linear branch's dA_i, dh_j and dz_j
  if (e == hipSuccess)
    e = sla::launch_bwd_prep(d, Q, dO, alpha, tr, dalpha, w.dOs, w.Dr, w.G, w.e, w.dzeta, stream);
  if (e == hipSuccess) e = sla::launch_bits_t(d, idx, w.kept_t, w.unsel_t, stream);
  if (e == hipSuccess)
    e = sla::launch_states(d, Q, w.G, w.zb2, nullptr, w.z_part2, nullptr, w.hj_bf, stream);
  if (e == hipSuccess) e = sla::launch_tsel(d, w.hj_bf, w.unsel_t, w.dh_bf, stream);
  if (e == hipSuccess) e = sla::launch_bwd_dz(d, w.dzeta, w.kept_t, w.dzt, w.dz, stream);
  // the gradients
  if (e == hipSuccess)
    e = sla::launch_bwd_dq(d, Q, K, V, idx, w.dOs, w.lse2, w.Dr, w.G, w.e, w.t_bf, w.Z, w.zb, dQ,
                           stream);
  if (e == hipSuccess)
    e = sla::launch_bwd_dkv(d, Q, K, V, w.kept_t, w.dOs, w.lse2, w.Dr, w.dh_bf, w.dz, dK, dV,
                            stream);
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

size_t sla_svoo_workspace_bytes(const sla_problem* p) {
  sla::Dims d;
  if (check_svoo(p, &d) != SLA_OK) return 0;
  return carve_svoo(d, nullptr, nullptr);
}

int sla_svoo_cluster(const sla_problem* p, const void* Q, const void* K, int32_t iters,
                     int32_t* q_assign, int32_t* k_assign, int32_t* perm_q, int32_t* perm_k,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  sla::Dims d;
  int st = check_svoo(p, &d);
  if (st != SLA_OK) return st;
  if (!Q || !K || !perm_q || !perm_k || !ws || iters < 1 || iters > 64) return SLA_ERR_INVALID;
  if ((int64_t)d.B * d.H > 65535) return SLA_ERR_UNSUPPORTED;  // grid y
  if (ws_bytes < carve_svoo(d, nullptr, nullptr)) return SLA_ERR_WORKSPACE;
  SvooWs w;
  carve_svoo(d, ws, &w);
  int32_t* qa = q_assign ? q_assign : w.qa;
  int32_t* ka = k_assign ? k_assign : w.ka;
  hipError_t e = sla::launch_pool_means(d, Q, K, w.q_hi, w.q_lo, w.k_hi, w.k_lo, stream);
  for (int it = 0; it < iters && e == hipSuccess; ++it) {
    // key step: keys by the query centroids, then the key centroids of the new clusters
    e = sla::launch_svoo_assign(d, K, w.q_hi, w.q_lo, ka, stream);
    if (e == hipSuccess) e = sla::launch_svoo_order(d, ka, w.hist, w.start, perm_k, stream);
    if (e == hipSuccess) e = sla::launch_svoo_centroids(d, K, perm_k, w.start, w.k_hi, w.k_lo, stream);
    // query step: queries by the updated key centroids (their centroids feed the next pass)
    if (e == hipSuccess) e = sla::launch_svoo_assign(d, Q, w.k_hi, w.k_lo, qa, stream);
    if (e == hipSuccess) e = sla::launch_svoo_order(d, qa, w.hist, w.start, perm_q, stream);
    if (e == hipSuccess && it + 1 < iters)
      e = sla::launch_svoo_centroids(d, Q, perm_q, w.start, w.q_hi, w.q_lo, stream);
  }
  if (e != hipSuccess) return hip_fail(e);
  return SLA_OK;
}

int sla_svoo_gather(const sla_problem* p, const void* X, int32_t row_bytes, const int32_t* perm,
                    void* Y, hipStream_t stream) {
  return permute_impl(p, X, row_bytes, perm, Y, 0, stream);
}

int sla_svoo_scatter(const sla_problem* p, const void* X, int32_t row_bytes, const int32_t* perm,
                     void* Y, hipStream_t stream) {
  return permute_impl(p, X, row_bytes, perm, Y, 1, stream);
}

const char* sla_status_string(int status) {
  switch (status) {
    case SLA_OK: return "ok";
    case SLA_ERR_INVALID: return "invalid argument";
    case SLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SLA_ERR_WORKSPACE: return "workspace too small";
    case SLA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int sla_validate_idx(const sla_problem* p, const int32_t* idx, hipStream_t stream) {
  sla::Dims d;
  int st = check_problem(p, &d);
  if (st != SLA_OK) return st;
  if (d.topk > 0 && !idx) return SLA_ERR_INVALID;
  return validate_idx_impl(d, idx, stream);
}

int sla_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
