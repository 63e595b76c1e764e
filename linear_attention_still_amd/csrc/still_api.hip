// Host side of libstill.so: argument validation, state / workspace layout and
// the launch sequences of still_prefill and still_decode_step. Validation
// makes no HIP call, so it runs (and is tested) without a GPU.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "still.h"
#include "still_decode.hip"
#include "still_prefill.hip"
#include "still_backward.hip"

namespace {

using still::bf16;

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Derived {
  int B, Hq, Hkv, G, D, W, C, m, t_max, lam, cap_chunks, R, P, esz;
  float eps, scale;
  double eps64, scale64;
  bool paged;  // STILL_FLAG_PAGED_POOL: the pool rows live in the caller's pages
  bool pool8;  // STILL_FLAG_POOL_FP8: pool rows as E4M3 codes, then a float32 scale per row
};

int derive(const still_params* p, Derived* d) {
  if (!p) return STILL_EINVAL;
  if (p->abi_version != STILL_ABI_VERSION) return STILL_EINVAL;
  if (p->dtype != STILL_DTYPE_F32 && p->dtype != STILL_DTYPE_BF16) return STILL_EINVAL;
  if (p->flags & ~(STILL_FLAG_FP32_OUT | STILL_FLAG_SOFTMAX_ONLY | STILL_FLAG_MERGE_SUM |
                   STILL_FLAG_PAGED_POOL | STILL_FLAG_POOL_FP8 | STILL_FLAG_ROUTE(15u)))
    return STILL_EINVAL;  // unknown flag bits
  if (STILL_ROUTE_OF(p->flags) > STILL_ROUTE_EXTERNAL) return STILL_EINVAL;
  if ((p->flags & STILL_FLAG_SOFTMAX_ONLY) && (p->flags & STILL_FLAG_MERGE_SUM))
    return STILL_EINVAL;  // two merges at once
  if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1) return STILL_EINVAL;
  if (p->n_q_heads % p->n_kv_heads != 0) return STILL_EINVAL;
  if (p->window < 1 || p->chunk < 1 || p->budget < p->window || p->t_max < 1) return STILL_EINVAL;
  if (p->head_dim < 1) return STILL_EINVAL;
  const int G = p->n_q_heads / p->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return STILL_EUNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return STILL_EUNSUPPORTED;
  if (p->dtype == STILL_DTYPE_F32 && p->head_dim != 64) return STILL_EUNSUPPORTED;
  if (p->chunk != 16 && p->chunk != 32 && p->chunk != 64 && p->chunk != 128)
    return STILL_EUNSUPPORTED;
  if (p->window > 256) return STILL_EUNSUPPORTED;
  if ((int64_t)p->budget - p->window > (1 << 20)) return STILL_EUNSUPPORTED;
  // the 8-bit pool: 16-bit data, rows in the state
  if ((p->flags & STILL_FLAG_POOL_FP8) &&
      (p->dtype != STILL_DTYPE_BF16 || (p->flags & STILL_FLAG_PAGED_POOL)))
    return STILL_EUNSUPPORTED;
  // the paged pool's table of a unit is staged in LDS (at most 256 pages)
  if ((p->flags & STILL_FLAG_PAGED_POOL) &&
      ((int64_t)p->budget - p->window + STILL_POOL_PAGE_ROWS - 1) / STILL_POOL_PAGE_ROWS > 256)
    return STILL_EUNSUPPORTED;
  d->B = p->batch;
  d->Hq = p->n_q_heads;
  d->Hkv = p->n_kv_heads;
  d->G = G;
  d->D = p->head_dim;
  d->W = p->window;
  d->C = p->chunk;
  d->m = p->budget;
  d->t_max = p->t_max;
  int lam = (p->budget - p->window) / p->t_max;
  if (lam > p->chunk) lam = p->chunk;
  d->lam = lam;
  d->cap_chunks = lam > 0 ? (p->budget - p->window) / lam : 0;
  d->R = p->window + 2 * p->chunk;
  d->P = p->budget - p->window;
  d->esz = p->dtype == STILL_DTYPE_F32 ? 4 : 2;
  d->paged = (p->flags & STILL_FLAG_PAGED_POOL) != 0;
  d->pool8 = (p->flags & STILL_FLAG_POOL_FP8) != 0;
  d->eps = p->eps > 0.f ? p->eps : 1e-6f;
  d->scale = p->sm_scale > 0.f ? p->sm_scale : 1.0f / sqrtf((float)p->head_dim);
  // float64 paths (score refinement, decode score): the default values are
  // taken in float64, a caller-given value as the float it was given as
  d->eps64 = p->eps > 0.f ? (double)p->eps : 1e-6;
  d->scale64 = p->sm_scale > 0.f ? (double)p->sm_scale : 1.0 / sqrt((double)p->head_dim);
  return STILL_OK;
}

void layout(const Derived& d, still_state_layout* s) {
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  s->S = take((int64_t)d.D * d.D * 4);
  s->z = take((int64_t)d.D * 4);
  // with the paged pool the rows live in the caller's pages (empty regions)
  const int64_t pool_bytes = d.paged ? 0 : d.pool8 ? (int64_t)d.P * (d.D + 1) : (int64_t)d.P * d.D * d.esz;
  s->pool_k = take(pool_bytes);
  s->pool_v = take(pool_bytes);
  s->pool_pos = take((int64_t)d.P * 4);
  s->ring_k = take((int64_t)d.R * d.D * d.esz);
  s->ring_v = take((int64_t)d.R * d.D * d.esz);
  s->ring_phi = take((int64_t)d.R * d.D * d.esz);
  s->ring_flag = take((int64_t)d.R * 4);
  s->pending = take((int64_t)d.C * 8);
  s->meta = take(4 * 8);
  s->unit_bytes = o;
  s->ring_slots = d.R;
  s->pool_slots = d.P;
}

static_assert(still::ROUTE_SALIENCY == STILL_ROUTE_SALIENCY && still::ROUTE_DIAG == STILL_ROUTE_DIAG &&
                  still::ROUTE_QK == STILL_ROUTE_QK && still::ROUTE_KEYNORM == STILL_ROUTE_KEYNORM &&
                  still::ROUTE_UNIFORM == STILL_ROUTE_UNIFORM && still::ROUTE_EXTERNAL == STILL_ROUTE_EXTERNAL,
              "routing metric numbers of the ABI and the kernels agree");

// Prefill launch geometry.
struct Plan {
  int L, T, n_dec, n_pend, K, NS, Gs, nHG, HPW;
  bool part;
  int64_t ws_ft, ws_score, ws_delta, ws_flag, ws_dS, ws_rl, ws_total;
};

// part: the walk keeps the two branches apart (one query head per wave,
// held in both head slots of the two-head walk).
Plan plan(const Derived& d, int64_t L, bool part) {
  Plan pl;
  pl.L = (int)L;
  pl.T = (int)((L + d.C - 1) / d.C);
  pl.n_dec = (int)((L - 1) / d.C);
  pl.n_pend = (int)(L - (int64_t)pl.n_dec * d.C);
  // 8 waves per attend workgroup, each one 16-query tile of HPW heads: two
  // heads per wave where that fills the 8 waves (the heads share every
  // key / value read and the workgroup's per-block work), else one
  const int n_qt = d.C / 16;
  int gs2 = 256 / d.C;
  if (gs2 > d.G) gs2 = d.G;
  bool two = gs2 >= 2 && (gs2 / 2) * n_qt == 8;
  if (const char* e = getenv("STILL_HEADS_PER_WAVE")) two = two && atoi(e) != 1;
  if (part) two = false;
  if (two) {
    pl.HPW = 2;
    pl.Gs = gs2;
  } else {
    int gs = 128 / d.C;  // at most 8 row tiles of 16 queries per workgroup
    if (gs < 1) gs = 1;
    if (gs > d.G) gs = d.G;
    pl.HPW = 1;
    pl.Gs = gs;
  }
  pl.nHG = d.G / pl.Gs;
  // chunks walked per workgroup: enough workgroups to fill the chip (about
  // four chunks each measured best at 16K, with one or two heads per wave)
  const int64_t units = (int64_t)d.B * d.Hkv * pl.nHG;
  int K = (int)((int64_t)pl.T * units * pl.HPW / 1024);
  if (K < 1) K = 1;
  if (K > 8) K = 8;
  if (const char* e = getenv("STILL_CHUNKS_PER_WG")) {
    const int k = atoi(e);
    if (k >= 1 && k <= 64) K = k;
  }
  if (K > pl.T) K = pl.T;
  pl.K = K;
  pl.NS = (pl.T + K - 1) / K;
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const int64_t nu = (int64_t)d.B * d.Hkv;
  pl.ws_ft = take((int64_t)d.Hkv * d.D * d.D * d.esz);
  pl.ws_score = take(nu * L * 4);
  pl.ws_delta = take(nu * L * 4);
  pl.ws_flag = take(nu * L);
  pl.ws_rl = take(nu * pl.T * (int64_t)(d.C + 1) * 4);
  pl.ws_dS = take(nu * pl.NS * ((int64_t)d.D * d.D + d.D) * 4);  // last: its size depends on NS
  pl.ws_total = o;
  pl.part = part;
  return pl;
}

// Workspace bytes that serve both walks (the separate-branch one included).
int64_t ws_bytes_any(const Derived& d, int64_t L) {
  const int64_t a = plan(d, L, false).ws_total, b = plan(d, L, true).ws_total;
  return a > b ? a : b;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// LDS-size attributes of the kernels that use more than 64 KiB of dynamic
// LDS, set once per (kernel family, device). The table is the library's only
// mutable host state; a mutex makes concurrent first calls safe.
constexpr int kMaxDevices = 64;
std::mutex g_attr_mu;
uint64_t g_attr_done[kMaxDevices];  // bit f: family f set on that device

template <typename T, int D>
void set_prefill_attrs(int family) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  if (g_attr_done[dev] & (1ull << family)) return;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::score_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::attend_kernel<T, D, 1>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)still::Blk<T, D>::bytes);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::attend_kernel<T, D, 2>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)still::Blk<T, D>::bytes);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::attend_kernel<T, D, 2, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)still::Blk<T, D>::bytes);
  // the forget-gate (decay) instantiations
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::attend_kernel<T, D, 1, false, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)still::Blk<T, D>::bytes);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::attend_kernel<T, D, 2, false, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)still::Blk<T, D>::bytes);
  if constexpr (sizeof(T) == 2) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::state_delta_kernel<T, D>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)still::SdLds<T, D>::bytes);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::state_delta_kernel<T, D, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)still::SdLds<T, D>::bytes);
  } else {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::state_delta_f32_kernel<D>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)still::Blk<T, D>::bytes);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::state_delta_f32_kernel<D, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)still::Blk<T, D>::bytes);
  }
  g_attr_done[dev] |= 1ull << family;
}

template <typename T, int D, int G>
void set_decode_attr(int family) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  if (g_attr_done[dev] & (1ull << family)) return;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::decode_kernel<T, D, G>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::decode_kernel<T, D, G, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if constexpr (sizeof(T) == 2)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::decode_kernel<T, D, G, false, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  g_attr_done[dev] |= 1ull << family;
}

// the chunk-boundary decode kernel (its fold's LDS passes 64 KiB at d = 128)
template <typename T, int D>
void set_boundary_attr(int family) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  if (g_attr_done[dev] & (1ull << family)) return;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::decode_boundary_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  g_attr_done[dev] |= 1ull << family;
}

// kernel family index of (element type, head dim[, group]) for the table
template <typename T, int D>
constexpr int prefill_family() { return (sizeof(T) == 4 ? 0 : 1) * 2 + (D == 128 ? 1 : 0); }
template <typename T, int D, int G>
constexpr int decode_family() {
  return 4 + ((sizeof(T) == 4 ? 0 : 1) * 2 + (D == 128 ? 1 : 0)) * 4 + (G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3);
}

template <typename T, int D>
void set_backward_attrs() {
  const int family = 20 + prefill_family<T, D>();
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  if (g_attr_done[dev] & (1ull << family)) return;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::bw_phi_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, still::BwRowLds<D>::bytes);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::bw_npmap_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, still::BwRowLds<D>::bytes);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::bw_query_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, still::BwQLds<D>::bytes);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&still::bw_key_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, still::BwKLds<D>::bytes);
  g_attr_done[dev] |= 1ull << family;
}

// Optional per-kernel events (still_prefill_timed).
struct Marks {
  void* const* ev;
  int n;
  hipStream_t s;
  void at(int i, int which) const {  // a null handle is skipped
    if (ev && i < n && ev[2 * i + which])
      (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[2 * i + which]), s);
  }
};

template <typename T, int D>
int launch_prefill(const Derived& d, const Plan& pl, still::PrefillArgs a, hipStream_t s,
                   const Marks& mk) {
  using namespace still;
  const int nkt = d.C / 16 + (d.W + 14) / 16;  // key tiles of the score kernel
  // the chunks are decided by the score kernel for the Self-Saliency route
  // with C <= 64 (its LDS then also holds the decision's arrays), else by
  // the select kernel
  const bool fuse = a.route == ROUTE_SALIENCY && d.C <= 64;
  a.fuse_sel = fuse ? 1 : 0;
  a.n_pend_grp = fuse ? (pl.n_pend + SCORE_PEND - 1) / SCORE_PEND : 0;
  const size_t lds_score =
      (size_t)nkt * 16 * (D + Pad<T>::v) * sizeof(T) + (size_t)(3 * d.G * d.C + nkt * 16 + 80) * 4 +
      (fuse ? (size_t)3 * d.C * 4 + score_decide_bytes(d.C, d.G, D) : 0);
  // select: float64 query rows, then for the undecided tokens their list,
  // per-head results and sums; for C <= 64 the per-wave counts, the shared
  // float64 list, per-head results and sums of SEL_CPW chunks; for C > 64
  // the chunk arrays, per-head results and sums
  const size_t lds_sel_pend = (size_t)4 * D * 8 + 16 + (size_t)SEL_PEND * d.G * 8 + (size_t)SEL_PEND * 8;
  const size_t lds_sel_chunk =
      d.C <= 64 ? (size_t)16 + 64 + (size_t)SEL_CPW * 64 * 4 + (size_t)SEL_CPW * 64 * d.G * 8 + (size_t)SEL_CPW * 64 * 8
                : (size_t)d.C * 8 + (size_t)(5 * d.C + 4) * 4 + (size_t)d.C * d.G * 8 + (size_t)d.C * 8;
  const size_t lds_sel = std::max(lds_sel_pend, (size_t)4 * D * 8 + lds_sel_chunk);
  const int n_sel = (pl.n_pend + SEL_PEND - 1) / SEL_PEND +
                    (d.C <= 64 ? (pl.n_dec + SEL_CPW - 1) / SEL_CPW : pl.n_dec) +
                    (d.C <= 64 && a.score_out ? (pl.n_dec + SEL_RCH - 1) / SEL_RCH : 0);
  set_prefill_attrs<T, D>(prefill_family<T, D>());
  // F^T is made by D*D/2048 extra workgroups of the score launch (its
  // events are recorded back to back)
  mk.at(0, 0);
  mk.at(0, 1);
  mk.at(1, 0);
  if (a.route == ROUTE_SALIENCY)
    score_kernel<T, D><<<dim3(a.n_pend_grp + pl.T + D * D / 2048, d.Hkv, d.B), dim3(256), lds_score, s>>>(a);
  else
    route_kernel<T, D><<<dim3(pl.T + D * D / 2048, d.Hkv, d.B), dim3(256), 4 * D * 8, s>>>(a);
  mk.at(1, 1);
  mk.at(2, 0);
  if (!fuse) select_kernel<T, D><<<dim3(n_sel, d.Hkv, d.B), dim3(256), lds_sel, s>>>(a);
  mk.at(2, 1);
  mk.at(3, 0);
  // the forget gate (a.decay) takes instantiations of its own, so the
  // plain layer's kernels carry none of its arithmetic
  const bool dk = a.decay != nullptr;
  if constexpr (sizeof(T) == 2) {
    if (dk) state_delta_kernel<T, D, true><<<dim3(pl.NS, d.Hkv, d.B), dim3(512), SdLds<T, D>::bytes, s>>>(a);
    else state_delta_kernel<T, D><<<dim3(pl.NS, d.Hkv, d.B), dim3(512), SdLds<T, D>::bytes, s>>>(a);
  } else {
    if (dk) state_delta_f32_kernel<D, true><<<dim3(pl.NS, d.Hkv, d.B), dim3(512), Blk<T, D>::bytes, s>>>(a);
    else state_delta_f32_kernel<D><<<dim3(pl.NS, d.Hkv, d.B), dim3(512), Blk<T, D>::bytes, s>>>(a);
  }
  mk.at(3, 1);
  mk.at(4, 0);
  // the scan and, as further workgroups of the same launch, the decode-state
  // export (its events are recorded back to back)
  const int n_scan = (D * D + D + 255) / 256;
  const int ring_lo = pl.L - d.R > 0 ? pl.L - d.R : 0;
  const int n_ring_grp = (pl.L - ring_lo + 63) / 64;
  const int n_pool = pool_count_at(pl.n_dec, d.lam, d.cap_chunks);
  const int n_pool_grp = n_pool > 0 ? (n_pool + 15) / 16 : 1;  // >= 1: it writes the position
  if (dk)
    state_scan_kernel<T, D, true><<<dim3(n_scan + n_ring_grp + n_pool_grp, d.Hkv, d.B), dim3(256),
                                    Blk<T, D>::ft_bytes, s>>>(a, n_scan);
  else
    state_scan_kernel<T, D><<<dim3(n_scan + n_ring_grp + n_pool_grp, d.Hkv, d.B), dim3(256), Blk<T, D>::ft_bytes,
                              s>>>(a, n_scan);
  mk.at(4, 1);
  mk.at(5, 0);
  if (pl.part)  // (the forget gate is refused with the separate branches on the host)
    attend_kernel<T, D, 2, true><<<dim3(pl.NS * d.Hkv * pl.nHG * d.B), dim3(512), Blk<T, D>::bytes, s>>>(a);
  else if (dk && pl.HPW == 2)
    attend_kernel<T, D, 2, false, true><<<dim3(pl.NS * d.Hkv * pl.nHG * d.B), dim3(512), Blk<T, D>::bytes, s>>>(a);
  else if (dk)
    attend_kernel<T, D, 1, false, true><<<dim3(pl.NS * d.Hkv * pl.nHG * d.B), dim3(512), Blk<T, D>::bytes, s>>>(a);
  else if (pl.HPW == 2)
    attend_kernel<T, D, 2><<<dim3(pl.NS * d.Hkv * pl.nHG * d.B), dim3(512), Blk<T, D>::bytes, s>>>(a);
  else
    attend_kernel<T, D, 1><<<dim3(pl.NS * d.Hkv * pl.nHG * d.B), dim3(512), Blk<T, D>::bytes, s>>>(a);
  mk.at(5, 1);
  mk.at(6, 0);
  mk.at(6, 1);
  return hipGetLastError() == hipSuccess ? STILL_OK : STILL_EHIP;
}

template <typename T, int D, int G>
int launch_decode_g(const Derived& d, still::DecodeArgs a, hipStream_t s) {
  using namespace still;
  const bool paged = a.pages.base != nullptr;
  const size_t lds = paged ? DecLds<T, D, G>::bytes_paged(d.W) : DecLds<T, D, G>::bytes(d.W);
  if (lds > 160 * 1024) return STILL_EUNSUPPORTED;
  set_decode_attr<T, D, G>(decode_family<T, D, G>());
  if (paged) {
    decode_kernel<T, D, G, true><<<dim3(d.Hkv, d.B), dim3(DEC_THREADS), lds, s>>>(a);
  } else if (a.pool8) {
    if constexpr (sizeof(T) == 2) decode_kernel<T, D, G, false, true><<<dim3(d.Hkv, d.B), dim3(DEC_THREADS), lds, s>>>(a);
    else return STILL_EUNSUPPORTED;
  } else {
    decode_kernel<T, D, G><<<dim3(d.Hkv, d.B), dim3(DEC_THREADS), lds, s>>>(a);
  }
  return hipGetLastError() == hipSuccess ? STILL_OK : STILL_EHIP;
}

template <typename T, int D>
int launch_decode(const Derived& d, still::DecodeArgs a, hipStream_t s) {
  using namespace still;
  if (a.boundary || a.pos) {  // per-row positions: every row's workgroups look
    // the fold's LDS: the float32 path's row groups, or the matrix-core
    // path's F, value block and features (16-bit data)
    const size_t fold = sizeof(T) == 2 ? BndFoldLds<D>::bytes : DecLds<T, D, 1>::fold_bytes;
    const size_t lds = DecLds<T, D, 1>::uni + fold;
    set_boundary_attr<T, D>(24 + prefill_family<T, D>());
    decode_boundary_kernel<T, D><<<dim3(d.Hkv, d.B), dim3(BND_THREADS), lds, s>>>(a);
    if (hipGetLastError() != hipSuccess) return STILL_EHIP;
  }
  switch (d.G) {
    case 1: return launch_decode_g<T, D, 1>(d, a, s);
    case 2: return launch_decode_g<T, D, 2>(d, a, s);
    case 4: return launch_decode_g<T, D, 4>(d, a, s);
    default: return launch_decode_g<T, D, 8>(d, a, s);
  }
}

void fill_state_offsets(const still_state_layout& L, long* unit, long* S, long* z, long* pk,
                        long* pv, long* pp, long* rk, long* rv, long* rp, long* rf, long* pend,
                        long* meta) {
  *unit = L.unit_bytes;
  *S = L.S;
  *z = L.z;
  *pk = L.pool_k;
  *pv = L.pool_v;
  *pp = L.pool_pos;
  *rk = L.ring_k;
  *rv = L.ring_v;
  *rp = L.ring_phi;
  *rf = L.ring_flag;
  *pend = L.pending;
  *meta = L.meta;
}

// Scratch of still_prefill_noalloc: a static device array, so that the call
// allocates nothing. Each GPU the library runs on holds its own copy until
// the process ends. In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress, taken once per device (with that
// device current) on the first call there and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return STILL_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return STILL_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return STILL_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return STILL_OK;
}

}  // namespace

// ---------------------------------------------------------------- backward
struct BwPlan {
  int64_t phq, phk, dphq, dphk, dz, lnN, delta, kept, cS, cR, total;
};

static BwPlan bw_plan(const Derived& d, int64_t L) {
  BwPlan w;
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const int64_t nq = (int64_t)d.B * d.Hq * L, nk = (int64_t)d.B * d.Hkv * L;
  w.phq = take(nq * d.D * 4);
  w.phk = take(nk * d.D * 4);
  w.dphq = take(nq * d.D * 4);
  w.dphk = take(nk * d.D * 4);
  w.dz = take((nq + nk) * d.D * 4);
  w.lnN = take(nq * 4);
  w.delta = take(nq * 4);
  w.kept = take(nk);
  const int64_t T = (L + d.C - 1) / d.C;
  w.cS = take((int64_t)d.B * d.Hkv * T * ((int64_t)d.D * d.D + d.D) * 4);
  w.cR = take((int64_t)d.B * d.Hkv * T * ((int64_t)d.D * d.D + d.D) * 4);
  w.total = o;
  return w;
}

template <typename T, int D>
static int launch_backward(const Derived& d, const BwPlan& w, still::BackwardArgs a, hipStream_t s) {
  using namespace still;
  set_backward_attrs<T, D>();
  const int L = a.L;
  bw_zero_kernel<<<dim3(1), dim3(BW_THREADS), 0, s>>>(a.dgate, d.Hq);
  bw_zero_kernel<<<dim3(64), dim3(BW_THREADS), 0, s>>>(a.dfmap, (int64_t)d.Hkv * D * D);
  const int64_t nk = (int64_t)d.B * d.Hkv * L;
  bw_flags_kernel<<<dim3((unsigned)std::min<int64_t>((nk + BW_THREADS - 1) / BW_THREADS, 4096)),
                    dim3(BW_THREADS), 0, s>>>(a);
  const dim3 rows_grid((L + BW_ROWS - 1) / BW_ROWS, d.B * (d.Hq + d.Hkv));
  bw_phi_kernel<T, D><<<rows_grid, dim3(BW_THREADS), BwRowLds<D>::bytes, s>>>(a);
  const int64_t nq = (int64_t)d.B * d.Hq * L;
  bw_rowstat_kernel<<<dim3((unsigned)((nq + 3) / 4)), dim3(BW_THREADS), 0, s>>>(a, D);
  bw_chunk_delta_kernel<T, D><<<dim3(a.T, d.B * d.Hkv, 2), dim3(BW_THREADS), 0, s>>>(a);
  bw_chunk_scan_kernel<<<dim3((D * D + D + BW_THREADS - 1) / BW_THREADS, 2 * d.B * d.Hkv), dim3(BW_THREADS), 0, s>>>(
      a, D);
  bw_query_kernel<T, D><<<dim3((L + BW_QT - 1) / BW_QT, d.Hq, d.B), dim3(BW_THREADS), BwQLds<D>::bytes, s>>>(a);
  bw_key_kernel<T, D><<<dim3((L + BW_KT - 1) / BW_KT, d.Hkv, d.B), dim3(BW_THREADS), BwKLds<D>::bytes, s>>>(a);
  const int n_kept = pool_count_at(a.n_dec, a.lam, a.cap_chunks);
  if (n_kept > 0)
    bw_pool_kernel<T, D><<<dim3((n_kept + BW_KT - 1) / BW_KT, d.Hkv,
                                d.B * d.G * ((L + BW_POOL_SEG - 1) / BW_POOL_SEG)),
                           dim3(BW_THREADS), BwKLds<D>::bytes, s>>>(a);
  bw_npmap_kernel<T, D><<<rows_grid, dim3(BW_THREADS), BwRowLds<D>::bytes, s>>>(a);
  const int64_t nrow = (int64_t)d.B * (d.G + 1) * L;
  bw_dfmap_kernel<T, D><<<dim3((unsigned)((nrow + BW_DF_ROWS - 1) / BW_DF_ROWS), d.Hkv), dim3(BW_THREADS), 0, s>>>(a);
  (void)w;
  return hipGetLastError() == hipSuccess ? STILL_OK : STILL_EHIP;
}

extern "C" {

int still_lambda(const still_params* p) {
  Derived d;
  const int rc = derive(p, &d);
  return rc == STILL_OK ? d.lam : rc;
}

int still_state_layout_get(const still_params* p, still_state_layout* out) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  if (!out) return STILL_EINVAL;
  layout(d, out);
  return STILL_OK;
}

int64_t still_state_bytes(const still_params* p) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  still_state_layout L;
  layout(d, &L);
  return L.unit_bytes * d.B * d.Hkv;
}

int64_t still_workspace_bytes(const still_params* p, int64_t seq_len) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  if (seq_len <= 0) return 0;
  if (seq_len > (int64_t)1 << 30) return STILL_EINVAL;
  return ws_bytes_any(d, seq_len);
}

// Branch partials of still_prefill_partials (all null for the other entries).
struct Partials {
  float *y_sa, *lse_sa, *y_la, *lse_la;
  bool any() const { return y_sa || lse_sa || y_la || lse_la; }
};

// The caller's pages of a paged pool (STILL_FLAG_PAGED_POOL).
struct PagesArg {
  void* base;
  const int32_t* table;
  int64_t n_pages;
};

// Paged params need the paged entries and the paged entries paged params;
// the arena is addressed with 31-bit byte offsets.
static int check_pages(const Derived& d, const PagesArg* pg) {
  if (d.paged != (pg != nullptr)) return STILL_EINVAL;
  if (!pg) return STILL_OK;
  if (!pg->base || !pg->table || misaligned(pg->base) || ((uintptr_t)pg->table & 3u)) return STILL_EINVAL;
  const int64_t page_bytes = (int64_t)2 * STILL_POOL_PAGE_ROWS * d.D * d.esz;
  if (pg->n_pages < 1 || pg->n_pages > ((int64_t)1 << 31) / page_bytes - 1) return STILL_EINVAL;
  return STILL_OK;
}

static still::PoolPages to_pool_pages(const Derived& d, const PagesArg& pg) {
  still::PoolPages r;
  r.base = reinterpret_cast<char*>(pg.base);
  r.table = pg.table;
  r.n_pages = (int)pg.n_pages;
  r.width = (d.P + STILL_POOL_PAGE_ROWS - 1) / STILL_POOL_PAGE_ROWS;
  return r;
}

static int prefill_impl(const still_params* p, int64_t seq_len, const void* q, const void* k,
                        const void* v, const void* fmap_w, const float* gate, void* out,
                        int32_t* sel_idx, float* score, void* state, void* workspace,
                        size_t ws_bytes, void* stream, void* const* events, int n_pairs,
                        Partials parts = Partials{nullptr, nullptr, nullptr, nullptr},
                        const void* out_gate = nullptr, const float* decay = nullptr,
                        const PagesArg* pages = nullptr) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  rc = check_pages(d, pages);
  if (rc != STILL_OK) return rc;
  if (seq_len < 1 || seq_len > ((int64_t)1 << 30)) return STILL_EINVAL;
  if ((int64_t)d.B * d.Hq * seq_len * d.D > ((int64_t)1 << 40)) return STILL_EINVAL;
  // one (batch row, head) sequence is addressed with 32-bit byte offsets
  if (seq_len * d.D * (int64_t)d.esz >= ((int64_t)1 << 31)) return STILL_EUNSUPPORTED;
  if (!q || !k || !v || !fmap_w || !gate || !out || !state || !workspace) return STILL_EINVAL;
  const int n_dec = (int)((seq_len - 1) / d.C);
  if (!sel_idx && n_dec > 0 && d.lam > 0) return STILL_EINVAL;
  if (STILL_ROUTE_OF(p->flags) == STILL_ROUTE_EXTERNAL && !score) return STILL_EINVAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(fmap_w) || misaligned(out) ||
      misaligned(state) || misaligned(workspace) || misaligned(gate))
    return STILL_EINVAL;
  if (misaligned(parts.y_sa) || misaligned(parts.y_la) || misaligned(out_gate) || misaligned(decay))
    return STILL_EINVAL;
  const bool merge_sum = (p->flags & STILL_FLAG_MERGE_SUM) != 0;
  const bool softmax_only = (p->flags & STILL_FLAG_SOFTMAX_ONLY) != 0;
  if (merge_sum && softmax_only) return STILL_EINVAL;
  if (decay && merge_sum) return STILL_EUNSUPPORTED;  // the forget gate takes the single-normaliser walk
  // the branches are kept apart for the sum merge and for the partials
  const Plan pl = plan(d, seq_len, merge_sum || parts.any());
  if ((int64_t)ws_bytes < pl.ws_total) return STILL_EWORKSPACE;
  still_state_layout SL;
  layout(d, &SL);

  still::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  char* ws = reinterpret_cast<char*>(workspace);
  a.q = q;
  a.k = k;
  a.v = v;
  a.fmap_w = fmap_w;
  a.gate = gate;
  a.out = out;
  a.out_gate = out_gate;
  a.decay = decay;
  if (pages) a.pages = to_pool_pages(d, *pages);
  a.sel = sel_idx;
  a.route = (int)STILL_ROUTE_OF(p->flags);
  if (a.route == still::ROUTE_EXTERNAL) {  // the caller's scores are an input here
    a.ext_score = score;
    score = nullptr;
  }
  a.score = score ? score : reinterpret_cast<float*>(ws + pl.ws_score);
  a.score_out = score ? 1 : 0;
  a.delta = reinterpret_cast<float*>(ws + pl.ws_delta);
  a.selflag = reinterpret_cast<uint8_t*>(ws + pl.ws_flag);
  a.ft = ws + pl.ws_ft;
  a.dS = reinterpret_cast<float*>(ws + pl.ws_dS);
  a.rlist = reinterpret_cast<int*>(ws + pl.ws_rl);
  a.state = reinterpret_cast<char*>(state);
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.L = pl.L;
  a.W = d.W;
  a.C = d.C;
  a.m = d.m;
  a.T = pl.T;
  a.n_dec = pl.n_dec;
  a.lam = d.lam;
  a.cap_chunks = d.cap_chunks;
  a.K = pl.K;
  a.NS = pl.NS;
  a.nHG = pl.nHG;
  a.Gs = pl.Gs;
  a.fp32_out = (p->flags & STILL_FLAG_FP32_OUT) ? 1 : 0;
  a.softmax_only = softmax_only ? 1 : 0;
  a.pool8 = d.pool8 ? 1 : 0;
  a.merge_sum = merge_sum ? 1 : 0;
  a.y_sa = parts.y_sa;
  a.lse_sa = parts.lse_sa;
  a.y_la = parts.y_la;
  a.lse_la = parts.lse_la;
  a.scale = d.scale;
  a.eps = d.eps;
  a.scale64 = d.scale64;
  a.eps64 = d.eps64;
  a.R = d.R;
  fill_state_offsets(SL, &a.st_unit, &a.st_S, &a.st_z, &a.st_pool_k, &a.st_pool_v,
                     &a.st_pool_pos, &a.st_ring_k, &a.st_ring_v, &a.st_ring_phi,
                     &a.st_ring_flag, &a.st_pending, &a.st_meta);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const Marks mk{events, n_pairs, s};
  if (p->dtype == STILL_DTYPE_BF16) {
    if (d.D == 128) return launch_prefill<bf16, 128>(d, pl, a, s, mk);
    return launch_prefill<bf16, 64>(d, pl, a, s, mk);
  }
  return launch_prefill<float, 64>(d, pl, a, s, mk);
}

int still_prefill(const still_params* p, int64_t seq_len, const void* q, const void* k,
                  const void* v, const void* fmap_w, const float* gate, void* out,
                  int32_t* sel_idx, float* score, void* state, void* workspace,
                  size_t ws_bytes, void* stream) {
  return prefill_impl(p, seq_len, q, k, v, fmap_w, gate, out, sel_idx, score, state, workspace,
                      ws_bytes, stream, nullptr, 0);
}

int still_prefill_gated(const still_params* p, int64_t seq_len, const void* q, const void* k,
                        const void* v, const void* fmap_w, const float* gate,
                        const void* out_gate, void* out, int32_t* sel_idx, float* score,
                        void* state, void* workspace, size_t ws_bytes, void* stream) {
  if (!out_gate) return STILL_EINVAL;
  return prefill_impl(p, seq_len, q, k, v, fmap_w, gate, out, sel_idx, score, state, workspace,
                      ws_bytes, stream, nullptr, 0, Partials{nullptr, nullptr, nullptr, nullptr},
                      out_gate);
}

int still_prefill_decay(const still_params* p, int64_t seq_len, const void* q, const void* k,
                        const void* v, const void* fmap_w, const float* gate, const float* decay,
                        void* out, int32_t* sel_idx, float* score, void* state, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (!decay) return STILL_EINVAL;
  return prefill_impl(p, seq_len, q, k, v, fmap_w, gate, out, sel_idx, score, state, workspace,
                      ws_bytes, stream, nullptr, 0, Partials{nullptr, nullptr, nullptr, nullptr},
                      nullptr, decay);
}

int still_prefill_paged(const still_params* p, int64_t seq_len, const void* q, const void* k,
                        const void* v, const void* fmap_w, const float* gate, void* out,
                        int32_t* sel_idx, float* score, void* state, void* pool_pages,
                        const int32_t* page_table, int64_t n_pages, void* workspace, size_t ws_bytes,
                        void* stream) {
  const PagesArg pg{pool_pages, page_table, n_pages};
  return prefill_impl(p, seq_len, q, k, v, fmap_w, gate, out, sel_idx, score, state, workspace,
                      ws_bytes, stream, nullptr, 0, Partials{nullptr, nullptr, nullptr, nullptr},
                      nullptr, nullptr, &pg);
}

int64_t still_pool_rows(const still_params* p, int64_t n_tokens) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  if (n_tokens < 0 || n_tokens > ((int64_t)1 << 30)) return STILL_EINVAL;
  const int n_dec = n_tokens > 0 ? (int)((n_tokens - 1) / d.C) : 0;
  return still::pool_count_at(n_dec, d.lam, d.cap_chunks);
}

int still_prefill_timed(const still_params* p, int64_t seq_len, const void* q, const void* k,
                        const void* v, const void* fmap_w, const float* gate, void* out,
                        int32_t* sel_idx, float* score, void* state, void* workspace,
                        size_t ws_bytes, void* stream, void* const* events, int n_pairs) {
  if (n_pairs < 0 || n_pairs > 7 || (n_pairs > 0 && !events)) return STILL_EINVAL;
  return prefill_impl(p, seq_len, q, k, v, fmap_w, gate, out, sel_idx, score, state, workspace,
                      ws_bytes, stream, events, n_pairs);
}

int still_prefill_partials(const still_params* p, int64_t seq_len, const void* q, const void* k,
                           const void* v, const void* fmap_w, const float* gate, void* out,
                           int32_t* sel_idx, float* score, void* state, void* workspace,
                           size_t ws_bytes, void* stream, float* y_sa, float* lse_sa, float* y_la,
                           float* lse_la) {
  if (!y_sa || !lse_sa || !y_la || !lse_la) return STILL_EINVAL;
  if (p && (p->flags & STILL_FLAG_SOFTMAX_ONLY)) return STILL_EINVAL;
  return prefill_impl(p, seq_len, q, k, v, fmap_w, gate, out, sel_idx, score, state, workspace,
                      ws_bytes, stream, nullptr, 0, Partials{y_sa, lse_sa, y_la, lse_la});
}

// Varlen prefill: the rows are prefilled one after another on the stream,
// each as a batch of one over its own length (row b's arrays start after
// the rows before it; its state units are b * Hkv .. b * Hkv + Hkv - 1 of
// the batch's state), sharing one workspace.
int64_t still_workspace_bytes_varlen(const still_params* p, const int64_t* seq_lens) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  if (!seq_lens) return STILL_EINVAL;
  still_params p1 = *p;
  p1.batch = 1;
  Derived d1;
  derive(&p1, &d1);
  int64_t ws = 0;
  for (int b = 0; b < d.B; ++b) {
    if (seq_lens[b] < 1 || seq_lens[b] > ((int64_t)1 << 30)) return STILL_EINVAL;
    const int64_t w = ws_bytes_any(d1, seq_lens[b]);
    ws = w > ws ? w : ws;
  }
  return ws;
}

int still_prefill_varlen(const still_params* p, const int64_t* seq_lens, const void* q,
                         const void* k, const void* v, const void* fmap_w, const float* gate,
                         void* out, int32_t* sel_idx, float* score, void* state, void* workspace,
                         size_t ws_bytes, void* stream) {
  const int64_t need = still_workspace_bytes_varlen(p, seq_lens);
  if (need < 0) return (int)need;
  if ((int64_t)ws_bytes < need) return STILL_EWORKSPACE;
  if (!q || !k || !v || !out || !state) return STILL_EINVAL;
  Derived d;
  derive(p, &d);
  still_params p1 = *p;
  p1.batch = 1;
  still_state_layout SL;
  layout(d, &SL);
  // checks that could fail on a later row are made before the first runs
  for (int b = 0; b < d.B; ++b) {
    if (seq_lens[b] * d.D * (int64_t)d.esz >= ((int64_t)1 << 31)) return STILL_EUNSUPPORTED;
    if (!sel_idx && d.lam > 0 && seq_lens[b] > d.C) return STILL_EINVAL;
  }
  const size_t osz = (p->flags & STILL_FLAG_FP32_OUT) ? 4 : d.esz;
  int64_t tok = 0, dec = 0;  // tokens and decided chunks of the rows before b
  for (int b = 0; b < d.B; ++b) {
    const int64_t L = seq_lens[b], n_dec = (L - 1) / d.C;
    const int rc = prefill_impl(
        &p1, L, reinterpret_cast<const char*>(q) + (size_t)tok * d.Hq * d.D * d.esz,
        reinterpret_cast<const char*>(k) + (size_t)tok * d.Hkv * d.D * d.esz,
        reinterpret_cast<const char*>(v) + (size_t)tok * d.Hkv * d.D * d.esz, fmap_w, gate,
        reinterpret_cast<char*>(out) + (size_t)tok * d.Hq * d.D * osz,
        sel_idx ? sel_idx + (size_t)dec * d.Hkv * d.lam : nullptr,
        score ? score + (size_t)tok * d.Hkv : nullptr,
        reinterpret_cast<char*>(state) + (size_t)b * d.Hkv * SL.unit_bytes, workspace, ws_bytes,
        stream, nullptr, 0);
    if (rc != STILL_OK) return rc;
    tok += L;
    dec += n_dec;
  }
  return STILL_OK;
}

int still_prefill_noalloc(const still_params* p, int64_t seq_len, const void* q, const void* k,
                          const void* v, const void* fmap_w, const float* gate, void* out,
                          int32_t* sel_idx, float* score, void* state, void* stream) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  if (d.paged) return STILL_EINVAL;  // the paged pool has its own entries
  if (seq_len < 1 || seq_len > ((int64_t)1 << 30)) return STILL_EINVAL;
  if (ws_bytes_any(d, seq_len) > (int64_t)kNoAllocScratchBytes) return STILL_ESCRATCH;
  void* ws = nullptr;
  const int rs = scratch_address(&ws);
  if (rs != STILL_OK) return rs;
  return prefill_impl(p, seq_len, q, k, v, fmap_w, gate, out, sel_idx, score, state, ws,
                      kNoAllocScratchBytes, stream, nullptr, 0);
}

int64_t still_noalloc_scratch_bytes(void) { return (int64_t)kNoAllocScratchBytes; }

// n_tokens decode steps: step s takes token s of q, k, v ([n][B][H][d])
// and writes out[s], sel_new[s]; row b's position is pos + s, or
// row_pos[b] + s with per-row positions (device array).
static int decode_impl(const still_params* p, int64_t pos, const int32_t* row_pos, int n_tokens,
                       const void* q, const void* k, const void* v, const void* fmap_w,
                       const float* gate, void* state, void* out, int32_t* sel_new, void* stream,
                       const void* out_gate = nullptr, const float* decay = nullptr,
                       const PagesArg* pages = nullptr) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  rc = check_pages(d, pages);
  if (rc != STILL_OK) return rc;
  if (p->flags & STILL_FLAG_MERGE_SUM) return STILL_EUNSUPPORTED;  // decode keeps one normaliser
  // the caller's scores are a prefill input only
  if (STILL_ROUTE_OF(p->flags) == STILL_ROUTE_EXTERNAL) return STILL_EUNSUPPORTED;
  if (n_tokens < 1 || n_tokens > (1 << 20)) return STILL_EINVAL;
  if (!row_pos && (pos < 1 || pos + n_tokens - 1 > ((int64_t)1 << 30))) return STILL_EINVAL;
  if (!q || !k || !v || !fmap_w || !gate || !state || !out) return STILL_EINVAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(fmap_w) || misaligned(out) ||
      misaligned(state) || misaligned(gate) || misaligned(out_gate) || misaligned(decay) ||
      ((uintptr_t)row_pos & 3u))
    return STILL_EINVAL;
  still_state_layout SL;
  layout(d, &SL);
  still::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.fmap_w = fmap_w;
  a.gate = gate;
  a.decay = decay;
  if (pages) a.pages = to_pool_pages(d, *pages);
  a.state = reinterpret_cast<char*>(state);
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.W = d.W;
  a.C = d.C;
  a.m = d.m;
  a.lam = d.lam;
  a.R = d.R;
  a.pos = row_pos;
  a.softmax_only = (p->flags & STILL_FLAG_SOFTMAX_ONLY) ? 1 : 0;
  a.pool8 = d.pool8 ? 1 : 0;
  a.route = (int)STILL_ROUTE_OF(p->flags);
  a.fp32_out = (p->flags & STILL_FLAG_FP32_OUT) ? 1 : 0;
  a.scale = d.scale;
  a.eps = d.eps;
  a.scale64 = d.scale64;
  a.eps64 = d.eps64;
  fill_state_offsets(SL, &a.st_unit, &a.st_S, &a.st_z, &a.st_pool_k, &a.st_pool_v,
                     &a.st_pool_pos, &a.st_ring_k, &a.st_ring_v, &a.st_ring_phi,
                     &a.st_ring_flag, &a.st_pending, &a.st_meta);
  const size_t qb = (size_t)d.B * d.Hq * d.D * d.esz, kb = (size_t)d.B * d.Hkv * d.D * d.esz;
  const size_t ob = (size_t)d.B * d.Hq * d.D * (a.fp32_out ? 4 : d.esz);
  const size_t sb = (size_t)d.B * d.Hkv * d.lam;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int i = 0; i < n_tokens; ++i) {
    a.q = reinterpret_cast<const char*>(q) + i * qb;
    a.k = reinterpret_cast<const char*>(k) + i * kb;
    a.v = reinterpret_cast<const char*>(v) + i * kb;
    a.out = reinterpret_cast<char*>(out) + i * ob;
    a.out_gate = out_gate ? reinterpret_cast<const char*>(out_gate) + i * qb : nullptr;
    a.sel_new = sel_new ? sel_new + i * sb : nullptr;
    a.t = row_pos ? i : (int)(pos + i);
    a.boundary = !row_pos && ((pos + i) % d.C) == 0 ? 1 : 0;
    if (p->dtype == STILL_DTYPE_BF16)
      rc = d.D == 128 ? launch_decode<bf16, 128>(d, a, s) : launch_decode<bf16, 64>(d, a, s);
    else
      rc = launch_decode<float, 64>(d, a, s);
    if (rc != STILL_OK) return rc;
  }
  return STILL_OK;
}

int still_decode_step(const still_params* p, int64_t pos, const void* q, const void* k,
                      const void* v, const void* fmap_w, const float* gate, void* state,
                      void* out, int32_t* sel_new, void* workspace, size_t ws_bytes,
                      void* stream) {
  (void)workspace;
  (void)ws_bytes;
  return decode_impl(p, pos, nullptr, 1, q, k, v, fmap_w, gate, state, out, sel_new, stream);
}

int still_decode_step_gated(const still_params* p, int64_t pos, const void* q, const void* k,
                            const void* v, const void* fmap_w, const float* gate,
                            const void* out_gate, void* state, void* out, int32_t* sel_new,
                            void* stream) {
  if (!out_gate) return STILL_EINVAL;
  return decode_impl(p, pos, nullptr, 1, q, k, v, fmap_w, gate, state, out, sel_new, stream,
                     out_gate);
}

int still_decode_step_decay(const still_params* p, int64_t pos, const void* q, const void* k,
                            const void* v, const void* fmap_w, const float* gate,
                            const float* decay, void* state, void* out, int32_t* sel_new,
                            void* stream) {
  if (!decay) return STILL_EINVAL;
  return decode_impl(p, pos, nullptr, 1, q, k, v, fmap_w, gate, state, out, sel_new, stream,
                     nullptr, decay);
}

int still_decode_step_paged(const still_params* p, int64_t pos, const void* q, const void* k,
                            const void* v, const void* fmap_w, const float* gate, void* state,
                            void* pool_pages, const int32_t* page_table, int64_t n_pages, void* out,
                            int32_t* sel_new, void* stream) {
  const PagesArg pg{pool_pages, page_table, n_pages};
  return decode_impl(p, pos, nullptr, 1, q, k, v, fmap_w, gate, state, out, sel_new, stream, nullptr,
                     nullptr, &pg);
}

int still_decode_tokens(const still_params* p, int64_t pos, const int32_t* row_pos, int n_tokens,
                        const void* q, const void* k, const void* v, const void* fmap_w,
                        const float* gate, void* state, void* out, int32_t* sel_new,
                        void* stream) {
  return decode_impl(p, pos, row_pos, n_tokens, q, k, v, fmap_w, gate, state, out, sel_new,
                     stream);
}

int64_t still_backward_workspace_bytes(const still_params* p, int64_t seq_len) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  if (seq_len < 1 || seq_len > ((int64_t)1 << 24)) return STILL_EINVAL;
  return bw_plan(d, seq_len).total;
}

int still_backward(const still_params* p, int64_t seq_len, const void* q, const void* k, const void* v,
                   const void* fmap_w, const float* gate, const int32_t* sel_idx, const float* y,
                   const float* lse_sa, const float* lse_la, const float* dy, float* dq, float* dk,
                   float* dv, float* dfmap, float* dgate, void* workspace, size_t ws_bytes,
                   void* stream) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != STILL_OK) return rc;
  // the gradients are those of the default merge (one normaliser)
  if (p->flags & (STILL_FLAG_SOFTMAX_ONLY | STILL_FLAG_MERGE_SUM)) return STILL_EUNSUPPORTED;
  if (seq_len < 1 || seq_len > ((int64_t)1 << 24)) return STILL_EINVAL;
  if ((int64_t)d.B * (d.Hq + d.Hkv) > 65535) return STILL_EUNSUPPORTED;  // grid rows
  const int n_dec = (int)((seq_len - 1) / d.C);
  if (!q || !k || !v || !fmap_w || !gate || !y || !lse_sa || !lse_la || !dy || !dq || !dk || !dv ||
      !dfmap || !dgate || !workspace)
    return STILL_EINVAL;
  if (!sel_idx && n_dec > 0 && d.lam > 0) return STILL_EINVAL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(fmap_w) || misaligned(y) ||
      misaligned(dy) || misaligned(dq) || misaligned(dk) || misaligned(dv) || misaligned(dfmap) ||
      misaligned(workspace))
    return STILL_EINVAL;
  const BwPlan w = bw_plan(d, seq_len);
  if ((int64_t)ws_bytes < w.total) return STILL_EWORKSPACE;
  char* ws = reinterpret_cast<char*>(workspace);
  still::BackwardArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.fmap_w = fmap_w;
  a.gate = gate;
  a.sel = sel_idx;
  a.y = y;
  a.lse_sa = lse_sa;
  a.lse_la = lse_la;
  a.dy = dy;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dfmap = dfmap;
  a.dgate = dgate;
  a.phq = reinterpret_cast<float*>(ws + w.phq);
  a.phk = reinterpret_cast<float*>(ws + w.phk);
  a.dphq = reinterpret_cast<float*>(ws + w.dphq);
  a.dphk = reinterpret_cast<float*>(ws + w.dphk);
  a.dz = reinterpret_cast<float*>(ws + w.dz);
  a.lnN = reinterpret_cast<float*>(ws + w.lnN);
  a.delta = reinterpret_cast<float*>(ws + w.delta);
  a.kept = reinterpret_cast<uint8_t*>(ws + w.kept);
  a.cS = reinterpret_cast<float*>(ws + w.cS);
  a.cR = reinterpret_cast<float*>(ws + w.cR);
  a.T = (int)((seq_len + d.C - 1) / d.C);
  a.cap_chunks = d.cap_chunks;
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.G;
  a.L = (int)seq_len;
  a.W = d.W;
  a.C = d.C;
  a.n_dec = d.lam > 0 ? n_dec : 0;
  a.lam = d.lam;
  a.scale = d.scale;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p->dtype == STILL_DTYPE_BF16)
    return d.D == 128 ? launch_backward<bf16, 128>(d, w, a, s) : launch_backward<bf16, 64>(d, w, a, s);
  return launch_backward<float, 64>(d, w, a, s);
}

const char* still_status_str(int status) {
  switch (status) {
    case STILL_OK: return "ok";
    case STILL_EINVAL: return "invalid argument";
    case STILL_EUNSUPPORTED: return "unsupported configuration";
    case STILL_EWORKSPACE: return "workspace too small";
    case STILL_EHIP: return "HIP launch failed";
    case STILL_ESTATE: return "decode position does not match the state";
    case STILL_ESCRATCH: return "problem needs more scratch than still_prefill_noalloc's static buffer";
    default: return "unknown status";
  }
}

}  // extern "C"
