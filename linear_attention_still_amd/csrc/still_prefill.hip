// Prefill kernels of one STILL layer (chunk-parallel form) for gfx950.
//
// Pages cited (short tag -> page title):
//   [P2] "NeurIPS 2026|层内混合注意力：告别位置「伪混合」，STILL首个内容感知的层内混合注意力架构",
//        sections 亮点一 (固定预算路由, 延迟选择与分块并行), 亮点二
//   [P3] "STILL: Content-Aware Intra-Layer Hybrid Attention for Efficient
//        LLM Linearization", sections "Content-Aware Routing with Fixed
//        Budget", "Delayed Chunk-Level Selection for Unified
//        Training-Inference Parallelism", "Self-Saliency Score",
//        "NP-Map: Norm-Preserving Feature Map"
//
// Launch sequence on one stream (host side in still_api.hip):
//   1. F^T copy         so MFMA fragments of F^T are 16-byte reads (extra
//                       workgroups of the score launch)
//   2. score            windowed Self-Saliency Score, float32, + error bound
//   3. select           per decided chunk: Top-lambda, float64 refinement of
//                       candidates the float32 bound cannot separate; float64
//                       scores of the undecided chunk (decode state)
//   4. state_delta      per super-chunk: sum of phi(k) v^T over the chunks it
//                       folds into the linear state (float64 for the rare
//                       keys whose float32 features are not accurate enough)
//   5. state_scan       exclusive prefix over super-chunks (in place) and the
//                       exported S, z (their total)
//   6. attend           per super-chunk, chunk by chunk: softmax over window
//                       + own chunk + kept pool, NP-Map linear attention over
//                       the state and the not-yet-folded band, one softmax-
//                       style normaliser over both, then fold the next chunk
//   7. export           decode state: kept pool, recent-token ring, position
//                       (extra workgroups of the scan launch: it needs only
//                       the selection and the inputs)
#include "still_common.h"

namespace still {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* fmap_w;
  const float* gate;
  void* out;
  int32_t* sel;      // [B][Hkv][n_dec][lam]
  float* score;      // [B][Hkv][L]
  float* delta;      // [B][Hkv][L]  float32 score error bound
  uint8_t* selflag;  // [B][Hkv][L]
  void* ft;          // [Hkv][D][D] F^T in T
  float* dS;         // [B][Hkv][NS][D*D + D]
  char* state;
  int B, Hq, Hkv, G, L, W, C, m, T, n_dec, lam, cap_chunks, K, NS, nHG, Gs, fp32_out;
  int score_out;  // the caller asked for the scores (score is theirs)
  int softmax_only, merge_sum;  // branch variants (linear branch dropped / sum merge)
  int pool8;                    // the decode state's pool rows as E4M3 codes + row scales
  float* y_sa;    // [B][Hq][L][D] softmax-branch output, or null (separate walk)
  float* lse_sa;  // [B][Hq][L] natural log of its normaliser, or null
  float* y_la;    // [B][Hq][L][D] linear-branch output (no gate), or null
  float* lse_la;  // [B][Hq][L] natural log of sum <phi(q), phi(k)>, or null
  int* rlist;     // [B][Hkv][T][C + 1] tokens whose exported score is refined
  int route;      // routing metric (ROUTE_*)
  const void* out_gate;    // [B][Hq][L][D] T: channel-wise output gate before the sigmoid, or null
  int fuse_sel;            // the score kernel decides the chunks (Self-Saliency route, C <= 64)
  const float* decay;      // [Hkv] forget factor of the linear state in (0, 1], or null (1)
  PoolPages pages;         // the decode state's pool rows in pages (base null: in the state)
  int n_pend_grp;          // with fuse_sel: score workgroups (first) for the undecided chunk's float64 scores
  const float* ext_score;  // [B][Hkv][L] the caller's scores (ROUTE_EXTERNAL)
  float scale, eps;
  double scale64, eps64;  // the same parameters for the float64 paths
  long st_unit, st_S, st_z, st_pool_k, st_pool_v, st_pool_pos, st_ring_k, st_ring_v,
      st_ring_phi, st_ring_flag, st_pending, st_meta;
  int R;
};

template <typename T>
struct Pad {
  static constexpr int v = 16 / sizeof(T);  // one 16-byte vector of padding
};

// ------------------------------------------------------------ 1. F^T ----
// Part bx (of D*D/2048) of F^T for kv head kv, by 256 threads; run by extra
// workgroups of the score launch (the score kernel does not read it).
template <typename T, int D>
__device__ __forceinline__ void fmap_transpose_part(const PrefillArgs& a, int bx, int kv) {
  // F^T in fragment order: element ((ft * D/32 + kb) * 64 + lane) * 8 + s
  // holds F[32 kb + 8 g + s][16 ft + r], lane = 16 g + r, i.e. the B operand
  // fragments of X F for feature tile ft and d block kb, 8 per lane.
  const T* F = reinterpret_cast<const T*>(a.fmap_w) + (size_t)kv * D * D;
  T* Ft = reinterpret_cast<T*>(a.ft) + (size_t)kv * D * D;
  const int base = bx * 256 * 8;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = base + q * 256 + threadIdx.x;
    const int sl = e & 7, lane = (e >> 3) & 63, pr = e >> 9;
    const int ftile = pr / (D / 32), kb = pr % (D / 32);
    Ft[e] = F[(size_t)(32 * kb + 8 * (lane >> 4) + sl) * D + 16 * ftile + (lane & 15)];
  }
}

// ----------------------------------------------------------- 2. score ----
// One workgroup per (chunk, kv head, batch row), 4 waves. Keys of the
// chunk's windows [cC-W+1, cC+C-1] are staged in LDS; each wave takes
// 16-query tiles of one head, computes window logits with MFMA, keeps an
// online max / total / non-self total and the self logit, and turns them
// into the two-point KL form of the score [P3 "Self-Saliency Score"]
// (reading: KL(a_diag || (1-eps) a_nodiag + eps delta_t)). The group's heads
// are summed through LDS and the float32 score is written with a bound on
// its float32 evaluation error.
template <typename T, int D>
__device__ void score_decide(const PrefillArgs& a, int b, int kv, int c, const T* Ks, int kbase, int KS,
                             const float* sc, const float* dl, const int* rl, int nrl, char* scr);
template <typename T, int D>
__device__ void score_pending(const PrefillArgs& a, int b, int kv, int x, const T* Ks, int kbase, int KS,
                              char* scr);
template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void score_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int npg = a.n_pend_grp;
  if ((int)blockIdx.x >= npg + a.T) {  // the extra workgroups: F^T (batch row 0's)
    if (blockIdx.z == 0) fmap_transpose_part<T, D>(a, (int)blockIdx.x - npg - a.T, (int)blockIdx.y);
    return;
  }
  // workgroups x < npg (first, so their float64 work overlaps the rest):
  // the undecided last chunk's float64 scores, from its window staged as
  // for that chunk
  const bool pend_grp = (int)blockIdx.x < npg;  // uniform
  const int c = pend_grp ? a.T - 1 : (int)blockIdx.x - npg, kv = blockIdx.y, b = blockIdx.z;
  const int L = a.L, C = a.C, W = a.W, G = a.G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // in an SGPR
  const int r16 = lane & 15, g4 = lane >> 4;
  constexpr int KS = D + Pad<T>::v;
  const int cC = c * C;
  const int kbase = cC - W + 1;
  // key tiles: row tile qt reads tiles qt .. qt + (W + 14) / 16 (its rows'
  // windows start at 16 qt + r - W + 1 relative to the chunk)
  const int nkt = C / 16 + (W + 14) / 16;
  T* Ks = reinterpret_cast<T*>(smem);
  float* part = reinterpret_cast<float*>(smem + (size_t)nkt * 16 * KS * sizeof(T));
  float* pdel = part + G * C;
  float* pest = pdel + G * C;
  float* knrm = pest + G * C;  // [nkt * 16 + 80] key norms (tiles past the last of a group of five read zeros)
  // with the decision in this kernel: the chunk's scores, bounds and listed
  // positions, then the decision's scratch
  float* sfin = knrm + nkt * 16 + 80;  // [C]
  float* dfin = sfin + C;              // [C]
  int* rll = reinterpret_cast<int*>(dfin + C);  // [C]

  const T* kg = reinterpret_cast<const T*>(a.k) + (size_t)(b * a.Hkv + kv) * L * D;
  constexpr int VEC = 16 / sizeof(T);
  const int nvec = nkt * 16 * (D / VEC);
  const int n_qt = C / 16;
  const int n_rt = G * n_qt;
  // query fragments of row tile rt (zeros past the sequence or the tiles):
  // the next tile's are loaded while this one is used
  const uint32_t qbytes = (uint32_t)((size_t)L * D * sizeof(T));
  auto load_q = [&](Frag<T>* f, int rt) {
    const int hl = rt / n_qt, qt = rt % n_qt;
    const int t = cC + 16 * qt + r16;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(
        reinterpret_cast<const T*>(a.q) + ((size_t)(b * a.Hq + kv * G + (rt < n_rt ? hl : 0)) * L) * D, qbytes);
    const uint32_t off = (rt < n_rt && t < L) ? (uint32_t)((t * D + 8 * g4) * sizeof(T)) : qbytes;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) f[kb] = ld_frag_buf<T>(qrs, off, 32 * kb * sizeof(T));
  };
  Frag<T> qnext[D / 32];
  load_q(qnext, wave);  // in flight while the keys are staged
  // keys into LDS: up to nine 16-byte loads per thread in flight at a time (all of them for
  // a 64-key window and chunk at d = 128); rows outside
  // [0, min(L, cC + C)) read past the buffer range (zeros)
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, qbytes);
  constexpr int NB = 9;
  for (int base = 0; base < nvec; base += NB * 256) {  // whole rows per lane group
    uint4 val[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int idx = base + u * 256 + tid;
      const int row = idx / (D / VEC), col = (idx % (D / VEC)) * VEC;
      const int j = kbase + row;
      const bool ok = idx < nvec && j >= 0 && j < L && j < cC + C;
      val[u] = ld_u4_buf(krs, ok ? (uint32_t)(((size_t)j * D + col) * sizeof(T)) : qbytes, 0);
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int idx = base + u * 256 + tid;
      const int row = idx / (D / VEC), col = (idx % (D / VEC)) * VEC;
      if (idx < nvec) *reinterpret_cast<uint4*>(Ks + row * KS + col) = val[u];
      // the key norm from the same vectors: D / VEC consecutive lanes hold a row
      const T* e = reinterpret_cast<const T*>(&val[u]);
      float q2 = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) q2 += to_f32(e[i]) * to_f32(e[i]);
      q2 = row_sum<D / VEC>(q2);
      if (idx < nvec && col == 0) knrm[row] = sqrtf(q2);
    }
  }
  for (int i = nkt * 16 + tid; i < nkt * 16 + 80; i += 256) knrm[i] = 0.f;
  __syncthreads();
  if (pend_grp) {
    score_pending<T, D>(a, b, kv, (int)blockIdx.x, Ks, kbase, KS, reinterpret_cast<char*>(rll + C));
    return;
  }

  for (int rt = wave; rt < n_rt; rt += 4) {
    const int hl = rt / n_qt, qt = rt % n_qt;
    const int t = cC + 16 * qt + r16;
    Frag<T> qf[D / 32];
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) qf[kb] = qnext[kb];
    load_q(qnext, rt + 4);
    float qn2 = 0.f;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) qn2 += frag_sumsq(qf[kb]);
    const float qn = sqrtf(sum_over_g(qn2));
    float mrun = STILL_NEG_INF, zall = 0.f, zoth = 0.f, sself = STILL_NEG_INF;
    // key-norm sums for the error bound: sum_j e_j |k_j| over the other keys
    // (same running rescale as zoth) and the self key's norm
    float zabs = 0.f, tself = 0.f;
    const int kt_lo = qt, kt_hi = qt + (W + 14) / 16;
    // key tiles in groups of NG: the group's logits first (its MFMAs back
    // to back), then one running-max update and the exponentials
    constexpr int NG = 5;
    for (int k0 = kt_lo; k0 <= kt_hi; k0 += NG) {
      f32x4 sg[NG];
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        sg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (k0 + u <= kt_hi) {  // uniform
#pragma unroll
          for (int kb = 0; kb < D / 32; ++kb)
            mma(sg[u], ld_frag(Ks + (16 * (k0 + u) + r16) * KS + 32 * kb + 8 * g4), qf[kb]);
        }
      }
      float mx = STILL_NEG_INF;
#pragma unroll
      for (int u = 0; u < NG; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kbase + 16 * (k0 + u) + 4 * g4 + i;
          const bool ok = k0 + u <= kt_hi && j >= 0 && j <= t && j >= t - W + 1;
          sg[u][i] = ok ? sg[u][i] * a.scale : STILL_NEG_INF;
          sself = ok && j == t ? sg[u][i] : sself;
          mx = fmax_nn(mx, sg[u][i]);
        }
      const float mn = fmax_nn(mrun, mx);
      // rows with nothing visible so far keep m = -inf and zero sums
      const float al = mrun == STILL_NEG_INF ? 0.f : __expf(mrun - mn);
      const float mo = mn == STILL_NEG_INF ? 0.f : mn;
      float ea = 0.f, eo = 0.f, et = 0.f;
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const f32x4 kn = *reinterpret_cast<const f32x4*>(knrm + 16 * (k0 + u) + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __expf(sg[u][i] - mo);  // 0 for masked keys
          const bool oth = kbase + 16 * (k0 + u) + 4 * g4 + i != t;
          ea += e;
          eo += oth ? e : 0.f;
          et += oth ? e * kn[i] : 0.f;
          tself = oth ? tself : kn[i];
        }
      }
      zall = zall * al + ea;
      zoth = zoth * al + eo;
      zabs = zabs * al + et;
      mrun = mn;
    }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      auto px = [&](float x) { return off == 16 ? xor16f(x) : xor32f(x); };
      const float m2 = px(mrun), za2 = px(zall), zo2 = px(zoth), zt2 = px(zabs), ss2 = px(sself),
                  ts2 = px(tself);
      const float mn = fmax_nn(mrun, m2);
      if (mn != STILL_NEG_INF) {
        const float f1 = (mrun == STILL_NEG_INF) ? 0.f : __expf(mrun - mn);
        const float f2 = (m2 == STILL_NEG_INF) ? 0.f : __expf(m2 - mn);
        zall = zall * f1 + za2 * f2;
        zoth = zoth * f1 + zo2 * f2;
        zabs = zabs * f1 + zt2 * f2;
      }
      mrun = mn;
      sself = fmax_nn(sself, ss2);
      tself = fmax_nn(tself, ts2);
    }
    float sc = 0.f, dl = 0.f, es = 0.f;
    if (t < L) {
      const float p = __expf(sself - mrun) / zall;
      const float pn = zoth / zall;
      const float lp = p > 0.f ? logf(p / a.eps) : 0.f;
      const float lpn = pn > 0.f ? logf(pn / (1.f - a.eps)) : 0.f;
      sc = (p > 0.f ? p * lp : 0.f) + (pn > 0.f ? pn * lpn : 0.f);
      // Bound on the float32 evaluation error of this head's score. Each
      // logit s_j carries at most ~2^-24 sum_i |q_i k_ji| <= 2^-24 |q| |k_j|
      // of MFMA accumulation error (measured on gfx950: at most 1.3x that;
      // taken as 4x with the scale), so p = a_t moves by at most p ((1-p)
      // ds_t + sum_{j!=t} a_j ds_j). The exponentials (argument rounding |x| 2^-24,
      // 2 ulps each) and the sums (one rounding per add: the lane's tiles,
      // two lane merges) move p and 1-p by rho relative. d score / d p =
      // lp - lpn, d score / d(p, pn) at most |lp| + |lpn| + 2. Doubled.
      const float cs = 4.f * 5.9604645e-8f * a.scale * qn;  // 4 * 2^-24 * scale * |q|
      const float dp = p * cs * ((1.f - p) * tself + zabs / zall);
      const float n_add = (float)(4 * (kt_hi - kt_lo + 1) + 2);
      const float rho = (fabsf(sself - mrun) + 2.f + n_add) * 5.9604645e-8f;
      dl = 2.f * (fabsf(lp - lpn) * dp + (fabsf(lp) + fabsf(lpn) + 2.f) * fmaxf(p, pn) * rho +
                  2.3841858e-7f * (fabsf(sc) + 1.f));
      // The typical size of the logit term (1x instead of 4x the MFMA
      // error scale, no doubling): measured against the float64 scores of
      // the workloads here it stays above the actual error, and the tokens
      // where it exceeds 3e-6 of the score (a few %) hold every error
      // above ~1e-6.
      es = fabsf(lp - lpn) * dp * 0.25f;
    }
    if (g4 == 0) {
      part[hl * C + 16 * qt + r16] = sc;
      pdel[hl * C + 16 * qt + r16] = dl;
      pest[hl * C + 16 * qt + r16] = es;
    }
  }
  // tokens whose exported score is recomputed in float64 by the refine
  // kernel (their estimated float32 error comes near 1e-5 of the score):
  // the chunk's list rlist[unit][c] = {count, positions in the chunk}
  int* rl = a.rlist + ((size_t)(b * a.Hkv + kv) * a.T + c) * (C + 1);
  int* n_list = reinterpret_cast<int*>(knrm);
  __syncthreads();  // every wave is done with the key norms
  if (tid == 0) *n_list = 0;
  __syncthreads();
  for (int qi = tid; qi < C; qi += 256) {
    const int t = cC + qi;
    if (t >= L) continue;
    float s = 0.f, d = 0.f, e = 0.f;
    for (int hl = 0; hl < G; ++hl) {
      s += part[hl * C + qi];
      d += pdel[hl * C + qi];
      e += pest[hl * C + qi];
    }
    const size_t o = (size_t)(b * a.Hkv + kv) * L + t;
    if (!(a.fuse_sel && c >= a.n_dec)) a.score[o] = s;  // (else the float64 score is written)
    a.delta[o] = d;
    if (a.fuse_sel) {
      sfin[qi] = s;
      dfin[qi] = d;
    }
    if (a.score_out && c * C + C < L && e > 6e-6f * fmaxf(1.f, fabsf(s))) {
      const int k = atomicAdd(n_list, 1);  // (the last chunk's are all recomputed)
      if (a.fuse_sel) rll[k] = qi;
      else rl[1 + k] = qi;
    }
  }
  __syncthreads();
  if (!a.fuse_sel) {
    if (tid == 0) rl[0] = *n_list;  // 0 unless the scores are exported
    return;
  }
  score_decide<T, D>(a, b, kv, c, Ks, kbase, KS, sfin, dfin, rll, *n_list,
                     reinterpret_cast<char*>(rll + C));
}

// Float64 score of head h (of the kv group) for token t [P3 "Self-Saliency
// Score"] by one wave. Lane j takes the window keys t - n + 1 + j, + 64, ...
// (rows read from global memory, 16 bytes at a time, the next read in flight
// while one is used); the query row
// is staged in LDS as float64 (qd: this wave's [D]); the logits are float64
// dot products (products of bf16 / float32 values are exact in float64);
// the softmax sums run online over the 64-key slots and the two-point KL
// form takes 1-p from the other keys. Every lane returns the head's score.
// diag: return the window softmax's weight on the token itself instead (the
// diagonal-attention routing metric). KL: the key rows come from LDS instead,
// row j at klds + (j - kbase) * kstride (the score kernel's staged window).
template <typename T, int D, bool KL = false>
__device__ double score_f64_head(const PrefillArgs& a, int b, int kv, int h, int t, double* qd,
                                 bool diag = false, const T* klds = nullptr, int kbase = 0,
                                 int kstride = D) {
  const int lane = threadIdx.x & 63;
  const int W = a.W, G = a.G, L = a.L;
  const int n = t - W + 1 > 0 ? W : t + 1;
  constexpr int VEC = 16 / sizeof(T), NV = D / VEC;
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  const T* qrow = reinterpret_cast<const T*>(a.q) + ((size_t)(b * a.Hq + kv * G + h) * L + t) * D;
  wave_sync();  // the previous call's reads of qd are done
  for (int c = lane; c < NV; c += 64) {
    const uint4 q4 = *reinterpret_cast<const uint4*>(qrow + c * VEC);
    const T* qe = reinterpret_cast<const T*>(&q4);
#pragma unroll
    for (int i = 0; i < VEC; ++i) qd[c * VEC + i] = (double)to_f32(qe[i]);
  }
  wave_sync();
  double m = -__builtin_huge_val(), za = 0.0, zo = 0.0, zt = 0.0;  // uniform
  for (int s = 0; 64 * s < n; ++s) {  // uniform
    const int j = lane + 64 * s;
    const int kj = t - n + 1 + (j < n ? j : 0);
    const T* krow = KL ? klds + (size_t)(kj - kbase) * kstride
                       : reinterpret_cast<const T*>(a.k) + ((size_t)(b * a.Hkv + kv) * L + kj) * D;
    // query doubles as 16-byte pairs (read here, not hoisted out of the loop)
    typedef double f64x2 __attribute__((ext_vector_type(2)));
    const f64x2* q2 = reinterpret_cast<const f64x2*>(lds_opaque_v(qd));
    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    // one 16-byte key vector and its VEC query doubles per step; the next
    // step's LDS reads are issued before this step's products
    uint4 kc = *reinterpret_cast<const uint4*>(krow);
    f64x2 qc[VEC / 2];
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) qc[i] = q2[i];
#pragma unroll 1
    for (int c = 0; c < NV; ++c) {
      const uint4 kx = kc;
      f64x2 qx[VEC / 2];
#pragma unroll
      for (int i = 0; i < VEC / 2; ++i) qx[i] = qc[i];
      if (c + 1 < NV) {
        kc = *reinterpret_cast<const uint4*>(krow + (c + 1) * VEC);
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) qc[i] = q2[(c + 1) * (VEC / 2) + i];
      }
      const T* ke = reinterpret_cast<const T*>(&kx);
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        acc[i & 7] = fma(qx[i / 2][i & 1], (double)to_f32(ke[i]), acc[i & 7]);
    }
    const double dot = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    const double xv = j < n ? a.scale64 * dot : -__builtin_huge_val();
    const double mx = wave_max_d(xv);
    const double mn = mx > m ? mx : m;
    const double al = m == -__builtin_huge_val() ? 0.0 : exp(m - mn);
    const double e = j < n ? exp(xv - mn) : 0.0;
    za = za * al + wave_sum_d(e);
    zo = zo * al + wave_sum_d(j == n - 1 ? 0.0 : e);
    zt = zt * al + wave_sum_d(j == n - 1 ? e : 0.0);
    m = mn;
  }
  const double p = zt / za, pn = zo / za;
  if (diag) return p;
  double sc = 0.0;
  if (p > 0.0) sc += p * log(p / a.eps64);
  if (pn > 0.0) sc += pn * log(pn / (1.0 - a.eps64));
  return sc;
}

// Float64 routing score of head h for token t by one wave (every lane gets
// it): the Self-Saliency Score or the metric a.route names. Metrics of the
// kv head (key norm, uniform, the caller's) are returned for h = 0 and 0
// for the other heads, so a sum over the group's heads is the metric.
template <typename T, int D>
__device__ double route_f64_head(const PrefillArgs& a, int b, int kv, int h, int t, double* qd) {
  const int unit = b * a.Hkv + kv;
  const T* krow = reinterpret_cast<const T*>(a.k) + ((size_t)unit * a.L + t) * D;
  switch (a.route) {  // uniform
    case ROUTE_DIAG:
      return score_f64_head<T, D>(a, b, kv, h, t, qd, true);
    case ROUTE_QK: {
      const T* qrow = reinterpret_cast<const T*>(a.q) + ((size_t)(b * a.Hq + kv * a.G + h) * a.L + t) * D;
      return a.scale64 * row_dot_f64<T, D>(qrow, krow);
    }
    case ROUTE_KEYNORM:
      return h == 0 ? sqrt(row_dot_f64<T, D>(krow, krow)) : 0.0;
    case ROUTE_UNIFORM:
      return h == 0 ? (double)uniform_mark(t % a.C, a.C, a.lam) : 0.0;
    case ROUTE_EXTERNAL:
      return h == 0 ? (double)a.ext_score[(size_t)unit * a.L + t] : 0.0;
    default:
      return score_f64_head<T, D>(a, b, kv, h, t, qd);
  }
}

// Routing scores other than the Self-Saliency Score, in place of the score
// kernel (same grid, the same extra F^T workgroups): one workgroup of 4
// waves per (chunk, kv head, batch row), one token per wave at a time, the
// group's heads summed in head order in float64 and rounded once. The bound
// written beside the float32 score covers that rounding (the select
// kernel's float64 ranking of near ties recomputes the same values); no
// exported score needs refining.
template <typename T, int D>
__global__ __launch_bounds__(256) void route_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) char smem[];
  if ((int)blockIdx.x >= a.T) {  // the extra workgroups: F^T (batch row 0's)
    if (blockIdx.z == 0) fmap_transpose_part<T, D>(a, (int)blockIdx.x - a.T, (int)blockIdx.y);
    return;
  }
  const int c = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  double* qd = reinterpret_cast<double*>(smem) + wave * D;  // this wave's float64 query row
  const int unit = b * a.Hkv + kv;
  for (int i = wave; i < a.C; i += 4) {  // wave-uniform
    const int t = c * a.C + i;
    if (t >= a.L) break;
    double s = 0.0;
    for (int h = 0; h < a.G; ++h) s += route_f64_head<T, D>(a, b, kv, h, t, qd);
    if (lane == 0) {
      const float s32 = (float)s;
      const size_t o = (size_t)unit * a.L + t;
      a.score[o] = s32;
      // |float32 - float64| plus the float64 evaluation error (far below)
      a.delta[o] = (float)(fabs((double)s32 - s) + fabs(s) * 0x1p-40) * (1.f + 0x1p-20f);
    }
  }
  if (tid == 0) a.rlist[((size_t)unit * a.T + c) * (a.C + 1)] = 0;
}

// Float64 scores of a list of tokens by a 4-wave workgroup: the (token,
// head) pairs are dealt to the waves, each head's score lands in res[i][h]
// and every token's sum is taken in head order (tok_t: the tokens; qd: [4][D]
// float64). Ends with a barrier; the sums are left in sum[i].
// KL: the Self-Saliency Score with the key rows from the score kernel's LDS
// window (klds, kbase, kstride as for score_f64_head).
template <typename T, int D, bool KL = false>
__device__ void score_f64_list(const PrefillArgs& a, int b, int kv, const int* tok_t, int n_tok,
                               double* qd, double* res, double* sum, const T* klds = nullptr,
                               int kbase = 0, int kstride = D) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, G = a.G;
  for (int pi = wave; pi < n_tok * G; pi += 4) {  // wave-uniform
    const int i = pi / G, h = pi % G, t = tok_t[i];
    const double s = KL ? score_f64_head<T, D, true>(a, b, kv, h, t, qd + wave * D, false, klds, kbase, kstride)
                        : route_f64_head<T, D>(a, b, kv, h, t, qd + wave * D);
    if (lane == 0) res[pi] = s;
  }
  __syncthreads();
  for (int i = tid; i < n_tok; i += 256) {
    double s = 0.0;
    for (int h = 0; h < G; ++h) s += res[i * G + h];
    sum[i] = s;
  }
  __syncthreads();
}

// ---------------------------------------------------------- 3. select ----
// Chunk c is decided [P3 "Delayed Chunk-Level Selection"]: keep lambda_c =
// lambda tokens while the pool of m - W slots has room [P2 固定预算路由],
// ranked by (score desc, position asc). The float32 scores with their error
// bounds give, for every token, an interval; tokens whose upper end is
// below the lambda-th largest lower end cannot be kept. If more than lambda
// tokens remain, their scores are recomputed in float64 and the ranking is
// made on those (their exported scores become the float64 values rounded
// once); the tokens the score kernel listed for export are recomputed in
// float64 as well. The float64 scores of the undecided last chunk's tokens
// go to the decode state.
// Workgroups, in launch order: for C <= 64 and exported scores, the
// recomputation of the listed exported scores of SEL_RCH chunks each; then
// SEL_PEND tokens of the undecided chunk each; then the decisions, for
// C <= 64 one chunk per wave (token j in lane j) and SEL_CPW chunks per
// workgroup, the four waves sharing the float64 scores their chunks need,
// so that the few chunks that need them finish within the same round as
// the others; for C > 64 one chunk per workgroup, which also recomputes its
// listed exported scores.
// The selection's intervals are [score - m dl, score + m dl] with the score
// kernel's bound dl widened by SEL_MARGIN: a wider interval only sends more
// tokens to the float64 ranking, a too narrow one could drop a token the
// float64 ranking keeps.
constexpr float SEL_MARGIN = 2.f;
constexpr int SEL_PEND = 2;  // undecided tokens per workgroup
constexpr int SEL_CPW = 4;   // chunks per workgroup for C <= 64 (one per wave)
constexpr int SEL_RCH = 2;   // chunks per workgroup of the exported-score recomputation

// the lam_c-th largest lower bound of a chunk's scores, ranked by (lower
// bound desc, index asc): one wave, token j in lane j (C <= 64), lam_c
// rounds of removing the largest; every lane gets it
__device__ __forceinline__ float lambda_lower_bound(float xl, bool gone, int lam_c) {
  const int lane = threadIdx.x & 63;
  float LBv = STILL_NEG_INF;
  for (int k = 0; k < lam_c; ++k) {
    float m = row_max<16>(gone ? STILL_NEG_INF : xl);
    m = fmax_nn(m, xor16f(m));
    m = fmax_nn(m, xor32f(m));
    const uint64_t at = __builtin_amdgcn_ballot_w64(!gone && xl == m);
    const int first = at ? (int)__builtin_ctzll(at) : 64;  // lowest index among the maxima
    if (lane == first) gone = true;
    LBv = m;
  }
  return LBv;
}

// Float64 scores of SEL_PEND tokens (group x) of the undecided last chunk of
// unit (kv, b) into the decode state's pending scores, and the exported
// scores; their kept flags are 0. LDS: [4][D] float64 query rows, then the
// list, per-head results and sums.
template <typename T, int D>
__device__ void pending_part(const PrefillArgs& a, int x, int kv, int b) {
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, C = a.C, L = a.L, G = a.G;
  const int unit = b * a.Hkv + kv;
  const size_t ub_off = (size_t)unit * L;
  const int c_last = (L - 1) / C, n_pend = L - c_last * C;
  double* qd = reinterpret_cast<double*>(smem);               // [4][D]
  int* list = reinterpret_cast<int*>(qd + 4 * D);            // [SEL_PEND]
  double* res = reinterpret_cast<double*>(list + 4);          // [SEL_PEND][G]
  double* sum = res + SEL_PEND * G;                           // [SEL_PEND]
  const int i0 = x * SEL_PEND, n = min(SEL_PEND, n_pend - i0);
  if (tid < n) list[tid] = c_last * C + i0 + tid;
  __syncthreads();
  score_f64_list<T, D>(a, b, kv, list, n, qd, res, sum);
  double* pend = reinterpret_cast<double*>(a.state + (size_t)unit * a.st_unit + a.st_pending);
  if (tid < n) {
    const int t = list[tid];
    pend[i0 + tid] = sum[tid];
    a.selflag[ub_off + t] = 0;
    if (a.score_out) a.score[ub_off + t] = (float)sum[tid];
  }
  if (x == 0)
    for (int i = n_pend + tid; i < C; i += 256) pend[i] = __builtin_nan("");
}

// Bytes of score_decide's LDS scratch.
__host__ __device__ constexpr size_t score_decide_bytes(int C, int G, int D) {
  return (size_t)8 * (4 * D + C * G + C + 2) + (size_t)4 * (C + 4);
}

// The decision of chunk c inside the score kernel's workgroup (the Self-
// Saliency route, C <= 64): the select kernel's interval test and float64
// ranking for one chunk (token j in lane j of wave 0), with the float64
// scores' key rows read from the window the score kernel staged in LDS
// (Ks: rows kbase, kbase + 1, ... of stride KS); the chunk's listed
// exported scores (rl: nrl positions) are recomputed in float64 in the same
// pass. sc, dl: the chunk's float32 scores and bounds; scr: LDS scratch of
// score_decide_bytes(C, G, D) bytes. The undecided last chunk only gets its
// kept flags (0): its float64 scores are made by pending_part. Called by
// every thread of the workgroup.
template <typename T, int D>
__device__ void score_decide(const PrefillArgs& a, int b, int kv, int c, const T* Ks, int kbase, int KS,
                             const float* sc, const float* dl, const int* rl, int nrl, char* scr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = a.C, L = a.L, lam = a.lam, G = a.G;
  const int unit = b * a.Hkv + kv;
  const size_t ub_off = (size_t)unit * L;
  const int base = c * C;
  if (c >= a.n_dec) {  // uniform
    for (int j = tid; j < C && base + j < L; j += 256) a.selflag[ub_off + base + j] = 0;
    return;
  }
  double* qd = reinterpret_cast<double*>(scr);           // [4][D]
  double* res = qd + 4 * D;                              // [C][G]
  double* sum = res + (size_t)C * G;                     // [C]
  uint64_t* msk = reinterpret_cast<uint64_t*>(sum + C);  // candidates, float64 tokens
  int* list = reinterpret_cast<int*>(msk + 2);           // [C]
  int* cnt = list + C;
  const int lam_c = ((c + 1) * lam <= a.m - a.W) ? lam : 0;
  const bool partial = lam_c > 0 && lam_c < C;  // else none or all are kept
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;  // lanes under this one
  if (wave == 0) {
    const float s = lane < C ? sc[lane] : 0.f, d = lane < C ? dl[lane] : 0.f;
    uint64_t cand = 0;
    bool rank64 = false;
    if (partial) {
      const float LB = lambda_lower_bound(lane < C ? s - SEL_MARGIN * d : STILL_NEG_INF, lane >= C, lam_c);
      cand = __builtin_amdgcn_ballot_w64(lane < C && s + SEL_MARGIN * d >= LB);
      rank64 = __builtin_popcountll(cand) > lam_c;
    }
    bool mine = false;
    for (int i = 0; i < nrl; ++i) mine = mine || rl[i] == lane;
    const uint64_t need = (rank64 ? cand : 0ull) | __builtin_amdgcn_ballot_w64(mine);
    if ((need >> lane) & 1ull) list[__builtin_popcountll(need & below)] = base + lane;
    if (lane == 0) {
      msk[0] = cand;
      msk[1] = need;
      *cnt = __builtin_popcountll(need);
    }
  }
  __syncthreads();
  const int total = *cnt;
  if (total > 0) score_f64_list<T, D, true>(a, b, kv, list, total, qd, res, sum, Ks, kbase, KS);  // uniform
  if (wave != 0) return;
  const uint64_t cand = msk[0], need = msk[1];
  const bool rank64 = partial && __builtin_popcountll(cand) > lam_c;
  const bool in_list = (need >> lane) & 1ull;
  const double s64 = in_list ? sum[__builtin_popcountll(need & below)] : 0.0;
  bool kept = lane < C && lam_c == C;
  if (partial) {
    kept = (cand >> lane) & 1ull;
    if (rank64) {  // uniform; every lane takes part in the shuffles
      int r = 0;
      for (uint64_t mm = cand; mm; mm &= mm - 1) {  // the candidates, in index order
        const int i = __builtin_ctzll(mm);
        const double si = __shfl(s64, i);
        r += (si > s64 || (si == s64 && i < lane)) ? 1 : 0;
      }
      kept = kept && r < lam_c;
    }
  }
  if (lane < C) a.selflag[ub_off + base + lane] = (uint8_t)kept;
  int32_t* selrow = a.sel + ((size_t)unit * a.n_dec + c) * lam;
  const uint64_t km = __builtin_amdgcn_ballot_w64(kept);
  if (kept) selrow[__builtin_popcountll(km & below)] = base + lane;
  for (int i = lam_c + lane; i < lam; i += 64) selrow[i] = -1;
  if (a.score_out && in_list) a.score[ub_off + base + lane] = (float)s64;
}

// The float64 scores of SCORE_PEND tokens (group x) of the undecided last
// chunk inside the score launch, with the key rows from the chunk's window
// staged in LDS (Ks, kbase, KS as for score_decide): into the decode state's
// pending scores and the exported scores. scr: score_decide's scratch.
constexpr int SCORE_PEND = 4;
template <typename T, int D>
__device__ void score_pending(const PrefillArgs& a, int b, int kv, int x, const T* Ks, int kbase, int KS,
                              char* scr) {
  const int tid = threadIdx.x, C = a.C, L = a.L, G = a.G;
  const int unit = b * a.Hkv + kv;
  const size_t ub_off = (size_t)unit * L;
  const int c_last = (L - 1) / C, n_pend = L - c_last * C;
  double* qd = reinterpret_cast<double*>(scr);           // [4][D]
  double* res = qd + 4 * D;                              // [SCORE_PEND][G]
  double* sum = res + SCORE_PEND * G;                    // [SCORE_PEND]
  int* list = reinterpret_cast<int*>(sum + SCORE_PEND);  // [SCORE_PEND]
  const int i0 = x * SCORE_PEND, n = min(SCORE_PEND, n_pend - i0);
  if (tid < n) list[tid] = c_last * C + i0 + tid;
  __syncthreads();
  score_f64_list<T, D, true>(a, b, kv, list, n, qd, res, sum, Ks, kbase, KS);
  double* pend = reinterpret_cast<double*>(a.state + (size_t)unit * a.st_unit + a.st_pending);
  if (tid < n) {
    pend[i0 + tid] = sum[tid];
    a.score[ub_off + list[tid]] = (float)sum[tid];
  }
  if (x == 0)
    for (int i = n_pend + tid; i < C; i += 256) pend[i] = __builtin_nan("");
}

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void select_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = a.C, L = a.L, lam = a.lam, G = a.G;
  const int unit = b * a.Hkv + kv;
  const size_t ub_off = (size_t)unit * L;
  const int c_last = (L - 1) / C, n_pend = L - c_last * C;
  const int n_pgrp = (n_pend + SEL_PEND - 1) / SEL_PEND;
  const int n_rgrp = C <= 64 && a.score_out ? (a.n_dec + SEL_RCH - 1) / SEL_RCH : 0;
  double* qd = reinterpret_cast<double*>(smem);  // [4][D] float64 query rows (one per wave)

  if ((int)blockIdx.x < n_rgrp) {
    // exported scores the score kernel listed for SEL_RCH chunks (estimated
    // float32 error near 1e-5 of the score): recomputed in float64, rounded
    // once; in workgroups of their own, first, so that their float64 work
    // spreads evenly and runs beside the selection's
    int* cnt = reinterpret_cast<int*>(qd + 4 * D);  // [4] tokens per wave
    int* list = cnt + 4 + 16;                      // [4 * 64] (after the mask slots)
    double* res = reinterpret_cast<double*>(list + 4 * 64);
    double* sum = res + (size_t)4 * 64 * G;
    const int c = (int)blockIdx.x * SEL_RCH + wave;
    const size_t rl0 = ((size_t)unit * a.T + c) * (C + 1);
    const int nr = wave < SEL_RCH && c < a.n_dec ? min(a.rlist[rl0], C) : 0;
    if (lane == 0) cnt[wave] = nr;
    __syncthreads();
    int off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      off += w < wave ? cnt[w] : 0;
      total += cnt[w];
    }
    if (lane < nr) list[off + lane] = c * C + a.rlist[rl0 + 1 + lane];
    __syncthreads();
    if (total == 0) return;  // uniform
    score_f64_list<T, D>(a, b, kv, list, total, qd, res, sum);
    for (int i = tid; i < total; i += 256) a.score[ub_off + list[i]] = (float)sum[i];
    return;
  }
  const int x = (int)blockIdx.x - n_rgrp;

  if (x < n_pgrp) {
    pending_part<T, D>(a, x, kv, b);
    return;
  }

  if (C <= 64) {
    // one chunk per wave
    int* cnt = reinterpret_cast<int*>(qd + 4 * D);                        // [4] float64 tokens per wave
    uint64_t* msk = reinterpret_cast<uint64_t*>(cnt + 4);                 // [4][2] candidates, float64 tokens
    int* list = reinterpret_cast<int*>(msk + 8);                          // [SEL_CPW * 64]
    double* res = reinterpret_cast<double*>(list + SEL_CPW * 64);         // [SEL_CPW * 64][G]
    double* sum = res + (size_t)SEL_CPW * 64 * G;                         // [SEL_CPW * 64]
    const int c = (x - n_pgrp) * SEL_CPW + wave;
    const bool act = c < a.n_dec;  // wave-uniform
    const int base = c * C;
    const int lam_c = ((c + 1) * lam <= a.m - a.W) ? lam : 0;
    const bool partial = act && lam_c > 0 && lam_c < C;  // else none or all are kept
    uint64_t cand = 0, need = 0;
    bool rank64 = false;
    if (act) {
      const float sc = lane < C ? a.score[ub_off + base + lane] : 0.f;
      const float dl = lane < C ? a.delta[ub_off + base + lane] : 0.f;
      if (partial) {
        const float LB = lambda_lower_bound(lane < C ? sc - SEL_MARGIN * dl : STILL_NEG_INF, lane >= C, lam_c);
        cand = __builtin_amdgcn_ballot_w64(lane < C && sc + SEL_MARGIN * dl >= LB);
        rank64 = __builtin_popcountll(cand) > lam_c;
      }
      if (rank64) need = cand;
    }
    if (lane == 0) {
      cnt[wave] = __builtin_popcountll(need);
      msk[2 * wave] = cand;
      msk[2 * wave + 1] = need;
    }
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) total += cnt[w];
    {
      int off = 0;
      for (int w = 0; w < wave; ++w) off += cnt[w];
      const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
      if ((need >> lane) & 1ull) list[off + __builtin_popcountll(need & below)] = base + lane;
    }
    __syncthreads();
    if (total > 0) score_f64_list<T, D>(a, b, kv, list, total, qd, res, sum);  // uniform
    if (!act) return;
    // (the masks come back from LDS: fewer registers live across the scores)
    cand = msk[2 * wave];
    need = msk[2 * wave + 1];
    int off = 0;
    for (int w = 0; w < wave; ++w) off += cnt[w];
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;  // lanes under this one
    const bool in_list = (need >> lane) & 1ull;
    const double s64 = in_list ? sum[off + __builtin_popcountll(need & below)] : 0.0;
    rank64 = partial && __builtin_popcountll(cand) > lam_c;
    bool kept = lane < C && lam_c == C;
    if (partial) {
      kept = (cand >> lane) & 1ull;
      if (rank64) {  // uniform; every lane takes part in the shuffles
        int r = 0;
        for (uint64_t mm = cand; mm; mm &= mm - 1) {  // the candidates, in index order
          const int i = __builtin_ctzll(mm);
          const double si = __shfl(s64, i);
          r += (si > s64 || (si == s64 && i < lane)) ? 1 : 0;
        }
        kept = kept && r < lam_c;
      }
    }
    if (lane < C) a.selflag[ub_off + base + lane] = (uint8_t)kept;
    int32_t* selrow = a.sel + ((size_t)unit * a.n_dec + c) * lam;
    const uint64_t km = __builtin_amdgcn_ballot_w64(kept);
    if (kept) selrow[__builtin_popcountll(km & below)] = base + lane;
    for (int i = lam_c + lane; i < lam; i += 64) selrow[i] = -1;
    if (a.score_out && in_list) a.score[ub_off + base + lane] = (float)s64;
    return;
  }

  // C > 64: one chunk per workgroup
  double* s64 = qd + 4 * D;                        // [C]
  float* sc = reinterpret_cast<float*>(s64 + C);   // [C]
  float* dl = sc + C;                              // [C]
  int* flag = reinterpret_cast<int*>(dl + C);      // [C] candidate
  int* keep = flag + C;                            // [C]
  int* list = keep + C;                            // [C] float64 tokens
  int* misc = list + C;  // [4], then (16-byte aligned) the per-head float64 results
  double* res = reinterpret_cast<double*>(misc + 4);  // [C][G] per-head float64 scores
  double* sum = res + (size_t)C * G;                  // [C]
  const int c = x - n_pgrp, base = c * C;
  const int lam_c = ((c + 1) * lam <= a.m - a.W) ? lam : 0;
  const bool partial = lam_c > 0 && lam_c < C;  // else none or all are kept
  int32_t* selrow = a.sel + ((size_t)unit * a.n_dec + c) * lam;
  for (int j = tid; j < C; j += 256) {
    sc[j] = a.score[ub_off + base + j];
    dl[j] = a.delta[ub_off + base + j];
  }
  if (tid == 0) {
    misc[0] = 0;  // candidates
    misc[1] = 0;  // float64 list
  }
  __syncthreads();
  // the lam_c-th largest lower bound, ranked by (lower bound desc, index asc)
  if (partial) {
    for (int j = tid; j < C; j += 256) {
      const float lj = sc[j] - SEL_MARGIN * dl[j];
      int r = 0;
      for (int i = 0; i < C; ++i) {
        const float li = sc[i] - SEL_MARGIN * dl[i];
        r += (li > lj || (li == lj && i < j)) ? 1 : 0;
      }
      if (r == lam_c - 1) misc[2] = __float_as_int(lj);
    }
  }
  __syncthreads();
  const float LB = __int_as_float(misc[2]);
  for (int j = tid; j < C; j += 256) {
    const bool cand = partial && sc[j] + SEL_MARGIN * dl[j] >= LB;
    flag[j] = cand ? 1 : 0;
    if (cand) atomicAdd(&misc[0], 1);
  }
  __syncthreads();
  const bool rank64 = partial && misc[0] > lam_c;  // uniform
  for (int j = tid; j < C; j += 256)
    if (rank64 && flag[j]) list[atomicAdd(&misc[1], 1)] = j;
  __syncthreads();
  const int n_list = misc[1];
  if (n_list > 0) {  // uniform: float64 scores, key rows read from global memory
    for (int i = tid; i < n_list; i += 256) list[i] += base;  // positions
    __syncthreads();
    score_f64_list<T, D>(a, b, kv, list, n_list, qd, res, sum);
    for (int i = tid; i < n_list; i += 256) {
      const int j = list[i] - base;
      s64[j] = sum[i];
      if (a.score_out) a.score[ub_off + base + j] = (float)sum[i];
    }
  }
  __syncthreads();
  for (int j = tid; j < C; j += 256) {
    bool kept = lam_c == C;
    if (partial) {
      kept = flag[j] != 0;
      if (rank64 && kept) {
        int r = 0;
        for (int i = 0; i < C; ++i)
          r += (flag[i] && (s64[i] > s64[j] || (s64[i] == s64[j] && i < j))) ? 1 : 0;
        kept = r < lam_c;
      }
    }
    keep[j] = kept ? 1 : 0;
  }
  __syncthreads();
  for (int j = tid; j < C; j += 256) {
    a.selflag[ub_off + base + j] = (uint8_t)keep[j];
    if (keep[j]) {
      int k = 0;
      for (int i = 0; i < j; ++i) k += keep[i];
      selrow[k] = base + j;
    }
  }
  for (int i = lam_c + tid; i < lam; i += 256) selrow[i] = -1;
  // exported scores the score kernel listed: recomputed in float64
  if (!a.score_out) return;
  const int* rl = a.rlist + ((size_t)unit * a.T + c) * (C + 1);
  const int nr = min(rl[0], C);
  if (nr <= 0) return;  // uniform
  __syncthreads();  // the ranking's reads of list are done
  for (int i = tid; i < nr; i += 256) list[i] = base + rl[1 + i];
  __syncthreads();
  score_f64_list<T, D>(a, b, kv, list, nr, qd, res, sum);
  for (int i = tid; i < nr; i += 256) a.score[ub_off + list[i]] = (float)sum[i];
}

// ----------------------------------------- shared block machinery (4-6) ----
// A workgroup of 8 waves streams 64-key blocks through LDS:
//   Ks    [64][D+pad] T         keys, row-major (A fragments of K)
//   VTs   values as H (fp16 next to bf16 data, float otherwise): for fp16
//         row-major [64][D+8], read as fragments by transposing LDS reads;
//         for float transposed [D][64+pad], keys permuted (perm_col)
//   WF    NP-Map features of the block's keys as H, the A fragments (rows =
//         keys) of <phi(k),phi(q)>: for fp16 feature-major [D][64+8] read
//         by transposing LDS reads; for float [4 kt][D/32] fragments
//   SP    float32 linear state S (d_k x d_v), fragment-linear: pair
//         p = (d_v tile vt, d_k 32-block bb) holds, per lane, the 8 values
//         {S[32bb + 4g + i][16vt + r], S[32bb + 16 + 4g + i][16vt + r]} as two
//         halves [p][h][lane][4] (the accumulators of tiles (2bb, vt) and
//         (2bb+1, vt)); read together they are the A operand of S^T for the
//         readout.
//   stat  per-key softmax statistics of the feature map
// At the start of a chunk the first region (Ks..WF) holds the state's
// fp16 readout fragments (RS; rows scaled by 1/z).
template <typename T, int D>
struct Blk {
  typedef typename HalfOf<T>::type H;
  // key rows padded by two 16-byte vectors (measured: fewer LDS bank
  // conflicts on the fragment reads than one)
  static constexpr int KS = D + 2 * Pad<T>::v;
  static constexpr int VS = 64 + Pad<H>::v;  // float data: values transposed
  // 16-bit H: values row-major [64][VR] and phi(K) feature-major [D][FKS],
  // read as MFMA fragments with transposing LDS reads
  static constexpr bool TR = sizeof(H) == 2;
  static constexpr int VR = D + 8;
  static constexpr int FKS = 64 + 8;
  static constexpr int NFT = D / 16;  // feature (and d_v) tiles
  static constexpr int NPAIR = (D / 16) * (D / 32);
  static constexpr int PCAP = 1024;   // pool positions staged in LDS per chunk
  static constexpr size_t ks_bytes = 64 * KS * sizeof(T);
  static constexpr size_t vs_bytes = TR ? (size_t)64 * VR * sizeof(H) : (size_t)D * VS * sizeof(H);
  static constexpr size_t wf_bytes = TR ? (size_t)D * FKS * sizeof(H) : (size_t)4 * (D / 32) * 64 * 8 * sizeof(H);
  // readout fragments of the state: [NPAIR][64][8] H
  static constexpr size_t rs_bytes = (size_t)NPAIR * 64 * 8 * sizeof(H);
  static constexpr size_t lo_bytes =
      (ks_bytes + vs_bytes + wf_bytes > rs_bytes ? ks_bytes + vs_bytes + wf_bytes : rs_bytes);
  static constexpr size_t sp_bytes = (size_t)NPAIR * 64 * 8 * sizeof(float);
  static constexpr size_t ft_bytes = (size_t)D * D * sizeof(T);
  static constexpr size_t stat_bytes = (8 * 64 * 2 + 64 * 3) * 4;
  static constexpr size_t meta_bytes = 64 * 4 + 16 + D * 8 + PCAP * 4;
  static constexpr size_t bytes = lo_bytes + sp_bytes + ft_bytes + stat_bytes + meta_bytes;
  static_assert(bytes <= 160 * 1024, "one workgroup's LDS");
};

template <typename T, int D>
struct BlkPtr {
  typedef typename HalfOf<T>::type H;
  T* Ks;
  H* VTs;
  H* WF;
  T* RS;
  float* SP;
  T* FT;         // F^T of the kv head in fragment order
  float* kmax;   // [8][64] per-wave partial max
  float* ksum;   // [8][64] per-wave partial sum of squares
  float* kstat;  // [3][64]: max, scale, |k|^2
  float* fmask;  // [64]
  uint32_t* selw;
  double* zs;     // running z of the walk, float64
  int32_t* pidx;  // [PCAP] kept-pool positions of the chunk
  // every region base is opaque (see lds_opaque)
  __device__ BlkPtr(char* smem) {
    using B_ = Blk<T, D>;
    Ks = lds_opaque(reinterpret_cast<T*>(smem));
    VTs = lds_opaque(reinterpret_cast<H*>(smem + B_::ks_bytes));
    WF = lds_opaque(reinterpret_cast<H*>(smem + B_::ks_bytes + B_::vs_bytes));
    RS = lds_opaque(reinterpret_cast<T*>(smem));
    SP = lds_opaque(reinterpret_cast<float*>(smem + B_::lo_bytes));
    FT = lds_opaque(reinterpret_cast<T*>(smem + B_::lo_bytes + B_::sp_bytes));
    char* st = smem + B_::lo_bytes + B_::sp_bytes + B_::ft_bytes;
    kmax = lds_opaque(reinterpret_cast<float*>(st));
    ksum = lds_opaque(reinterpret_cast<float*>(st + 8 * 64 * 4));
    kstat = lds_opaque(reinterpret_cast<float*>(st + 16 * 64 * 4));
    fmask = lds_opaque(reinterpret_cast<float*>(st + 19 * 64 * 4));
    selw = lds_opaque(reinterpret_cast<uint32_t*>(st + 20 * 64 * 4));
    zs = lds_opaque(reinterpret_cast<double*>(st + 20 * 64 * 4 + 16));
    pidx = lds_opaque(reinterpret_cast<int32_t*>(st + 20 * 64 * 4 + 16 + D * 8));
  }
  // half h (0: d_k rows 32bb + 4g + i, 1: rows 32bb + 16 + 4g + i) of pair p
  __device__ float* pair(int p, int h) const {
    return SP + ((size_t)(2 * p + h) * 64 + (opaque_tid() & 63)) * 4;
  }
  __device__ H* wf(int kt, int bb) const { return WF + ((size_t)(kt * (D / 32) + bb) * 64) * 8; }
  // Fragment of V^T for d_v tile dt and key half kb2: lane (r, g) holds
  // V[32 kb2 + perm(g, s)][16 dt + r], s = 0..7 (A operand of O^T += V^T P^T,
  // B operand of the fold).
  // (lane: the caller's lane index, so that the lane-dependent part of the
  // address is computed once where the caller reads many fragments)
  __device__ Frag<H> ld_v(int dt, int kb2) const { return ld_v(dt, kb2, opaque_tid() & 63); }
  __device__ Frag<H> ld_v(int dt, int kb2, int lane) const {
    using B_ = Blk<T, D>;
    const int r16 = lane & 15, g4 = lane >> 4;
    if constexpr (B_::TR) {
      const H* p = VTs + (32 * kb2 + 4 * g4 + (r16 >> 2)) * B_::VR + 16 * dt + 4 * (r16 & 3);
      return tr_frag(p, 16 * B_::VR);
    } else {
      return ld_frag(VTs + (16 * dt + r16) * B_::VS + 32 * kb2 + 8 * g4);
    }
  }
  // A fragment of phi(K) (rows = keys 16 kt + r, depth = features 32 bb + perm(g, s)).
  __device__ Frag<H> ld_wk(int kt, int bb) const { return ld_wk(kt, bb, opaque_tid() & 63); }
  __device__ Frag<H> ld_wk(int kt, int bb, int lane) const {
    using B_ = Blk<T, D>;
    const int r16 = lane & 15, g4 = lane >> 4;
    if constexpr (B_::TR) {
      const H* p = WF + (32 * bb + 4 * g4 + (r16 >> 2)) * B_::FKS + 16 * kt + 4 * (r16 & 3);
      return tr_frag(p, 16 * B_::FKS);
    } else {
      return ld_frag(wf(kt, bb) + lane * 8);
    }
  }
  // fragment (feature tile ft, d block kb) of F^T: B operand of X F
  __device__ const T* ft(int ftile, int kb) const { return ft(ftile, kb, opaque_tid() & 63); }
  __device__ const T* ft(int ftile, int kb, int lane) const {
    return FT + ((size_t)(ftile * (D / 32) + kb) * 64 + lane) * 8;
  }
};

// Copies F^T of one kv head (fragment order, D*D elements) into LDS.
template <typename T, int D, int NT>
__device__ __forceinline__ void load_ft(const BlkPtr<T, D>& P, const T* ftg) {
  constexpr int N16 = D * D * (int)sizeof(T) / 16;
  for (int e = opaque_tid(); e < N16; e += NT)
    reinterpret_cast<uint4*>(P.FT)[e] = reinterpret_cast<const uint4*>(ftg)[e];
}

// A block of 64 keys/values in flight: the global loads of a block are
// issued into registers (issue_block) while the previous block is still
// being used, and written to LDS after it (commit_block). Positions come
// from a gather list (kept pool) or a range; absent rows read past the
// buffer range and load zeros.
template <typename T, int D, int NT>
struct BlkRegs {
  static constexpr int VEC = 16 / sizeof(T), CPR = D / VEC;  // 16-byte chunks per row
  static constexpr int KIT = (64 * CPR + NT - 1) / NT;       // key chunks per thread
  static constexpr int VIT = (32 * CPR + NT - 1) / NT;       // value chunk pairs per thread
  static constexpr bool TR = sizeof(typename HalfOf<T>::type) == 2;
  uint4 k[KIT];
  uint4 vr[TR ? KIT : 1];     // values, same row chunks as the keys
  uint4 v[TR ? 1 : VIT][2];   // values as key pairs (transposed layout)
  int pos;  // threads < 64: position of key tid (-1: none)
  int sel;  // threads < 64: kept flag of key tid
};

// Where the positions of a block's keys come from: a range [lo, hi), a
// list in LDS or a list in global memory (entries from `first`).
struct BlkSrc {
  int mode;  // 0 range, 1 LDS list, 2 global list
  int lo, hi;
  const int32_t* lds;             // mode 1
  __amdgpu_buffer_rsrc_t glist;   // mode 2
  int first, n;                   // list entries first .. first + n
};
__device__ __forceinline__ BlkSrc blk_range(int lo, int hi) {
  BlkSrc s{};
  s.mode = 0; s.lo = lo; s.hi = hi;
  return s;
}

template <typename T, int D, int NT>
__device__ __forceinline__ void issue_block(BlkRegs<T, D, NT>& R, __amdgpu_buffer_rsrc_t kr,
                                            __amdgpu_buffer_rsrc_t vr, uint32_t kv_bytes,
                                            __amdgpu_buffer_rsrc_t sfr, const BlkSrc& src) {
  using BR = BlkRegs<T, D, NT>;
  constexpr int VEC = BR::VEC, CPR = BR::CPR;
  // lane-dependent addresses are recomputed here rather than kept live
  // across the caller's loop (they would be hoisted out of it and spilled)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  auto pos_of = [&](int kk) -> int {
    if (src.mode == 0) return src.lo + kk < src.hi ? src.lo + kk : -1;
    if (kk >= src.n) return -1;
    if (src.mode == 1)
      return ((const __attribute__((address_space(3))) int32_t*)(lds_char*)(char*)src.lds)[src.first + kk];
    return (int)__builtin_amdgcn_raw_buffer_load_b32(src.glist, (uint32_t)(src.first + kk) * 4, 0, 0);
  };
  auto row_off = [&](int j) { return j >= 0 ? (uint32_t)j * (uint32_t)(D * sizeof(T)) : kv_bytes; };
  // all row positions first (list entries are read before any row load is
  // issued, so waiting for them does not wait for the row loads)
  uint32_t koff[BR::KIT], voff[BR::VIT][2];
#pragma unroll
  for (int it = 0; it < BR::KIT; ++it) {
    const int idx = tid + it * NT;
    koff[it] = idx < 64 * CPR ? row_off(pos_of(idx / CPR)) + (idx % CPR) * VEC * sizeof(T) : kv_bytes;
  }
#pragma unroll
  for (int it = 0; it < (BR::TR ? 0 : BR::VIT); ++it) {
    const int idx = tid + it * NT;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      voff[it][i] = idx < 32 * CPR ? row_off(pos_of(2 * (idx / CPR) + i)) + (idx % CPR) * VEC * sizeof(T)
                                   : kv_bytes;
  }
  // threads < 64: position and kept flag of key tid (the flag byte is read
  // by every thread, past the range where there is no key: no branch)
  R.pos = pos_of(tid & 63);
  const int flag = (int)__builtin_amdgcn_raw_buffer_load_b8(sfr, R.pos >= 0 ? (uint32_t)R.pos : 0xffffffffu, 0, 0);
  R.sel = src.mode == 0 ? flag : (R.pos >= 0 ? 1 : 0);
#pragma unroll
  for (int it = 0; it < BR::KIT; ++it) R.k[it] = ld_u4_buf(kr, koff[it], 0);
  if constexpr (BR::TR) {
#pragma unroll
    for (int it = 0; it < BR::KIT; ++it) R.vr[it] = ld_u4_buf(vr, koff[it], 0);
  } else {
#pragma unroll
    for (int it = 0; it < BR::VIT; ++it)
#pragma unroll
      for (int i = 0; i < 2; ++i) R.v[it][i] = ld_u4_buf(vr, voff[it][i], 0);
  }
}

// Writes an issued block to LDS: keys row-major into Ks, values transposed
// (as H) into VTs with keys 2a, 2a+1 in adjacent permuted columns, the kept
// flags as a 64-bit mask, the fold mask and (with want_norm, uniform: for
// blocks whose NP-Map features are computed) the keys' squared norms.
template <typename T, int D, int NT>
__device__ __forceinline__ void commit_block(const BlkPtr<T, D>& P, const BlkRegs<T, D, NT>& R,
                                             int fold_lo, int fold_hi, bool want_norm = true) {
  using B_ = Blk<T, D>;
  using BR = BlkRegs<T, D, NT>;
  typedef typename HalfOf<T>::type H;
  constexpr int VEC = BR::VEC, CPR = BR::CPR;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // as in issue_block
  if (tid < 64) {
    P.fmask[tid] = (R.pos >= fold_lo && R.pos < fold_hi && !R.sel) ? 1.f : 0.f;
    const uint64_t bits = __ballot(R.sel != 0);
    if (tid == 0) {
      P.selw[0] = (uint32_t)bits;
      P.selw[1] = (uint32_t)(bits >> 32);
    }
  }
#pragma unroll
  for (int it = 0; it < BR::KIT; ++it) {
    const int idx = tid + it * NT;
    if (BR::KIT * NT > 64 * CPR && idx >= 64 * CPR) break;  // uniform per wave
    const int kk = idx / CPR, col = (idx % CPR) * VEC;
    *reinterpret_cast<uint4*>(P.Ks + kk * B_::KS + col) = R.k[it];
    if (!want_norm) continue;
    // |k|^2 for the feature map: CPR consecutive lanes hold one row
    const T* ke = reinterpret_cast<const T*>(&R.k[it]);
    float q2 = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) q2 += to_f32(ke[e]) * to_f32(ke[e]);
    q2 = row_sum<CPR>(q2);
    if (col == 0) P.kstat[128 + kk] = q2;
  }
  if constexpr (B_::TR) {  // values row-major as H, 16-byte writes
#pragma unroll
    for (int it = 0; it < BR::KIT; ++it) {
      const int idx = tid + it * NT;
      if (BR::KIT * NT > 64 * CPR && idx >= 64 * CPR) break;
      const int kk = idx / CPR, col = (idx % CPR) * VEC;
      const T* ve = reinterpret_cast<const T*>(&R.vr[it]);
      H w[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) w[e] = from_f32<H>(to_f32(ve[e]));
      *reinterpret_cast<uint4*>(P.VTs + kk * B_::VR + col) = *reinterpret_cast<uint4*>(w);
    }
    return;
  }
#pragma unroll
  for (int it = 0; it < BR::VIT; ++it) {
    const int idx = tid + it * NT;
    if (BR::VIT * NT > 32 * CPR && idx >= 32 * CPR) break;
    const int a2 = idx / CPR, col = (idx % CPR) * VEC;
    const T* v0 = reinterpret_cast<const T*>(&R.v[it][0]);
    const T* v1 = reinterpret_cast<const T*>(&R.v[it][1]);
    const int pc = perm_col(2 * a2);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      H w2[2] = {from_f32<H>(to_f32(v0[e])), from_f32<H>(to_f32(v1[e]))};
      if constexpr (sizeof(H) == 2)
        *reinterpret_cast<uint32_t*>(P.VTs + (col + e) * B_::VS + pc) = *reinterpret_cast<uint32_t*>(w2);
      else
        *reinterpret_cast<uint2*>(P.VTs + (col + e) * B_::VS + pc) = *reinterpret_cast<uint2*>(w2);
    }
  }
}

// NP-Map [P3 "NP-Map: Norm-Preserving Feature Map"], reading: direction =
// softmax(x F) scaled to unit L2 norm, magnitude = ||x||. Computes, for one
// 16-row tile whose B fragments of X^T are xf[], the feature values in the
// accumulator layout of (X F)^T: out[ft][i] = phi(x_r)[16 ft + 4g + i].
template <typename T, int D>
__device__ __forceinline__ void np_map_tile(const BlkPtr<T, D>& P, const Frag<T>* xf, f32x4* out) {
  const int lane = opaque_tid() & 63, r16 = lane & 15, g4 = lane >> 4;
  float xn2 = 0.f;
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) xn2 += frag_sumsq(xf[kb]);
  xn2 = sum_over_g(xn2);
  float mx = STILL_NEG_INF;
#pragma unroll
  for (int ft = 0; ft < D / 16; ++ft) {
    out[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      mma(out[ft], ld_frag(P.ft(ft, kb, lane)), xf[kb]);
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmax_nn(mx, out[ft][i]);
  }
  mx = max_over_g(mx);
  float ss = 0.f;
#pragma unroll
  for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = exp_acc<T>(out[ft][i] - mx);
      out[ft][i] = e;
      ss += e * e;
    }
  ss = sum_over_g(ss);
  const float f = sqrtf(xn2) / sqrtf(ss);
#pragma unroll
  for (int ft = 0; ft < D / 16; ++ft) out[ft] *= f;
}

// Orders the LDS reads and MFMAs of the enclosing scheduling region (one
// basic block): AHEAD reads first, then N times M MFMAs followed by R reads,
// then TAIL MFMAs. The reads then run that far ahead of the MFMAs that use
// them and their latency is covered; other instructions are placed freely.
template <int AHEAD, int N, int M, int R, int TAIL>
__device__ __forceinline__ void lds_mfma_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);  // MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, TAIL, 0);
}

// np_map_tile for NX tiles at once: each F^T fragment read from LDS serves
// every tile.
template <typename T, int D, int NX>
__device__ __forceinline__ void np_map_tiles(const BlkPtr<T, D>& P, const Frag<T> (&xf)[NX][D / 32],
                                             f32x4 (&out)[NX][D / 16]) {
  const int lane = opaque_tid() & 63;
  float xn2[NX], mx[NX], ss[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    xn2[x] = 0.f;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) xn2[x] += frag_sumsq(xf[x][kb]);
    xn2[x] = sum_over_g(xn2[x]);
    mx[x] = STILL_NEG_INF;
    ss[x] = 0.f;
  }
#pragma unroll
  for (int ft = 0; ft < D / 16; ++ft) {
#pragma unroll
    for (int x = 0; x < NX; ++x) out[x][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      const Frag<T> f = ld_frag(P.ft(ft, kb, lane));
#pragma unroll
      for (int x = 0; x < NX; ++x) mma(out[x][ft], f, xf[x][kb]);
    }
#pragma unroll
    for (int x = 0; x < NX; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[x] = fmax_nn(mx[x], out[x][ft][i]);
  }
  if constexpr (sizeof(T) == 2)  // F^T reads two feature tiles ahead
    lds_mfma_pipeline<2 * (D / 32), (D / 16 - 2) * (D / 32), NX, 1, 2 * (D / 32) * NX>();
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    mx[x] = max_over_g(mx[x]);
#pragma unroll
    for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp_acc<T>(out[x][ft][i] - mx[x]);
        out[x][ft][i] = e;
        ss[x] += e * e;
      }
    ss[x] = sum_over_g(ss[x]);
    const float f = sqrtf(xn2[x]) / sqrtf(ss[x]);
#pragma unroll
    for (int ft = 0; ft < D / 16; ++ft) out[x][ft] *= f;
  }
}

// Max / sum over the 16 lanes sharing g (the 16 columns of a C tile).
__device__ __forceinline__ float max_over_r(float x) {
  x = row_max<16>(x);
  return x;
}
__device__ __forceinline__ float sum_over_r(float x) {
  x = row_sum<16>(x);
  return x;
}

// NP-Map features of the block's 64 keys, computed once by the waves
// w < D/16, wave w holding feature tile w of every key in the accumulator
// layout of K F: ph[kt][i] = phi(k_{16kt+4g+i})[16w + r]. Per-key softmax
// statistics are combined across waves through LDS: each wave's max and sum
// of squares relative to it, then one factor per (wave, key). With want_w
// the features are also written as H A fragments (rows = keys) to WF. One
// workgroup barrier (two with want_w); every thread must call it with the
// same want_w.
template <typename T, int D>
__device__ __forceinline__ void block_phi(const BlkPtr<T, D>& P, f32x4 (&ph)[4],
                                          bool want_w) {
  using B_ = Blk<T, D>;
  typedef typename HalfOf<T>::type H;
  const int tid = opaque_tid(), wave = tid >> 6, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const bool mine = wave < B_::NFT;  // wave-uniform
  if (mine) {
    Frag<T> fb[D / 32];
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) fb[kb] = ld_frag(P.ft(wave, kb));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      ph[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        mma(ph[kt], ld_frag(P.Ks + (16 * kt + r16) * B_::KS + 32 * kb + 8 * g4), fb[kb]);
    }
    if constexpr (sizeof(T) == 2)  // F^T and two key tiles ahead
      lds_mfma_pipeline<3 * (D / 32), 2 * (D / 32), 1, 1, 2 * (D / 32)>();
    // per key: this wave's max over its 16 features and its sum of squared
    // exponentials relative to that max; the 16 keys of a lane are reduced
    // side by side (independent chains), then one lane per row stores them
    f32x4 mk[4], sk[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mk[kt][i] = max_over_r(ph[kt][i]);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp_acc<T>(ph[kt][i] - mk[kt][i]);
        ph[kt][i] = e;
        sk[kt][i] = e * e;
      }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sk[kt][i] = sum_over_r(sk[kt][i]);
    if (r16 == 0) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        *reinterpret_cast<f32x4*>(P.kmax + wave * 64 + 16 * kt + 4 * g4) = mk[kt];
        *reinterpret_cast<f32x4*>(P.ksum + wave * 64 + 16 * kt + 4 * g4) = sk[kt];
      }
    }
  }
  __syncthreads();
  if (mine) {
    // Combine the waves per key (lane = key): the maximum M of the waves'
    // maxima, the sum S of squares relative to it, and this wave's factor
    // exp(m_w - M) |k| / sqrt(S). Every wave computes the key statistics
    // itself, so no further workgroup barrier is needed; each lane then
    // takes the factors of its 16 keys from the lanes that hold them.
    float M = STILL_NEG_INF;
#pragma unroll
    for (int w = 0; w < B_::NFT; ++w) M = fmax_nn(M, P.kmax[w * 64 + lane]);
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < B_::NFT; ++w)
      S += P.ksum[w * 64 + lane] * exp_acc<T>(2.f * (P.kmax[w * 64 + lane] - M));
    const float base = sqrtf(P.kstat[128 + lane]) / sqrtf(S);
    const float fac = exp_acc<T>(P.kmax[wave * 64 + lane] - M) * base;
    const int f = 16 * wave + r16, bb = f >> 5, o = f & 31;
    const int gp = (o & 15) >> 2, sl = (o & 3) + ((o >> 4) << 2);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ph[kt][i] *= __shfl(fac, 16 * kt + 4 * g4 + i);
      if (want_w) {
        if constexpr (B_::TR) {  // feature-major: 4 keys of feature f, 8 bytes
          H w4[4] = {from_f32<H>(ph[kt][0]), from_f32<H>(ph[kt][1]), from_f32<H>(ph[kt][2]),
                     from_f32<H>(ph[kt][3])};
          *reinterpret_cast<uint2*>(P.WF + f * B_::FKS + 16 * kt + 4 * g4) = *reinterpret_cast<uint2*>(w4);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            P.wf(kt, bb)[(16 * gp + ((4 * g4 + i) & 15)) * 8 + sl] = from_f32<H>(ph[kt][i]);
        }
      }
    }
  }
  if (want_w) __syncthreads();  // WF is read by every wave
}

// The block's contribution phi(K)^T diag(fmask) V to the d_k tile of wave w
// (< D/16): acc[vt] for every d_v tile, key halves kb2 in [kb_lo, kb_hi).
// phi is split into two H parts (fp16 hi + lo keep ~22 significant bits;
// values are exact in H), so the products keep float32 accuracy.
template <typename T, int D>
__device__ __forceinline__ void fold_tile(const BlkPtr<T, D>& P, const f32x4 (&ph)[4], int kb_lo,
                                          int kb_hi, f32x4 (&acc)[D / 16]) {
  using B_ = Blk<T, D>;
  typedef typename HalfOf<T>::type H;
  const int lane = opaque_tid() & 63, r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    if (kb2 < kb_lo || kb2 >= kb_hi) continue;
    f32x4 x0 = ph[2 * kb2], x1 = ph[2 * kb2 + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x0[i] *= P.fmask[32 * kb2 + 4 * g4 + i];
      x1[i] *= P.fmask[32 * kb2 + 16 + 4 * g4 + i];
    }
    Frag<H> hi, lo;
    split2_frag<H>(x0, x1, hi, lo);
#pragma unroll
    for (int vt = 0; vt < D / 16; ++vt) {
      const Frag<H> bv = P.ld_v(vt, kb2, lane);
      mma(acc[vt], hi, bv);
      if constexpr (sizeof(H) == 2) mma(acc[vt], lo, bv);
    }
  }
}

// The block's contribution to z for feature 16w + r (lanes with g == 0).
template <typename T, int D>
__device__ __forceinline__ float fold_zsum(const BlkPtr<T, D>& P, const f32x4 (&ph)[4]) {
  const int lane = opaque_tid() & 63, g4 = lane >> 4;
  float z = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) z += P.fmask[16 * kt + 4 * g4 + i] * ph[kt][i];
  return sum_over_g(z);
}

// Fold the block into the walk's state in LDS (SP += contribution, z += ...);
// wave w updates the d_k tile w, i.e. half e = w % 2 of the pairs (vt, w/2).
// DK: with the forget gate, fS is its factor on the state before the
// block's keys are added (their features come weighted already).
template <typename T, int D, bool DK = false>
__device__ __forceinline__ void block_fold(const BlkPtr<T, D>& P, const f32x4 (&ph)[4], float fS = 1.f) {
  using B_ = Blk<T, D>;
  const int wave = opaque_tid() >> 6, lane = opaque_tid() & 63, r16 = lane & 15, g4 = lane >> 4;
  if (wave >= B_::NFT) return;
  f32x4 acc[D / 16];
#pragma unroll
  for (int vt = 0; vt < D / 16; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  fold_tile<T, D>(P, ph, 0, 2, acc);
#pragma unroll
  for (int vt = 0; vt < D / 16; ++vt) {
    float* sp = P.pair(vt * (D / 32) + (wave >> 1), wave & 1);
    if constexpr (DK) *reinterpret_cast<f32x4*>(sp) = *reinterpret_cast<const f32x4*>(sp) * fS + acc[vt];
    else *reinterpret_cast<f32x4*>(sp) += acc[vt];
  }
  const float z = fold_zsum<T, D>(P, ph);
  if (g4 == 0) {
    if constexpr (DK) P.zs[16 * wave + r16] = P.zs[16 * wave + r16] * (double)fS + (double)z;
    else P.zs[16 * wave + r16] += (double)z;
  }
}

// Super-chunk states in the workspace use the fragment-linear layout of SP
// (element (p*64 + lane)*8 + slot), so moving them is a straight copy; the
// exported state is row-major S[d_k][d_v].
template <typename T, int D>
__device__ __forceinline__ void load_state(const BlkPtr<T, D>& P, const float* Sfl) {
  for (int e = opaque_tid() * 4; e < D * D; e += 512 * 4)
    *reinterpret_cast<f32x4*>(P.SP + e) = *reinterpret_cast<const f32x4*>(Sfl + e);
}

// ---------------------------------------------------- 4. state_delta ----
// Super-chunk s folds the chunks [cf(sK), cf(sK+K)) into the state, cf(c) =
// chunks wholly before the window of chunk c; the last super-chunk's delta
// runs to cf(T-1), so that the sum of all deltas is the exported state. This
// kernel sums their unkept tokens' phi(k) v^T (and phi(k)) so the scan can
// give every super-chunk its starting state and the decode state its S, z.
// Every 32-key group lands in float64 sums on its own: a single 8x-norm token
// can make a group's sum ~1e4, where one float32 rounding is already ~5e-4.
//
// Keys with |k|^2 max|v| >= BIG_KV fold through a float64 path instead of
// the MFMAs: the bf16 MFMA accumulates the 128 products of a feature logit
// x.F with an error of up to about 2^-24 times the sum of their magnitudes
// (measured on gfx950), i.e. ~1e-5 absolute for a key of norm ~300, which
// moves phi(k) by ~1e-5 relative and the state entry it dominates (~1e4) by
// ~1e-1. Such keys are rare (the largest 1-2 % of |k|^2 max|v| in the
// workloads here); their logits, NP-Map and rank-1 update are float64.
constexpr float BIG_KV = 16384.f;

template <typename T, int D>
struct BigScratch {  // in the state region SP, which state_delta does not use
  double* part;  // [512 / D][D] partial logits
  double* phi;   // [D]
  double* red;   // [8]
  float* vmx;    // [64] max |v| per key
  uint32_t* bits;  // [2] big keys of the block
  __device__ BigScratch(const BlkPtr<T, D>& P) {
    char* b = reinterpret_cast<char*>(P.SP);
    part = reinterpret_cast<double*>(b);
    phi = part + 512;
    red = phi + D;
    vmx = reinterpret_cast<float*>(red + 8);
    bits = reinterpret_cast<uint32_t*>(vmx + 64);
  }
};

// value c of key kk of the block in LDS, as float
template <typename T, int D>
__device__ __forceinline__ float blk_v(const BlkPtr<T, D>& P, int kk, int c) {
  using B_ = Blk<T, D>;
  if constexpr (B_::TR) return to_f32(P.VTs[kk * B_::VR + c]);
  else return to_f32(P.VTs[c * B_::VS + perm_col(kk)]);
}

// Marks the block's fold keys with |k|^2 max|v| >= BIG_KV: clears their
// fmask (the MFMA fold skips them) and returns them as a bit mask (same in
// every thread). Ends with a barrier.
template <typename T, int D>
__device__ __forceinline__ uint64_t mark_big_keys(const BlkPtr<T, D>& P, const BigScratch<T, D>& Z) {
  const int tid = threadIdx.x;
  {  // 8 threads per key, D/8 values each
    const int kk = tid >> 3, part = tid & 7;
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) m = fmaxf(m, fabsf(blk_v<T, D>(P, kk, part * (D / 8) + c)));
    m = row_max<8>(m);
    if (part == 0) Z.vmx[kk] = m;
  }
  __syncthreads();
  if (tid < 64) {
    const bool big = P.fmask[tid] != 0.f && P.kstat[128 + tid] * Z.vmx[tid] >= BIG_KV;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(big);
    if (big) P.fmask[tid] = 0.f;
    if (tid == 0) {
      Z.bits[0] = (uint32_t)bits;
      Z.bits[1] = (uint32_t)(bits >> 32);
    }
  }
  __syncthreads();
  return ((uint64_t)Z.bits[1] << 32) | Z.bits[0];
}

// Float64 fold of key kk of the block: logits x.F (every product of bf16 /
// float32 inputs is exact in float64), NP-Map [P3 "NP-Map: Norm-Preserving
// Feature Map"] and the rank-1 update of the calling thread's state entries
// sum[vt][i] = S[16w + 4g + i][16vt + r] (waves w < D/16) and z[16w + r]
// (lanes g == 0). Every thread calls it; it contains barriers.
template <typename T, int D>
__device__ __forceinline__ void big_key_fold(const BlkPtr<T, D>& P, const BigScratch<T, D>& Z, int kk,
                                             double (&sum)[D / 16][4], double& zsum, double wgt = 1.0) {
  using B_ = Blk<T, D>;
  constexpr int NPART = 512 / D, TP = D / NPART;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  {
    const int j = tid % D, part = tid / D;
    double u = 0.0;
#pragma unroll 8
    for (int ii = 0; ii < TP; ++ii) {
      const int i = part * TP + ii;
      const int kb = i >> 5, g = (i & 31) >> 3, s = i & 7;
      const float f = to_f32(P.FT[(((j >> 4) * (D / 32) + kb) * 64 + 16 * g + (j & 15)) * 8 + s]);
      u += (double)to_f32(P.Ks[kk * B_::KS + i]) * (double)f;
    }
    Z.part[part * D + j] = u;
  }
  __syncthreads();
  double uj = 0.0, e = 0.0, k2 = 0.0;
  if (tid < D) {
#pragma unroll
    for (int p = 0; p < NPART; ++p) uj += Z.part[p * D + tid];
    const double kx = (double)to_f32(P.Ks[kk * B_::KS + tid]);
    const double mx = wave_max_d(uj);
    k2 = wave_sum_d(kx * kx);
    if (lane == 0) {
      Z.red[2 * wave] = mx;
      Z.red[2 * wave + 1] = k2;
    }
  }
  __syncthreads();
  if (tid < D) {
    double mx = Z.red[0];
    k2 = Z.red[1];
#pragma unroll
    for (int w = 1; w < D / 64; ++w) {
      mx = Z.red[2 * w] > mx ? Z.red[2 * w] : mx;
      k2 += Z.red[2 * w + 1];
    }
    e = exp(uj - mx);
    const double ss = wave_sum_d(e * e);
    if (lane == 0) Z.red[4 + wave] = ss;
  }
  __syncthreads();
  if (tid < D) {
    double ss = 0.0;
#pragma unroll
    for (int w = 0; w < D / 64; ++w) ss += Z.red[4 + w];
    Z.phi[tid] = wgt * (sqrt(k2) * e / sqrt(ss));  // wgt: the key's forget factor
  }
  __syncthreads();
  if (wave < B_::NFT) {
#pragma unroll
    for (int vt = 0; vt < D / 16; ++vt) {
      const double vv = (double)blk_v<T, D>(P, kk, 16 * vt + r16);
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[vt][i] += Z.phi[16 * wave + 4 * g4 + i] * vv;
    }
    if (g4 == 0) zsum += Z.phi[16 * wave + r16];
  }
}

// float32 data: in blocks of 64 keys through the attention kernel's block
// helpers (features of feature tile w by wave w, per-key statistics combined
// across the waves through LDS).
template <int D, bool DK = false>
__global__ __launch_bounds__(512) void state_delta_f32_kernel(PrefillArgs a) {
  using T = float;
  using B_ = Blk<T, D>;
  extern __shared__ __align__(16) char smem[];
  const BlkPtr<T, D> P(smem);
  const BigScratch<T, D> Z(P);
  const int s = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int unit = b * a.Hkv + kv;
  const uint32_t kv_bytes = (uint32_t)((size_t)a.L * D * sizeof(T));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(reinterpret_cast<const T*>(a.k) + (size_t)unit * a.L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(reinterpret_cast<const T*>(a.v) + (size_t)unit * a.L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t sfr = make_rsrc(a.selflag + (size_t)unit * a.L, (uint32_t)a.L);
  load_ft<T, D, 512>(P, reinterpret_cast<const T*>(a.ft) + (size_t)kv * D * D);
  double sum[D / 16][4];
#pragma unroll
  for (int vt = 0; vt < D / 16; ++vt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[vt][i] = 0.0;
  double zsum = 0.0;
  const int lo = full_chunks_before(s * a.K, a.W, a.C) * a.C;
  const int hi = (s == a.NS - 1 ? full_chunks_before(a.T - 1, a.W, a.C)
                                : full_chunks_before(s * a.K + a.K, a.W, a.C)) * a.C;
  // forget gate: the delta is held at hi, key j weighted gamma^(hi - j)
  const double l2g64 = DK ? log2((double)a.decay[kv]) : 0.0;
  const float l2g = (float)l2g64;
  // block blo + 64 is issued as soon as block blo is in LDS (past hi the
  // loads read zeros past the buffer range)
  BlkRegs<T, D, 512> R;
  issue_block<T, D, 512>(R, kr, vr, kv_bytes, sfr, blk_range(lo, hi));
  for (int blo = lo; blo < hi; blo += 64) {
    __syncthreads();
    commit_block<T, D, 512>(P, R, lo, hi);
    issue_block<T, D, 512>(R, kr, vr, kv_bytes, sfr, blk_range(blo + 64, hi));
    __syncthreads();
    const uint64_t big = mark_big_keys<T, D>(P, Z);
    f32x4 ph[4];
    block_phi<T, D>(P, ph, false);
    if constexpr (DK) {  // key j weighted gamma^(hi - j)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) ph[kt][i] *= exp2f((float)(hi - (blo + 16 * kt + 4 * g4 + i)) * l2g);
    }
    if (wave < B_::NFT) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x4 acc[D / 16];
#pragma unroll
        for (int vt = 0; vt < D / 16; ++vt) acc[vt] = f32x4{0.f, 0.f, 0.f, 0.f};
        fold_tile<T, D>(P, ph, kb2, kb2 + 1, acc);
#pragma unroll
        for (int vt = 0; vt < D / 16; ++vt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sum[vt][i] += (double)acc[vt][i];
      }
      zsum += (double)fold_zsum<T, D>(P, ph);
    }
    for (uint64_t m = big; m; m &= m - 1) {  // uniform
      const int kk = (int)__builtin_ctzll(m);
      big_key_fold<T, D>(P, Z, kk, sum, zsum, DK ? exp2((double)(hi - (blo + kk)) * l2g64) : 1.0);
    }
  }
  float* dst = a.dS + ((size_t)unit * a.NS + s) * (D * D + D);
  if (wave < B_::NFT) {
#pragma unroll
    for (int vt = 0; vt < D / 16; ++vt) {
      float* o = dst + ((size_t)(2 * (vt * (D / 32) + (wave >> 1)) + (wave & 1)) * 64 + lane) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (float)sum[vt][i];
    }
    if (g4 == 0) dst[D * D + 16 * wave + r16] = (float)zsum;
  }
}

// 16-bit data: blocks of SD_BK = 128 keys (eight 16-key tiles), one
// workgroup of 8 waves per super-chunk.
//  * Wave w computes phi(k) of key tile w over all D features (X F by MFMA
//    with the features on the lanes): a key's softmax statistics then reduce
//    over the wave's own registers and the 16 lanes of a row, with no
//    exchange between waves. Keys that do not fold (kept, past the range,
//    or large, see below) get zero features. The features go to LDS
//    feature-major in float32.
//  * Wave w then folds feature tile w % (D/16) against the block's values
//    for its d_v tiles: phi as fp16 hi + lo parts (~22 significant bits),
//    values exact in fp16; the block's float32 sums are added to float64
//    ones.
//  * Large keys (|k|^2 max|v| >= BIG_KV, a few per block) take the float64
//    path: logits split over all threads (each D / (512 / D) products),
//    NP-Map and rank-1 update, in rounds of up to SD_NBK keys with two
//    barriers per round.
constexpr int SD_BK = 128;
constexpr int SD_NBK = 8;

template <typename T, int D>
struct SdLds {
  static constexpr int VS = D + 8;       // value row (fp16 elements)
  static constexpr int PS = SD_BK + 4;   // feature row (floats)
  static constexpr size_t ft_bytes = (size_t)D * D * sizeof(T);
  static constexpr size_t v_bytes = (size_t)SD_BK * VS * 2;
  static constexpr size_t ph_bytes = (size_t)D * PS * 4;
  static constexpr size_t vmx_bytes = SD_BK * 4;
  static constexpr size_t bits_bytes = 32;
  static constexpr size_t bst_bytes = (size_t)SD_NBK * (8 * 2 + 2) * 8;  // + |k|^2, forget factor
  static constexpr size_t bphi_bytes = (size_t)SD_NBK * D * 8;
  static constexpr size_t krow_bytes = (size_t)16 * D * sizeof(T);  // two large-key rows per wave
  static constexpr size_t kn2_bytes = (size_t)SD_BK * 8;              // float64 |k|^2 of large keys
  static constexpr size_t bytes =
      ft_bytes + v_bytes + ph_bytes + vmx_bytes + bits_bytes + bst_bytes + bphi_bytes + krow_bytes + kn2_bytes;
  static_assert(bytes <= 160 * 1024, "one workgroup's LDS");
};

// sum over groups of N consecutive lanes (N = 4 or 8), float64
template <int N>
__device__ __forceinline__ double group_sum_d(double x) {
  x += dppd<0xB1>(x);
  x += dppd<0x4E>(x);
  if constexpr (N >= 8) x += dppd<0x141>(x);
  static_assert(N == 4 || N == 8, "groups of 4 or 8 lanes");
  return x;
}

template <typename T, int D, bool DK = false>
__global__ __launch_bounds__(512) void state_delta_kernel(PrefillArgs a) {
  static_assert(sizeof(T) == 2, "16-bit data");
  using L_ = SdLds<T, D>;
  constexpr int NFT = D / 16;            // feature (and d_v) tiles
  constexpr int VPW = NFT * NFT / 8;     // d_v tiles folded per wave
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int VIT = SD_BK * CPR / 512; // value chunks per thread
  constexpr int NP = 512 / D;            // threads per float64 logit
  constexpr int TPP = D / NP;            // products per thread
  extern __shared__ __align__(16) char smem[];
  T* FT = lds_opaque(reinterpret_cast<T*>(smem));
  f16* VR = lds_opaque(reinterpret_cast<f16*>(smem + L_::ft_bytes));
  float* PH = lds_opaque(reinterpret_cast<float*>(smem + L_::ft_bytes + L_::v_bytes));
  char* misc = smem + L_::ft_bytes + L_::v_bytes + L_::ph_bytes;
  float* vmx = lds_opaque(reinterpret_cast<float*>(misc));
  uint32_t* bigw = lds_opaque(reinterpret_cast<uint32_t*>(misc + L_::vmx_bytes));
  double* bst = lds_opaque(reinterpret_cast<double*>(misc + L_::vmx_bytes + L_::bits_bytes));
  double* bk2 = bst + SD_NBK * 16;
  double* bphi = lds_opaque(reinterpret_cast<double*>(misc + L_::vmx_bytes + L_::bits_bytes + L_::bst_bytes));
  T* krows = lds_opaque(reinterpret_cast<T*>(misc + L_::vmx_bytes + L_::bits_bytes + L_::bst_bytes + L_::bphi_bytes));
  double* kn2d = lds_opaque(
      reinterpret_cast<double*>(misc + L_::vmx_bytes + L_::bits_bytes + L_::bst_bytes + L_::bphi_bytes + L_::krow_bytes));

  const int s = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = b * a.Hkv + kv;
  const uint32_t kv_bytes = (uint32_t)((size_t)a.L * D * sizeof(T));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(reinterpret_cast<const T*>(a.k) + (size_t)unit * a.L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(reinterpret_cast<const T*>(a.v) + (size_t)unit * a.L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t sfr = make_rsrc(a.selflag + (size_t)unit * a.L, (uint32_t)a.L);
  {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.ft) + (size_t)kv * D * D);
    for (int e = tid; e < (int)(L_::ft_bytes / 16); e += 512) reinterpret_cast<uint4*>(FT)[e] = src[e];
  }
  const int lo = full_chunks_before(s * a.K, a.W, a.C) * a.C;
  const int hi = (s == a.NS - 1 ? full_chunks_before(a.T - 1, a.W, a.C)
                                : full_chunks_before(s * a.K + a.K, a.W, a.C)) * a.C;
  // forget gate: the delta is held at hi, key j weighted gamma^(hi - j)
  const double l2g64 = DK ? log2((double)a.decay[kv]) : 0.0;
  const float l2g = (float)l2g64;
  // fold ownership: feature tile ft, d_v tiles vt0 .. vt0 + VPW - 1
  const int ft = wave % NFT, vt0 = (wave / NFT) * VPW;
  double sum[VPW][4];
#pragma unroll
  for (int v = 0; v < VPW; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[v][i] = 0.0;
  double zsum = 0.0;

  // loads of a block: wave w's key tile as MFMA A fragments (row r16), its
  // keys' kept flags, and the values (every thread VIT row chunks); rows at
  // or past hi read zeros (keys) or are not folded
  Frag<T> kn[D / 32];
  int sn;
  uint4 vn[VIT];
  auto issue = [&](int blo) __attribute__((always_inline)) {
    const int row = blo + 16 * wave + r16;
    const uint32_t off = row < hi ? (uint32_t)((size_t)row * D * sizeof(T)) : kv_bytes;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) kn[kb] = ld_frag_buf<T>(kr, off + 8 * g4 * sizeof(T), 32 * kb * sizeof(T));
    sn = (int)__builtin_amdgcn_raw_buffer_load_b8(sfr, row < hi ? (uint32_t)row : 0xffffffffu, 0, 0);
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = tid + it * 512, vrow = blo + idx / CPR;
      vn[it] = ld_u4_buf(vr, vrow < hi ? (uint32_t)(((size_t)vrow * D + (idx % CPR) * 8) * sizeof(T)) : kv_bytes, 0);
    }
  };
  if (lo < hi) issue(lo);
  for (int blo = lo; blo < hi; blo += SD_BK) {
    __syncthreads();  // the previous block's fold and large keys are done with VR, PH
    // values as fp16, row-major, and each key's largest |v|
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int idx = tid + it * 512, row = idx / CPR, col = (idx % CPR) * 8;
      const T* ve = reinterpret_cast<const T*>(&vn[it]);
      f16 w[8];
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = to_f32(ve[e]);
        w[e] = (f16)x;
        m = fmaxf(m, fabsf(x));
      }
      *reinterpret_cast<uint4*>(VR + row * L_::VS + col) = *reinterpret_cast<uint4*>(w);
      m = row_max<CPR>(m);
      if (col == 0) vmx[row] = m;
    }
    Frag<T> kc[D / 32];
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) kc[kb] = kn[kb];
    const int sc = sn;
    if (blo + SD_BK < hi) issue(blo + SD_BK);
    __syncthreads();  // VR, vmx

    // phi of key tile `wave`: ph[f][i] = logit of key 4g + i, feature 16 f + r
    {
      f32x4 ph[NFT];
#pragma unroll
      for (int f = 0; f < NFT; ++f) {
        ph[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
          mma(ph[f], kc[kb], ld_frag(FT + ((size_t)(f * (D / 32) + kb) * 64 + lane) * 8));
      }
      lds_mfma_pipeline<2 * (D / 32), (NFT - 2) * (D / 32), 1, 1, 2 * (D / 32)>();
      // |k|^2 of key r16 (every g; packed bf16 dot products), and whether
      // it folds / is large
      float n2 = 0.f;
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) n2 = frag_dot2_sumsq(kc[kb], n2);
      n2 = sum_over_g(n2);
      const int row = blo + 16 * wave + r16;
      const bool fold = row < hi && sc == 0;
      const bool big = fold && n2 * vmx[16 * wave + r16] >= BIG_KV;
      const uint32_t use16 = (uint32_t)__builtin_amdgcn_ballot_w64(fold && !big) & 0xffffu;
      const uint32_t big16 = (uint32_t)__builtin_amdgcn_ballot_w64(big) & 0xffffu;
      if (lane == 0) bigw[wave] = big16;
      // the rows of the tile's first two large keys and their float64
      // |k|^2, for the float64 path
      if (big16) {  // uniform
        double d2 = 0.0;
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double x = (double)to_f32(kc[kb].v[e]);
            d2 += x * x;
          }
        d2 += xor16d(d2);
        d2 += xor32d(d2);
        const int q = __builtin_popcount(big16 & ((1u << r16) - 1u));
        if (big && q < 2) {
#pragma unroll
          for (int kb = 0; kb < D / 32; ++kb) st_frag(krows + (2 * wave + q) * D + 32 * kb + 8 * g4, kc[kb]);
        }
        if (big && g4 == 0) kn2d[16 * wave + r16] = d2;
      }
      // softmax over the features in base 2 (exp2(x log2 e - m log2 e): the
      // offset's rounding is common to a key's features and cancels in the
      // normalisation), the factor |k| / sqrt(sum e^2) from the hardware
      // square root and reciprocal square root (~1 ulp each)
      float nm[4], ss[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = ph[0][i];
#pragma unroll
        for (int f = 1; f < NFT; ++f) m = fmax_nn(m, ph[f][i]);
        nm[i] = -row_max<16>(m) * STILL_LOG2E;
        ss[i] = 0.f;
      }
#pragma unroll
      for (int f = 0; f < NFT; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(ph[f][i], STILL_LOG2E, nm[i]));
          ph[f][i] = e;
          ss[i] = fmaf(e, e, ss[i]);
        }
      float fac[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s2 = row_sum<16>(ss[i]);
        const float k2 = __shfl(n2, 4 * g4 + i);
        fac[i] = ((use16 >> (4 * g4 + i)) & 1u) ? __builtin_amdgcn_sqrtf(k2) * __builtin_amdgcn_rsqf(s2) : 0.f;
        if constexpr (DK) fac[i] *= exp2f((float)(hi - (row - r16 + 4 * g4 + i)) * l2g);
      }
#pragma unroll
      for (int f = 0; f < NFT; ++f) {
        const f32x4 o = {ph[f][0] * fac[0], ph[f][1] * fac[1], ph[f][2] * fac[2], ph[f][3] * fac[3]};
        *reinterpret_cast<f32x4*>(PH + (16 * f + r16) * L_::PS + 16 * wave + 4 * g4) = o;
      }
    }
    __syncthreads();  // PH, bigw

    // fold: S[16 ft + 4g + i][16 vt + r] over the block's keys
    {
      f32x4 acc[VPW];
#pragma unroll
      for (int v = 0; v < VPW; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
      float zl = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < SD_BK / 32; ++kb2) {
        const float* pr = PH + (16 * ft + r16) * L_::PS + 32 * kb2 + 4 * g4;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(pr);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(pr + 16);
        zl += ((x0[0] + x0[1]) + (x0[2] + x0[3])) + ((x1[0] + x1[1]) + (x1[2] + x1[3]));
        Frag<f16> fh, fl;
        split2_frag<f16>(x0, x1, fh, fl);
#pragma unroll
        for (int v = 0; v < VPW; ++v) {
          const Frag<f16> bv =
              tr_frag(VR + (32 * kb2 + 4 * g4 + (r16 >> 2)) * L_::VS + 16 * (vt0 + v) + 4 * (r16 & 3), 16 * L_::VS);
          mma(acc[v], fh, bv);
          mma(acc[v], fl, bv);
        }
      }
#pragma unroll
      for (int v = 0; v < VPW; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[v][i] += (double)acc[v][i];
      if (vt0 == 0) zsum += (double)sum_over_g(zl);
    }

    // large keys, float64, in rounds of up to SD_NBK
    uint64_t bl = 0, bh = 0;  // the block's large keys (uniform)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      bl |= (uint64_t)bigw[w] << (16 * w);
      bh |= (uint64_t)bigw[4 + w] << (16 * w);
    }
    while (bl | bh) {
      // this round: the first SD_NBK of them (masks rl, rh; key n of the
      // round is the n-th set bit)
      uint64_t rl = 0, rh = 0;
      int nb = 0;
      for (; nb < SD_NBK && (bl | bh); ++nb) {
        if (bl) {
          rl |= bl & (~bl + 1);
          bl &= bl - 1;
        } else {
          rh |= bh & (~bh + 1);
          bh &= bh - 1;
        }
      }
      auto next_key = [](uint64_t& ml, uint64_t& mh) {
        int k;
        if (ml) {
          k = __builtin_ctzll(ml);
          ml &= ml - 1;
        } else {
          k = 64 + __builtin_ctzll(mh);
          mh &= mh - 1;
        }
        return k;
      };
      // logits: thread (j, part) sums TPP products of feature j, the NP
      // threads of a feature are consecutive lanes; the logit goes to bphi
      // (turned into the feature after the barrier), the wave's maximum
      // and sum of exp(2 (u - m)) over its features to bst, |k|^2 to bk2
      const int j = tid / NP, part = tid % NP;
      uint64_t ml = rl, mh = rh;
#pragma unroll 1
      for (int n = 0; n < nb; ++n) {
        const int kk = next_key(ml, mh), wo = kk >> 4;
        const int slot = __builtin_popcount(bigw[wo] & ((1u << (kk & 15)) - 1u));  // uniform
        const T* krow = krows + (2 * wo + slot) * D;
        const int row = blo + kk;
        double u = 0.0;
#pragma unroll
        for (int q = 0; q < TPP / 8; ++q) {
          const int i0 = part * TPP + 8 * q;
          const uint4 k8 = slot < 2 ? *reinterpret_cast<const uint4*>(krow + i0)
                                    : ld_u4_buf(kr, (uint32_t)(((size_t)row * D + i0) * sizeof(T)), 0);
          const T* ke = reinterpret_cast<const T*>(&k8);
          const Frag<T> f8 =
              ld_frag(FT + ((size_t)(((j >> 4) * (D / 32) + (i0 >> 5)) * 64) + 16 * ((i0 & 31) >> 3) + (j & 15)) * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) u += (double)to_f32(ke[e]) * (double)to_f32(f8.v[e]);
        }
        u = group_sum_d<NP>(u);
        const double m = wave_max_d(u);
        const double se = wave_sum_d(part == 0 ? exp(2.0 * (u - m)) : 0.0);
        if (part == 0) bphi[n * D + j] = u;
        if (lane == 0) {
          bst[(n * 8 + wave) * 2] = m;
          bst[(n * 8 + wave) * 2 + 1] = se;
          if (wave == 0) {
            bk2[n] = kn2d[kk];
            if constexpr (DK) bk2[SD_NBK + n] = exp2((double)(hi - row) * l2g64);  // gamma^(hi - j)
          }
        }
      }
      __syncthreads();
      // the key's maximum M over the waves' maxima and S = sum of
      // exp(2 (u - M)): lane w < 8 rescales wave w's sum, a sum over the
      // row's 8 lanes and a broadcast give S; then phi_j (one exponential
      // per lane)
#pragma unroll 1
      for (int n = 0; n < nb; ++n) {
        const int w8 = lane & 7;
        const double mw = bst[(n * 8 + w8) * 2];
        double M = mw;
        M = fmax(M, dppd<0xB1>(M));
        M = fmax(M, dppd<0x4E>(M));
        M = fmax(M, dppd<0x141>(M));
        const double S = group_sum_d<8>(bst[(n * 8 + w8) * 2 + 1] * exp(2.0 * (mw - M)));
        if (part == 0) {
          if constexpr (DK) bphi[n * D + j] = bk2[SD_NBK + n] * (sqrt(bk2[n]) * exp(bphi[n * D + j] - M) / sqrt(S));
          else bphi[n * D + j] = sqrt(bk2[n]) * exp(bphi[n * D + j] - M) / sqrt(S);
        }
      }
      __syncthreads();
      ml = rl;
      mh = rh;
#pragma unroll 1
      for (int n = 0; n < nb; ++n) {
        const f16* vrow = VR + next_key(ml, mh) * L_::VS;
#pragma unroll
        for (int v = 0; v < VPW; ++v) {
          const double vv = (double)(float)vrow[16 * (vt0 + v) + r16];
#pragma unroll
          for (int i = 0; i < 4; ++i) sum[v][i] += bphi[n * D + 16 * ft + 4 * g4 + i] * vv;
        }
        if (vt0 == 0) zsum += bphi[n * D + 16 * ft + r16];
      }
    }
  }
  float* dst = a.dS + ((size_t)unit * a.NS + s) * (D * D + D);
#pragma unroll
  for (int v = 0; v < VPW; ++v) {
    const int vt = vt0 + v;
    const f32x4 o = {(float)sum[v][0], (float)sum[v][1], (float)sum[v][2], (float)sum[v][3]};
    *reinterpret_cast<f32x4*>(dst + ((size_t)(2 * (vt * (D / 32) + (ft >> 1)) + (ft & 1)) * 64 + lane) * 4) = o;
  }
  if (vt0 == 0 && g4 == 0) dst[D * D + 16 * ft + r16] = (float)zsum;
}

// ----------------------------------------------------- 5. state_scan ----
// Exclusive prefix over the super-chunk deltas, in place (the starting state
// of every super-chunk), and their total, the exported state S (row-major)
// and z, each rounded to float32 once from a float64 running sum.
// Part bx of the scan for unit (blockIdx.y, blockIdx.z): 256 of the D*D + D
// state entries.
template <int D, bool DK>
__device__ __forceinline__ void state_scan_part(const PrefillArgs& a, int bx) {
  float* dS = a.dS;
  const int NS = a.NS;
  constexpr int n_elem = D * D + D;
  const int e = bx * 256 + threadIdx.x;
  if (e >= n_elem) return;
  const int unit = blockIdx.y + gridDim.y * blockIdx.z;
  float* base = dS + (size_t)unit * NS * n_elem + e;
  // forget gate: super-chunk s's delta is held at the end hi_s of its key
  // range and the running sum at the start lo_s = hi_{s-1}, so it moves on
  // by gamma^(hi_s - lo_s) before the delta is added
  const double l2g = DK ? log2((double)a.decay[blockIdx.y]) : 0.0;
  auto key_end = [&](int s2) {
    return (s2 == NS - 1 ? full_chunks_before(a.T - 1, a.W, a.C) : full_chunks_before(s2 * a.K + a.K, a.W, a.C)) *
           a.C;
  };
  double run = 0.0;  // float64 running sum: one float32 rounding per start
  constexpr int NB = 32;  // loads of a batch in flight together (indices
                          // past the end re-read the last entry, unused)
  for (int s0 = 0; s0 < NS; s0 += NB) {
    float x[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) x[i] = base[(size_t)min(s0 + i, NS - 1) * n_elem];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (s0 + i < NS) {
        base[(size_t)(s0 + i) * n_elem] = (float)run;
        if constexpr (DK) {
          const int s2 = s0 + i, lo_s = full_chunks_before(s2 * a.K, a.W, a.C) * a.C;
          run *= exp2((double)(key_end(s2) - lo_s) * l2g);
        }
        run += (double)x[i];
      }
  }
  char* st = a.state + (size_t)unit * a.st_unit;
  if (e < D * D) {
    // fragment-linear index ((2p + h) * 64 + lane) * 4 + i, pair p = vt *
    // (D/32) + bb, lane = 16g + r: S[32bb + 16h + 4g + i][16vt + r]
    const int i = e & 3, ln = (e >> 2) & 63, ph = e >> 8;
    const int h = ph & 1, p = ph >> 1, vt = p / (D / 32), bb = p % (D / 32);
    const int row = 32 * bb + 16 * h + 4 * (ln >> 4) + i, col = 16 * vt + (ln & 15);
    reinterpret_cast<float*>(st + a.st_S)[row * D + col] = (float)run;
  } else {
    reinterpret_cast<float*>(st + a.st_z)[e - D * D] = (float)run;
  }
}

// The scan (workgroups x < n_scan) and the decode-state export (the rest,
// x - n_scan as the export's workgroup index) in one launch: the export
// depends only on the selection and the inputs, so it runs beside the scan
// instead of after the attention walk.
template <typename T, int D>
__device__ void export_part(const PrefillArgs& a, int x);
template <typename T, int D, bool DK = false>
__global__ __launch_bounds__(256) void state_scan_kernel(PrefillArgs a, int n_scan) {
  if ((int)blockIdx.x < n_scan)
    state_scan_part<D, DK>(a, (int)blockIdx.x);
  else
    export_part<T, D>(a, (int)blockIdx.x - n_scan);
}

// ---------------------------------------------------------- 6. attend ----
// One workgroup per (super-chunk, kv head x head group, batch row); 8 waves,
// each owning one 16-query row tile (one head, 16 positions), so a
// workgroup holds at most 8 row tiles (head groups split the heads of a kv
// head across workgroups). Workgroups are ordered so that consecutive ids of
// one (batch, kv head, head group) unit share an XCD (ids are dealt to the 8
// XCDs round robin), keeping that unit's kept pool, F^T and state in one L2.
// For each chunk of the super-chunk, in order:
//  * phi(Q) and the state readout S^T phi(Q)^T, z . phi(q): the linear
//    state enters as one virtual key of weight g*z.phi(q) and value
//    S^T phi(q) / z.phi(q) [P3 "NP-Map ..."];
//  * kept-pool keys below the band (all visible) [P2 固定预算路由];
//  * band keys from the first chunk not yet folded to the chunk's end: a key
//    is softmax-visible if it is in the window, in the query's own chunk or
//    kept; otherwise (decided, unkept, out of the window) it is a linear key
//    with weight g <phi(q), phi(k)>;
//  * every weight enters one running max / sum in the log domain (reading:
//    a single normaliser over softmax and gated linear weights);
//  * the next chunk's newly folded tokens are added to the state.
// Precision: logits from exact bf16 products; the readout as one fp16
// product of S with rows scaled by 1/z_i against z_i phi(q)_i / z.phi(q)
// (both bounded, see the readout); <phi(k),phi(q)> with both features in
// fp16 (all terms are positive, so the relative error stays within 2^-11);
// softmax weights and values in fp16 (11-bit significands, bf16 values
// exact), the weights below 2^8 by the lazily moved offset.
// A wave holds HPW heads of one 16-query tile: the key, value and phi(K)
// fragments it reads from LDS serve every head it holds.
// PART: the two branches kept apart. The wave's two head slots then hold one
// query head twice: slot 0 accumulates the softmax branch alone (the kept,
// window and own-chunk keys), slot 1 the linear branch alone (linear keys and
// the state, without the gate); the output is their merge (the single
// normaliser, or the sum y_SA + g y_LA), and the branch partials (normalised
// outputs and natural-log normalisers) are written when asked for.
template <typename T, int D, int HPW, bool PART = false, bool DK = false>
__global__ __launch_bounds__(512) void attend_kernel(PrefillArgs a) {
  static_assert(!PART || HPW == 2, "the separate-branch walk uses both head slots");
  using B_ = Blk<T, D>;
  typedef typename HalfOf<T>::type H;
  extern __shared__ __align__(16) char smem[];
  const BlkPtr<T, D> P(smem);
  // XCD-grouped order: logical id = xcd * (n / 8) + (id / 8)
  const int n_units = a.Hkv * a.nHG * a.B;
  const int n_wg = a.NS * n_units;
  int id = blockIdx.x;
  if ((n_wg & 7) == 0) id = (id & 7) * (n_wg >> 3) + (id >> 3);
  // super-chunks in descending order: later ones walk larger kept pools and
  // take longer, so the longest start first and the short ones fill in
  const int s = a.NS - 1 - id % a.NS;
  const int u3 = id / a.NS;  // (b, kv, hg)
  const int hg = u3 % a.nHG, kv = (u3 / a.nHG) % a.Hkv, b = u3 / (a.nHG * a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // in an SGPR
  const int L = a.L, C = a.C, W = a.W;
  const int unit = b * a.Hkv + kv;
  const uint32_t kv_bytes = (uint32_t)((size_t)L * D * sizeof(T));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(reinterpret_cast<const T*>(a.k) + (size_t)unit * L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(reinterpret_cast<const T*>(a.v) + (size_t)unit * L * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t sfr = make_rsrc(a.selflag + (size_t)unit * L, (uint32_t)L);
  const int32_t* selu = a.sel + (size_t)unit * a.n_dec * a.lam;
  const __amdgpu_buffer_rsrc_t selr = make_rsrc(selu, (uint32_t)((size_t)a.n_dec * a.lam * 4));
  load_ft<T, D, 512>(P, reinterpret_cast<const T*>(a.ft) + (size_t)kv * D * D);
  const int n_qt = C / 16;
  constexpr int RH = PART ? 1 : HPW;  // query heads per wave
  const bool act = wave < (a.Gs / RH) * n_qt;  // wave-uniform
  const int hl = act ? wave / n_qt : 0, qt = act ? wave % n_qt : 0;
  // log-weights are kept in base 2: logits times scale * log2(e), linear
  // weights log2(g) + log2 <phi(q), phi(k)>
  const float scale2 = a.scale * STILL_LOG2E;
  int hh[HPW];
  float gg[HPW], lgate2[HPW];
  __amdgpu_buffer_rsrc_t qr[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    hh[j] = kv * a.G + hg * a.Gs + (PART ? hl : hl * HPW + j);
    gg[j] = a.softmax_only ? 0.f : a.gate[hh[j]];
    if constexpr (PART) gg[j] = j == 0 ? 0.f : 1.f;  // slot 0: no linear key; slot 1: gate-free
    lgate2[j] = gg[j] > 0.f ? log2_acc<T>(gg[j]) : STILL_NEG_INF;
    qr[j] = make_rsrc(reinterpret_cast<const T*>(a.q) + ((size_t)(b * a.Hq + hh[j]) * L) * D, kv_bytes);
  }
  // forget gate of the linear state (0: none), base 2
  const float l2g = DK ? log2f(a.decay[kv]) : 0.f;
  // the output gates of the wave's heads (only read with a.out_gate)
  __amdgpu_buffer_rsrc_t gr[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j)
    gr[j] = make_rsrc(a.out_gate ? reinterpret_cast<const T*>(a.out_gate) + ((size_t)(b * a.Hq + hh[j]) * L) * D
                                 : nullptr,
                      a.out_gate ? kv_bytes : 0u);

  const float* Sst = a.dS + ((size_t)unit * a.NS + s) * (D * D + D);
  load_state<T, D>(P, Sst);
  if (tid < D) P.zs[tid] = (double)Sst[D * D + tid];

  const int c_begin = s * a.K;
  const int c_end = min(c_begin + a.K, a.T);
  for (int c = c_begin; c < c_end; ++c) {
    __syncthreads();
    const int lane = opaque_tid() & 63, r16 = lane & 15, g4 = lane >> 4;  // see opaque_tid
    const int cC = c * C;
    const bool fold = c + 1 < c_end;
    const int cf = full_chunks_before(c, W, C);
    const int fold_lo = cf * C;
    const int fold_hi = fold ? full_chunks_before(c + 1, W, C) * C : fold_lo;
    const int band_lo = cf * C;
    const int band_hi = min(cC + C, L);
    const int n_oob = pool_count_at(cf, a.lam, a.cap_chunks);
    const int t = cC + 16 * qt + r16;

    // kept-pool positions of the chunk: gather indices of the pool blocks
    for (int i = tid; i < min(n_oob, B_::PCAP); i += 512) P.pidx[i] = selu[i];

    // query fragments, phi(q) (F^T from LDS), state readout
    Frag<T> qf[HPW][D / 32];
    Frag<H> pq[HPW][D / 32];  // phi(q) as H for <phi(k), phi(q)> (linear blocks)
#pragma unroll
    for (int j = 0; j < HPW; ++j)
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)
        qf[j][kb] = ld_frag_buf_p<T, CPOL_NT>(qr[j], act ? (uint32_t)(t * D + 8 * g4) * sizeof(T) : kv_bytes,
                                              32 * kb * sizeof(T));  // read once
    // the first band block's loads are in flight during the readout (issued
    // after the query loads: waits on those then leave them outstanding)
    BlkRegs<T, D, 512> R;
    issue_block<T, D, 512>(R, kr, vr, kv_bytes, sfr, blk_range(band_lo, band_hi));
    f32x4 O[HPW][D / 16];
    float mrun[HPW];
    f32x4 lacc[HPW];  // running sums, the same in all four entries (ones-row MFMA)
    {
      // Readout o = S^T phi(q) / dz, dz = z . phi(q). 16-bit data: one fp16
      // MFMA per tile on a rescaled pair, row i of S times 1/z_i and phi(q)_i
      // times z_i / dz. |S_ij| <= z_i max|v| (S and z sum the same
      // non-negative features), so the scaled state is bounded by the largest
      // value magnitude and the scaled features are weights in [0, 1] that
      // sum to 1: both sit well inside fp16, and each product carries about
      // 2^-10 relative error. float32 data: the float32 MFMA on S and phi(q).
      [[maybe_unused]] Frag<H> pz[HPW][D / 32];
      [[maybe_unused]] Frag<T> phq[HPW][D / 32];
      float dz[HPW];
      {
        f32x4 ph[HPW][D / 16];
        np_map_tiles<T, D, HPW>(P, qf, ph);
#pragma unroll
        for (int j = 0; j < HPW; ++j)
#pragma unroll
          for (int bb = 0; bb < D / 32; ++bb) {
            pq[j][bb] = frag_from<H>(ph[j][2 * bb], ph[j][2 * bb + 1]);
            if constexpr (sizeof(T) == 4) phq[j][bb] = frag_from<T>(ph[j][2 * bb], ph[j][2 * bb + 1]);
          }
        float z_[HPW];
#pragma unroll
        for (int j = 0; j < HPW; ++j) z_[j] = 0.f;
#pragma unroll
        for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float zi = (float)P.zs[16 * ft + 4 * g4 + i];
#pragma unroll
            for (int j = 0; j < HPW; ++j) {
              ph[j][ft][i] *= zi;  // z_i phi(q)_i
              z_[j] += ph[j][ft][i];
            }
          }
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          dz[j] = sum_over_g(z_[j]);
          if constexpr (sizeof(T) == 2) {
            const float inv = dz[j] > 0.f ? 1.f / dz[j] : 0.f;
#pragma unroll
            for (int bb = 0; bb < D / 32; ++bb) pz[j][bb] = frag_from<H>(ph[j][2 * bb] * inv, ph[j][2 * bb + 1] * inv);
          }
        }
      }
      if constexpr (sizeof(T) == 2) {
        // 1/z_i per state row (kmax is scratch of block_phi, free here)
        if (tid < D) {
          const double z = P.zs[tid];
          P.kmax[tid] = z > 0.0 ? (float)(1.0 / z) : 0.f;
        }
        __syncthreads();
        // the scaled state as fp16 fragments, split once and shared by
        // every wave (the region of the key / value blocks is free here)
        H* RSh = reinterpret_cast<H*>(P.RS);
        for (int e = tid; e < B_::NPAIR * 64; e += 512) {
          const int pl = e >> 6, ln = e & 63, g = ln >> 4, bb = pl % (D / 32);
          const float* sp = P.SP + ((size_t)2 * pl * 64 + ln) * 4;
          f32x4 x0 = *reinterpret_cast<const f32x4*>(sp), x1 = *reinterpret_cast<const f32x4*>(sp + 256);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x0[i] *= P.kmax[32 * bb + 4 * g + i];
            x1[i] *= P.kmax[32 * bb + 16 + 4 * g + i];
          }
          st_frag(RSh + ((size_t)pl * 64 + ln) * 8, frag_from<H>(x0, x1));
        }
        __syncthreads();
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
          for (int j = 0; j < HPW; ++j) O[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int bb = 0; bb < D / 32; ++bb) {
            const Frag<H> sf = ld_frag(RSh + ((size_t)(dt * (D / 32) + bb) * 64 + lane) * 8);
#pragma unroll
            for (int j = 0; j < HPW; ++j) mma(O[j][dt], sf, pz[j][bb]);
          }
        }
        lds_mfma_pipeline<2 * (D / 32), (D / 16 - 2) * (D / 32), HPW, 1, 2 * (D / 32) * HPW>();
      } else {
        // float32 S fragments straight from the state region
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
          for (int j = 0; j < HPW; ++j) O[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int bb = 0; bb < D / 32; ++bb) {
            const int pl = dt * (D / 32) + bb;
            const Frag<T> sf = frag_from<T>(*reinterpret_cast<const f32x4*>(P.pair(pl, 0)),
                                            *reinterpret_cast<const f32x4*>(P.pair(pl, 1)));
#pragma unroll
            for (int j = 0; j < HPW; ++j) mma(O[j][dt], sf, phq[j][bb]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        if (gg[j] > 0.f && dz[j] > 0.f) {
          // the state is held at band_lo: the forget gate weights it
          // gamma^(t - band_lo) at this query
          mrun[j] = log2_acc<T>(gg[j] * dz[j]);
          if constexpr (DK) mrun[j] += (float)(t - band_lo) * l2g;
          lacc[j] = f32x4{1.f, 1.f, 1.f, 1.f};
          if constexpr (sizeof(T) == 4) {
            const float inv = 1.f / dz[j];
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) O[j][dt] *= inv;
          }
        } else {
          mrun[j] = STILL_NEG_INF;
          lacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) O[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }

    // key blocks: the band first (linear-attention weights, fold), then the
    // kept pool below the band
    const int n_pool_blk = (n_oob + 63) / 64;
    const int n_band_blk = (band_hi - band_lo + 63) / 64;
    // softmax / linear weights of one block in LDS folded into (m, l, O)
    auto attend_block = [&](const bool is_pool, const int blo, const int nvalid, const bool la_blk)
                            __attribute__((always_inline)) {
      // region bases made opaque again per block: the per-lane fragment
      // addresses are then recomputed here instead of held across the loop
      const int lane = opaque_tid() & 63, r16 = lane & 15, g4 = lane >> 4;
      BlkPtr<T, D> Pb = P;
      Pb.Ks = lds_opaque_v(P.Ks);
      Pb.VTs = lds_opaque_v(P.VTs);
      Pb.WF = lds_opaque_v(P.WF);
      const uint64_t selbits = ((uint64_t)P.selw[1] << 32) | P.selw[0];
      // QK^T of the block; the schedule keeps the key fragment reads two
      // 16-key tiles ahead of their MFMAs, so their LDS latency is covered
      f32x4 st[HPW][4];
      Frag<T> kf[4][D / 32];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) kf[kt][kb] = ld_frag(Pb.Ks + (16 * kt + r16) * B_::KS + 32 * kb + 8 * g4);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int j = 0; j < HPW; ++j) st[j][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
#pragma unroll
          for (int j = 0; j < HPW; ++j) mma(st[j][kt], kf[kt][kb], qf[j][kb]);
      }
      if constexpr (sizeof(T) == 2) lds_mfma_pipeline<2 * (D / 32), 2 * (D / 32), HPW, 1, 2 * HPW * (D / 32)>();
      // st holds raw logits (scaled into the base-2 domain inside the
      // exponential); linear keys hold their log-weight / scale2, masked
      // keys -inf. scale2 > 0, so the row maximum commutes with the scaling.
      float mx[HPW];
#pragma unroll
      for (int j = 0; j < HPW; ++j) mx[j] = STILL_NEG_INF;
      if constexpr (PART) {  // slot 1 (the linear branch) takes no kept key
        if (is_pool)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) st[1][kt] = f32x4{STILL_NEG_INF, STILL_NEG_INF, STILL_NEG_INF, STILL_NEG_INF};
      }
      if (is_pool) {
        if (nvalid < 64) {  // uniform: only a last, partial pool block is masked
          const uint64_t v_s = low_bits(nvalid) >> (4 * g4);
#pragma unroll
          for (int j = 0; j < HPW; ++j)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                st[j][kt][i] = ((v_s >> (16 * kt + i)) & 1ull) ? st[j][kt][i] : STILL_NEG_INF;
        }
      } else {
        // per-lane key masks (bit kk = key blo + kk): visible keys are those
        // up to the query; softmax-visible ones are in the window / own
        // chunk or kept; the rest of the visible ones are linear
        const uint64_t valid_m = low_bits(min(nvalid, t - blo + 1));
        const uint64_t sa_m = valid_m & (~low_bits(min(t - W + 1, cC) - blo) | selbits);
        const uint64_t sa_s = sa_m >> (4 * g4), la_s = (valid_m & ~sa_m) >> (4 * g4);
        const float inv_scale2 = 1.f / scale2;
        f32x4 wt[HPW][4];
        if (la_blk) {
          // <phi(k), phi(q)> of every key and row: each phi(K) fragment read
          // serves all heads of the wave
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int j = 0; j < HPW; ++j) wt[j][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int bb = 0; bb < D / 32; ++bb) {
              const Frag<H> wk = Pb.ld_wk(kt, bb, lane);
#pragma unroll
              for (int j = 0; j < HPW; ++j) mma(wt[j][kt], wk, pq[j][bb]);
            }
          }
          // one key tile ahead (two transposing reads per fragment)
          if constexpr (sizeof(T) == 2) lds_mfma_pipeline<2 * (D / 32), 3 * (D / 32), HPW, 2, HPW * (D / 32)>();
        }
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = ((sa_s >> (16 * kt + i)) & 1ull) && !(PART && j == 1) ? st[j][kt][i] : STILL_NEG_INF;
              if (la_blk) {
                const float w = wt[j][kt][i];
                const bool la = ((la_s >> (16 * kt + i)) & 1ull) && w > 0.f;
                if constexpr (DK)
                  x = la ? (lgate2[j] + log2_acc<T>(fmax_nn(w, 1e-37f)) +
                            (float)(t - (blo + 16 * kt + 4 * g4 + i)) * l2g) * inv_scale2
                         : x;
                else
                  x = la ? (lgate2[j] + log2_acc<T>(fmax_nn(w, 1e-37f))) * inv_scale2 : x;
              }
              st[j][kt][i] = x;
            }
        }
      }
#pragma unroll
      for (int j = 0; j < HPW; ++j)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          mx[j] = fmax_nn(mx[j], fmax_nn(fmax_nn(st[j][kt][0], st[j][kt][1]), fmax_nn(st[j][kt][2], st[j][kt][3])));
      // the first value tile is read while the weights are formed
      Frag<H> vf[D / 16][2];
      vf[0][0] = Pb.ld_v(0, 0, lane);
      vf[0][1] = Pb.ld_v(0, 1, lane);
      // weights as H hi + lo parts (fp16: ~22 significant bits; one fp16
      // part alone moves y by up to 2^-12 of the value spread)
      Frag<H> pf[HPW][2], pl[HPW][2];
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const float mxj = max_over_g(mx[j]) * scale2;
        // The offset m is moved only when some row's block maximum passes it
        // by more than 2^RESCALE_SLACK (wave-uniform test): weights then stay
        // below 2^8, well inside fp16, and O and l are rescaled on few blocks
        // instead of on almost every one. y = O / l does not depend on m.
        // Rows with nothing visible so far keep m = -inf, O = 0, l = 0; the
        // exponent's offset is finite either way (exp2(-inf) = 0).
        constexpr float RESCALE_SLACK = 8.f;
        if (__builtin_amdgcn_ballot_w64(mxj > mrun[j] + RESCALE_SLACK)) {
          const float mn = fmax_nn(mrun[j], mxj);
          const float al = mrun[j] == STILL_NEG_INF ? 0.f : exp2_acc<T>(mrun[j] - mn);
          mrun[j] = mn;
          lacc[j] *= al;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) O[j][dt] *= al;
        }
        const float nmn = mrun[j] == STILL_NEG_INF ? 0.f : -mrun[j];
        f32x4 pv[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[kt][i] = exp2_acc<T>(fmaf(st[j][kt][i], scale2, nmn));
        // weights as H; the running sum comes from the same rounded weights
        // through a ones-row MFMA
        split2_frag<H>(pv[0], pv[1], pf[j][0], pl[j][0]);
        split2_frag<H>(pv[2], pv[3], pf[j][1], pl[j][1]);
        const Frag<H> one = ones_frag<H>();
        mma(lacc[j], one, pf[j][0]);
        mma(lacc[j], one, pf[j][1]);
        if constexpr (sizeof(H) == 2) {
          mma(lacc[j], one, pl[j][0]);
          mma(lacc[j], one, pl[j][1]);
        }
      }
#pragma unroll
      for (int dt = 1; dt < D / 16; ++dt) {
        vf[dt][0] = Pb.ld_v(dt, 0, lane);
        vf[dt][1] = Pb.ld_v(dt, 1, lane);
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          mma(O[j][dt], vf[dt][0], pf[j][0]);
          mma(O[j][dt], vf[dt][1], pf[j][1]);
          if constexpr (sizeof(H) == 2) {
            mma(O[j][dt], vf[dt][0], pl[j][0]);
            mma(O[j][dt], vf[dt][1], pl[j][1]);
          }
        }
      // value tiles 1 and 2 first (tile 0 is in flight), then each tile's
      // MFMAs with the reads of the tile three ahead (two transposing reads
      // per fragment)
      if constexpr (sizeof(T) == 2) lds_mfma_pipeline<8, 2 * (D / 16 - 3), 2 * HPW, 2, 3 * 4 * HPW>();
    };
    auto issue_pool = [&](int pb) __attribute__((always_inline)) {
      const int blo = 64 * pb;
      BlkSrc src{};
      src.mode = blo + 64 <= B_::PCAP ? 1 : 2;  // positions staged in LDS, else global
      src.lds = P.pidx;
      src.glist = selr;
      src.first = blo;
      src.n = min(64, n_oob - blo);
      issue_block<T, D, 512>(R, kr, vr, kv_bytes, sfr, src);
    };
    // one stream of blocks, the band's then the pool's: block i + 1 is
    // issued as soon as block i is in LDS, so its loads are in flight while
    // block i is used. The band blocks below the chunk (linear weights, the
    // only users of phi(q) after the readout) come first, in a loop of their
    // own, so phi(q) is not held through the rest.
    const int nblk = n_band_blk + n_pool_blk;
    const int n_la_blk = min(n_band_blk, max(0, (cC - band_lo + 63) / 64));
    auto process = [&](int i, auto la_phase) __attribute__((always_inline)) {
      constexpr bool LA = decltype(la_phase)::value;
      const bool band = i < n_band_blk;  // uniform
      const int blo = band ? band_lo + 64 * i : 64 * (i - n_band_blk);
      __syncthreads();  // the previous block (or the readout) is done with LDS
      commit_block<T, D, 512>(P, R, band ? fold_lo : 0, band ? fold_hi : 0, band);
      if (i + 1 < n_band_blk)
        issue_block<T, D, 512>(R, kr, vr, kv_bytes, sfr, blk_range(blo + 64, band_hi));
      else if (i + 1 < nblk)
        issue_pool(i + 1 - n_band_blk);
      __syncthreads();
      const bool la_blk = LA && band && blo < cC;
      const bool do_fold = band && fold && blo < fold_hi;
      if (la_blk || do_fold) {
        f32x4 phk[4];
        block_phi<T, D>(P, phk, la_blk);  // WF is complete on return
        // the fold writes only SP / zs, which this chunk no longer reads;
        // with the forget gate the state moves from blo to the block's
        // end re (factor gamma^(re - blo)) and key j enters at gamma^(re - j)
        if (do_fold) {
          const int re = min(blo + 64, fold_hi);
          if constexpr (DK) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
              for (int i = 0; i < 4; ++i) phk[kt][i] *= exp2f((float)(re - (blo + 16 * kt + 4 * g4 + i)) * l2g);
            block_fold<T, D, true>(P, phk, exp2f((float)(re - blo) * l2g));
          } else {
            block_fold<T, D>(P, phk);
          }
        }
      }
      // one call site, whatever the block (the accumulators then stay in
      // place); idle waves run it too on a copy of wave 0's rows and store
      // nothing
      attend_block(!band, blo, min(64, (band ? band_hi : n_oob) - blo), la_blk);
    };
    for (int i = 0; i < n_la_blk; ++i) process(i, std::true_type{});
    for (int i = n_la_blk; i < nblk; ++i) process(i, std::false_type{});

    if constexpr (PART) {
      // the branch outputs and their natural-log normalisers (base-2 log of
      // the weight sum plus the offset, times ln 2), then the merge
      const float l0 = lacc[0][0], l1 = lacc[1][0];
      const float lse_sa = l0 > 0.f ? (mrun[0] + log2_acc<T>(l0)) * 0.6931471805599453f : STILL_NEG_INF;
      const float lse_la = l1 > 0.f ? (mrun[1] + log2_acc<T>(l1)) * 0.6931471805599453f : STILL_NEG_INF;
      const float i0 = l0 > 0.f ? 1.f / l0 : 0.f, i1 = l1 > 0.f ? 1.f / l1 : 0.f;
      const float g = a.gate[hh[0]];
      // single normaliser: y = a y_SA + (1 - a) y_LA, a = Z / (Z + g D);
      // sum merge: y = y_SA + g y_LA
      float w_sa = 1.f, w_la = 0.f;
      if (a.merge_sum) {
        w_la = g;
      } else if (g > 0.f && lse_la != STILL_NEG_INF) {
        const float r = exp_acc<T>(log_acc<T>(g) + lse_la - lse_sa);  // g D / Z
        w_sa = 1.f / (1.f + r);
        w_la = r * w_sa;
      }
      if (act && t < L) {
        const size_t ob = ((size_t)(b * a.Hq + hh[0]) * L + t) * D;
        const size_t orow = (size_t)(b * a.Hq + hh[0]) * L + t;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const f32x4 ys = O[0][dt] * i0, yl = O[1][dt] * i1;
          f32x4 y = ys * w_sa + yl * w_la;
          const int col = 16 * dt + 4 * g4;
          if (a.out_gate) y *= sigmoid_gate4<T>(gr[0], (uint32_t)(t * D + col) * sizeof(T));
          if (sizeof(T) == 4 || a.fp32_out) {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + ob + col) = y;
          } else {
            bf16 y4[4] = {(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
            *reinterpret_cast<uint2*>(reinterpret_cast<bf16*>(a.out) + ob + col) = *reinterpret_cast<uint2*>(y4);
          }
          if (a.y_sa) *reinterpret_cast<f32x4*>(a.y_sa + ob + col) = ys;
          if (a.y_la) *reinterpret_cast<f32x4*>(a.y_la + ob + col) = yl;
        }
        if (g4 == 0) {
          if (a.lse_sa) a.lse_sa[orow] = lse_sa;
          if (a.lse_la) a.lse_la[orow] = lse_la;
        }
      }
      continue;
    }
    // outputs: normalise; bf16 rows go through LDS for full-line stores
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const float inv = 1.f / lacc[j][0];
      const size_t ob = ((size_t)(b * a.Hq + hh[j]) * L) * D;
      if constexpr (sizeof(T) == 2) {
        if (!a.fp32_out) {
          if (j == 0) __syncthreads();  // Ks / VTs are free again
          constexpr int OS = D + 8;  // padded row, elements
          bf16* tile = reinterpret_cast<bf16*>(smem) + (size_t)wave * 16 * OS;
          if (act) {
            // wave-local: the tile is written and read by this wave only
            auto wave_sync = [] {
              __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
              __builtin_amdgcn_wave_barrier();
              __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            };
            if (j > 0) wave_sync();  // the previous head's rows are read
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
              f32x4 y = O[j][dt] * inv;
              if (a.out_gate) y *= sigmoid_gate4<T>(gr[j], (uint32_t)(t * D + 16 * dt + 4 * g4) * sizeof(T));
              bf16 y4[4] = {(bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
              *reinterpret_cast<uint2*>(tile + r16 * OS + 16 * dt + 4 * g4) = *reinterpret_cast<uint2*>(y4);
            }
            wave_sync();
            constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
            for (int it = 0; it < 16 * CPR / 64; ++it) {
              const int e = it * 64 + lane, row = e / CPR, ch = e % CPR;
              const int tr = cC + 16 * qt + row;
              if (tr < L)
                __builtin_nontemporal_store(  // written once
                    *reinterpret_cast<const u32x4*>(tile + row * OS + 8 * ch),
                    reinterpret_cast<u32x4*>(reinterpret_cast<bf16*>(a.out) + ob + (size_t)tr * D + 8 * ch));
            }
          }
        } else if (act && t < L) {
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) {
            f32x4 y = O[j][dt] * inv;
            if (a.out_gate) y *= sigmoid_gate4<T>(gr[j], (uint32_t)(t * D + 16 * dt + 4 * g4) * sizeof(T));
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + ob + (size_t)t * D + 16 * dt + 4 * g4) = y;
          }
        }
      } else if (act && t < L) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          f32x4 y = O[j][dt] * inv;
          if (a.out_gate) y *= sigmoid_gate4<T>(gr[j], (uint32_t)(t * D + 16 * dt + 4 * g4) * sizeof(T));
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + ob + (size_t)t * D + 16 * dt + 4 * g4) = y;
        }
      }
    }
  }
}

// ---------------------------------------------------------- 7. export ----
// Decode state after the prefill: ring slots of the last R positions (keys,
// values, NP-Map features, kept flags), the kept pool, and the position
// (workgroups of the scan launch, see state_scan_kernel).
template <typename T, int D>
__device__ void export_part(const PrefillArgs& a, int x) {
  extern __shared__ __align__(16) char smem[];
  const int kv = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, L = a.L, R = a.R;
  const int unit = b * a.Hkv + kv;
  char* st = a.state + (size_t)unit * a.st_unit;
  const T* kg = reinterpret_cast<const T*>(a.k) + (size_t)unit * L * D;
  const T* vg = reinterpret_cast<const T*>(a.v) + (size_t)unit * L * D;
  constexpr int VEC = 16 / sizeof(T), CPR = D / VEC;  // 16-byte chunks per row
  const int ring_lo = L - R > 0 ? L - R : 0;
  const int n_ring_grp = (L - ring_lo + 63) / 64;
  if (x < n_ring_grp) {
    // 64 ring keys per workgroup, 16 per wave: NP-Map [P3 "NP-Map:
    // Norm-Preserving Feature Map"] by MFMA against F^T (fragment order, in
    // LDS), keys, values and kept flags copied to their slots
    BlkPtr<T, D> P(smem);
    P.FT = lds_opaque(reinterpret_cast<T*>(smem));
    load_ft<T, D, 256>(P, reinterpret_cast<const T*>(a.ft) + (size_t)kv * D * D);
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = lane >> 4;
    const uint32_t kv_bytes = (uint32_t)((size_t)L * D * sizeof(T));
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kg, kv_bytes);
    const int p = ring_lo + 64 * x + 16 * wave + r16;  // key row of lane (r, g)
    Frag<T> xf[D / 32];
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      xf[kb] = ld_frag_buf<T>(kr, p < L ? (uint32_t)((p * D + 8 * g4) * sizeof(T)) : kv_bytes,
                              32 * kb * sizeof(T));
    __syncthreads();  // F^T in LDS
    f32x4 ph[D / 16];
    np_map_tile<T, D>(P, xf, ph);
    T* rk = reinterpret_cast<T*>(st + a.st_ring_k);
    T* rv = reinterpret_cast<T*>(st + a.st_ring_v);
    T* rp = reinterpret_cast<T*>(st + a.st_ring_phi);
    int32_t* rf = reinterpret_cast<int32_t*>(st + a.st_ring_flag);
    if (p < L) {
      const int slot = p % R;
#pragma unroll
      for (int ft = 0; ft < D / 16; ++ft) {
        T w4[4] = {from_f32<T>(ph[ft][0]), from_f32<T>(ph[ft][1]), from_f32<T>(ph[ft][2]),
                   from_f32<T>(ph[ft][3])};
        T* dst = rp + (size_t)slot * D + 16 * ft + 4 * g4;
        if constexpr (sizeof(T) == 2) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<uint2*>(w4);
        else *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<uint4*>(w4);
      }
      if (g4 == 0) rf[slot] = a.selflag[(size_t)unit * L + p];
    }
    for (int e = tid; e < 64 * CPR; e += 256) {
      const int r = e / CPR, c = (e % CPR) * VEC, q = ring_lo + 64 * x + r;
      if (q >= L) continue;
      const int slot = q % R;
      *reinterpret_cast<uint4*>(rk + (size_t)slot * D + c) = *reinterpret_cast<const uint4*>(kg + (size_t)q * D + c);
      *reinterpret_cast<uint4*>(rv + (size_t)slot * D + c) = *reinterpret_cast<const uint4*>(vg + (size_t)q * D + c);
    }
    return;
  }
  // kept pool rows, 16 per workgroup
  const int n_pool = pool_count_at(a.n_dec, a.lam, a.cap_chunks);
  const int i0 = (x - n_ring_grp) * 16;
  const int32_t* selu = a.sel + (size_t)unit * a.n_dec * a.lam;
  T* pk = reinterpret_cast<T*>(st + a.st_pool_k);
  T* pvv = reinterpret_cast<T*>(st + a.st_pool_v);
  int32_t* pp = reinterpret_cast<int32_t*>(st + a.st_pool_pos);
  for (int e = tid; e < 16 * CPR; e += 256) {
    const int r = e / CPR, c = (e % CPR) * VEC, i = i0 + r;
    if (i >= n_pool) continue;
    const int q = selu[i];
    if (a.pages.base) {  // the row's page of the arena (unmapped: the error word below)
      const long ok = pool_page_off(a.pages, unit, i, 0, D * sizeof(T));
      const long ov = pool_page_off(a.pages, unit, i, 1, D * sizeof(T));
      if (ok >= 0) {
        *reinterpret_cast<uint4*>(a.pages.base + ok + c * sizeof(T)) =
            *reinterpret_cast<const uint4*>(kg + (size_t)q * D + c);
        *reinterpret_cast<uint4*>(a.pages.base + ov + c * sizeof(T)) =
            *reinterpret_cast<const uint4*>(vg + (size_t)q * D + c);
      }
    } else if (sizeof(T) == 2 && a.pool8) {
      // the 8-bit store: the row's CPR lanes (consecutive, aligned) share
      // its largest magnitude; codes of x / 2^e, the exponent bytes after
      // the P rows
      const int P = a.m - a.W;
      const T* kr = kg + (size_t)q * D + c;
      const T* vr = vg + (size_t)q * D + c;
      float km = 0.f, vm = 0.f;
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        km = fmaxf(km, fabsf(to_f32(kr[j])));
        vm = fmaxf(vm, fabsf(to_f32(vr[j])));
      }
      const int ek = e4m3_row_exp(group_max<CPR>(km)), ev = e4m3_row_exp(group_max<CPR>(vm));
      const float rk = pow2_int(-ek), rv = pow2_int(-ev);  // x / 2^e, exact
      uint32_t kc[VEC / 4], vc[VEC / 4];
#pragma unroll
      for (int j = 0; j < VEC / 4; ++j) {
        kc[j] = vc[j] = 0u;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          kc[j] |= e4m3_code(to_f32(kr[4 * j + e2]) * rk) << (8 * e2);
          vc[j] |= e4m3_code(to_f32(vr[4 * j + e2]) * rv) << (8 * e2);
        }
      }
      uint8_t* k8 = reinterpret_cast<uint8_t*>(st + a.st_pool_k);
      uint8_t* v8 = reinterpret_cast<uint8_t*>(st + a.st_pool_v);
#pragma unroll
      for (int j = 0; j < VEC / 4; ++j) {
        *reinterpret_cast<uint32_t*>(k8 + (size_t)i * D + c + 4 * j) = kc[j];
        *reinterpret_cast<uint32_t*>(v8 + (size_t)i * D + c + 4 * j) = vc[j];
      }
      if (c == 0) {
        k8[(size_t)P * D + i] = (uint8_t)(ek + 127);
        v8[(size_t)P * D + i] = (uint8_t)(ev + 127);
      }
    } else {
      *reinterpret_cast<uint4*>(pk + (size_t)i * D + c) = *reinterpret_cast<const uint4*>(kg + (size_t)q * D + c);
      *reinterpret_cast<uint4*>(pvv + (size_t)i * D + c) = *reinterpret_cast<const uint4*>(vg + (size_t)q * D + c);
    }
    if (c == 0) pp[i] = q;
  }
  if (x == n_ring_grp && tid == 0) {
    int64_t* meta = reinterpret_cast<int64_t*>(st + a.st_meta);
    meta[0] = L;
    meta[1] = n_pool;
    int64_t err = 0;
    if (a.pages.base)  // every pool row needs a page of the arena
      for (int i = 0; i < n_pool; i += POOL_PAGE_ROWS)
        if (pool_page_off(a.pages, unit, i, 0, 1) < 0) err = -5;
    meta[2] = err;
    meta[3] = 0;
  }
}

}  // namespace still
