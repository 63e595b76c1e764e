// Decode step of one STILL layer for gfx950: one new token per sequence.
//
// Pages cited (short tag -> page title):
//   [P2] "NeurIPS 2026|层内混合注意力：告别位置「伪混合」，STILL首个内容感知的层内混合注意力架构",
//        sections 亮点一 (固定预算路由, 延迟选择与分块并行)
//   [P3] "STILL: Content-Aware Intra-Layer Hybrid Attention for Efficient
//        LLM Linearization", sections "Content-Aware Routing with Fixed
//        Budget", "Delayed Chunk-Level Selection for Unified
//        Training-Inference Parallelism", "Self-Saliency Score",
//        "NP-Map: Norm-Preserving Feature Map"
//
// The step applies the same routing and memory update as the prefill
// [P3 "Delayed Chunk-Level Selection ..."]. One workgroup (4 waves) per
// (kv head, batch row) unit:
//   1. when a new chunk begins: Top-lambda of the finished chunk over its
//      float64 scores, kept tokens appended to the pool [P2 固定预算路由];
//      the chunk(s) now wholly before the window folded into S, z;
//   2. the new token enters the ring (key, value, NP-Map feature);
//   3. its float64 score joins the undecided chunk's scores;
//   4. every query head of the group attends: softmax over kept tokens
//      below the window and over the window / own-chunk tokens in the ring,
//      gated linear weights over ring tokens already out of the window but
//      not yet folded, and the state S, z as one virtual key; all weights
//      share one normaliser (reading of the branch merge).
#include "still_common.h"

namespace still {

struct DecodeArgs {
  const void* q;  // [B][Hq][D]
  const void* k;  // [B][Hkv][D]
  const void* v;
  const void* fmap_w;  // [Hkv][D][D]
  const float* gate;
  char* state;
  void* out;         // [B][Hq][D]
  int32_t* sel_new;  // [B][Hkv][lam] or null
  int B, Hq, Hkv, G, W, C, m, lam, R, t, boundary, fp32_out, n_keys_max;
  float scale, eps;
  double scale64, eps64;  // the same parameters for the float64 score
  long st_unit, st_S, st_z, st_pool_k, st_pool_v, st_pool_pos, st_ring_k, st_ring_v,
      st_ring_phi, st_ring_flag, st_pending, st_meta;
};

__device__ __forceinline__ float block_sum256(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ float block_max256(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// NP-Map of n rows of xs (float32, stride D) into ph [P3 "NP-Map"]; reading:
// ||x|| * softmax(x F) / ||softmax(x F)||. All 256 threads; us is scratch.
template <typename T, int D>
__device__ __forceinline__ void np_map_rows(const T* F, const float* xs, int n, float* us,
                                            float* ph, float* rowinfo) {
  const int tid = threadIdx.x;
  for (int e = tid; e < n * D; e += 256) {
    const int r = e / D, j = e % D;
    float u = 0.f;
    for (int i = 0; i < D; ++i) u += xs[r * D + i] * to_f32(F[(size_t)i * D + j]);
    us[r * D + j] = u;
  }
  __syncthreads();
  for (int r = tid; r < n; r += 256) {
    float mx = STILL_NEG_INF, xn = 0.f;
    for (int j = 0; j < D; ++j) mx = fmaxf(mx, us[r * D + j]);
    for (int i = 0; i < D; ++i) xn += xs[r * D + i] * xs[r * D + i];
    float ss = 0.f;
    for (int j = 0; j < D; ++j) {
      const float e = expf(us[r * D + j] - mx);
      ss += e * e;
    }
    rowinfo[2 * r] = mx;
    rowinfo[2 * r + 1] = sqrtf(xn) / sqrtf(ss);
  }
  __syncthreads();
  for (int e = tid; e < n * D; e += 256) {
    const int r = e / D;
    ph[e] = expf(us[e] - rowinfo[2 * r]) * rowinfo[2 * r + 1];
  }
  __syncthreads();
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int unit = b * a.Hkv + kv;
  const int G = a.G, W = a.W, C = a.C, R = a.R, t = a.t;
  char* st = a.state + (size_t)unit * a.st_unit;
  int64_t* meta = reinterpret_cast<int64_t*>(st + a.st_meta);
  float* S = reinterpret_cast<float*>(st + a.st_S);
  float* z = reinterpret_cast<float*>(st + a.st_z);
  T* pool_k = reinterpret_cast<T*>(st + a.st_pool_k);
  T* pool_v = reinterpret_cast<T*>(st + a.st_pool_v);
  int32_t* pool_pos = reinterpret_cast<int32_t*>(st + a.st_pool_pos);
  T* ring_k = reinterpret_cast<T*>(st + a.st_ring_k);
  T* ring_v = reinterpret_cast<T*>(st + a.st_ring_v);
  T* ring_phi = reinterpret_cast<T*>(st + a.st_ring_phi);
  int32_t* ring_flag = reinterpret_cast<int32_t*>(st + a.st_ring_flag);
  double* pend = reinterpret_cast<double*>(st + a.st_pending);
  const T* F = reinterpret_cast<const T*>(a.fmap_w) + (size_t)kv * D * D;

  // LDS carve-up
  float* qs = reinterpret_cast<float*>(smem);  // [G][D]
  float* phq = qs + G * D;                      // [G][D]
  float* xs = phq + G * D;                      // [16][D]  rows to map
  float* us = xs + 16 * D;                      // [16][D]  scratch
  float* ph = us + 16 * D;                      // [16][D]  features
  float* vs = ph + 16 * D;                      // [16][D]  values (fold)
  float* rowinfo = vs + 16 * D;                 // [32]
  float* red = rowinfo + 32;                    // [8]
  float* headv = red + 8;                       // [8][4]  per-head scalars
  float* nst = headv + 32;                      // [G][D]  state readout
  float* acc2 = nst + G * D;                    // [256/D][G][D] partial sums
  int* ibuf = reinterpret_cast<int*>(acc2 + 256 * G);    // [C + 8]
  double* d64 = reinterpret_cast<double*>(ibuf + C + 8);  // [G*W + C + 8]
  float* lw = reinterpret_cast<float*>(d64 + G * W + C + 8);  // [G][n_keys_max]
  const int NK = a.n_keys_max;

  if (meta[0] != t || meta[2] != 0) {
    __syncthreads();
    if (tid == 0 && meta[2] == 0) meta[2] = -5;
    return;
  }
  int n_pool = (int)meta[1];
  const int c = t / C, cC = c * C;

  // ---- 1. chunk boundary: decide chunk c-1, append kept, fold -------------
  int lam_c = 0;
  if (a.boundary) {
    double* ps = d64;  // [C]
    int* kept = ibuf;  // [C]
    for (int j = tid; j < C; j += 256) ps[j] = pend[j];
    __syncthreads();
    lam_c = (n_pool + a.lam <= a.m - W) ? a.lam : 0;
    for (int j = tid; j < C; j += 256) {
      int r = 0;
      for (int i = 0; i < C; ++i) r += (ps[i] > ps[j] || (ps[i] == ps[j] && i < j)) ? 1 : 0;
      kept[j] = r < lam_c ? 1 : 0;
    }
    __syncthreads();
    const int base = cC - C;
    for (int j = tid; j < C; j += 256) {
      if (!kept[j]) continue;
      int k2 = 0;
      for (int i = 0; i < j; ++i) k2 += kept[i];
      const int pos = base + j, slot = pos % R, row = n_pool + k2;
      for (int e = 0; e < D; ++e) {
        pool_k[(size_t)row * D + e] = ring_k[(size_t)slot * D + e];
        pool_v[(size_t)row * D + e] = ring_v[(size_t)slot * D + e];
      }
      pool_pos[row] = pos;
      ring_flag[slot] = 1;
      if (a.sel_new) a.sel_new[(size_t)unit * a.lam + k2] = pos;
    }
    if (a.sel_new)
      for (int i = lam_c + tid; i < a.lam; i += 256) a.sel_new[(size_t)unit * a.lam + i] = -1;
    for (int j = tid; j < C; j += 256) pend[j] = __builtin_nan("");
    n_pool += lam_c;
    __syncthreads();

    // fold chunks [cf(c-1), cf(c)) into S, z (float32 features)
    const int f_lo = full_chunks_before(c - 1, W, C) * C;
    const int f_hi = full_chunks_before(c, W, C) * C;
    float dacc[D * D / 256];
    for (int q2 = 0; q2 < D * D / 256; ++q2) dacc[q2] = 0.f;
    float dz = 0.f;
    for (int g0 = f_lo; g0 < f_hi; g0 += 16) {
      const int n = min(16, f_hi - g0);
      for (int e = tid; e < 16 * D; e += 256) {
        const int r = e / D, i = e % D, pos = g0 + r;
        const int slot = pos % R;
        const bool use = r < n && ring_flag[slot] == 0;
        xs[e] = use ? to_f32(ring_k[(size_t)slot * D + i]) : 0.f;
        vs[e] = use ? to_f32(ring_v[(size_t)slot * D + i]) : 0.f;
      }
      __syncthreads();
      np_map_rows<T, D>(F, xs, 16, us, ph, rowinfo);
      for (int q2 = 0; q2 < D * D / 256; ++q2) {
        const int e = tid + 256 * q2, i = e / D, jv = e % D;
        float s = 0.f;
        for (int r = 0; r < 16; ++r) s += ph[r * D + i] * vs[r * D + jv];
        dacc[q2] += s;
      }
      if (tid < D)
        for (int r = 0; r < 16; ++r) dz += ph[r * D + tid];
      __syncthreads();
    }
    if (f_hi > f_lo) {
      for (int q2 = 0; q2 < D * D / 256; ++q2) S[tid + 256 * q2] += dacc[q2];
      if (tid < D) z[tid] += dz;
    }
    __syncthreads();
  } else if (a.sel_new) {
    for (int i = tid; i < a.lam; i += 256) a.sel_new[(size_t)unit * a.lam + i] = -1;
  }

  // ---- 2. the new token enters the ring ------------------------------------
  const T* kin = reinterpret_cast<const T*>(a.k) + (size_t)unit * D;
  const T* vin = reinterpret_cast<const T*>(a.v) + (size_t)unit * D;
  const int slot_t = t % R;
  for (int i = tid; i < D; i += 256) {
    xs[i] = to_f32(kin[i]);
    ring_k[(size_t)slot_t * D + i] = kin[i];
    ring_v[(size_t)slot_t * D + i] = vin[i];
  }
  if (tid == 0) ring_flag[slot_t] = 0;
  for (int e = tid; e < G * D; e += 256) {
    const int hl = e / D, i = e % D;
    qs[e] = to_f32(reinterpret_cast<const T*>(a.q)[((size_t)b * a.Hq + kv * G + hl) * D + i]);
  }
  __syncthreads();
  np_map_rows<T, D>(F, xs, 1, us, ph, rowinfo);
  for (int i = tid; i < D; i += 256) ring_phi[(size_t)slot_t * D + i] = from_f32<T>(ph[i]);

  // ---- 3. float64 score of token t [P3 "Self-Saliency Score"] -------------
  {
    const int lo = t - W + 1 > 0 ? t - W + 1 : 0;
    const int n = t - lo + 1;
    double* lg = d64;  // [G][W]
    for (int p = tid; p < G * n; p += 256) {
      const int hl = p / n, jj = p % n, pos = lo + jj;
      const T* kr = ring_k + (size_t)(pos % R) * D;
      double s = 0.0;
      for (int i = 0; i < D; ++i) {
        const double kx = pos == t ? (double)xs[i] : (double)to_f32(kr[i]);
        s += (double)qs[hl * D + i] * kx;
      }
      lg[hl * W + jj] = a.scale64 * s;
    }
    __syncthreads();
    double* hs = d64 + G * W;
    if (tid < G) {
      const double* x = lg + tid * W;
      double mx = x[0];
      for (int j = 1; j < n; ++j) mx = x[j] > mx ? x[j] : mx;
      double za = 0.0, zo = 0.0;
      for (int j = 0; j < n; ++j) {
        const double e = exp(x[j] - mx);
        za += e;
        if (j != n - 1) zo += e;
      }
      const double p = exp(x[n - 1] - mx) / za, pn = zo / za;
      double sc = 0.0;
      if (p > 0.0) sc += p * log(p / a.eps64);
      if (pn > 0.0) sc += pn * log(pn / (1.0 - a.eps64));
      hs[tid] = sc;
    }
    __syncthreads();
    if (tid == 0) {
      double tot = 0.0;
      for (int h = 0; h < G; ++h) tot += hs[h];
      pend[t - cC] = tot;
    }
  }

  // ---- 4. attention ---------------------------------------------------------
  // phi(q) of each head of the group
  for (int hl = 0; hl < G; ++hl) {
    __syncthreads();
    for (int i = tid; i < D; i += 256) xs[i] = qs[hl * D + i];
    __syncthreads();
    np_map_rows<T, D>(F, xs, 1, us, ph, rowinfo);
    for (int i = tid; i < D; i += 256) phq[hl * D + i] = ph[i];
  }
  __syncthreads();
  int lo = t - W + 1 < cC ? t - W + 1 : cC;
  if (lo < 0) lo = 0;
  // kept tokens below lo: pool positions ascending
  if (tid == 0) ibuf[0] = 0;
  __syncthreads();
  for (int i = tid; i < n_pool; i += 256)
    if (pool_pos[i] < lo) atomicAdd(&ibuf[0], 1);
  __syncthreads();
  const int n_oob = ibuf[0];
  const int n_win = t - lo + 1;
  const int la_lo = full_chunks_before(c, W, C) * C;
  const int la_hi = min(t - W, cC - 1);  // inclusive
  const int n_la = la_hi >= la_lo ? la_hi - la_lo + 1 : 0;
  const int n_keys = n_oob + n_win + n_la;

  // log-weights
  for (int kk = tid; kk < n_keys; kk += 256) {
    if (kk < n_oob + n_win) {
      const T* kr = kk < n_oob ? pool_k + (size_t)kk * D
                               : ring_k + (size_t)((lo + kk - n_oob) % R) * D;
      for (int hl = 0; hl < G; ++hl) {
        float s = 0.f;
        for (int i = 0; i < D; ++i) s += qs[hl * D + i] * to_f32(kr[i]);
        lw[hl * NK + kk] = s * a.scale;
      }
    } else {
      const int pos = la_lo + (kk - n_oob - n_win);
      const int slot = pos % R;
      const bool la = ring_flag[slot] == 0;
      const T* pr = ring_phi + (size_t)slot * D;
      for (int hl = 0; hl < G; ++hl) {
        float w = 0.f;
        for (int i = 0; i < D; ++i) w += phq[hl * D + i] * to_f32(pr[i]);
        const float g = a.gate[kv * G + hl];
        lw[hl * NK + kk] = (la && w > 0.f && g > 0.f) ? __logf(g) + __logf(w) : STILL_NEG_INF;
      }
    }
  }
  // state readout: nst[h][f] = sum_i phi_h[i] S[i][f], dz_h = phi_h . z
  {
    const int f = tid % D, half = tid / D;  // D = 64: 4 quarters, D = 128: 2 halves
    const int parts = 256 / D;
    float accs[8];
    for (int hl = 0; hl < G; ++hl) accs[hl] = 0.f;
    for (int i = half; i < D; i += parts) {
      const float sv = S[(size_t)i * D + f];
      for (int hl = 0; hl < G; ++hl) accs[hl] += phq[hl * D + i] * sv;
    }
    for (int hl = 0; hl < G; ++hl) acc2[(half * G + hl) * D + f] = accs[hl];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    float s = 0.f;
    for (int p = 0; p < 256 / D; ++p) s += acc2[(p * G) * D + e];
    nst[e] = s;
  }
  for (int hl = 0; hl < G; ++hl) {
    float part = 0.f;
    for (int i = tid; i < D; i += 256) part += phq[hl * D + i] * z[i];
    const float dzh = block_sum256(part, red);
    if (tid == 0) headv[hl * 4 + 0] = dzh;
  }
  __syncthreads();
  // per head: max over all log-weights (state included), then weights
  for (int hl = 0; hl < G; ++hl) {
    const float g = a.gate[kv * G + hl];
    const float dzh = headv[hl * 4 + 0];
    const float lws = (g > 0.f && dzh > 0.f) ? __logf(g * dzh) : STILL_NEG_INF;
    float mx = lws;
    for (int kk = tid; kk < n_keys; kk += 256) mx = fmaxf(mx, lw[hl * NK + kk]);
    mx = block_max256(mx, red);
    float sum = 0.f;
    for (int kk = tid; kk < n_keys; kk += 256) {
      const float x = lw[hl * NK + kk];
      const float e = x == STILL_NEG_INF ? 0.f : __expf(x - mx);
      lw[hl * NK + kk] = e;
      sum += e;
    }
    sum = block_sum256(sum, red);
    if (tid == 0) {
      const float es = lws == STILL_NEG_INF ? 0.f : __expf(lws - mx);
      headv[hl * 4 + 1] = es;
      headv[hl * 4 + 2] = sum + es;
    }
  }
  __syncthreads();
  // weighted values
  {
    const int f = tid % D, part = tid / D, parts = 256 / D;
    float accs[8];
    for (int hl = 0; hl < G; ++hl) accs[hl] = 0.f;
    for (int kk = part; kk < n_keys; kk += parts) {
      const T* vr;
      if (kk < n_oob) vr = pool_v + (size_t)kk * D;
      else if (kk < n_oob + n_win) vr = ring_v + (size_t)((lo + kk - n_oob) % R) * D;
      else vr = ring_v + (size_t)((la_lo + kk - n_oob - n_win) % R) * D;
      const float x = to_f32(vr[f]);
      for (int hl = 0; hl < G; ++hl) accs[hl] += lw[hl * NK + kk] * x;
    }
    __syncthreads();
    for (int hl = 0; hl < G; ++hl) acc2[(part * G + hl) * D + f] = accs[hl];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int hl = e / D;
    float s = 0.f;
    for (int p = 0; p < 256 / D; ++p) s += acc2[(p * G) * D + e];
    const float es = headv[hl * 4 + 1], tot = headv[hl * 4 + 2];
    const float dzh = headv[hl * 4 + 0];
    if (es > 0.f) s += es * nst[e] / dzh;
    const float y = s / tot;
    const size_t o = ((size_t)b * a.Hq + kv * G + hl) * D + (e % D);
    if (a.fp32_out) reinterpret_cast<float*>(a.out)[o] = y;
    else reinterpret_cast<T*>(a.out)[o] = from_f32<T>(y);
  }
  __syncthreads();
  if (tid == 0) {
    meta[1] = n_pool;
    meta[0] = t + 1;
  }
}

}  // namespace still
