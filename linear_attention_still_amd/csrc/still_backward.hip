// Backward of one STILL layer for gfx950: gradients of the output with
// respect to q, k, v, the NP-Map weights and the gates.
//
// Pages cited (short tag -> page title):
//   [P3] "STILL: Content-Aware Intra-Layer Hybrid Attention for Efficient
//        LLM Linearization", sections "Delayed Chunk-Level Selection for
//        Unified Training-Inference Parallelism", "Content-Aware Routing with
//        Fixed Budget", "NP-Map: Norm-Preserving Feature Map"
//
// Training runs the same chunk-parallel layer as inference [P3 "Delayed
// Chunk-Level Selection ..."]; the routing (which tokens are kept) is a
// discrete decision and is held fixed (reading): the kept set comes from the
// forward's selection. With it, every query t has fixed key sets A(t)
// (window, own chunk, kept tokens of earlier chunks: softmax) and B(t) (the
// other earlier tokens: linear), and
//   y_t = (sum_A e^{s_tj} v_j + g sum_B w_tj v_j) / N_t,
//   N_t = sum_A e^{s_tj} + g sum_B w_tj,  s = scale q.k,  w = phi(q).phi(k).
// With e_tj = dy_t . v_j and delta_t = dy_t . y_t:
//   d s_tj = e^{s_tj} / N_t (e_tj - delta_t)         (j in A(t))
//   d w_tj = g / N_t (e_tj - delta_t)                 (j in B(t))
//   dv_j   = sum_t (weight_tj / N_t) dy_t
//   dg     = sum_t sum_B w_tj / N_t (e_tj - delta_t)
// and the features' gradients go through the NP-Map Jacobian to q, k and F.
// N_t comes from the forward's log-normalisers (the branch partials), y_t
// from its float32 output.
//
// Dense form: every (query, key) pair on or below the diagonal is visited,
// in float32 on the vector ALUs, tiles staged in LDS. The cost grows as
// L^2 (the forward's is linear in L).
//
// Kernels, in launch order:
//   0. zero the accumulated outputs (dgate, dfmap); kept flags from sel
//   1. NP-Map features of every q and k row
//   2. query side: per 16-query tile, all earlier keys: the softmax part of
//      dq, d phi(q), dg; the rows' ln N and delta for step 3
//   3. key side: per 32-key tile, all later queries of the group's heads:
//      the softmax part of dk, d phi(k), dv
//   4. NP-Map backward of every row: dq, dk += J^T d phi; dz = d(x F)
//   5. dF = sum over rows of x^T dz, per kv head
#include "still_common.h"

namespace still {

struct BackwardArgs {
  const void *q, *k, *v, *fmap_w;  // T: [B][Hq][L][D], [B][Hkv][L][D] x2, [Hkv][D][D]
  const float* gate;               // [Hq]
  const int32_t* sel;              // [B][Hkv][n_dec][lam] kept positions (-1: none)
  const float* y;                  // [B][Hq][L][D] forward output (float32)
  const float *lse_sa, *lse_la;    // [B][Hq][L] forward log-normalisers of the branches
  const float* dy;                 // [B][Hq][L][D]
  float *dq, *dk, *dv;             // outputs, float32, shaped as q, k, v
  float *dfmap, *dgate;            // [Hkv][D][D], [Hq]
  float *phq, *phk, *dphq, *dphk;  // workspace: features and their gradients
  float *lnN, *delta;              // [B][Hq][L]
  float* dz;                       // [B*Hq*L + B*Hkv*L][D] gradients of x F
  uint8_t* kept;                   // [B][Hkv][L]
  int B, Hq, Hkv, G, L, W, C, n_dec, lam;
  float scale;
};

constexpr int BW_THREADS = 256;
constexpr int BW_PAD = 4;  // floats of padding per LDS row

__global__ __launch_bounds__(BW_THREADS) void bw_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * BW_THREADS + threadIdx.x; i < n; i += (int64_t)gridDim.x * BW_THREADS)
    p[i] = 0.f;
}

// kept[b][kv][j] = 1 where j is listed in its chunk's selection row
__global__ __launch_bounds__(BW_THREADS) void bw_flags_kernel(BackwardArgs a) {
  const int64_t n = (int64_t)a.B * a.Hkv * a.L;
  for (int64_t i = (int64_t)blockIdx.x * BW_THREADS + threadIdx.x; i < n; i += (int64_t)gridDim.x * BW_THREADS) {
    const int j = (int)(i % a.L);
    const int64_t unit = i / a.L;
    const int c = j / a.C;
    uint8_t f = 0;
    if (c < a.n_dec) {
      const int32_t* row = a.sel + (unit * a.n_dec + c) * a.lam;
      for (int e = 0; e < a.lam; ++e) f |= row[e] == j ? 1 : 0;
    }
    a.kept[i] = f;
  }
}

// Row r of the stacked q and k rows: its input, feature and gradient rows
// and its kv head.
template <typename T, int D>
struct BwRow {
  const T* x;
  float *ph, *dph, *dx;
  int kv;
  __device__ BwRow(const BackwardArgs& a, int64_t r) {
    const int64_t nq = (int64_t)a.B * a.Hq * a.L;
    if (r < nq) {
      const int h = (int)((r / a.L) % a.Hq);
      x = reinterpret_cast<const T*>(a.q) + r * D;
      ph = a.phq + r * D;
      dph = a.dphq + r * D;
      dx = a.dq + r * D;
      kv = h / a.G;
    } else {
      const int64_t rk = r - nq;
      x = reinterpret_cast<const T*>(a.k) + rk * D;
      ph = a.phk + rk * D;
      dph = a.dphk + rk * D;
      dx = a.dk + rk * D;
      kv = (int)((rk / a.L) % a.Hkv);
    }
  }
};

// Row kernels (features and their backward): one workgroup per (64 rows of
// one (batch row, head) sequence, sequence); the sequences are the q rows
// of every (b, h), then the k rows of every (b, kv). F of the sequence's
// kv head is staged in LDS as float, rows padded to D + 1 (reads along a
// row or down a column are both conflict-free); 4 waves, one row at a time.
constexpr int BW_ROWS = 64;
template <int D>
struct BwRowLds {
  static constexpr int FS = D + 1;
  static constexpr int bytes = (D * FS + 8 * D) * 4;
};

template <typename T, int D>
__device__ __forceinline__ int bw_stage_f(const BackwardArgs& a, float* Fs, int seq) {
  const int kv = seq < a.B * a.Hq ? (seq % a.Hq) / a.G : (seq - a.B * a.Hq) % a.Hkv;
  const T* F = reinterpret_cast<const T*>(a.fmap_w) + (size_t)kv * D * D;
  for (int e = threadIdx.x; e < D * D; e += BW_THREADS) Fs[(e / D) * (D + 1) + e % D] = to_f32(F[e]);
  __syncthreads();
  return kv;
}

// NP-Map of one row by one wave [P3 "NP-Map"], reading of the layer:
// phi(x) = ||x|| u / ||u||, u = softmax(x F). Lane l holds features
// l + 64 c; xs: the row in LDS; Fs: F in LDS. Returns, per lane, u, and the
// norms ||u||, ||x||.
template <int D>
__device__ __forceinline__ void bw_npmap_row(const float* Fs, const float* xs, float (&u)[D / 64], float& nu,
                                             float& nx) {
  const int lane = threadIdx.x & 63;
  float z[D / 64];
#pragma unroll
  for (int c = 0; c < D / 64; ++c) z[c] = 0.f;
  for (int i = 0; i < D; ++i) {
    const float xi = xs[i];
#pragma unroll
    for (int c = 0; c < D / 64; ++c) z[c] = fmaf(xi, Fs[i * (D + 1) + lane + 64 * c], z[c]);
  }
  float mx = z[0];
#pragma unroll
  for (int c = 1; c < D / 64; ++c) mx = fmaxf(mx, z[c]);
  mx = wave_max(mx);
  float su = 0.f, xx = 0.f;
#pragma unroll
  for (int c = 0; c < D / 64; ++c) {
    u[c] = expf(z[c] - mx);
    su += u[c];
    const float xv = xs[lane + 64 * c];
    xx += xv * xv;
  }
  su = wave_sum(su);
  float uu = 0.f;
#pragma unroll
  for (int c = 0; c < D / 64; ++c) {
    u[c] /= su;
    uu += u[c] * u[c];
  }
  nu = sqrtf(wave_sum(uu));
  nx = sqrtf(wave_sum(xx));
}

// 1. features of every q row and k row
template <typename T, int D>
__global__ __launch_bounds__(BW_THREADS) void bw_phi_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) char smem[];
  float* Fs = reinterpret_cast<float*>(smem);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* xs = Fs + D * (D + 1) + wave * D;
  const int seq = blockIdx.y;
  bw_stage_f<T, D>(a, Fs, seq);
  const int64_t row0 = (int64_t)seq * a.L;
  for (int i = wave; i < BW_ROWS; i += 4) {  // wave-uniform
    const int t = blockIdx.x * BW_ROWS + i;
    if (t >= a.L) break;
    const BwRow<T, D> R(a, row0 + t);
    __builtin_amdgcn_wave_barrier();  // the previous row's reads of xs are done
#pragma unroll
    for (int c = 0; c < D / 64; ++c) xs[lane + 64 * c] = to_f32(R.x[lane + 64 * c]);
    __builtin_amdgcn_wave_barrier();
    float u[D / 64], nu, nx;
    bw_npmap_row<D>(Fs, xs, u, nu, nx);
#pragma unroll
    for (int c = 0; c < D / 64; ++c) R.ph[lane + 64 * c] = nu > 0.f ? nx * u[c] / nu : 0.f;
  }
}

// The LDS rows of one tile: n rows of D floats, padded.
template <int D>
__device__ __forceinline__ float* bw_tile(float* base, int i, int n) {
  return base + (size_t)i * n * (D + BW_PAD);
}

// Is key j a softmax key of query t (j <= t)? Window, own chunk, or kept
// in an earlier chunk [P3 "Content-Aware Routing with Fixed Budget"].
__device__ __forceinline__ bool bw_is_sa(int t, int j, int W, int C, bool kept) {
  return j >= t - W + 1 || j / C == t / C || kept;
}

// Pair values of query row qi (LDS rows Q, PQ, DY) and key row kk (K, PK,
// V): s (unscaled), w, e.
template <int D>
__device__ __forceinline__ void bw_dots(const float* q, const float* pq, const float* dy, const float* k,
                                        const float* pk, const float* v, float& s, float& w, float& e) {
  float s0 = 0.f, w0 = 0.f, e0 = 0.f;
#pragma unroll 8
  for (int d = 0; d < D; d += 4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(q + d), b = *reinterpret_cast<const f32x4*>(k + d);
    const f32x4 c = *reinterpret_cast<const f32x4*>(pq + d), f = *reinterpret_cast<const f32x4*>(pk + d);
    const f32x4 g = *reinterpret_cast<const f32x4*>(dy + d), h = *reinterpret_cast<const f32x4*>(v + d);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0 = fmaf(a[i], b[i], s0);
      w0 = fmaf(c[i], f[i], w0);
      e0 = fmaf(g[i], h[i], e0);
    }
  }
  s = s0;
  w = w0;
  e = e0;
}

// 2. query side: one workgroup per (16-query tile, query head, batch row)
constexpr int BW_QT = 16, BW_KT = 32;
template <int D>
struct BwQLds {
  static constexpr int RS = D + BW_PAD;
  static constexpr int bytes = (3 * BW_QT * RS + 3 * BW_KT * RS + 2 * BW_QT * (BW_KT + 1) + 2 * BW_QT) * 4 + BW_KT;
};

template <typename T, int D>
__global__ __launch_bounds__(BW_THREADS) void bw_query_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int RS = D + BW_PAD, DPT = D / 16;
  float* Qs = reinterpret_cast<float*>(smem);
  float* PQs = Qs + BW_QT * RS;
  float* DYs = PQs + BW_QT * RS;
  float* Ks = DYs + BW_QT * RS;
  float* PKs = Ks + BW_KT * RS;
  float* Vs = PKs + BW_KT * RS;
  float* DS = Vs + BW_KT * RS;          // [QT][KT + 1]
  float* DW = DS + BW_QT * (BW_KT + 1);  // [QT][KT + 1]
  float* rowN = DW + BW_QT * (BW_KT + 1);  // ln N of the tile's rows
  float* rowD = rowN + BW_QT;             // delta
  uint8_t* kp = reinterpret_cast<uint8_t*>(rowD + BW_QT);  // [KT] kept flags
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * BW_QT, h = blockIdx.y, b = blockIdx.z;
  const int L = a.L, kv = h / a.G;
  const float g = a.gate[h];
  const size_t qrow0 = ((size_t)b * a.Hq + h) * L;  // row index of (b, h, 0)
  const size_t krow0 = ((size_t)b * a.Hkv + kv) * L;
  // query tile: q (as float), phi(q), dy; rows past L are zeros
  for (int e = tid; e < BW_QT * D; e += BW_THREADS) {
    const int i = e / D, d = e % D, t = t0 + i;
    const bool in = t < L;
    Qs[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.q)[(qrow0 + t) * D + d]) : 0.f;
    PQs[i * RS + d] = in ? a.phq[(qrow0 + t) * D + d] : 0.f;
    DYs[i * RS + d] = in ? a.dy[(qrow0 + t) * D + d] : 0.f;
  }
  // row constants: delta = dy . y, ln N = ln(Z + g D) from the branch
  // log-normalisers (wave w: rows 4w .. 4w + 3)
  for (int i = wave * (BW_QT / 4); i < (wave + 1) * (BW_QT / 4); ++i) {
    const int t = t0 + i;
    float dd = 0.f;
    if (t < L)
      for (int d = lane; d < D; d += 64) dd += a.dy[(qrow0 + t) * D + d] * a.y[(qrow0 + t) * D + d];
    dd = wave_sum(dd);
    if (lane == 0) {
      float ln = 0.f;
      if (t < L) {
        const float ls = a.lse_sa[qrow0 + t], ll = a.lse_la[qrow0 + t];
        ln = (g > 0.f && ll != STILL_NEG_INF) ? ls + log1pf(g * expf(ll - ls)) : ls;
        a.lnN[qrow0 + t] = ln;
        a.delta[qrow0 + t] = dd;
      }
      rowN[i] = ln;
      rowD[i] = dd;
    }
  }
  const int qi = tid >> 4, sub = tid & 15;  // row of the tile; key pair / column group
  const int t = t0 + qi;
  float dqa[DPT], dpa[DPT], dg = 0.f;
#pragma unroll
  for (int c = 0; c < DPT; ++c) dqa[c] = dpa[c] = 0.f;
  const int j_end = min(t0 + BW_QT, L);
  for (int j0 = 0; j0 < j_end; j0 += BW_KT) {
    __syncthreads();  // the previous tile is done with Ks .. DW
    for (int e = tid; e < BW_KT * D; e += BW_THREADS) {
      const int i = e / D, d = e % D, j = j0 + i;
      const bool in = j < L;
      Ks[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.k)[(krow0 + j) * D + d]) : 0.f;
      PKs[i * RS + d] = in ? a.phk[(krow0 + j) * D + d] : 0.f;
      Vs[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.v)[(krow0 + j) * D + d]) : 0.f;
    }
    if (tid < BW_KT) kp[tid] = j0 + tid < L ? a.kept[krow0 + j0 + tid] : 0;
    __syncthreads();
    // pair gradients of (t, keys 2 sub, 2 sub + 1)
    const float lnN = rowN[qi], dl = rowD[qi];
    const float rN = expf(-lnN);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = 2 * sub + u, j = j0 + kk;
      float ds = 0.f, dw = 0.f;
      if (t < L && j <= t) {
        float s, w, e;
        bw_dots<D>(Qs + qi * RS, PQs + qi * RS, DYs + qi * RS, Ks + kk * RS, PKs + kk * RS, Vs + kk * RS, s, w,
                   e);
        if (bw_is_sa(t, j, a.W, a.C, kp[kk] != 0)) {
          ds = expf(a.scale * s - lnN) * (e - dl);
        } else {
          dw = g * rN * (e - dl);
          dg += w * rN * (e - dl);
        }
      }
      DS[qi * (BW_KT + 1) + kk] = ds;
      DW[qi * (BW_KT + 1) + kk] = dw;
    }
    __syncthreads();
    // dq += ds K, d phi(q) += dw phi(K) over the tile's keys (columns
    // sub + 16 c of the row)
    for (int kk = 0; kk < BW_KT; ++kk) {
      const float ds = DS[qi * (BW_KT + 1) + kk], dw = DW[qi * (BW_KT + 1) + kk];
#pragma unroll
      for (int c = 0; c < DPT; ++c) {
        dqa[c] = fmaf(ds, Ks[kk * RS + sub + 16 * c], dqa[c]);
        dpa[c] = fmaf(dw, PKs[kk * RS + sub + 16 * c], dpa[c]);
      }
    }
  }
  if (t < L) {
#pragma unroll
    for (int c = 0; c < DPT; ++c) {
      a.dq[(qrow0 + t) * D + sub + 16 * c] = a.scale * dqa[c];
      a.dphq[(qrow0 + t) * D + sub + 16 * c] = dpa[c];
    }
  }
  // dg over the workgroup, one atomic add
  dg = wave_sum(dg);
  __syncthreads();
  if (lane == 0) rowN[wave] = dg;
  __syncthreads();
  if (tid == 0) atomicAdd(a.dgate + h, rowN[0] + rowN[1] + rowN[2] + rowN[3]);
}

// 3. key side: one workgroup per (32-key tile, kv head, batch row); the
// group's query heads and every later 16-query tile in turn
template <int D>
struct BwKLds {
  static constexpr int RS = D + BW_PAD;
  static constexpr int bytes = (3 * BW_KT * RS + 3 * BW_QT * RS + 3 * BW_KT * (BW_QT + 1) + 2 * BW_QT) * 4 + BW_KT;
};

template <typename T, int D>
__global__ __launch_bounds__(BW_THREADS) void bw_key_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int RS = D + BW_PAD, DPT = D / 8;
  float* Ks = reinterpret_cast<float*>(smem);
  float* PKs = Ks + BW_KT * RS;
  float* Vs = PKs + BW_KT * RS;
  float* Qs = Vs + BW_KT * RS;
  float* PQs = Qs + BW_QT * RS;
  float* DYs = PQs + BW_QT * RS;
  float* PS = DYs + BW_QT * RS;          // [KT][QT + 1] weight / N
  float* DS = PS + BW_KT * (BW_QT + 1);  // [KT][QT + 1]
  float* DW = DS + BW_KT * (BW_QT + 1);  // [KT][QT + 1]
  float* rowN = DW + BW_KT * (BW_QT + 1);
  float* rowD = rowN + BW_QT;
  uint8_t* kp = reinterpret_cast<uint8_t*>(rowD + BW_QT);
  const int tid = threadIdx.x;
  const int j0 = blockIdx.x * BW_KT, kv = blockIdx.y, b = blockIdx.z;
  const int L = a.L;
  const size_t krow0 = ((size_t)b * a.Hkv + kv) * L;
  for (int e = tid; e < BW_KT * D; e += BW_THREADS) {
    const int i = e / D, d = e % D, j = j0 + i;
    const bool in = j < L;
    Ks[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.k)[(krow0 + j) * D + d]) : 0.f;
    PKs[i * RS + d] = in ? a.phk[(krow0 + j) * D + d] : 0.f;
    Vs[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.v)[(krow0 + j) * D + d]) : 0.f;
  }
  if (tid < BW_KT) kp[tid] = j0 + tid < L ? a.kept[krow0 + j0 + tid] : 0;
  const int qi = tid >> 4, sub = tid & 15;  // phase 1: query row, key pair
  const int kk2 = tid >> 3, part = tid & 7;  // phase 2: key row, column group
  float dka[DPT], dpa[DPT], dva[DPT];
#pragma unroll
  for (int c = 0; c < DPT; ++c) dka[c] = dpa[c] = dva[c] = 0.f;
  for (int hl = 0; hl < a.G; ++hl) {
    const int h = kv * a.G + hl;
    const float g = a.gate[h];
    const size_t qrow0 = ((size_t)b * a.Hq + h) * L;
    for (int t0 = (j0 / BW_QT) * BW_QT; t0 < L; t0 += BW_QT) {
      __syncthreads();  // the previous query tile is done with Qs .. DW
      for (int e = tid; e < BW_QT * D; e += BW_THREADS) {
        const int i = e / D, d = e % D, t = t0 + i;
        const bool in = t < L;
        Qs[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.q)[(qrow0 + t) * D + d]) : 0.f;
        PQs[i * RS + d] = in ? a.phq[(qrow0 + t) * D + d] : 0.f;
        DYs[i * RS + d] = in ? a.dy[(qrow0 + t) * D + d] : 0.f;
      }
      if (tid < BW_QT) {
        const int t = t0 + tid;
        rowN[tid] = t < L ? a.lnN[qrow0 + t] : 0.f;
        rowD[tid] = t < L ? a.delta[qrow0 + t] : 0.f;
      }
      __syncthreads();
      const int t = t0 + qi;
      const float lnN = rowN[qi], dl = rowD[qi], rN = expf(-lnN);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kk = 2 * sub + u, j = j0 + kk;
        float p = 0.f, ds = 0.f, dw = 0.f;
        if (t < L && j < L && j <= t) {
          float s, w, e;
          bw_dots<D>(Qs + qi * RS, PQs + qi * RS, DYs + qi * RS, Ks + kk * RS, PKs + kk * RS, Vs + kk * RS, s,
                     w, e);
          if (bw_is_sa(t, j, a.W, a.C, kp[kk] != 0)) {
            p = expf(a.scale * s - lnN);
            ds = p * (e - dl);
          } else {
            p = g * w * rN;
            dw = g * rN * (e - dl);
          }
        }
        PS[kk * (BW_QT + 1) + qi] = p;
        DS[kk * (BW_QT + 1) + qi] = ds;
        DW[kk * (BW_QT + 1) + qi] = dw;
      }
      __syncthreads();
      // dk += ds q, d phi(k) += dw phi(q), dv += p dy over the tile's queries
      for (int i = 0; i < BW_QT; ++i) {
        const float p = PS[kk2 * (BW_QT + 1) + i], ds = DS[kk2 * (BW_QT + 1) + i], dw = DW[kk2 * (BW_QT + 1) + i];
#pragma unroll
        for (int c = 0; c < DPT; ++c) {
          dka[c] = fmaf(ds, Qs[i * RS + part + 8 * c], dka[c]);
          dpa[c] = fmaf(dw, PQs[i * RS + part + 8 * c], dpa[c]);
          dva[c] = fmaf(p, DYs[i * RS + part + 8 * c], dva[c]);
        }
      }
    }
  }
  const int j = j0 + kk2;
  if (j < L) {
#pragma unroll
    for (int c = 0; c < DPT; ++c) {
      a.dk[(krow0 + j) * D + part + 8 * c] = a.scale * dka[c];
      a.dphk[(krow0 + j) * D + part + 8 * c] = dpa[c];
      a.dv[(krow0 + j) * D + part + 8 * c] = dva[c];
    }
  }
}

// 4. NP-Map backward of every row (one wave per row): with phi = n u / nu,
// n = ||x||, u = softmax(z), z = x F, nu = ||u||:
//   dn = dphi . u / nu, du = n (dphi - (u / nu)(u / nu . dphi)) / nu,
//   dz = u (du - u . du), dx = F dz + dn x / n.
// dx is added to the row's softmax-part gradient; dz is kept for dF.
template <typename T, int D>
__global__ __launch_bounds__(BW_THREADS) void bw_npmap_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) char smem[];
  float* Fs = reinterpret_cast<float*>(smem);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* xs = Fs + D * (D + 1) + wave * D;
  float* dzs = Fs + D * (D + 1) + 4 * D + wave * D;
  const int seq = blockIdx.y;
  bw_stage_f<T, D>(a, Fs, seq);
  const int64_t row0 = (int64_t)seq * a.L;
  for (int ii = wave; ii < BW_ROWS; ii += 4) {  // wave-uniform
    const int t = blockIdx.x * BW_ROWS + ii;
    if (t >= a.L) break;
    const int64_t r = row0 + t;
    const BwRow<T, D> R(a, r);
    __builtin_amdgcn_wave_barrier();  // the previous row's reads of xs, dzs are done
#pragma unroll
    for (int c = 0; c < D / 64; ++c) xs[lane + 64 * c] = to_f32(R.x[lane + 64 * c]);
    __builtin_amdgcn_wave_barrier();
    float u[D / 64], nu, nx;
    bw_npmap_row<D>(Fs, xs, u, nu, nx);
    const float inu = nu > 0.f ? 1.f / nu : 0.f;
    float dph[D / 64], udp = 0.f;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      dph[c] = R.dph[lane + 64 * c];
      udp += u[c] * dph[c];
    }
    udp = wave_sum(udp) * inu;  // (u / nu) . dphi = dn
    float du[D / 64], uddu = 0.f;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      du[c] = nx * (dph[c] - u[c] * inu * udp) * inu;
      uddu += u[c] * du[c];
    }
    uddu = wave_sum(uddu);
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const float dzv = u[c] * (du[c] - uddu);
      dzs[lane + 64 * c] = dzv;
      a.dz[r * D + lane + 64 * c] = dzv;
    }
    __builtin_amdgcn_wave_barrier();
    const float dnx = nx > 0.f ? udp / nx : 0.f;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const int i = lane + 64 * c;
      float acc = 0.f;
      for (int jj = 0; jj < D; ++jj) acc = fmaf(Fs[i * (D + 1) + jj], dzs[jj], acc);
      R.dx[i] += acc + dnx * xs[i];
    }
  }
}

// 5. dF[kv] = sum over the kv head's rows of x^T dz: one workgroup per
// (chunk of BW_DF_ROWS rows, kv head); thread (i, part) owns F[i][part OPT
// .. part OPT + OPT - 1]; one atomic add per owned entry per workgroup
constexpr int BW_DF_ROWS = 512;
template <typename T, int D>
__global__ __launch_bounds__(BW_THREADS) void bw_dfmap_kernel(BackwardArgs a) {
  __shared__ float xs[16][D];
  __shared__ float dzs[16][D];
  constexpr int OPT = D * D / BW_THREADS;  // outputs per thread
  const int kv = blockIdx.y, tid = threadIdx.x;
  const int i = tid / (BW_THREADS / D), j0 = (tid % (BW_THREADS / D)) * OPT;
  // the kv head's rows: q rows of its G heads in every batch row, then its
  // k rows; row index n -> stacked row
  const int64_t nrow_q = (int64_t)a.B * a.G * a.L, nrow = nrow_q + (int64_t)a.B * a.L;
  auto stacked = [&](int64_t n) -> int64_t {
    if (n < nrow_q) {
      const int64_t bb = n / ((int64_t)a.G * a.L), rem = n % ((int64_t)a.G * a.L);
      const int64_t hh = kv * a.G + rem / a.L, t = rem % a.L;
      return (bb * a.Hq + hh) * a.L + t;
    }
    const int64_t m = n - nrow_q, bb = m / a.L, t = m % a.L;
    return (int64_t)a.B * a.Hq * a.L + (bb * a.Hkv + kv) * a.L + t;
  };
  float acc[OPT];
#pragma unroll
  for (int c = 0; c < OPT; ++c) acc[c] = 0.f;
  const int64_t n0 = (int64_t)blockIdx.x * BW_DF_ROWS, n1 = min(n0 + BW_DF_ROWS, nrow);
  for (int64_t nb = n0; nb < n1; nb += 16) {
    __syncthreads();
    for (int e = tid; e < 16 * D; e += BW_THREADS) {
      const int rr = e / D, d = e % D;
      const int64_t n = nb + rr;
      float xv = 0.f, dv = 0.f;
      if (n < n1) {
        const int64_t s = stacked(n);
        const BwRow<T, D> R(a, s);
        xv = to_f32(R.x[d]);
        dv = a.dz[s * D + d];
      }
      xs[rr][d] = xv;
      dzs[rr][d] = dv;
    }
    __syncthreads();
    for (int rr = 0; rr < 16; ++rr) {
      const float xi = xs[rr][i];
#pragma unroll
      for (int c = 0; c < OPT; ++c) acc[c] = fmaf(xi, dzs[rr][j0 + c], acc[c]);
    }
  }
  float* dF = a.dfmap + (size_t)kv * D * D + (size_t)i * D + j0;
#pragma unroll
  for (int c = 0; c < OPT; ++c) atomicAdd(dF + c, acc[c]);
}

}  // namespace still
