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
// Chunked form, linear in L like the forward: with the routing fixed, the
// linear keys of a query t of chunk c are the unkept tokens before the
// chunk-level boundary b_c = cf(c) C (the forward's folded state) plus some
// band keys in [b_c, t]; so the linear part of the query side is the chunk's
// prefix state P_c = sum_{unkept j < b_c} phi(k_j) v_j^T (and z_c):
//   d phi(q_t) += (g / N_t)(P_c dy_t - z_c delta_t),
//   dg += (1 / N_t)(phi(q_t)^T P_c dy_t - delta_t phi(q_t) . z_c),
// and the linear part of the key side, for an unkept key j, is a suffix over
// the query chunks that hold j in their state, R = sum (g / N_t) phi(q_t)
// dy_t^T and r = sum (g / N_t) delta_t phi(q_t) (over those chunks' queries
// and the group's heads):
//   d phi(k_j) += R v_j - r,  dv_j += R^T phi(k_j).
// The remaining pairs are visited one by one: the band pairs (key in
// [b_c, t]) from both sides, and the kept-pool pairs (softmax keys of every
// later chunk) from the query side and, for dk and dv, from a pass over the
// kept keys. Float32 on the vector ALUs, tiles in LDS, float64 scans.
//
// Kernels, in launch order:
//   0. zero dgate, dfmap; kept flags from sel
//   1. NP-Map features of every q and k row; per query row ln N and delta
//   2. per chunk: the state delta (unkept keys) and the query-side delta
//      (R, r); a float64 prefix scan of the first, suffix scan of the second
//   3. query side, per 16-query tile: band and pool pairs, the state term:
//      dq (softmax part), d phi(q), dg
//   4. key side, per 16-key tile: band pairs of the group's heads, the
//      suffix-state term: dk (softmax part), d phi(k), dv
//   5. kept keys, per 16 pool entries: their softmax pairs with the later
//      chunks' queries: dk, dv +=
//   6. NP-Map backward of every row: dq, dk += J^T d phi; dz = d(x F)
//   7. dF = sum over rows of x^T dz, per kv head
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
  float* cS;                       // [B][Hkv][T][D*D + D] chunk state deltas -> prefix
  float* cR;                       // [B][Hkv][T][D*D + D] chunk query deltas -> suffix
  int B, Hq, Hkv, G, L, W, C, n_dec, lam, T, cap_chunks;
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

// per query row: delta = dy . y and ln N = ln(Z + g D) from the branch
// log-normalisers (one wave per row)
__global__ __launch_bounds__(BW_THREADS) void bw_rowstat_kernel(BackwardArgs a, int D) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave, rows = (int64_t)a.B * a.Hq * a.L;
  if (r >= rows) return;  // wave-uniform
  const int h = (int)((r / a.L) % a.Hq);
  float dd = 0.f;
  for (int d = lane; d < D; d += 64) dd += a.dy[r * D + d] * a.y[r * D + d];
  dd = wave_sum(dd);
  if (lane == 0) {
    const float g = a.gate[h], ls = a.lse_sa[r], ll = a.lse_la[r];
    a.lnN[r] = (g > 0.f && ll != STILL_NEG_INF) ? ls + log1pf(g * expf(ll - ls)) : ls;
    a.delta[r] = dd;
  }
}

// 2a. per chunk c: cS[c] = sum over its unkept keys of phi(k) v^T (row-major
// D x D) and phi(k) (D); cR[c] = sum over its queries and the group's heads
// of (g / N) phi(q) dy^T and (g / N) delta phi(q). Thread (i, part) owns
// entries [i][part OPT .. + OPT) and, for part 0, the vector entry i.
template <typename T, int D>
__global__ __launch_bounds__(BW_THREADS) void bw_chunk_delta_kernel(BackwardArgs a) {
  __shared__ float xa[16][D];
  __shared__ float xb[16][D];
  __shared__ float cf_[16];  // per-row factor
  constexpr int OPT = D * D / BW_THREADS;
  const int c = blockIdx.x, kv = blockIdx.y % a.Hkv, b = blockIdx.y / a.Hkv, side = blockIdx.z;
  const int tid = threadIdx.x, i = tid / (BW_THREADS / D), j0 = (tid % (BW_THREADS / D)) * OPT;
  const int L = a.L, C = a.C;
  const size_t unit = (size_t)b * a.Hkv + kv;
  float acc[OPT], vec = 0.f;
#pragma unroll
  for (int e = 0; e < OPT; ++e) acc[e] = 0.f;
  // side 0: rows = the chunk's keys (factor: unkept); side 1: rows = the
  // chunk's queries of every head of the group (factor g / N)
  const int nrows = side == 0 ? C : C * a.G;
  for (int r0 = 0; r0 < nrows; r0 += 16) {
    __syncthreads();
    for (int e = tid; e < 16 * D; e += BW_THREADS) {
      const int rr = e / D, d = e % D, r = r0 + rr;
      float va = 0.f, vb = 0.f;
      if (side == 0) {
        const int t = c * C + r;
        if (r < nrows && t < L) {
          va = a.phk[(unit * L + t) * D + d];
          vb = to_f32(reinterpret_cast<const T*>(a.v)[(unit * L + t) * D + d]);
        }
      } else {
        const int hl = r / C, t = c * C + r % C;
        if (r < nrows && t < L) {
          const size_t row = ((size_t)b * a.Hq + kv * a.G + hl) * L + t;
          va = a.phq[row * D + d];
          vb = a.dy[row * D + d];
        }
      }
      xa[rr][d] = va;
      xb[rr][d] = vb;
    }
    if (tid < 16) {
      const int r = r0 + tid;
      float f = 0.f;
      if (side == 0) {
        const int t = c * C + r;
        if (r < nrows && t < L) f = a.kept[unit * L + t] ? 0.f : 1.f;
      } else {
        const int hl = r / C, t = c * C + r % C;
        if (r < nrows && t < L) {
          const int h = kv * a.G + hl;
          const size_t row = ((size_t)b * a.Hq + h) * L + t;
          const float g = a.gate[h];
          f = g > 0.f ? g * expf(-a.lnN[row]) : 0.f;
        }
      }
      cf_[tid] = f;
    }
    __syncthreads();
    for (int rr = 0; rr < 16; ++rr) {
      const float f = cf_[rr];
      if (f == 0.f) continue;  // uniform across the workgroup
      const float xi = f * xa[rr][i];
#pragma unroll
      for (int e = 0; e < OPT; ++e) acc[e] = fmaf(xi, xb[rr][j0 + e], acc[e]);
      if (j0 == 0) {
        float w = 1.f;
        if (side == 1) {
          const int r = r0 + rr, hl = r / C, t = c * C + r % C;
          w = a.delta[((size_t)b * a.Hq + kv * a.G + hl) * L + t];
        }
        vec = fmaf(xi, w, vec);
      }
    }
  }
  float* dst = (side == 0 ? a.cS : a.cR) + (unit * a.T + c) * (size_t)(D * D + D);
#pragma unroll
  for (int e = 0; e < OPT; ++e) dst[(size_t)i * D + j0 + e] = acc[e];
  if (j0 == 0) dst[D * D + i] = vec;
}

// 2b. scans over chunks, float64 running sums: cS inclusive prefix (the
// state of the chunks <= c), cR inclusive suffix (chunks >= c).
__global__ __launch_bounds__(BW_THREADS) void bw_chunk_scan_kernel(BackwardArgs a, int D) {
  const int n_elem = D * D + D;
  const int e = blockIdx.x * BW_THREADS + threadIdx.x;
  if (e >= n_elem) return;
  const size_t unit = (size_t)blockIdx.y % (a.B * a.Hkv);
  const bool suffix = blockIdx.y >= (unsigned)(a.B * a.Hkv);
  float* base = (suffix ? a.cR : a.cS) + unit * a.T * (size_t)n_elem + e;
  double run = 0.0;
  for (int k = 0; k < a.T; ++k) {
    const int c = suffix ? a.T - 1 - k : k;
    run += (double)base[(size_t)c * n_elem];
    base[(size_t)c * n_elem] = (float)run;
  }
}

// Tile helpers of the pair kernels (LDS rows of D floats, padded).
constexpr int BW_QT = 16, BW_KT = 16;

// Loads the rows `pos[i]` (-1: zeros) of a [L][D] array of type S into LDS.
template <typename S, int D>
__device__ __forceinline__ void bw_load_rows(float* dst, const S* src, const int* pos, int n) {
  constexpr int RS = D + BW_PAD;
  for (int e = threadIdx.x; e < n * D; e += BW_THREADS) {
    const int i = e / D, d = e % D, p = pos[i];
    dst[i * RS + d] = p >= 0 ? to_f32(src[(size_t)p * D + d]) : 0.f;
  }
}

// Pair gradients of query row t (of head with gate g, ln N, delta) and key
// j: softmax pair -> (p, ds, 0), linear pair -> (p, 0, dw) and its dg term.
struct BwPair {
  float p, ds, dw, dg;
};
__device__ __forceinline__ BwPair bw_pair(bool sa, float s, float w, float e, float g, float lnN, float dl,
                                          float scale) {
  BwPair r{0.f, 0.f, 0.f, 0.f};
  if (sa) {
    r.p = expf(scale * s - lnN);
    r.ds = r.p * (e - dl);
  } else {
    const float rN = expf(-lnN);
    r.p = g * w * rN;
    r.dw = g * rN * (e - dl);
    r.dg = w * rN * (e - dl);
  }
  return r;
}

// 3. query side: one workgroup per (16-query tile, query head, batch row);
// the tile lies in one chunk c (C is a multiple of 16)
template <int D>
struct BwQLds {
  static constexpr int RS = D + BW_PAD;
  static constexpr int KT = 32;
  static constexpr int bytes =
      (3 * BW_QT * RS + 3 * KT * RS + 2 * BW_QT * (KT + 1) + 2 * BW_QT + KT) * 4 + KT * 4;
};

template <typename T, int D>
__global__ __launch_bounds__(BW_THREADS) void bw_query_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int RS = D + BW_PAD, DPT = D / 16, KT = BwQLds<D>::KT;
  float* Qs = reinterpret_cast<float*>(smem);
  float* PQs = Qs + BW_QT * RS;
  float* DYs = PQs + BW_QT * RS;
  float* Ks = DYs + BW_QT * RS;
  float* PKs = Ks + KT * RS;
  float* Vs = PKs + KT * RS;
  float* DS = Vs + KT * RS;            // [QT][KT + 1]
  float* DW = DS + BW_QT * (KT + 1);   // [QT][KT + 1]
  float* rowN = DW + BW_QT * (KT + 1);
  float* rowD = rowN + BW_QT;
  int* kpos = reinterpret_cast<int*>(rowD + BW_QT);  // [KT] key positions (-1: none)
  int* ksa = kpos + KT;                              // [KT] kept (pool) flags
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.x * BW_QT, h = blockIdx.y, b = blockIdx.z;
  const int L = a.L, C = a.C, kv = h / a.G;
  const float g = a.gate[h];
  const size_t qrow0 = ((size_t)b * a.Hq + h) * L;
  const size_t unit = (size_t)b * a.Hkv + kv, krow0 = unit * L;
  const int c = t0 / C, cf = full_chunks_before(c, a.W, C), bc = cf * C;
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
  const int qi = tid >> 4, sub = tid & 15;
  const int t = t0 + qi;
  float dqa[DPT], dpa[DPT], dg = 0.f;
#pragma unroll
  for (int cc = 0; cc < DPT; ++cc) dqa[cc] = dpa[cc] = 0.f;
  // key tiles: the band [bc, min(t0 + 15, L - 1)] in order, then the kept
  // pool's entries (sel rows of the chunks before cf, all valid)
  const int band_hi = min(t0 + BW_QT, L);
  const int n_band = (band_hi - bc + KT - 1) / KT;
  const int n_pool = pool_count_at(cf, a.lam, a.cap_chunks);
  const int32_t* pool = a.sel + unit * (size_t)a.n_dec * a.lam;
  const int n_tiles = n_band + (n_pool + KT - 1) / KT;
  for (int it = 0; it < n_tiles; ++it) {
    __syncthreads();  // the previous tile is done with Ks .. kpos
    const bool band = it < n_band;
    if (tid < KT) {
      int p = -1;
      if (band) {
        const int j = bc + it * KT + tid;
        p = j < band_hi ? j : -1;
      } else {
        const int e = (it - n_band) * KT + tid;
        p = e < n_pool ? pool[e] : -1;
      }
      kpos[tid] = p;
      ksa[tid] = band ? (p >= 0 ? a.kept[krow0 + p] : 0) : 1;
    }
    __syncthreads();
    bw_load_rows<T, D>(Ks, reinterpret_cast<const T*>(a.k) + krow0 * D, kpos, KT);
    bw_load_rows<float, D>(PKs, a.phk + krow0 * D, kpos, KT);
    bw_load_rows<T, D>(Vs, reinterpret_cast<const T*>(a.v) + krow0 * D, kpos, KT);
    __syncthreads();
    const float lnN = rowN[qi], dl = rowD[qi];
#pragma unroll
    for (int u = 0; u < KT / 16; ++u) {
      const int kk = (KT / 16) * sub + u, j = kpos[kk];
      float ds = 0.f, dw = 0.f;
      if (t < L && j >= 0 && j <= t) {
        float s, w, e;
        bw_dots<D>(Qs + qi * RS, PQs + qi * RS, DYs + qi * RS, Ks + kk * RS, PKs + kk * RS, Vs + kk * RS, s, w,
                   e);
        const bool sa = band ? bw_is_sa(t, j, a.W, C, ksa[kk] != 0) : true;
        const BwPair pr = bw_pair(sa, s, w, e, g, lnN, dl, a.scale);
        ds = pr.ds;
        dw = pr.dw;
        dg += pr.dg;
      }
      DS[qi * (KT + 1) + kk] = ds;
      DW[qi * (KT + 1) + kk] = dw;
    }
    __syncthreads();
    for (int kk = 0; kk < KT; ++kk) {
      const float ds = DS[qi * (KT + 1) + kk], dw = DW[qi * (KT + 1) + kk];
#pragma unroll
      for (int cc = 0; cc < DPT; ++cc) {
        dqa[cc] = fmaf(ds, Ks[kk * RS + sub + 16 * cc], dqa[cc]);
        dpa[cc] = fmaf(dw, PKs[kk * RS + sub + 16 * cc], dpa[cc]);
      }
    }
  }
  // the state term: P = state of the chunks < cf (prefix entry cf - 1);
  // dg needs it whatever the gate
  if (cf > 0 && t < L) {
    const float* P = a.cS + (unit * a.T + (cf - 1)) * (size_t)(D * D + D);
    const float lnN = rowN[qi], dl = rowD[qi], rN = expf(-lnN);
    const float* dyr = DYs + qi * RS;
    float pu = 0.f, pz = 0.f;
#pragma unroll
    for (int cc = 0; cc < DPT; ++cc) {
      const int i = sub + 16 * cc;
      const float* Pi = P + (size_t)i * D;
      float u = 0.f;
      for (int k = 0; k < D; k += 4) {
        const f32x4 pv = *reinterpret_cast<const f32x4*>(Pi + k);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(dyr + k);
        u = fmaf(pv[0], dv[0], fmaf(pv[1], dv[1], fmaf(pv[2], dv[2], fmaf(pv[3], dv[3], u))));
      }
      const float zi = P[D * D + i];
      dpa[cc] += g * rN * (u - zi * dl);
      pu += PQs[qi * RS + i] * u;
      pz += PQs[qi * RS + i] * zi;
    }
    dg += rN * (pu - dl * pz);
  }
  if (t < L) {
#pragma unroll
    for (int cc = 0; cc < DPT; ++cc) {
      a.dq[(qrow0 + t) * D + sub + 16 * cc] = a.scale * dqa[cc];
      a.dphq[(qrow0 + t) * D + sub + 16 * cc] = dpa[cc];
    }
  }
  dg = wave_sum(dg);
  __syncthreads();
  if (lane == 0) rowN[wave] = dg;
  __syncthreads();
  if (tid == 0) atomicAdd(a.dgate + h, rowN[0] + rowN[1] + rowN[2] + rowN[3]);
}

// Last chunk whose queries hold key chunk cj in their band (cf(c) <= cj).
__device__ __forceinline__ int bw_band_last_chunk(int cj, int W, int C, int T) {
  int c = cj;
  while (c + 1 < T && full_chunks_before(c + 1, W, C) <= cj) ++c;
  return c;
}

// 4. key side: one workgroup per (16-key tile, kv head, batch row); the
// tile lies in one chunk cj. Band queries: chunks cj .. c_hi (cf <= cj),
// every head of the group; then the suffix state of the chunks after c_hi
// for the unkept keys.
template <int D>
struct BwKLds {
  static constexpr int RS = D + BW_PAD;
  static constexpr int bytes = (3 * BW_KT * RS + 3 * BW_QT * RS + 3 * BW_KT * (BW_QT + 1) + 2 * BW_QT) * 4 + BW_KT * 4;
};

template <typename T, int D>
__global__ __launch_bounds__(BW_THREADS) void bw_key_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int RS = D + BW_PAD, DPT = D / 16;
  float* Ks = reinterpret_cast<float*>(smem);
  float* PKs = Ks + BW_KT * RS;
  float* Vs = PKs + BW_KT * RS;
  float* Qs = Vs + BW_KT * RS;
  float* PQs = Qs + BW_QT * RS;
  float* DYs = PQs + BW_QT * RS;
  float* PS = DYs + BW_QT * RS;          // [KT][QT + 1]
  float* DS = PS + BW_KT * (BW_QT + 1);  // [KT][QT + 1]
  float* DW = DS + BW_KT * (BW_QT + 1);  // [KT][QT + 1]
  float* rowN = DW + BW_KT * (BW_QT + 1);
  float* rowD = rowN + BW_QT;
  int* kp = reinterpret_cast<int*>(rowD + BW_QT);  // [KT] kept flags
  const int tid = threadIdx.x;
  const int j0 = blockIdx.x * BW_KT, kv = blockIdx.y, b = blockIdx.z;
  const int L = a.L, C = a.C;
  const size_t unit = (size_t)b * a.Hkv + kv, krow0 = unit * L;
  const int cj = j0 / C, c_hi = bw_band_last_chunk(cj, a.W, C, a.T);
  for (int e = tid; e < BW_KT * D; e += BW_THREADS) {
    const int i = e / D, d = e % D, j = j0 + i;
    const bool in = j < L;
    Ks[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.k)[(krow0 + j) * D + d]) : 0.f;
    PKs[i * RS + d] = in ? a.phk[(krow0 + j) * D + d] : 0.f;
    Vs[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.v)[(krow0 + j) * D + d]) : 0.f;
  }
  if (tid < BW_KT) kp[tid] = j0 + tid < L ? a.kept[krow0 + j0 + tid] : 0;
  const int qi = tid >> 4, sub = tid & 15;   // phase 1: query row, key
  const int kk2 = tid >> 4, part = tid & 15;  // phase 2: key row, columns part + 16 c
  float dka[DPT], dpa[DPT], dva[DPT];
#pragma unroll
  for (int cc = 0; cc < DPT; ++cc) dka[cc] = dpa[cc] = dva[cc] = 0.f;
  const int t_end = min(L, (c_hi + 1) * C);
  for (int hl = 0; hl < a.G; ++hl) {
    const int h = kv * a.G + hl;
    const float g = a.gate[h];
    const size_t qrow0 = ((size_t)b * a.Hq + h) * L;
    for (int t0 = j0; t0 < t_end; t0 += BW_QT) {
      __syncthreads();  // the previous query tile is done with Qs .. DW
      for (int e = tid; e < BW_QT * D; e += BW_THREADS) {
        const int i = e / D, d = e % D, t = t0 + i;
        const bool in = t < t_end;
        Qs[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.q)[(qrow0 + t) * D + d]) : 0.f;
        PQs[i * RS + d] = in ? a.phq[(qrow0 + t) * D + d] : 0.f;
        DYs[i * RS + d] = in ? a.dy[(qrow0 + t) * D + d] : 0.f;
      }
      if (tid < BW_QT) {
        const int t = t0 + tid;
        rowN[tid] = t < t_end ? a.lnN[qrow0 + t] : 0.f;
        rowD[tid] = t < t_end ? a.delta[qrow0 + t] : 0.f;
      }
      __syncthreads();
      const int t = t0 + qi, kk = sub, j = j0 + kk;
      BwPair pr{0.f, 0.f, 0.f, 0.f};
      if (t < t_end && j < L && j <= t) {
        float s, w, e;
        bw_dots<D>(Qs + qi * RS, PQs + qi * RS, DYs + qi * RS, Ks + kk * RS, PKs + kk * RS, Vs + kk * RS, s, w,
                   e);
        pr = bw_pair(bw_is_sa(t, j, a.W, C, kp[kk] != 0), s, w, e, g, rowN[qi], rowD[qi], a.scale);
      }
      PS[kk * (BW_QT + 1) + qi] = pr.p;
      DS[kk * (BW_QT + 1) + qi] = pr.ds;
      DW[kk * (BW_QT + 1) + qi] = pr.dw;
      __syncthreads();
      for (int i = 0; i < BW_QT; ++i) {
        const float p = PS[kk2 * (BW_QT + 1) + i], ds = DS[kk2 * (BW_QT + 1) + i], dw = DW[kk2 * (BW_QT + 1) + i];
#pragma unroll
        for (int cc = 0; cc < DPT; ++cc) {
          dka[cc] = fmaf(ds, Qs[i * RS + part + 16 * cc], dka[cc]);
          dpa[cc] = fmaf(dw, PQs[i * RS + part + 16 * cc], dpa[cc]);
          dva[cc] = fmaf(p, DYs[i * RS + part + 16 * cc], dva[cc]);
        }
      }
    }
  }
  // suffix state of the chunks after c_hi (their queries hold key j in the
  // state when j is unkept): d phi(k) += R v - r, dv += R^T phi(k)
  const int j = j0 + kk2;
  if (c_hi + 1 < a.T && j < L && !kp[kk2]) {
    const float* R = a.cR + (unit * a.T + (c_hi + 1)) * (size_t)(D * D + D);
    const float* vr = Vs + kk2 * RS;
    const float* pr = PKs + kk2 * RS;
    float u[DPT], w[DPT];
#pragma unroll
    for (int cc = 0; cc < DPT; ++cc) u[cc] = w[cc] = 0.f;
#pragma unroll 2
    for (int k = 0; k < D; ++k) {
      const float vk = vr[k], pk = pr[k];
#pragma unroll
      for (int cc = 0; cc < DPT; ++cc) {
        const int i = part + 16 * cc;
        u[cc] = fmaf(R[(size_t)i * D + k], vk, u[cc]);  // (R v)_i
        w[cc] = fmaf(R[(size_t)k * D + i], pk, w[cc]);  // (R^T phi(k))_i
      }
    }
#pragma unroll
    for (int cc = 0; cc < DPT; ++cc) {
      dpa[cc] += u[cc] - R[D * D + part + 16 * cc];
      dva[cc] += w[cc];
    }
  }
  if (j < L) {
#pragma unroll
    for (int cc = 0; cc < DPT; ++cc) {
      a.dk[(krow0 + j) * D + part + 16 * cc] = a.scale * dka[cc];
      a.dphk[(krow0 + j) * D + part + 16 * cc] = dpa[cc];
      a.dv[(krow0 + j) * D + part + 16 * cc] = dva[cc];
    }
  }
}

// 5. kept keys: one workgroup per (16 consecutive entries of the unit's
// selection, kv head, (batch row, query head of the group, query segment)).
// Entry j (kept, chunk cj) is a softmax key of every query of the chunks
// after bw_band_last_chunk(cj) (the band pairs were taken by the key-side
// kernel); each workgroup adds its segment's share of dk, dv atomically.
constexpr int BW_POOL_SEG = 512;  // queries per segment
template <typename T, int D>
__global__ __launch_bounds__(BW_THREADS) void bw_pool_kernel(BackwardArgs a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int RS = D + BW_PAD, DPT = D / 16;
  float* Ks = reinterpret_cast<float*>(smem);
  float* PKs = Ks + BW_KT * RS;  // (unused; keeps the key kernel's layout)
  float* Vs = PKs + BW_KT * RS;
  float* Qs = Vs + BW_KT * RS;
  float* PQs = Qs + BW_QT * RS;
  float* DYs = PQs + BW_QT * RS;
  float* PS = DYs + BW_QT * RS;
  float* DS = PS + BW_KT * (BW_QT + 1);
  float* DW = DS + BW_KT * (BW_QT + 1);
  float* rowN = DW + BW_KT * (BW_QT + 1);
  float* rowD = rowN + BW_QT;
  int* kpos = reinterpret_cast<int*>(rowD + BW_QT);  // [KT]
  __shared__ int tstart[BW_KT];
  const int tid = threadIdx.x;
  const int L = a.L, C = a.C;
  const int n_seg = (L + BW_POOL_SEG - 1) / BW_POOL_SEG;
  const int e0 = blockIdx.x * BW_KT, kv = blockIdx.y;
  const int seg = blockIdx.z % n_seg, hl = (blockIdx.z / n_seg) % a.G, b = blockIdx.z / (n_seg * a.G);
  const size_t unit = (size_t)b * a.Hkv + kv, krow0 = unit * L;
  const int n_kept = pool_count_at(a.n_dec, a.lam, a.cap_chunks);
  const int32_t* pool = a.sel + unit * (size_t)a.n_dec * a.lam;
  if (tid < BW_KT) {
    const int e = e0 + tid;
    const int j = e < n_kept ? pool[e] : -1;
    kpos[tid] = j;
    tstart[tid] = j >= 0 ? (bw_band_last_chunk(j / C, a.W, C, a.T) + 1) * C : L;
  }
  __syncthreads();
  bw_load_rows<T, D>(Ks, reinterpret_cast<const T*>(a.k) + krow0 * D, kpos, BW_KT);
  bw_load_rows<T, D>(Vs, reinterpret_cast<const T*>(a.v) + krow0 * D, kpos, BW_KT);
  int t_first = L;
  for (int i = 0; i < BW_KT; ++i) t_first = min(t_first, tstart[i]);
  t_first = max(t_first / BW_QT * BW_QT, seg * BW_POOL_SEG);
  const int t_last = min(L, (seg + 1) * BW_POOL_SEG);
  const int qi = tid >> 4, sub = tid & 15;
  const int kk2 = tid >> 4, part = tid & 15;
  float dka[DPT], dva[DPT];
#pragma unroll
  for (int cc = 0; cc < DPT; ++cc) dka[cc] = dva[cc] = 0.f;
  {
    const int h = kv * a.G + hl;
    const size_t qrow0 = ((size_t)b * a.Hq + h) * L;
    for (int t0 = t_first; t0 < t_last; t0 += BW_QT) {
      __syncthreads();
      for (int e = tid; e < BW_QT * D; e += BW_THREADS) {
        const int i = e / D, d = e % D, t = t0 + i;
        const bool in = t < t_last;
        Qs[i * RS + d] = in ? to_f32(reinterpret_cast<const T*>(a.q)[(qrow0 + t) * D + d]) : 0.f;
        DYs[i * RS + d] = in ? a.dy[(qrow0 + t) * D + d] : 0.f;
      }
      if (tid < BW_QT) {
        const int t = t0 + tid;
        rowN[tid] = t < t_last ? a.lnN[qrow0 + t] : 0.f;
        rowD[tid] = t < t_last ? a.delta[qrow0 + t] : 0.f;
      }
      __syncthreads();
      const int t = t0 + qi, kk = sub;
      float p = 0.f, ds = 0.f;
      if (t < t_last && kpos[kk] >= 0 && t >= tstart[kk]) {
        float s = 0.f, e = 0.f;
        const float *q = Qs + qi * RS, *k = Ks + kk * RS, *dy = DYs + qi * RS, *v = Vs + kk * RS;
        for (int d = 0; d < D; d += 4) {
          const f32x4 qa = *reinterpret_cast<const f32x4*>(q + d), ka = *reinterpret_cast<const f32x4*>(k + d);
          const f32x4 ya = *reinterpret_cast<const f32x4*>(dy + d), va = *reinterpret_cast<const f32x4*>(v + d);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s = fmaf(qa[i], ka[i], s);
            e = fmaf(ya[i], va[i], e);
          }
        }
        p = expf(a.scale * s - rowN[qi]);
        ds = p * (e - rowD[qi]);
      }
      PS[kk * (BW_QT + 1) + qi] = p;
      DS[kk * (BW_QT + 1) + qi] = ds;
      __syncthreads();
      for (int i = 0; i < BW_QT; ++i) {
        const float pp = PS[kk2 * (BW_QT + 1) + i], dd = DS[kk2 * (BW_QT + 1) + i];
#pragma unroll
        for (int cc = 0; cc < DPT; ++cc) {
          dka[cc] = fmaf(dd, Qs[i * RS + part + 16 * cc], dka[cc]);
          dva[cc] = fmaf(pp, DYs[i * RS + part + 16 * cc], dva[cc]);
        }
      }
    }
  }
  const int j = kpos[kk2];
  if (j >= 0 && t_first < t_last) {
#pragma unroll
    for (int cc = 0; cc < DPT; ++cc) {
      atomicAdd(a.dk + (krow0 + j) * D + part + 16 * cc, a.scale * dka[cc]);
      atomicAdd(a.dv + (krow0 + j) * D + part + 16 * cc, dva[cc]);
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
