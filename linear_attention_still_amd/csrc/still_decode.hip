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
// [P3 "Delayed Chunk-Level Selection ..."]. One workgroup (8 waves) per
// (kv head, batch row) unit:
//   1. when a new chunk begins: Top-lambda of the finished chunk over its
//      float64 scores, kept tokens appended to the pool [P2 固定预算路由];
//      the chunk(s) now wholly before the window folded into S, z;
//   2. the new token enters the ring (key, value, NP-Map feature);
//   3. every query head of the group attends: softmax over kept tokens
//      below the window and over the window / own-chunk tokens in the ring,
//      gated linear weights over ring tokens already out of the window but
//      not yet folded, and the state S, z as one virtual key; all weights
//      share one normaliser (reading of the branch merge);
//   4. the new token's float64 score joins the undecided chunk's scores
//      (its window logits come from the same pass over the ring keys).
//
// The step is bound by HBM reads (pool and ring K/V, S): rows are read as
// 16-byte vectors, D / (16 / sizeof(T)) consecutive lanes per row, several
// rows in flight per lane, and partial sums are combined through LDS once.
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

constexpr int DEC_THREADS = 512;
constexpr int DEC_WAVES = DEC_THREADS / 64;
constexpr int DEC_MAP_ROWS = 16;  // rows per NP-Map batch

// LDS carve-up of the decode kernel, in bytes from the base.
template <typename T, int D, int G>
struct DecLds {
  static constexpr size_t qs = 0;                                  // f32 [G][D]
  static constexpr size_t phq = qs + (size_t)G * D * 4;            // f32 [G][D]
  static constexpr size_t hv = phq + (size_t)G * D * 4;            // f32 [G][4]
  static constexpr size_t ibuf = hv + (size_t)G * 4 * 4;           // int [2 + 130]
  static constexpr size_t d64 = ibuf + (2 + 130) * 4;              // f64 [128 + 8]
  static constexpr size_t rowst = d64 + (128 + 8) * 8;             // f32 [16][2]
  static constexpr size_t uni = rowst + DEC_MAP_ROWS * 2 * 4;      // union below
  // union member 1 (NP-Map and fold): xs, us, ph, vs f32 [16][D] each
  static constexpr size_t map_bytes = (size_t)4 * DEC_MAP_ROWS * D * 4;
  // union member 2 (value and state partial sums): f32 [2][waves][G][D]
  static constexpr size_t red_bytes = (size_t)2 * DEC_WAVES * G * D * 4;
  static constexpr size_t uni_bytes = map_bytes > red_bytes ? map_bytes : red_bytes;
  static constexpr size_t lg = uni + uni_bytes;                    // f64 [G][W] (runtime W)
  __host__ __device__ static size_t lw(int W) { return lg + (size_t)G * W * 8; }  // f32 [G][NK]
  __host__ __device__ static size_t bytes(int W, int NK) { return lw(W) + (size_t)G * NK * 4; }
};

// 16 bytes of a row as floats.
template <typename T>
struct RowVec;
template <>
struct RowVec<bf16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void get(const uint4& u, float (&x)[8]) {
    const bf16* e = reinterpret_cast<const bf16*>(&u);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)e[i];
  }
};
template <>
struct RowVec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void get(const uint4& u, float (&x)[4]) {
    const float* e = reinterpret_cast<const float*>(&u);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = e[i];
  }
};

// Sum over the n consecutive lanes (n a power of two) that hold one row.
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
#pragma unroll
  for (int o = 1; o < N; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
template <int N>
__device__ __forceinline__ double sum_lanes_f64(double x) {
#pragma unroll
  for (int o = 1; o < N; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// NP-Map [P3 "NP-Map: Norm-Preserving Feature Map"] of n <= 16 rows of xs
// (float32, row stride D) into ph; reading: ||x|| * softmax(x F) /
// ||softmax(x F)||, exact expf. us is scratch; rowst holds (max, scale).
// All threads; ends with a barrier.
template <typename T, int D>
__device__ __forceinline__ void np_map_rows(const T* F, const float* xs, int n, float* us,
                                            float* ph, float* rowst) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < n * D; e += DEC_THREADS) {
    const int r = e / D, j = e % D;
    const float* x = xs + r * D;
    float u0 = 0.f, u1 = 0.f;
#pragma unroll 8
    for (int i = 0; i < D; i += 2) {
      u0 += x[i] * to_f32(F[(size_t)i * D + j]);
      u1 += x[i + 1] * to_f32(F[(size_t)(i + 1) * D + j]);
    }
    us[e] = u0 + u1;
  }
  __syncthreads();
  for (int r = wave; r < n; r += DEC_WAVES) {
    float mx = STILL_NEG_INF, xn = 0.f;
    for (int j = lane; j < D; j += 64) {
      mx = fmaxf(mx, us[r * D + j]);
      xn += xs[r * D + j] * xs[r * D + j];
    }
    mx = wave_max(mx);
    xn = wave_sum(xn);
    float ss = 0.f;
    for (int j = lane; j < D; j += 64) {
      const float e = expf(us[r * D + j] - mx);
      ss += e * e;
    }
    ss = wave_sum(ss);
    if (lane == 0) {
      rowst[2 * r] = mx;
      rowst[2 * r + 1] = sqrtf(xn) / sqrtf(ss);
    }
  }
  __syncthreads();
  for (int e = tid; e < n * D; e += DEC_THREADS) {
    const int r = e / D;
    ph[e] = expf(us[e] - rowst[2 * r]) * rowst[2 * r + 1];
  }
  __syncthreads();
}


// Chunk boundary (position t = cC): decide chunk c-1 by Top-lambda over its
// float64 scores, append the kept tokens to the pool [P2 固定预算路由], and
// fold the chunks that are now wholly before the window into S, z. Runs
// before decode_kernel of the same step; on a position mismatch it does
// nothing (decode_kernel then flags the error).
template <typename T, int D>
__global__ __launch_bounds__(DEC_THREADS) void decode_boundary_kernel(DecodeArgs a) {
  using LD = DecLds<T, D, 1>;
  constexpr int VEC = RowVec<T>::N;
  constexpr int LPK = D / VEC;
  extern __shared__ __align__(16) char smem[];
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int unit = b * a.Hkv + kv;
  const int W = a.W, C = a.C, R = a.R, t = a.t;
  char* st = a.state + (size_t)unit * a.st_unit;
  int64_t* meta = reinterpret_cast<int64_t*>(st + a.st_meta);
  float* S = reinterpret_cast<float*>(st + a.st_S);
  float* z = reinterpret_cast<float*>(st + a.st_z);
  T* pool_k = reinterpret_cast<T*>(st + a.st_pool_k);
  T* pool_v = reinterpret_cast<T*>(st + a.st_pool_v);
  int32_t* pool_pos = reinterpret_cast<int32_t*>(st + a.st_pool_pos);
  T* ring_k = reinterpret_cast<T*>(st + a.st_ring_k);
  T* ring_v = reinterpret_cast<T*>(st + a.st_ring_v);
  int32_t* ring_flag = reinterpret_cast<int32_t*>(st + a.st_ring_flag);
  double* pend = reinterpret_cast<double*>(st + a.st_pending);
  const T* F = reinterpret_cast<const T*>(a.fmap_w) + (size_t)kv * D * D;
  int* ibuf = reinterpret_cast<int*>(smem + LD::ibuf);
  double* d64 = reinterpret_cast<double*>(smem + LD::d64);
  float* rowst = reinterpret_cast<float*>(smem + LD::rowst);
  float* xs = reinterpret_cast<float*>(smem + LD::uni);
  float* us = xs + DEC_MAP_ROWS * D;
  float* ph = us + DEC_MAP_ROWS * D;
  float* vs = ph + DEC_MAP_ROWS * D;
  if (meta[0] != t || meta[2] != 0) return;
  int n_pool = (int)meta[1];
  const int c = t / C, cC = c * C;
  double* ps = d64;      // [C] scores of the finished chunk
  int* kept = ibuf + 2;  // [C] rank among kept, or -1
  for (int j = tid; j < C; j += DEC_THREADS) ps[j] = pend[j];
  __syncthreads();
  const int lam_c = (n_pool + a.lam <= a.m - W) ? a.lam : 0;
  for (int j = tid; j < C; j += DEC_THREADS) {
    int r = 0;  // rank by (score desc, position asc)
    for (int i = 0; i < C; ++i) r += (ps[i] > ps[j] || (ps[i] == ps[j] && i < j)) ? 1 : 0;
    kept[j] = r < lam_c ? 1 : 0;
  }
  __syncthreads();
  if (tid == 0) {  // kept positions in ascending order -> pool rows
    int k2 = 0;
    for (int j = 0; j < C; ++j) kept[j] = kept[j] ? k2++ : -1;
  }
  __syncthreads();
  const int base = cC - C;
  for (int e = tid; e < C * LPK; e += DEC_THREADS) {
    const int j = e / LPK, part = e % LPK;
    if (kept[j] < 0) continue;
    const int pos = base + j, slot = pos % R, row = n_pool + kept[j];
    const size_t src = (size_t)slot * D + part * VEC, dst = (size_t)row * D + part * VEC;
    *reinterpret_cast<uint4*>(pool_k + dst) = *reinterpret_cast<const uint4*>(ring_k + src);
    *reinterpret_cast<uint4*>(pool_v + dst) = *reinterpret_cast<const uint4*>(ring_v + src);
    if (part == 0) {
      pool_pos[row] = pos;
      ring_flag[slot] = 1;
      if (a.sel_new) a.sel_new[(size_t)unit * a.lam + kept[j]] = pos;
    }
  }
  if (a.sel_new)
    for (int i = lam_c + tid; i < a.lam; i += DEC_THREADS) a.sel_new[(size_t)unit * a.lam + i] = -1;
  for (int j = tid; j < C; j += DEC_THREADS) pend[j] = __builtin_nan("");
  n_pool += lam_c;
  __syncthreads();
  if (tid == 0) meta[1] = n_pool;

  // fold chunks [cf(c-1), cf(c)) into S, z (float32 features, exact expf)
  const int f_lo = full_chunks_before(c - 1, W, C) * C;
  const int f_hi = full_chunks_before(c, W, C) * C;
  constexpr int PER = D * D / DEC_THREADS;
  float dacc[PER];
#pragma unroll
  for (int q2 = 0; q2 < PER; ++q2) dacc[q2] = 0.f;
  float dz = 0.f;
  for (int g0 = f_lo; g0 < f_hi; g0 += DEC_MAP_ROWS) {
    const int n = min(DEC_MAP_ROWS, f_hi - g0);
    for (int e = tid; e < DEC_MAP_ROWS * D; e += DEC_THREADS) {
      const int r = e / D, i = e % D, pos = g0 + r;
      const int slot = pos % R;
      const bool use = r < n && ring_flag[slot] == 0;
      xs[e] = use ? to_f32(ring_k[(size_t)slot * D + i]) : 0.f;
      vs[e] = use ? to_f32(ring_v[(size_t)slot * D + i]) : 0.f;
    }
    __syncthreads();
    np_map_rows<T, D>(F, xs, DEC_MAP_ROWS, us, ph, rowst);
    // thread tid owns S[i][jv] for jv = tid % D and i = tid / D + q2 * (512 / D)
#pragma unroll 1
    for (int r = 0; r < DEC_MAP_ROWS; ++r) {
      const float vr = vs[r * D + tid % D];
      const float* pr = ph + r * D + tid / D;
#pragma unroll
      for (int q2 = 0; q2 < PER; ++q2) dacc[q2] += pr[q2 * (DEC_THREADS / D)] * vr;
    }
    if (tid < D)
      for (int r = 0; r < DEC_MAP_ROWS; ++r) dz += ph[r * D + tid];
    __syncthreads();
  }
  if (f_hi > f_lo) {
#pragma unroll
    for (int q2 = 0; q2 < PER; ++q2) S[tid + DEC_THREADS * q2] += dacc[q2];
    if (tid < D) z[tid] += dz;
  }
  __syncthreads();
}

template <typename T, int D, int G>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(DecodeArgs a) {
  using LD = DecLds<T, D, G>;
  constexpr int VEC = RowVec<T>::N;  // elements per 16-byte vector
  constexpr int LPK = D / VEC;       // lanes per K/V row
  constexpr int KPW = 64 / LPK;      // rows per wave and vector load
  constexpr int SL = D / 4;          // lanes per S row (float4)
  constexpr int RPW = 64 / SL;       // S rows per wave and vector load
  constexpr int U = G >= 8 ? 2 : 4;  // rows in flight per lane
  extern __shared__ __align__(16) char smem[];
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int unit = b * a.Hkv + kv;
  const int W = a.W, C = a.C, R = a.R, t = a.t;
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

  float* qs = reinterpret_cast<float*>(smem + LD::qs);
  float* phq = reinterpret_cast<float*>(smem + LD::phq);
  float* hv = reinterpret_cast<float*>(smem + LD::hv);
  int* ibuf = reinterpret_cast<int*>(smem + LD::ibuf);
  double* d64 = reinterpret_cast<double*>(smem + LD::d64);
  float* rowst = reinterpret_cast<float*>(smem + LD::rowst);
  float* xs = reinterpret_cast<float*>(smem + LD::uni);
  float* us = xs + DEC_MAP_ROWS * D;
  float* ph = us + DEC_MAP_ROWS * D;
  float* vs = ph + DEC_MAP_ROWS * D;
  float* red = reinterpret_cast<float*>(smem + LD::uni);  // [2][waves][G][D]
  double* lg = reinterpret_cast<double*>(smem + LD::lg);
  float* lw = reinterpret_cast<float*>(smem + LD::lw(W));
  const int NK = a.n_keys_max;

  if (meta[0] != t || meta[2] != 0) {
    __syncthreads();
    if (tid == 0 && meta[2] == 0) meta[2] = -5;
    return;
  }
  int n_pool = (int)meta[1];
  const int c = t / C, cC = c * C;

  if (a.sel_new && !a.boundary)
    for (int i = tid; i < a.lam; i += DEC_THREADS) a.sel_new[(size_t)unit * a.lam + i] = -1;

  // ---- 2. the new token enters the ring; phi(q_h), phi(k_t) ---------------
  const T* kin = reinterpret_cast<const T*>(a.k) + (size_t)unit * D;
  const T* vin = reinterpret_cast<const T*>(a.v) + (size_t)unit * D;
  const int slot_t = t % R;
  for (int i = tid; i < D; i += DEC_THREADS) {
    xs[G * D + i] = to_f32(kin[i]);
    ring_k[(size_t)slot_t * D + i] = kin[i];
    ring_v[(size_t)slot_t * D + i] = vin[i];
  }
  if (tid == 0) ring_flag[slot_t] = 0;
  for (int e = tid; e < G * D; e += DEC_THREADS) {
    const float x = to_f32(reinterpret_cast<const T*>(a.q)[((size_t)b * a.Hq + kv * G) * D + e]);
    qs[e] = x;
    xs[e] = x;
  }
  __syncthreads();
  np_map_rows<T, D>(F, xs, G + 1, us, ph, rowst);
  for (int e = tid; e < G * D; e += DEC_THREADS) phq[e] = ph[e];
  for (int i = tid; i < D; i += DEC_THREADS) ring_phi[(size_t)slot_t * D + i] = from_f32<T>(ph[G * D + i]);

  // key sets [P3 "Content-Aware Routing ..."]: kept tokens below lo, the ring
  // from lo to t (window and own chunk), ring tokens [la_lo, la_hi] that are
  // out of the window and unkept (linear), then S, z.
  int lo = t - W + 1 < cC ? t - W + 1 : cC;
  if (lo < 0) lo = 0;
  if (tid == 0) ibuf[0] = 0;
  __syncthreads();
  {
    int cnt = 0;  // pool positions ascend: count those below lo
    for (int i = tid; i < n_pool; i += DEC_THREADS) cnt += pool_pos[i] < lo ? 1 : 0;
    cnt = (int)wave_sum((float)cnt);
    if (lane == 0 && cnt) atomicAdd(&ibuf[0], cnt);
  }
  __syncthreads();
  const int n_oob = ibuf[0];
  const int n_win = t - lo + 1;
  const int n_sa = n_oob + n_win;
  const int la_lo = full_chunks_before(c, W, C) * C;
  const int la_hi = min(t - W, cC - 1);  // inclusive
  const int n_la = la_hi >= la_lo ? la_hi - la_lo + 1 : 0;
  const int n_keys = n_sa + n_la;
  const int sc_lo = t - W + 1 > 0 ? t - W + 1 : 0;  // score window

  const int part = lane % LPK, grp = lane / LPK;
  auto key_row = [&](int kk) -> const T* {
    return kk < n_oob ? pool_k + (size_t)kk * D : ring_k + (size_t)((lo + kk - n_oob) % R) * D;
  };
  auto val_row = [&](int kk) -> const T* {
    if (kk < n_oob) return pool_v + (size_t)kk * D;
    if (kk < n_sa) return ring_v + (size_t)((lo + kk - n_oob) % R) * D;
    return ring_v + (size_t)((la_lo + kk - n_sa) % R) * D;
  };

  // ---- 3a. softmax logits (float32) and window logits (float64) -----------
  {
    float qv[G][VEC];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) qv[h][e] = qs[h * D + part * VEC + e];
    for (int k0 = wave * KPW * U; k0 < n_sa; k0 += DEC_WAVES * KPW * U) {
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k0 + u * KPW + grp;
        raw[u] = kk < n_sa ? *reinterpret_cast<const uint4*>(key_row(kk) + part * VEC)
                           : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k0 + u * KPW + grp;
        float x[VEC];
        RowVec<T>::get(raw[u], x);
        const int pos = kk < n_oob ? -1 : lo + kk - n_oob;
        const bool in_sc = kk < n_sa && pos >= sc_lo;  // uniform over the row's lanes
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) s += qv[h][e] * x[e];
          s = sum_lanes<LPK>(s);
          if (part == 0 && kk < n_sa) lw[h * NK + kk] = s * a.scale;
          if (in_sc) {  // products of bf16/f32 values are exact in float64
            double s64 = 0.0;
#pragma unroll
            for (int e = 0; e < VEC; ++e) s64 += (double)qv[h][e] * (double)x[e];
            s64 = sum_lanes_f64<LPK>(s64);
            if (part == 0) lg[h * W + (pos - sc_lo)] = a.scale64 * s64;
          }
        }
      }
    }
  }
  // ---- 3b. gated linear weights of the unfolded ring tokens ----------------
  {
    float pv[G][VEC];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) pv[h][e] = phq[h * D + part * VEC + e];
    for (int k0 = wave * KPW; k0 < n_la; k0 += DEC_WAVES * KPW) {
      const int kk = k0 + grp;
      const int slot = (la_lo + kk) % R;
      uint4 raw = uint4{0, 0, 0, 0};
      bool la = false;
      if (kk < n_la) {
        raw = *reinterpret_cast<const uint4*>(ring_phi + (size_t)slot * D + part * VEC);
        la = ring_flag[slot] == 0;
      }
      float x[VEC];
      RowVec<T>::get(raw, x);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float w = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) w += pv[h][e] * x[e];
        w = sum_lanes<LPK>(w);
        const float g = a.gate[kv * G + h];
        if (part == 0 && kk < n_la)
          lw[h * NK + n_sa + kk] = (la && w > 0.f && g > 0.f) ? __logf(g) + __logf(w) : STILL_NEG_INF;
      }
    }
  }
  __syncthreads();

  // ---- 4. float64 score of token t [P3 "Self-Saliency Score"] and the
  //         normaliser of each head (wave h) --------------------------------
  if (wave < G) {
    const int h = wave;
    // score: KL(a_diag || (1-eps) a_nodiag + eps delta_t) in float64
    {
      const int n = t - sc_lo + 1;
      const double* x = lg + h * W;
      double mx = -__builtin_huge_val();
      for (int j = lane; j < n; j += 64) mx = x[j] > mx ? x[j] : mx;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_xor(mx, o);
        mx = y > mx ? y : mx;
      }
      double za = 0.0, zo = 0.0;
      for (int j = lane; j < n; j += 64) {
        const double e = exp(x[j] - mx);
        za += e;
        if (j != n - 1) zo += e;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        za += __shfl_xor(za, o);
        zo += __shfl_xor(zo, o);
      }
      if (lane == 0) {
        const double p = exp(x[n - 1] - mx) / za, pn = zo / za;
        double sc = 0.0;
        if (p > 0.0) sc += p * log(p / a.eps64);
        if (pn > 0.0) sc += pn * log(pn / (1.0 - a.eps64));
        d64[128 + h] = sc;
      }
    }
    // state as a virtual key: log-weight log(g * phi(q).z)
    float dz = 0.f;
    for (int i = lane; i < D; i += 64) dz += phq[h * D + i] * z[i];
    dz = wave_sum(dz);
    const float g = a.gate[kv * G + h];
    const float lws = (g > 0.f && dz > 0.f) ? __logf(g * dz) : STILL_NEG_INF;
    float mx = lws;
    for (int kk = lane; kk < n_keys; kk += 64) mx = fmaxf(mx, lw[h * NK + kk]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int kk = lane; kk < n_keys; kk += 64) {
      const float x = lw[h * NK + kk];
      const float e = x == STILL_NEG_INF ? 0.f : __expf(x - mx);
      lw[h * NK + kk] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      const float es = lws == STILL_NEG_INF ? 0.f : __expf(lws - mx);
      hv[h * 4 + 0] = dz;
      hv[h * 4 + 1] = es;
      hv[h * 4 + 2] = sum + es;
    }
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int h = 0; h < G; ++h) tot += d64[128 + h];
    pend[t - cC] = tot;
  }

  // ---- 5. weighted values and the state readout ---------------------------
  {
    float acc[G][VEC];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
    for (int k0 = wave * KPW * U; k0 < n_keys; k0 += DEC_WAVES * KPW * U) {
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k0 + u * KPW + grp;
        raw[u] = kk < n_keys ? *reinterpret_cast<const uint4*>(val_row(kk) + part * VEC)
                             : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k0 + u * KPW + grp;
        if (kk >= n_keys) continue;
        float x[VEC];
        RowVec<T>::get(raw[u], x);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float w = lw[h * NK + kk];
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] += w * x[e];
        }
      }
    }
    // the row groups of a wave, then the waves (through LDS)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int o = LPK; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o);
    if (grp == 0)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) red[(wave * G + h) * D + part * VEC + e] = acc[h][e];
  }
  {
    // nst[h][f] = sum_i phi_h[i] S[i][f]: rows of S as float4 vectors
    float acc[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;
    const int sp = lane % SL, sg = lane / SL;
    constexpr int ROUNDS = D / (DEC_WAVES * RPW);
    f32x4 sv[ROUNDS];
#pragma unroll
    for (int rr = 0; rr < ROUNDS; ++rr) {
      const int i = (rr * DEC_WAVES + wave) * RPW + sg;
      sv[rr] = *reinterpret_cast<const f32x4*>(S + (size_t)i * D + sp * 4);
    }
#pragma unroll
    for (int rr = 0; rr < ROUNDS; ++rr) {
      const int i = (rr * DEC_WAVES + wave) * RPW + sg;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = phq[h * D + i];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[h][e] += p * sv[rr][e];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int o = SL; o < 64; o <<= 1) acc[h][e] += __shfl_xor(acc[h][e], o);
    float* red2 = red + DEC_WAVES * G * D;
    if (sg == 0)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) red2[(wave * G + h) * D + sp * 4 + e] = acc[h][e];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += DEC_THREADS) {
    const int h = e / D, f = e % D;
    float sv = 0.f, ns = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      sv += red[(w * G + h) * D + f];
      ns += red[((DEC_WAVES + w) * G + h) * D + f];
    }
    const float dz = hv[h * 4 + 0], es = hv[h * 4 + 1], tot = hv[h * 4 + 2];
    if (es > 0.f) sv += es * ns / dz;
    const float y = sv / tot;
    const size_t o = ((size_t)b * a.Hq + kv * G + h) * D + f;
    if (a.fp32_out) reinterpret_cast<float*>(a.out)[o] = y;
    else reinterpret_cast<T*>(a.out)[o] = from_f32<T>(y);
  }
  if (tid == 0) {
    meta[1] = n_pool;
    meta[0] = t + 1;
  }
}

}  // namespace still
