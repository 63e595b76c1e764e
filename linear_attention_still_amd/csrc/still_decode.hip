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
// (kv head, batch row) unit, two per CU; chunk-boundary work runs in its own
// kernel (8 waves) before the step:
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
//      (its window logits from a second, cached pass over the window rows).
//
// The step is bound by HBM reads (pool and ring K/V, S): rows are read as
// tiles of 16 keys per wave, two tiles in flight; logits by MFMA, values by
// per-lane column slices; partial sums are combined through LDS once. Two
// 4-wave workgroups fit on a CU, so every unit of a 512-unit step is
// resident at once.
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
  int B, Hq, Hkv, G, W, C, m, lam, R, t, boundary, fp32_out;
  // per-row positions: row b's token is at pos[b] + t (device [B]), or null
  // (every row at t); with them the boundary kernel runs for every row and
  // returns where pos[b] + t is not a chunk start
  const int32_t* pos;
  int softmax_only;  // the linear branch dropped (every gate taken as 0)
  int pool8;         // pool rows as E4M3 codes, then a float32 scale per row
  int route;         // routing metric (ROUTE_*; not ROUTE_EXTERNAL)
  const void* out_gate;  // [B][Hq][D] T: channel-wise output gate before the sigmoid, or null
  const float* decay;    // [Hkv] forget factor of the linear state in (0, 1], or null (1)
  PoolPages pages;       // the pool rows in pages (base null: in the state)
  float scale, eps;
  double scale64, eps64;  // the same parameters for the float64 score
  long st_unit, st_S, st_z, st_pool_k, st_pool_v, st_pool_pos, st_ring_k, st_ring_v,
      st_ring_phi, st_ring_flag, st_pending, st_meta;
};

constexpr int DEC_THREADS = 256;  // per-token kernel: 4 waves, two workgroups per CU
constexpr int DEC_WAVES = DEC_THREADS / 64;
constexpr int BND_THREADS = 512;  // chunk-boundary kernel
constexpr int BND_WAVES = BND_THREADS / 64;

// LDS carve-up of the decode kernel, in bytes from the base.
template <typename T, int D, int G>
struct DecLds {
  static constexpr size_t qs = 0;                                  // f32 [G][D]
  static constexpr size_t phq = qs + (size_t)G * D * 4;            // f32 [G][D]
  static constexpr size_t hv = phq + (size_t)G * D * 4;            // f32 [G][12]
  static constexpr size_t ml = hv + (size_t)G * 12 * 4;            // f32 [waves][G][2]
  static constexpr size_t pw = ml + (size_t)DEC_WAVES * G * 2 * 4;  // f32 [waves][17][8]
  static constexpr size_t ibuf = pw + (size_t)DEC_WAVES * 17 * 8 * 4;  // int [2 + 130]
  static constexpr size_t d64 = ibuf + (2 + 130) * 4;              // f64 [128 + 8]
  static constexpr size_t rowst = d64 + (128 + 8) * 8;             // f32 [16][2]
  static constexpr size_t uni = rowst + 16 * 2 * 4;                // union below
  // union member 1 (NP-Map and fold): xs, us, ph, vs [8][D] and red8
  // [waves][8][D] f32 in the boundary kernel; xs, us, ph [G+1][D] and red8
  // [waves][G+1][D] per token
  static constexpr int FOLD_ROWS = 8;  // rows per fold group of the boundary kernel
  static constexpr size_t fold_bytes = (size_t)(4 + BND_WAVES) * FOLD_ROWS * D * 4;
  static constexpr size_t mapg_bytes = (size_t)(3 + DEC_WAVES) * (G + 1) * D * 4;
  // union member 2 (value and state partial sums): f32 [2][waves][G][D]
  static constexpr size_t red_bytes = (size_t)2 * DEC_WAVES * G * D * 4;
  static constexpr size_t uni_bytes = mapg_bytes > red_bytes ? mapg_bytes : red_bytes;
  static constexpr size_t lg = uni + uni_bytes;                    // f64 [G][W] (runtime W)
  // then int [W + 256]: ring flags of the linear keys (at most R = W + 2C)
  __host__ __device__ static size_t lfl(int W) { return lg + (size_t)G * W * 8; }
  __host__ __device__ static size_t bytes(int W) { return lfl(W) + (size_t)(W + 256) * 4; }
  // paged pool: the unit's page table (at most MAX_PAGE_TABLE entries)
  static constexpr int MAX_PAGE_TABLE = 256;
  __host__ __device__ static size_t ptab(int W) { return bytes(W); }
  __host__ __device__ static size_t bytes_paged(int W) { return bytes(W) + (size_t)MAX_PAGE_TABLE * 4; }
};

// 8 bytes of a row as floats: rows are read as 8-byte vectors, so a row of
// D elements spans D * sizeof(T) / 8 lanes.
template <typename T>
struct RowVec;
template <>
struct RowVec<bf16> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void get(const uint2& u, float (&x)[4]) {
    const bf16* e = reinterpret_cast<const bf16*>(&u);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)e[i];
  }
};
template <>
struct RowVec<float> {
  static constexpr int N = 2;
  __device__ __forceinline__ static void get(const uint2& u, float (&x)[2]) {
    const float* e = reinterpret_cast<const float*>(&u);
    x[0] = e[0];
    x[1] = e[1];
  }
};
__device__ __forceinline__ uint2 ld8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// Sum over the n consecutive lanes (n a power of two) that hold one row.
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
  x = row_sum<(N < 16 ? N : 16)>(x);
  if constexpr (N >= 32) x += xor16f(x);
  if constexpr (N >= 64) x += xor32f(x);
  return x;
}
// partner value at lane ^ o, o = 16 or 32
template <int O>
__device__ __forceinline__ float xorf(float x) {
  static_assert(O == 16 || O == 32, "row-group exchange");
  return O == 16 ? xor16f(x) : xor32f(x);
}
__device__ __forceinline__ float wave_max(float x) {
  x = row_max<16>(x);
  x = fmax_nn(x, xor16f(x));
  return fmax_nn(x, xor32f(x));
}
__device__ __forceinline__ float wave_sum(float x) { return sum_lanes<64>(x); }

// NP-Map [P3 "NP-Map: Norm-Preserving Feature Map"] of NR <= 16 rows, reading:
// ||x|| * softmax(x F) / ||softmax(x F)|| with exact expf. u = x F with the rows
// of F read once as 8-byte vectors (all loads of a lane in flight at once),
// partial sums over the F rows reduced across lanes and then across waves
// through red8 [waves][NR][D]. xs, us, ph are [NR][D] float32 in LDS. All
// threads; ends with a barrier.
// The rows of F one lane reads for np_map_vec (issued early by callers).
template <typename T, int D, int NT>
struct FRows {
  static constexpr int NW = NT / 64;
  static constexpr int VEC = RowVec<T>::N, LPK = D / VEC, KPW = 64 / LPK;
  static constexpr int ITS = D / (NW * KPW);  // F rows per lane
  uint2 raw[ITS];
  __device__ __forceinline__ void load(const T* F) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int part = lane % LPK, grp = lane / LPK;
#pragma unroll
    for (int it = 0; it < ITS; ++it) raw[it] = ld8(F + (size_t)((it * NW + wave) * KPW + grp) * D + part * VEC);
  }
};

// one element through a buffer resource (zero past its range)
template <typename T>
__device__ __forceinline__ T ld_elem_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  if constexpr (sizeof(T) == 2) return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0));
  else return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

// element e of the 8 consecutive columns a fragment holds, as float32
__device__ __forceinline__ float frag_at(const Frag<bf16>& f, int e) { return (float)f.v[e]; }
__device__ __forceinline__ float frag_at(const Frag<f16>& f, int e) { return (float)f.v[e]; }
__device__ __forceinline__ float frag_at(const Frag<float>& f, int e) { return e < 4 ? f.lo[e] : f.hi[e - 4]; }

template <typename T, int D, int NR, int NT>
__device__ __forceinline__ void np_map_vec(const FRows<T, D, NT>& FR_, const float* xs, float* red8,
                                           float* us, float* ph, float* rowst) {
  constexpr int NW = NT / 64;
  constexpr int VEC = RowVec<T>::N, LPK = D / VEC, KPW = 64 / LPK;
  constexpr int ITS = D / (NW * KPW);  // F rows per lane
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int part = lane % LPK, grp = lane / LPK;
  float acc[NR][VEC];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[r][e] = 0.f;
  const uint2* raw = FR_.raw;
#pragma unroll
  for (int it = 0; it < ITS; ++it) {
    const int i = (it * NW + wave) * KPW + grp;
    float f[VEC];
    RowVec<T>::get(raw[it], f);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float x = xs[r * D + i];
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[r][e] += x * f[e];
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < VEC; ++e)
    {
      if constexpr (LPK <= 16) acc[r][e] += xorf<16>(acc[r][e]);
      acc[r][e] += xorf<32>(acc[r][e]);
    }
  if (grp == 0)
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < VEC; ++e) red8[(wave * NR + r) * D + part * VEC + e] = acc[r][e];
  __syncthreads();
  for (int e = tid; e < NR * D; e += NT) {
    float u = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) u += red8[w * NR * D + e];
    us[e] = u;
  }
  __syncthreads();
  for (int r = wave; r < NR; r += NW) {
    float mx = STILL_NEG_INF, xn = 0.f;
    for (int j = lane; j < D; j += 64) {
      mx = fmax_nn(mx, us[r * D + j]);
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
  for (int e = tid; e < NR * D; e += NT) {
    const int r = e / D;
    ph[e] = expf(us[e] - rowst[2 * r]) * rowst[2 * r + 1];
  }
  __syncthreads();
}

// Fold of the ring rows [f_lo, f_hi) that are not kept into S, z for 16-bit
// data, on the matrix cores, in blocks of BFB = 32 keys [P3 "NP-Map:
// Norm-Preserving Feature Map"]: F staged row-major in LDS (the B fragments
// of X F by transposing reads); waves 0-1 each compute phi of one 16-key
// tile over all D features (features on the lanes, so a key's softmax
// statistics reduce inside the wave), the features go to LDS feature-major
// in float32; then wave w folds feature tile w % (D/16) against the block's
// values for its d_v tiles (phi as fp16 hi + lo, ~22 significant bits;
// values exact in fp16) and adds its float32 sums to S, z once at the end
// (each entry by one thread). Every thread calls it; barriers inside. The
// 32-key blocks keep the kernel's LDS under 80 KiB: two workgroups per CU.
constexpr int BFB = 32;
template <int D>
struct BndFoldLds {
  static constexpr int FS = D + 8, VS = D + 8, PS = BFB + 4;  // row strides (elements)
  static constexpr size_t f_bytes = (size_t)D * FS * 2;
  static constexpr size_t v_bytes = (size_t)BFB * VS * 2;
  static constexpr size_t ph_bytes = (size_t)D * PS * 4;
  static constexpr size_t bytes = f_bytes + v_bytes + ph_bytes;
};

template <typename T, int D>
__device__ __forceinline__ void boundary_fold_mfma(const DecodeArgs& a, char* st, const T* F, int f_lo, int f_hi,
                                                   char* lds, float l2g) {
  static_assert(sizeof(T) == 2, "16-bit data");
  using BL = BndFoldLds<D>;
  constexpr int NFT = D / 16, VPW = NFT * NFT / 8, CPR = D / 8;
  T* Fl = reinterpret_cast<T*>(lds);
  f16* Vl = reinterpret_cast<f16*>(lds + BL::f_bytes);
  float* PH = reinterpret_cast<float*>(lds + BL::f_bytes + BL::v_bytes);
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.R;
  const T* ring_k = reinterpret_cast<const T*>(st + a.st_ring_k);
  const T* ring_v = reinterpret_cast<const T*>(st + a.st_ring_v);
  const int32_t* ring_flag = reinterpret_cast<const int32_t*>(st + a.st_ring_flag);
  float* S = reinterpret_cast<float*>(st + a.st_S);
  float* z = reinterpret_cast<float*>(st + a.st_z);
  for (int e = tid; e < D * CPR; e += BND_THREADS) {
    const int row = e / CPR, c = (e % CPR) * 8;
    *reinterpret_cast<uint4*>(Fl + row * BL::FS + c) = *reinterpret_cast<const uint4*>(F + (size_t)row * D + c);
  }
  // fold ownership: feature tile ft, d_v tiles vt0 .. vt0 + VPW - 1
  const int ft = wave % NFT, vt0 = (wave / NFT) * VPW;
  f32x4 acc[VPW];
#pragma unroll
  for (int v = 0; v < VPW; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zl = 0.f;
  for (int blo = f_lo; blo < f_hi; blo += BFB) {
    __syncthreads();  // F is staged; the previous block's fold is done with Vl, PH
    for (int e = tid; e < BFB * CPR; e += BND_THREADS) {
      const int r = e / CPR, c = (e % CPR) * 8, pos = blo + r;
      uint4 v8 = {0u, 0u, 0u, 0u};
      if (pos < f_hi) v8 = *reinterpret_cast<const uint4*>(ring_v + (size_t)(pos % R) * D + c);
      const T* ve = reinterpret_cast<const T*>(&v8);
      f16 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = (f16)to_f32(ve[i]);
      *reinterpret_cast<uint4*>(Vl + r * BL::VS + c) = *reinterpret_cast<uint4*>(w);
    }
    if (wave < BFB / 16) {
      // key tile `wave`: A fragments of the key rows with the depth order of
      // the transposing reads (slots 0-3: d = 32kb + 4g + s, slots 4-7: d =
      // 32kb + 16 + 4g + s - 4)
      const int pos = blo + 16 * wave + r16;
      const bool inr = pos < f_hi;
      const int slot = pos % R;
      const bool fold = inr && ring_flag[slot] == 0;
      const T* krow = ring_k + (size_t)slot * D;
      Frag<T> kf[D / 32];
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const uint2 x0 = inr ? ld8(krow + 32 * kb + 4 * g4) : uint2{0u, 0u};
        const uint2 x1 = inr ? ld8(krow + 32 * kb + 16 + 4 * g4) : uint2{0u, 0u};
        const uint4 x = {x0.x, x0.y, x1.x, x1.y};
        kf[kb].v = __builtin_bit_cast(decltype(kf[kb].v), x);
      }
      f32x4 ph[NFT];
#pragma unroll
      for (int f = 0; f < NFT; ++f) {
        ph[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb)
          mma(ph[f], kf[kb],
              tr_frag_bf16(reinterpret_cast<const bf16*>(Fl) + (32 * kb + 4 * g4 + (r16 >> 2)) * BL::FS + 16 * f +
                               4 * (r16 & 3),
                           16 * BL::FS));
      }
      // |k|^2 of key r16 (every g); softmax over the features in base 2,
      // factor |k| / sqrt(sum e^2), zero for keys that do not fold
      float n2 = 0.f;
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) n2 = frag_dot2_sumsq(kf[kb], n2);
      n2 = sum_over_g(n2);
      const uint32_t use16 = (uint32_t)__builtin_amdgcn_ballot_w64(fold) & 0xffffu;
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
        // forget gate: key j enters the state held at f_hi as gamma^(f_hi - j)
        if (l2g != 0.f) fac[i] *= exp2f((float)(f_hi - (pos - r16 + 4 * g4 + i)) * l2g);
      }
#pragma unroll
      for (int f = 0; f < NFT; ++f) {
        const f32x4 o = {ph[f][0] * fac[0], ph[f][1] * fac[1], ph[f][2] * fac[2], ph[f][3] * fac[3]};
        *reinterpret_cast<f32x4*>(PH + (16 * f + r16) * BL::PS + 16 * wave + 4 * g4) = o;
      }
    }
    __syncthreads();  // Vl, PH
#pragma unroll
    for (int kb2 = 0; kb2 < BFB / 32; ++kb2) {
      const float* pr = PH + (16 * ft + r16) * BL::PS + 32 * kb2 + 4 * g4;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(pr);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(pr + 16);
      zl += ((x0[0] + x0[1]) + (x0[2] + x0[3])) + ((x1[0] + x1[1]) + (x1[2] + x1[3]));
      Frag<f16> fh, fl;
      split2_frag<f16>(x0, x1, fh, fl);
#pragma unroll
      for (int v = 0; v < VPW; ++v) {
        const Frag<f16> bv =
            tr_frag(Vl + (32 * kb2 + 4 * g4 + (r16 >> 2)) * BL::VS + 16 * (vt0 + v) + 4 * (r16 & 3), 16 * BL::VS);
        mma(acc[v], fh, bv);
        mma(acc[v], fl, bv);
      }
    }
  }
  // the state moves from f_lo to f_hi: factor gamma^(f_hi - f_lo) (1 without the gate)
  const float fS = l2g != 0.f ? exp2f((float)(f_hi - f_lo) * l2g) : 1.f;
#pragma unroll
  for (int v = 0; v < VPW; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* e = S + (size_t)(16 * ft + 4 * g4 + i) * D + 16 * (vt0 + v) + r16;
      *e = *e * fS + acc[v][i];
    }
  if (vt0 == 0) {
    zl = sum_over_g(zl);
    if (g4 == 0) z[16 * ft + r16] = z[16 * ft + r16] * fS + zl;
  }
}

// Chunk boundary (position t = cC): decide chunk c-1 by Top-lambda over its
// float64 scores, append the kept tokens to the pool [P2 固定预算路由], and
// fold the chunks that are now wholly before the window into S, z. Runs
// before decode_kernel of the same step; on a position mismatch it does
// nothing (decode_kernel then flags the error).
template <typename T, int D>
__global__ __launch_bounds__(BND_THREADS) void decode_boundary_kernel(DecodeArgs a) {
  using LD = DecLds<T, D, 1>;
  constexpr int VEC = RowVec<T>::N;
  constexpr int LPK = D / VEC;
  extern __shared__ __align__(16) char smem[];
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int unit = b * a.Hkv + kv;
  const int W = a.W, C = a.C, R = a.R, t = a.pos ? a.pos[b] + a.t : a.t;
  if (a.pos && (t < 1 || t % C != 0)) return;  // this row is not at a chunk start
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
  constexpr int FR = LD::FOLD_ROWS;  // rows per fold group
  float* xs = reinterpret_cast<float*>(smem + LD::uni);  // [FR][D]
  float* us = xs + FR * D;
  float* ph = us + FR * D;
  float* vs = ph + FR * D;
  float* red8 = vs + FR * D;  // [waves][FR][D]
  if (meta[0] != t || meta[2] != 0) return;
  int n_pool = (int)meta[1];
  const int c = t / C, cC = c * C;
  double* ps = d64;      // [C] scores of the finished chunk
  int* kept = ibuf + 2;  // [C] rank among kept, or -1
  for (int j = tid; j < C; j += BND_THREADS) ps[j] = pend[j];
  __syncthreads();
  const int lam_c = (n_pool + a.lam <= a.m - W) ? a.lam : 0;
  if (a.pages.base) {  // uniform: the rows this step appends need pages of the arena
    bool bad = false;
    for (int i = n_pool; i < n_pool + lam_c; ++i) bad = bad || pool_page_off(a.pages, unit, i, 0, 1) < 0;
    if (bad) {
      if (tid == 0) meta[2] = -5;  // STILL_ESTATE; decode_kernel then skips the step
      return;
    }
  }
  for (int j = tid; j < C; j += BND_THREADS) {
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
  for (int e = tid; e < C * LPK; e += BND_THREADS) {
    const int j = e / LPK, part = e % LPK;
    if (kept[j] < 0) continue;
    const int pos = base + j, slot = pos % R, row = n_pool + kept[j];
    const size_t src = (size_t)slot * D + part * VEC, dst = (size_t)row * D + part * VEC;
    if (a.pages.base) {  // (mapped: checked above)
      const long ok = pool_page_off(a.pages, unit, row, 0, D * sizeof(T));
      const long ov = pool_page_off(a.pages, unit, row, 1, D * sizeof(T));
      *reinterpret_cast<uint2*>(a.pages.base + ok + part * VEC * sizeof(T)) = ld8(ring_k + src);
      *reinterpret_cast<uint2*>(a.pages.base + ov + part * VEC * sizeof(T)) = ld8(ring_v + src);
    } else if (sizeof(T) == 2 && a.pool8) {
      // the 8-bit store: the row's LPK lanes (consecutive, aligned) share
      // its largest magnitude; codes of x / 2^e, the exponent bytes after
      // the P rows
      const uint2 kw = ld8(ring_k + src), vw = ld8(ring_v + src);
      const T* kt = reinterpret_cast<const T*>(&kw);
      const T* vt = reinterpret_cast<const T*>(&vw);
      float km = 0.f, vm = 0.f;
#pragma unroll
      for (int e2 = 0; e2 < VEC; ++e2) {
        km = fmaxf(km, fabsf(to_f32(kt[e2])));
        vm = fmaxf(vm, fabsf(to_f32(vt[e2])));
      }
      const int ek = e4m3_row_exp(group_max<LPK>(km)), ev = e4m3_row_exp(group_max<LPK>(vm));
      const float rk = pow2_int(-ek), rv = pow2_int(-ev);  // x / 2^e, exact
      uint32_t kc = 0u, vc = 0u;
#pragma unroll
      for (int e2 = 0; e2 < VEC; ++e2) {
        kc |= e4m3_code(to_f32(kt[e2]) * rk) << (8 * e2);
        vc |= e4m3_code(to_f32(vt[e2]) * rv) << (8 * e2);
      }
      uint8_t* k8 = reinterpret_cast<uint8_t*>(st + a.st_pool_k);
      uint8_t* v8 = reinterpret_cast<uint8_t*>(st + a.st_pool_v);
      static_assert(sizeof(T) != 2 || VEC == 4, "four codes per lane");
      *reinterpret_cast<uint32_t*>(k8 + dst) = kc;
      *reinterpret_cast<uint32_t*>(v8 + dst) = vc;
      if (part == 0) {
        k8[(size_t)(a.m - W) * D + row] = (uint8_t)(ek + 127);
        v8[(size_t)(a.m - W) * D + row] = (uint8_t)(ev + 127);
      }
    } else {
      *reinterpret_cast<uint2*>(pool_k + dst) = ld8(ring_k + src);
      *reinterpret_cast<uint2*>(pool_v + dst) = ld8(ring_v + src);
    }
    if (part == 0) {
      pool_pos[row] = pos;
      ring_flag[slot] = 1;
      if (a.sel_new) a.sel_new[(size_t)unit * a.lam + kept[j]] = pos;
    }
  }
  if (a.sel_new)
    for (int i = lam_c + tid; i < a.lam; i += BND_THREADS) a.sel_new[(size_t)unit * a.lam + i] = -1;
  for (int j = tid; j < C; j += BND_THREADS) pend[j] = __builtin_nan("");
  n_pool += lam_c;
  __syncthreads();
  if (tid == 0) meta[1] = n_pool;

  // fold chunks [cf(c-1), cf(c)) into S, z: 16-bit data on the matrix cores,
  // float32 data with float32 features and exact expf on the VALU
  const int f_lo = full_chunks_before(c - 1, W, C) * C;
  const int f_hi = full_chunks_before(c, W, C) * C;
  // forget gate of the linear state (base 2; 0: none): the state held at
  // f_lo moves to f_hi, key j enters at gamma^(f_hi - j)
  const float l2g = a.decay ? log2f(a.decay[kv]) : 0.f;
  if constexpr (sizeof(T) == 2) {
    if (f_hi > f_lo) boundary_fold_mfma<T, D>(a, st, F, f_lo, f_hi, smem + LD::uni, l2g);  // uniform
    __syncthreads();
    return;
  }
  constexpr int PER = D * D / BND_THREADS;
  float dacc[PER];
#pragma unroll
  for (int q2 = 0; q2 < PER; ++q2) dacc[q2] = 0.f;
  float dz = 0.f;
  FRows<T, D, BND_THREADS> fr;  // F rows, read once for every group
  fr.load(F);
  const __amdgpu_buffer_rsrc_t st_r = make_rsrc(st, (uint32_t)a.st_unit);
  for (int g0 = f_lo; g0 < f_hi; g0 += FR) {
    const int n = min(FR, f_hi - g0);
    // rows of the group (unkept ones; absent or kept rows read zeros past
    // the state's range): buffer loads, all issued before any is used
    constexpr int PT = FR * D / BND_THREADS;
    T kx[PT], vx[PT];
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int e = tid + u * BND_THREADS, r = e / D, i = e % D, pos = g0 + r;
      const int slot = pos % R;
      const bool use = (ring_flag[slot] == 0) & (r < n);  // slot is in range: no branch
      const uint32_t off = (uint32_t)(slot * D + i) * sizeof(T);
      kx[u] = ld_elem_buf<T>(st_r, use ? (uint32_t)a.st_ring_k + off : (uint32_t)a.st_unit);
      vx[u] = ld_elem_buf<T>(st_r, use ? (uint32_t)a.st_ring_v + off : (uint32_t)a.st_unit);
    }
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      xs[tid + u * BND_THREADS] = to_f32(kx[u]);
      vs[tid + u * BND_THREADS] = to_f32(vx[u]);
    }
    __syncthreads();
    np_map_vec<T, D, FR, BND_THREADS>(fr, xs, red8, us, ph, rowst);
    // thread tid owns S[i][jv] for jv = tid % D and i = tid / D + q2 * (512 / D)
#pragma unroll 1
    for (int r = 0; r < FR; ++r) {
      const float wr = l2g != 0.f ? exp2f((float)(f_hi - (g0 + r)) * l2g) : 1.f;
      const float vr = vs[r * D + tid % D] * wr;
      const float* pr = ph + r * D + tid / D;
#pragma unroll
      for (int q2 = 0; q2 < PER; ++q2) dacc[q2] += pr[q2 * (BND_THREADS / D)] * vr;
    }
    if (tid < D)
      for (int r = 0; r < FR; ++r) dz += ph[r * D + tid] * (l2g != 0.f ? exp2f((float)(f_hi - (g0 + r)) * l2g) : 1.f);
    __syncthreads();
  }
  if (f_hi > f_lo) {
    const float fS = l2g != 0.f ? exp2f((float)(f_hi - f_lo) * l2g) : 1.f;
#pragma unroll
    for (int q2 = 0; q2 < PER; ++q2) S[tid + BND_THREADS * q2] = S[tid + BND_THREADS * q2] * fS + dacc[q2];
    if (tid < D) z[tid] = z[tid] * fS + dz;
  }
  __syncthreads();
}

template <typename T, int D, int G, bool PAGED = false, bool P8 = false>
__global__ __launch_bounds__(DEC_THREADS) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(DecodeArgs a) {
  static_assert(!P8 || (sizeof(T) == 2 && !PAGED), "8-bit pool: 16-bit data in the state");
  using LD = DecLds<T, D, G>;
  constexpr int VEC = RowVec<T>::N;  // elements per 8-byte vector
  constexpr int LPK = D / VEC;       // lanes per K/V row
  constexpr int KPW = 64 / LPK;      // rows per wave and vector load
  constexpr int U = 4;               // rows in flight per lane
  extern __shared__ __align__(16) char smem[];
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index in an SGPR
  const int unit = b * a.Hkv + kv;
  const int W = a.W, C = a.C, R = a.R, t = a.pos ? a.pos[b] + a.t : a.t;
  const bool boundary = t % C == 0;  // row b's token starts a chunk
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
  float* xs = reinterpret_cast<float*>(smem + LD::uni);  // [G+1][D] q rows, then k
  float* us = xs + (G + 1) * D;
  float* ph = us + (G + 1) * D;
  float* red8 = ph + (G + 1) * D;  // [waves][G+1][D]
  float* red = reinterpret_cast<float*>(smem + LD::uni);  // [2][waves][G][D]
  double* lg = reinterpret_cast<double*>(smem + LD::lg);

  // loads that depend on nothing else go first, so their latencies overlap,
  // in the order they are needed (a wait for one is a wait for all issued
  // before it): the position and pool count, the first pool positions, the
  // queries and the new key / value, the gate, z and the ring flags of the
  // linear keys. Buffer loads return zero past their range, so none of them
  // needs a branch.
  const __amdgpu_buffer_rsrc_t st_r = make_rsrc(st, (uint32_t)a.st_unit);
  const u32x4 mv = __builtin_amdgcn_raw_buffer_load_b128(st_r, 0, (uint32_t)a.st_meta, 0);
  const u32x4 me = __builtin_amdgcn_raw_buffer_load_b128(st_r, 0, (uint32_t)a.st_meta + 16, 0);
  constexpr int PPT = 2;  // pool positions per thread read ahead
  int ppos[PPT];
#pragma unroll
  for (int u = 0; u < PPT; ++u)
    ppos[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(st_r, (uint32_t)(tid + u * DEC_THREADS) * 4,
                                                          (uint32_t)a.st_pool_pos, 0);
  const __amdgpu_buffer_rsrc_t q_r =
      make_rsrc(reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Hq + kv * G) * D, G * D * sizeof(T));
  const __amdgpu_buffer_rsrc_t k_r = make_rsrc(reinterpret_cast<const T*>(a.k) + (size_t)unit * D, D * sizeof(T));
  const __amdgpu_buffer_rsrc_t v_r = make_rsrc(reinterpret_cast<const T*>(a.v) + (size_t)unit * D, D * sizeof(T));
  constexpr int QPT = (G * D + DEC_THREADS - 1) / DEC_THREADS;
  constexpr int KPT = (D + DEC_THREADS - 1) / DEC_THREADS;
  T qraw[QPT], kreg[KPT], vreg[KPT];
#pragma unroll
  for (int u = 0; u < QPT; ++u) qraw[u] = ld_elem_buf<T>(q_r, (uint32_t)(tid + u * DEC_THREADS) * sizeof(T));
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    kreg[u] = ld_elem_buf<T>(k_r, (uint32_t)(tid + u * DEC_THREADS) * sizeof(T));
    vreg[u] = ld_elem_buf<T>(v_r, (uint32_t)(tid + u * DEC_THREADS) * sizeof(T));
  }
  // key sets [P3 "Content-Aware Routing ..."]: kept tokens below lo, the ring
  // from lo to t (window and own chunk), ring tokens [la_lo, la_hi] that are
  // out of the window and unkept (linear), then S, z.
  const int c = t / C, cC = c * C;
  int lo = t - W + 1 < cC ? t - W + 1 : cC;
  if (lo < 0) lo = 0;
  const int n_win = t - lo + 1;
  const int la_lo = full_chunks_before(c, W, C) * C;
  const int la_hi = min(t - W, cC - 1);  // inclusive
  const float lng = a.decay ? logf(a.decay[kv]) : 0.f;  // forget gate, natural log (0: none)
  const int n_la = la_hi >= la_lo ? la_hi - la_lo + 1 : 0;
  const int sc_lo = t - W + 1 > 0 ? t - W + 1 : 0;  // score window
  // ring slots of consecutive positions: one modulo each, then a wrap
  const int lo_slot = lo % R, la_slot = la_lo % R;
  auto wrap = [R](int s_) { return s_ >= R ? s_ - R : s_; };
  // the gate of head r = lane % 16 (zero for r >= G) and this lane's
  // entries l, l + 64, ... of z
  const float g_load = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.gate + kv * G, G * 4), (lane & 15) * 4, 0, 0));
  const float g_lane = a.softmax_only ? 0.f : g_load;
  float zreg[D / 64];
#pragma unroll
  for (int u = 0; u < D / 64; ++u)
    zreg[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(st_r, (lane + 64 * u) * 4,
                                                                              (uint32_t)a.st_z, 0));
  // the ring flags of the linear keys (n_la < R <= W + 256)
  constexpr int FPT = 2;
  int flg[FPT];
#pragma unroll
  for (int u = 0; u < FPT; ++u) {
    const int i = tid + u * DEC_THREADS;
    flg[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(st_r, (uint32_t)((la_slot + i) % R) * 4,
                                                         (uint32_t)a.st_ring_flag, 0);
  }

  // meta: position, pool count, error (int64 each)
  const uint32_t pos_lo = __builtin_amdgcn_readfirstlane(mv[0]), pos_hi = __builtin_amdgcn_readfirstlane(mv[1]);
  const uint32_t err_or = __builtin_amdgcn_readfirstlane(me[0] | me[1]);
  if (pos_lo != (uint32_t)t || pos_hi != 0u || err_or != 0u) {
    // the loads above are used on this path too, so the compiler keeps them
    // ahead of the branch instead of moving them behind it (where they
    // would wait for the meta data)
#pragma unroll
    for (int u = 0; u < PPT; ++u) asm volatile("" ::"v"(ppos[u]));
#pragma unroll
    for (int u = 0; u < QPT; ++u) asm volatile("" ::"v"(to_f32(qraw[u])));
#pragma unroll
    for (int u = 0; u < KPT; ++u) asm volatile("" ::"v"(to_f32(kreg[u])), "v"(to_f32(vreg[u])));
#pragma unroll
    for (int u = 0; u < FPT; ++u) asm volatile("" ::"v"(flg[u]));
#pragma unroll
    for (int u = 0; u < D / 64; ++u) asm volatile("" ::"v"(zreg[u]));
    asm volatile("" ::"v"(g_lane));
    __syncthreads();
    if (tid == 0 && err_or == 0u) meta[2] = -5;
    return;
  }
  int n_pool = (int)__builtin_amdgcn_readfirstlane(mv[2]);
  if constexpr (PAGED) {  // every pool row read needs a page of the arena (uniform)
    bool bad = false;
    for (int p = lane; p < (n_pool + POOL_PAGE_ROWS - 1) / POOL_PAGE_ROWS; p += 64) {
      const int pg = a.pages.table[(size_t)unit * a.pages.width + p];
      bad = bad || pg < 0 || pg >= a.pages.n_pages;
    }
    if (__builtin_amdgcn_ballot_w64(bad)) {
      if (tid == 0) meta[2] = -5;  // STILL_ESTATE
      return;
    }
  }

  if (a.sel_new && !boundary)
    for (int i = tid; i < a.lam; i += DEC_THREADS) a.sel_new[(size_t)unit * a.lam + i] = -1;

  const int part = lane % LPK, grp = lane / LPK;

  {
    int cnt = 0;  // pool positions ascend: count those below lo
#pragma unroll
    for (int u = 0; u < PPT; ++u) cnt += (tid + u * DEC_THREADS < n_pool && ppos[u] < lo) ? 1 : 0;
    for (int i = tid + PPT * DEC_THREADS; i < n_pool; i += DEC_THREADS) cnt += pool_pos[i] < lo ? 1 : 0;
    cnt = (int)wave_sum((float)cnt);
    if (lane == 0) ibuf[1 + wave] = cnt;
  }

  // ---- 2. the new token enters the ring; phi(q_h), phi(k_t) ---------------
  const int slot_t = t % R;
#pragma unroll
  for (int u = 0; u < (D + DEC_THREADS - 1) / DEC_THREADS; ++u) {
    const int i = tid + u * DEC_THREADS;
    if (i < D) {
      xs[G * D + i] = to_f32(kreg[u]);
      ring_k[(size_t)slot_t * D + i] = kreg[u];
      ring_v[(size_t)slot_t * D + i] = vreg[u];
    }
  }
  if (tid == 0) ring_flag[slot_t] = 0;
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int e = tid + u * DEC_THREADS;
    if (e < G * D) {
      qs[e] = to_f32(qraw[u]);
      xs[e] = to_f32(qraw[u]);
    }
  }
  int* lfl = reinterpret_cast<int*>(smem + LD::lfl(W));
#pragma unroll
  for (int u = 0; u < FPT; ++u)
    if (tid + u * DEC_THREADS < n_la) lfl[tid + u * DEC_THREADS] = flg[u];
  int* ptab = reinterpret_cast<int*>(smem + LD::ptab(W));  // paged pool: the unit's pages
  if constexpr (PAGED)
    for (int i = tid; i < (n_pool + POOL_PAGE_ROWS - 1) / POOL_PAGE_ROWS; i += DEC_THREADS)
      ptab[i] = a.pages.table[(size_t)unit * a.pages.width + i];
  __syncthreads();
  int n_oob = 0;
#pragma unroll
  for (int w = 0; w < DEC_WAVES; ++w) n_oob += ibuf[1 + w];
  const int n_sa = n_oob + n_win;

  const int r16 = lane & 15, g4 = lane >> 4;
  constexpr int DV = D / 64;  // value columns per lane
  // paged pool: a pool row's offset is in the arena, tagged with bit 31
  // (the arena and the state blob both stay below 2^31 bytes)
  auto pool_row = [&](int kk, int v) -> uint32_t {
    return 0x80000000u | (uint32_t)(((ptab[kk / POOL_PAGE_ROWS] * 2 + v) * POOL_PAGE_ROWS + kk % POOL_PAGE_ROWS) *
                                    (D * (int)sizeof(T)));
  };
  auto krow_sa = [&](int kk) -> uint32_t {  // byte offset of key row kk in the state blob
    if constexpr (PAGED)
      if (kk < n_oob) return pool_row(kk, 0);
    return kk < n_oob ? (uint32_t)a.st_pool_k + (uint32_t)kk * (D * sizeof(T))
                      : (uint32_t)a.st_ring_k + (uint32_t)wrap(lo_slot + kk - n_oob) * (D * sizeof(T));
  };
  // value rows as byte offsets into this unit's state blob (one buffer
  // resource, the row offset a scalar)
  const uint32_t pv_off = (uint32_t)a.st_pool_v, rv_off = (uint32_t)a.st_ring_v;
  auto vrow_sa = [&](int kk) -> uint32_t {
    if constexpr (PAGED)
      if (kk < n_oob) return pool_row(kk, 1);
    return kk < n_oob ? pv_off + (uint32_t)kk * (D * sizeof(T))
                      : rv_off + (uint32_t)wrap(lo_slot + kk - n_oob) * (D * sizeof(T));
  };
  // 16-bit data: PV on the matrix cores (v_mfma_f32_16x16x16_bf16: the
  // weights, heads x 16 keys, are the A operand exactly in the lanes the
  // logit product leaves them in; the B operand of value block (blk, par)
  // holds, in lane (n, g), keys 4g .. 4g + 3 at dim 32 blk + 2 n + par, so
  // one 4-byte load per (key, blk) serves both parities). float32 data:
  // per-lane value columns on the vector ALUs.
  static constexpr bool PV_MFMA = sizeof(T) == 2;
  static constexpr int NVW = PV_MFMA ? 4 * (D / 32) : 16;
  struct TileRegs0 {
    Frag<T> af[D / 32];
    uint32_t vw[NVW];
    uint32_t sc[P8 ? 2 : 1];  // 8-bit pool: exponent bytes (+127): the word holding key row kk0 + r's, the value keys 4g + i
  };
  TileRegs0 TA0;

  // ---- 3b. the keys in 16-key tiles, one tile per wave at a time: logits by
  //         MFMA (keys as A rows against the heads' query columns), a running
  //         max m and sum l per head in lanes r = h, the tile's weights
  //         through a per-wave LDS slot to every lane, which owns D/64 value
  //         columns; softmax keys take logits, linear keys log(g) +
  //         log <phi(q), phi(k)> -------------------------------------------
  float* pwv = reinterpret_cast<float*>(smem + LD::pw) + wave * 17 * 8;  // [16 keys + al][8]
  float mh = STILL_NEG_INF, lh = 0.f;  // lanes r16 = h < G
  float acc[PV_MFMA ? 1 : G][DV];  // float32 data: per head, this lane's value columns
  f32x4 accm[PV_MFMA ? D / 32 : 1][2];  // 16-bit data: O[heads 4g + i][dim 32 blk + 2 r + par]
#pragma unroll
  for (int h = 0; h < (PV_MFMA ? 1 : G); ++h)
#pragma unroll
    for (int e = 0; e < DV; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int blk = 0; blk < (PV_MFMA ? D / 32 : 1); ++blk)
    accm[blk][0] = accm[blk][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // query-side B fragments: lane (r, g) holds x_r[32 kb + 8 g .. + 8] for
  // rows r < G of src (float32 in LDS), zero above; with a split, the part
  // the first rounding lost
  auto qfrag = [&](const float* src, int kb, bool lo_part) {
    // every lane reads (rows past G read row 0, then drop it): no branch
    // around the LDS reads
    const float* row = src + (r16 < G ? r16 : 0) * D + 32 * kb + 8 * g4;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(row), x1 = *reinterpret_cast<const f32x4*>(row + 4);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = r16 < G ? (e < 4 ? x0[e] : x1[e - 4]) : 0.f;
      v[e] = lo_part ? x - to_f32(from_f32<T>(x)) : x;
    }
    return frag_from<T>(f32x4{v[0], v[1], v[2], v[3]}, f32x4{v[4], v[5], v[6], v[7]});
  };
  // a tile in flight: A fragments of its 16 key rows and, per row, this
  // lane's DV value columns (DV * sizeof(T) <= 4 bytes)
  using TileRegs = TileRegs0;
  TileRegs& TA = TA0;
  TileRegs TB;
  // key rows: flat loads (a tile may span the pool and the ring); value
  // columns: buffer loads with the row in the scalar offset, so the 16 rows
  // of a tile need no per-row address registers
  // p8: std::true_type where the first n_oob keys are the kept pool's
  // 8-bit store (the softmax walk with P8), else std::false_type
  auto load_tile = [&](TileRegs& X, int kk0, int n, auto krow, auto vrow, auto p8) {
    constexpr bool Q8 = decltype(p8)::value;
    if constexpr (PAGED) {
      // rows in the state blob or, offsets tagged with bit 31, in the
      // arena's pages: loads through addresses; absent rows read a row that
      // exists and are zeroed after the load
      auto rowp = [&](uint32_t o) -> const char* {
        return (o & 0x80000000u) ? a.pages.base + (o & 0x7fffffffu) : st + o;
      };
      const int kr_ = kk0 + r16;
      const bool kin = kr_ < n;
      const char* kp = rowp(kin ? krow(kr_) : (uint32_t)a.st_ring_k) + 8 * g4 * sizeof(T);
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const Frag<T> f = ld_frag(reinterpret_cast<const T*>(kp + 32 * kb * sizeof(T)));
        X.af[kb] = kin ? f : zero_frag<T>();
      }
      if constexpr (PV_MFMA) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = kk0 + 4 * g4 + i;
          const bool vin = kk < n;
          const char* vp = rowp(vin ? vrow(kk) : (uint32_t)a.st_ring_v);
#pragma unroll
          for (int blk = 0; blk < D / 32; ++blk) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(vp + (32 * blk + 2 * r16) * sizeof(T));
            X.vw[i * (D / 32) + blk] = vin ? w : 0u;
          }
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int kk = kk0 + jj;  // uniform
          const bool vin = kk < n;
          const char* vp = rowp(vin ? vrow(kk) : (uint32_t)a.st_ring_v) + lane * DV * sizeof(T);
          uint32_t w;
          if constexpr (DV * sizeof(T) == 4) w = *reinterpret_cast<const uint32_t*>(vp);
          else w = *reinterpret_cast<const uint16_t*>(vp);
          X.vw[jj] = vin ? w : 0u;
        }
      }
      return;
    }
    // absent rows read at the end of the blob, past the range: zeros
    const uint32_t oob = (uint32_t)a.st_unit;
    const int kr_ = kk0 + r16;
    if constexpr (Q8) {
      // keys below n_oob: E4M3 codes (converted exactly to bf16) and row
      // scales; the rest: bf16 rows of the ring. One load per lane from its
      // row's store, of the same width (a code load reads 8 bytes past the
      // lane's 8 codes, inside the blob or past its range)
      const uint32_t P = (uint32_t)(a.m - a.W);
      const bool in8 = kr_ < n_oob;
      const uint32_t koff = in8 ? (uint32_t)a.st_pool_k + (uint32_t)kr_ * D + 8 * g4
                                : (kr_ < n ? krow(kr_) : oob) + 8 * g4 * sizeof(T);
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb)  // raw: converted where the tile is used
        X.af[kb] = ld_frag_buf<T>(st_r, koff + (in8 ? 32 : 64) * kb, 0);
      // exponent bytes: of the lane's key row kr_ (in its aligned word), and
      // of its value keys ks .. ks + 3
      const int ks = kk0 + 4 * g4;
      const uint32_t eko = in8 ? (uint32_t)a.st_pool_k + P * D + (uint32_t)(kr_ & ~3) : oob;
      const uint32_t evo = ks < n_oob ? (uint32_t)a.st_pool_v + P * D + (uint32_t)ks : oob;
      X.sc[0] = __builtin_amdgcn_raw_buffer_load_b32(st_r, eko, 0, 0);
      X.sc[1] = __builtin_amdgcn_raw_buffer_load_b32(st_r, evo, 0, 0);
      // values: dims 32 blk + 2 r, + 1 of key ks + i; an 8-bit row's two
      // codes sit in the aligned 4 bytes at 32 blk + 4 (r / 2), half r % 2
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = ks + i;
        const bool v8 = kk < n_oob;
        const uint32_t roff = v8 ? (uint32_t)a.st_pool_v + (uint32_t)kk * D + 4 * (r16 >> 1)
                                 : (kk < n ? vrow(kk) : oob) + 2 * r16 * sizeof(T);
#pragma unroll
        for (int blk = 0; blk < D / 32; ++blk) {
          X.vw[i * (D / 32) + blk] = __builtin_amdgcn_raw_buffer_load_b32(st_r, roff + (v8 ? 32 : 64) * blk, 0, 0);
        }
      }
      return;
    }
    const uint32_t koff = (kr_ < n ? krow(kr_) : oob) + 8 * g4 * sizeof(T);
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) X.af[kb] = ld_frag_buf<T>(st_r, koff, 32 * kb * sizeof(T));
    if constexpr (PV_MFMA) {
      // keys 4g + i of the tile, dims 32 blk + 2 r, + 1 (4 bytes)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = kk0 + 4 * g4 + i;
        const uint32_t roff = kk < n ? vrow(kk) : oob;
#pragma unroll
        for (int blk = 0; blk < D / 32; ++blk)
          X.vw[i * (D / 32) + blk] =
              __builtin_amdgcn_raw_buffer_load_b32(st_r, roff + (32 * blk + 2 * r16) * sizeof(T), 0, 0);
      }
    } else {
      const uint32_t voff = lane * DV * sizeof(T);
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int kk = kk0 + jj;  // uniform
        const uint32_t soff = __builtin_amdgcn_readfirstlane(kk < n ? vrow(kk) : oob);
        if constexpr (DV * sizeof(T) == 4) X.vw[jj] = __builtin_amdgcn_raw_buffer_load_b32(st_r, voff, soff, 0);
        else X.vw[jj] = __builtin_amdgcn_raw_buffer_load_b16(st_r, voff, soff, 0);
      }
    }
  };
  // one tile: weight(c, kk) turns a product into a log-weight
  auto tile = [&](const TileRegs& X, int kk0, int n, const Frag<T>* qb, const Frag<T>* qb2,
                  auto weight, int sc_first, auto p8) {
    constexpr bool Q8 = decltype(p8)::value;
    if (kk0 + 16 > sc_first) {  // wave-uniform: score-window keys in the tile
      // float64 logits of the new token's score: the products of bf16/f32
      // values are exact in float64; lane (r, g) sums its 8 columns per
      // block, then the four g lanes of row r combine
      const int kk = kk0 + r16;
#pragma unroll 1
      for (int h = 0; h < G; ++h) {  // one head at a time keeps few registers live
        const float* qh = lds_opaque(qs) + h * D + 8 * g4;
        double d = 0.0;
#pragma unroll
        for (int kb = 0; kb < D / 32; ++kb) {
          const f32x4 q0 = *reinterpret_cast<const f32x4*>(qh + 32 * kb);
          const f32x4 q1 = *reinterpret_cast<const f32x4*>(qh + 32 * kb + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) d += (double)(e < 4 ? q0[e] : q1[e - 4]) * (double)frag_at(X.af[kb], e);
        }
        d += xor16d(d);
        d += xor32d(d);
        if (g4 == 0 && kk >= sc_first && kk < n) lg[h * W + kk - sc_first] = a.scale64 * d;
      }
    }
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    // 8-bit pool: the lane's key row kk0 + r below n_oob holds codes (the
    // first 8 bytes of its load), converted here, where the tile is used
    const bool k8 = Q8 && kk0 + r16 < n_oob;
    float ks8 = 1.f;  // 2^e of the lane's key row
    if constexpr (Q8) ks8 = __uint_as_float(((X.sc[0] >> (8 * ((kk0 + r16) & 3))) & 255u) << 23);
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      Frag<T> af = X.af[kb];
      if constexpr (Q8) af = e4m3x8_or_raw<T>(p8, k8, af, ks8);
      mma(c, af, qb[kb]);
      if (qb2) mma(c, af, qb2[kb]);
    }
    // c[i] = <key kk0 + 4g + i, query-side column r>; an 8-bit key's
    // product times its row scale (1 for the others)
    float mx = STILL_NEG_INF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = kk0 + 4 * g4 + i;
      const bool ok = r16 < G && kk < n;
      const float w = weight(c[i], ok ? kk : kk0);  // evaluated in every lane: no branch
      c[i] = ok ? w : STILL_NEG_INF;
      mx = fmax_nn(mx, c[i]);
    }
    mx = fmax_nn(mx, xor16f(mx));
    mx = fmax_nn(mx, xor32f(mx));
    const float mn = fmax_nn(mh, mx);
    const float al = (mh == STILL_NEG_INF || mn == STILL_NEG_INF) ? 0.f : __expf(mh - mn);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = c[i] == STILL_NEG_INF ? 0.f : __expf(c[i] - mn);
      ls += c[i];
    }
    ls += xor16f(ls);
    ls += xor32f(ls);
    lh = lh * al + ls;
    mh = mn;
    if constexpr (PV_MFMA) {
      // rescale factors of the O rows (heads 4g + i) from lanes r = head,
      // only when some head's maximum moved (wave-uniform)
      if (__builtin_amdgcn_ballot_w64(r16 < G && al != 1.f)) {
        if (r16 < 8 && g4 == 0) pwv[128 + r16] = al;
        wave_sync();
        float ar[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ar[i] = 4 * g4 + i < G ? pwv[128 + 4 * g4 + i] : 0.f;
#pragma unroll
        for (int blk = 0; blk < D / 32; ++blk)
#pragma unroll
          for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int i = 0; i < 4; ++i) accm[blk][par][i] *= ar[i];
        wave_sync();  // the slot is written again by the next tile
      }
      // weights as bf16 hi (the top 16 bits) + lo (the remainder's top 16
      // bits): ~16 significant bits; A operand: row = head r, keys 4g + i
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      s16x4 ahi, alo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u = __float_as_uint(c[i]) & 0xFFFF0000u;
        ahi[i] = (short)(u >> 16);
        alo[i] = (short)(__float_as_uint(c[i] - __uint_as_float(u)) >> 16);
      }
#pragma unroll
      for (int blk = 0; blk < D / 32; ++blk) {
        uint32_t w0 = X.vw[blk], w1 = X.vw[(D / 32) + blk];
        uint32_t w2 = X.vw[2 * (D / 32) + blk], w3 = X.vw[3 * (D / 32) + blk];
        if constexpr (Q8) {  // an 8-bit row's two codes (half r % 2 of its aligned 4 bytes) times 2^e
          const int k0 = kk0 + 4 * g4, sh = 16 * (r16 & 1);
          const uint32_t ev = X.sc[1];
          w0 = k0 < n_oob ? e4m3x2_scaled_bf16x2(w0 >> sh, __uint_as_float((ev & 255u) << 23)) : w0;
          w1 = k0 + 1 < n_oob ? e4m3x2_scaled_bf16x2(w1 >> sh, __uint_as_float(((ev >> 8) & 255u) << 23)) : w1;
          w2 = k0 + 2 < n_oob ? e4m3x2_scaled_bf16x2(w2 >> sh, __uint_as_float(((ev >> 16) & 255u) << 23)) : w2;
          w3 = k0 + 3 < n_oob ? e4m3x2_scaled_bf16x2(w3 >> sh, __uint_as_float((ev >> 24) << 23)) : w3;
        }
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          // keys 0..3 of the lane's group at dim 32 blk + 2 r + par
          const uint32_t sel = par ? 0x07060302u : 0x05040100u;
          const uint32_t b01 = __builtin_amdgcn_perm(w1, w0, sel), b23 = __builtin_amdgcn_perm(w3, w2, sel);
          s16x4 bv;
          bv[0] = (short)(b01 & 0xffffu);
          bv[1] = (short)(b01 >> 16);
          bv[2] = (short)(b23 & 0xffffu);
          bv[3] = (short)(b23 >> 16);
          accm[blk][par] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bv, accm[blk][par], 0, 0, 0);
          accm[blk][par] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, bv, accm[blk][par], 0, 0, 0);
        }
      }
    } else {
      if (r16 < 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pwv[(4 * g4 + i) * 8 + r16] = c[i];
        if (g4 == 0) pwv[128 + r16] = al;
      }
      wave_sync();
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float a_h = pwv[128 + h];
#pragma unroll
        for (int e = 0; e < DV; ++e) acc[h][e] *= a_h;
      }
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        float v[DV];
        const T* ve = reinterpret_cast<const T*>(&X.vw[jj]);
#pragma unroll
        for (int e = 0; e < DV; ++e) v[e] = to_f32(ve[e]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pj = pwv[jj * 8 + h];
#pragma unroll
          for (int e = 0; e < DV; ++e) acc[h][e] += pj * v[e];
        }
      }
      wave_sync();  // the slot is written again by the next tile
    }
  };
  // the tiles of wave w: w, w + waves, ...; two in flight
  auto run_tiles = [&](TileRegs& A, TileRegs& B, bool a_loaded, int n, auto krow, auto vrow,
                       const Frag<T>* qb, const Frag<T>* qb2, auto weight, int sc_first, auto p8) {
    constexpr int STEP = 16 * DEC_WAVES;
    const int first = 16 * wave;
    // loads are issued whether or not their tile exists (absent rows read
    // zeros past the range): a load on one side of a branch only would make
    // the next wait one for every load in flight
    if (!a_loaded) load_tile(A, first, n, krow, vrow, p8);
    for (int kk0 = first; kk0 < n; kk0 += 2 * STEP) {  // wave-uniform
      load_tile(B, kk0 + STEP, n, krow, vrow, p8);
      tile(A, kk0, n, qb, qb2, weight, sc_first, p8);
      if (kk0 + STEP >= n) break;
      load_tile(A, kk0 + 2 * STEP, n, krow, vrow, p8);
      tile(B, kk0 + STEP, n, qb, qb2, weight, sc_first, p8);
    }
  };
  // ---- 3b. NP-Map phi(q_h), phi(k_t), with the wave's state rows and its
  //         first softmax-key tile in flight --------------------------------
  FRows<T, D, DEC_THREADS> frows;
  frows.load(F);
  // state rows 16 j .. 16 j + 15 for j = wave, wave + waves, ...: lane l
  // holds columns l * DV .. + DV of each
  constexpr int SJ = D / (16 * DEC_WAVES);
  using SRow = typename std::conditional<DV == 2, uint2, uint32_t>::type;
  SRow srow[SJ][16];
#pragma unroll
  for (int j = 0; j < SJ; ++j)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const uint32_t soff = (uint32_t)a.st_S + (uint32_t)((16 * (j * DEC_WAVES + wave) + jj) * D * 4);
      if constexpr (DV == 2) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(st_r, lane * 8, soff, 0);
        srow[j][jj] = uint2{x[0], x[1]};
      } else {
        srow[j][jj] = __builtin_amdgcn_raw_buffer_load_b32(st_r, lane * 4, soff, 0);
      }
    }
  using SaP8 = std::integral_constant<bool, P8>;  // the softmax walk reads the 8-bit pool
  load_tile(TA, 16 * wave, n_sa, krow_sa, vrow_sa, SaP8{});

  np_map_vec<T, D, G + 1, DEC_THREADS>(frows, xs, red8, us, ph, rowst);
  for (int e = tid; e < G * D; e += DEC_THREADS) phq[e] = ph[e];
  for (int i = tid; i < D; i += DEC_THREADS) ring_phi[(size_t)slot_t * D + i] = from_f32<T>(ph[G * D + i]);

  float* redA = red;                                          // [waves][G][D]
  float* redS = red + DEC_WAVES * G * D;                      // [waves][G][D]
  float* mlw = reinterpret_cast<float*>(smem + LD::ml);       // [waves][G][2]
  __syncthreads();  // phq complete; the NP-Map scratch (aliased by red) is free

  // ---- 3c. state readout partials: sum_i phi_h[i] S[i][f] over the wave's
  //         rows -----------------------------------------------------------
  {
    float accS[G][DV];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < DV; ++e) accS[h][e] = 0.f;
#pragma unroll
    for (int j = 0; j < SJ; ++j)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int i = 16 * (j * DEC_WAVES + wave) + jj;
        const float* sr = reinterpret_cast<const float*>(&srow[j][jj]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = phq[h * D + i];
#pragma unroll
          for (int e = 0; e < DV; ++e) accS[h][e] += p * sr[e];
        }
      }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < DV; ++e) redS[(wave * G + h) * D + lane * DV + e] = accS[h][e];
  }

  // ---- 3d. softmax keys: logits q.k scaled; the float64 score-window
  //         logits come from the same key fragments; the wave's first
  //         linear-key tile is loaded meanwhile (up to four heads: with
  //         eight the registers do not hold it) -----------------------------
  auto krow_la = [&](int kk) -> uint32_t {
    return (uint32_t)a.st_ring_phi + (uint32_t)wrap(la_slot + kk) * (D * sizeof(T));
  };
  auto vrow_la = [&](int kk) -> uint32_t { return rv_off + (uint32_t)wrap(la_slot + kk) * (D * sizeof(T)); };
  // (not with the 8-bit or the paged pool: their softmax tiles carry more
  // registers, and a third tile live through that walk would spill)
  constexpr bool LA_EARLY = G <= 4 && !P8 && !PAGED;
  TileRegs TC;
  if constexpr (LA_EARLY) load_tile(TC, 16 * wave, n_la, krow_la, vrow_la, std::false_type{});
  {
    Frag<T> qb[D / 32];
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) qb[kb] = qfrag(qs, kb, false);
    const float scale = a.scale;
    const int n_sc = t - sc_lo + 1;  // the score window: the last n_sc keys
    run_tiles(TA, TB, true, n_sa, krow_sa, vrow_sa, qb, (const Frag<T>*)nullptr,
              [&](float x, int) { return x * scale; }, n_sa - n_sc, SaP8{});
  }

  // ---- 3e. linear keys: log-weight log(g) + log <phi(q), phi(k)> --------
  if (n_la > 0) {
    // phi(q) as T hi + lo parts (float32 data: exact in one part)
    Frag<T> pb[D / 32], pb2[D / 32];
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
      pb[kb] = qfrag(phq, kb, false);
      pb2[kb] = qfrag(phq, kb, true);
    }
    const float g_r = g_lane;  // zero for r >= G
    const float lgate = g_r > 0.f ? __logf(g_r) : STILL_NEG_INF;
    // forget gate: linear key la_lo + kk weighted gamma^(t - la_lo - kk)
    auto weight = [&](float w, int kk) {
      const bool la = lfl[kk] == 0;
      return (la && w > 0.f) ? lgate + __logf(w) + (float)(t - la_lo - kk) * lng : STILL_NEG_INF;
    };
    run_tiles(LA_EARLY ? TC : TA, TB, LA_EARLY, n_la, krow_la, vrow_la, pb,
              sizeof(T) == 2 ? pb2 : (const Frag<T>*)nullptr, weight, INT_MAX, std::false_type{});
  }
  // publish per wave: (m, l) per head from lanes r = h, the value slices
  if constexpr (PV_MFMA) {
#pragma unroll
    for (int blk = 0; blk < D / 32; ++blk)
#pragma unroll
      for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * g4 + i;
          if (h < G) redA[(wave * G + h) * D + 32 * blk + 2 * r16 + par] = accm[blk][par][i];
        }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < DV; ++e) redA[(wave * G + h) * D + lane * DV + e] = acc[h][e];
  }
  if (g4 == 0 && r16 < G) {
    mlw[(wave * G + r16) * 2] = mh;
    mlw[(wave * G + r16) * 2 + 1] = lh;
  }
  __syncthreads();

  // ---- 4. float64 score of token t [P3 "Self-Saliency Score"] and the
  //         normaliser of each head (one wave per head) ------------------
  for (int h = wave; h < G; h += DEC_WAVES) {  // wave-uniform
    {  // score: KL(a_diag || (1-eps) a_nodiag + eps delta_t) in float64
      const int n = t - sc_lo + 1;
      const double* x = lg + h * W;
      double mx = -__builtin_huge_val();
      for (int j = lane; j < n; j += 64) mx = x[j] > mx ? x[j] : mx;
      mx = wave_max_d(mx);
      double za = 0.0, zo = 0.0;
      for (int j = lane; j < n; j += 64) {
        const double e = exp(x[j] - mx);
        za += e;
        if (j != n - 1) zo += e;
      }
      za = wave_sum_d(za);
      zo = wave_sum_d(zo);
      // the routing metric (metrics of the kv head counted on head 0 only)
      double kn = 0.0;
      if (a.route == ROUTE_KEYNORM && h == 0) {  // wave-uniform
        const T* kt = reinterpret_cast<const T*>(a.k) + (size_t)unit * D;
        kn = sqrt(row_dot_f64<T, D>(kt, kt));
      }
      if (lane == 0) {
        const double p = exp(x[n - 1] - mx) / za, pn = zo / za;
        double sc = 0.0;
        if (a.route == ROUTE_DIAG) {
          sc = p;
        } else if (a.route == ROUTE_QK) {
          sc = x[n - 1];
        } else if (a.route == ROUTE_KEYNORM) {
          sc = kn;
        } else if (a.route == ROUTE_UNIFORM) {
          sc = h == 0 ? (double)uniform_mark(t - cC, C, a.lam) : 0.0;
        } else {
          if (p > 0.0) sc += p * log(p / a.eps64);
          if (pn > 0.0) sc += pn * log(pn / (1.0 - a.eps64));
        }
        d64[128 + h] = sc;
      }
    }
    // the state as a virtual key: log-weight log(g * phi(q).z), value
    // S^T phi(q) / phi(q).z; one normaliser over the waves' partials
    float dz = 0.f;
#pragma unroll
    for (int u = 0; u < D / 64; ++u) dz += phq[h * D + lane + 64 * u] * zreg[u];
    dz = wave_sum(dz);
    const float g = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g_lane), h));
    // (the state is held at la_lo: the forget gate weights it gamma^(t - la_lo))
    const float lws = (g > 0.f && dz > 0.f) ? __logf(g * dz) + (float)(t - la_lo) * lng : STILL_NEG_INF;
    float mx = lws;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) mx = fmax_nn(mx, mlw[(w * G + h) * 2]);
    if (lane < DEC_WAVES) {
      const float mw = mlw[(lane * G + h) * 2];
      hv[h * 12 + 4 + lane] = mw == STILL_NEG_INF ? 0.f : __expf(mw - mx);
    }
    if (lane == 0) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < DEC_WAVES; ++w) {
        const float mw = mlw[(w * G + h) * 2];
        tot += mw == STILL_NEG_INF ? 0.f : mlw[(w * G + h) * 2 + 1] * __expf(mw - mx);
      }
      const float es = lws == STILL_NEG_INF ? 0.f : __expf(lws - mx);
      hv[h * 12 + 0] = dz;
      hv[h * 12 + 1] = es;
      hv[h * 12 + 2] = tot + es;
    }
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int h = 0; h < G; ++h) tot += d64[128 + h];
    pend[t - cC] = tot;
  }
  for (int e = tid; e < G * D; e += DEC_THREADS) {
    const int h = e / D, f = e % D;
    float sv = 0.f, ns = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      sv += redA[(w * G + h) * D + f] * hv[h * 12 + 4 + w];
      ns += redS[(w * G + h) * D + f];
    }
    const float dz = hv[h * 12 + 0], es = hv[h * 12 + 1], tot = hv[h * 12 + 2];
    if (es > 0.f) sv += es * ns / dz;
    float y = sv / tot;
    const size_t o = ((size_t)b * a.Hq + kv * G + h) * D + f;
    if (a.out_gate) y *= sigmoid_gate(to_f32(reinterpret_cast<const T*>(a.out_gate)[o]));
    if (a.fp32_out) reinterpret_cast<float*>(a.out)[o] = y;
    else reinterpret_cast<T*>(a.out)[o] = from_f32<T>(y);
  }
  if (tid == 0) {
    meta[1] = n_pool;
    meta[0] = t + 1;
  }
}

}  // namespace still
