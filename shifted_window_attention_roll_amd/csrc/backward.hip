// Backward pass of the shifted-window attention sub-layer: from dL/dy to the
// gradients of x, the QKV and projection weights and biases, the relative
// position bias table and (V2) tau.
//
// Pages: "Boosting Swin Transformer Speed", Training Optimization (the fused
// MHA and the shift / partition kernels serve training, so the sub-layer is
// differentiated through all of them); "Swin Transformer V2" summary, How It
// Works (cosine logits divided by max(tau, 0.01), plus the position bias).
//
// Pipeline (window order, row-major slots, float32 intermediates):
//   xw  = partition+shift(x),  dyw = partition+shift(dy)        (index maps)
//   qkv = xw Wqkv^T + bqkv,    do  = dyw Wp                      (bwd_gemm)
//   per (window, head): recompute S, P and O; dq, dk, dv; table and tau
//   gradients                                                     (attn_bwd)
//   dWp = dyw^T o, dWqkv = dqkv^T xw (split over tokens, atomics) (bwd_gemm)
//   dbp, dbqkv = column sums of dyw, dqkv (in the same two GEMMs)
//   dxw = dqkv Wqkv, dx = reverse+unshift(dxw)                    (bwd_gemm,
//                                                                   index map)
// The inverse of a permutation is its adjoint, so the index maps of the
// forward carry the gradients between the image and window orders.
#include "kv_frag.hpp"
#include "launch.hpp"

namespace swin {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) { return (float)p[i]; }

// v[0..8) = p[off .. off+8) as float for the first `valid` elements (<= 8), 0
// after; one 16-byte (16-bit) or two (float) loads when all 8 are valid.  The
// full-run path needs off % 8 == 0 and a 16-byte aligned p.
template <typename T>
__device__ __forceinline__ void load_run8(const T* p, int64_t off, int valid, float (&v)[8]) {
  if (valid >= 8) {
    if constexpr (sizeof(T) == 4) {
      const float4 a = *reinterpret_cast<const float4*>(p + off);
      const float4 b = *reinterpret_cast<const float4*>(p + off + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const vec8<T> a = *reinterpret_cast<const vec8<T>*>(p + off);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = i < valid ? (float)p[off + i] : 0.f;
  }
}

__device__ __forceinline__ void store_row8(float* d, const float (&v)[8]) {
  *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Matrix-core type of a product of TA and TB elements: float16 when both are
// float16 (each product exact in float32), else bfloat16.
template <typename TA, typename TB>
using mma_type_t = typename std::conditional<std::is_same<TA, h16>::value &&
                                                 std::is_same<TB, h16>::value,
                                             h16, b16>::type;

// Terms of the product type per operand element: one when the element type is
// the product type, else two, hi = MT(x) and lo = MT(x - hi) (x - hi is exact
// in float32).  hi + lo equals a float16 x exactly and a float x to about
// 2^-17 relative.
template <typename T, typename MT>
constexpr int terms_of() {
  return std::is_same<T, MT>::value ? 1 : 2;
}

template <typename MT, int P>
__device__ __forceinline__ void split8(const float (&v)[8], vec8<MT> (&t)[P]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const MT hi = from_f32<MT>(v[e]);
    t[0][e] = hi;
    if constexpr (P == 2) t[1][e] = from_f32<MT>(v[e] - (float)hi);
  }
}

// C[m][n] (+)= sum_k A(m, k) B(k, n) (+ bias[n]) with element strides, on the
// 16-bit matrix cores with float32 accumulation (16x16x32 products).  With two
// terms per operand the product of a pair is hi_a hi_b + hi_a lo_b + lo_a hi_b
// (lo_a lo_b, about 2^-18 of it, left out): about 2^-16 relative per product
// for float operands, against 2^-24 for a float32 product.  64 x 64 tile per
// workgroup of 4 waves, 32 x 32 per wave; K in steps of 32 through LDS, the
// next step's global loads in flight during the current step's products.
// Each thread stages runs of 8 elements along an operand's unit stride with
// one 16-byte store per term: an operand whose unit stride is k is stored
// [row][k] (80-byte rows: the fragment reads of 8 consecutive rows hit
// distinct bank groups) and read as rows; one whose unit stride is its row
// index is stored [k][row] (144-byte rows) and read by transposing loads, which
// give the lane of fragment row 4a + b of 32-row pair half t the row 8a + 4t +
// b (undone in the epilogue).  blockIdx.z takes the K range [z*kc,
// (z+1)*kc).  ATOMIC adds the tile into C (float) instead of storing it; then
// only z = 0 adds bias.
constexpr int kGT = 64, kGK = 32, kGP = kGK + 8, kTP = kGT + 8;
static_assert(kGK * kTP <= kGT * kGP, "one plane size for both layouts");

template <typename TA, typename TB, typename TC, bool ATOMIC>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(BwdGemm a) {
  using MT = mma_type_t<TA, TB>;
  constexpr int PA = terms_of<TA, MT>(), PB = terms_of<TB, MT>();
  __shared__ __attribute__((aligned(16))) MT As[PA][kGT * kGP];  // [m][k] per term
  __shared__ __attribute__((aligned(16))) MT Bs[PB][kGT * kGP];  // [n][k] per term
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * kGT;
  const int n0 = blockIdx.x * kGT;
  const int64_t k0 = (int64_t)blockIdx.z * a.kc;
  const int64_t k1 = k0 + a.kc < a.K ? k0 + a.kc : a.K;
  const TA* A = static_cast<const TA*>(a.A);
  const TB* B = static_cast<const TB*>(a.B);
  const bool a_k_unit = a.sak == 1, b_n_unit = a.sbn == 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row sums of A (the bias gradient of a weight-gradient product), from the
  // staged runs of the first column tile's workgroups.
  const bool rows_sum = ATOMIC && a.rowsum && !a_k_unit && blockIdx.x == 0;
  float rs[8] = {};
  // Each thread loads one run of 8 elements of each operand along its
  // unit-stride dimension (k, or the row dimension m / n) of step kb.
  float va[8], vb[8];
  auto load = [&](int64_t kb) {
    if (a_k_unit) {
      const int mm = tid >> 2, kk = (tid & 3) * 8;
      const int64_t m = m0 + mm, k = kb + kk;
      load_run8(A, m * a.sam + k, m < a.M ? (int)min<int64_t>(k1 - k, 8) : 0, va);
    } else {
      const int kk = tid >> 3, mm = (tid & 7) * 8;
      const int64_t m = m0 + mm, k = kb + kk;
      load_run8(A, m + k * a.sak, k < k1 ? (int)min<int64_t>(a.M - m, 8) : 0, va);
    }
    if (!b_n_unit) {
      const int nn = tid >> 2, kk = (tid & 3) * 8;
      const int n = n0 + nn;
      const int64_t k = kb + kk;
      load_run8(B, (int64_t)n * a.sbn + k, n < a.N ? (int)min<int64_t>(k1 - k, 8) : 0, vb);
    } else {
      const int kk = tid >> 3, nn = (tid & 7) * 8;
      const int n = n0 + nn;
      const int64_t k = kb + kk;
      load_run8(B, n + k * a.sbk, k < k1 ? (int)min<int64_t>(a.N - n, 8) : 0, vb);
    }
  };
  // The loaded runs, split into their terms, into LDS.
  auto stage = [&]() {
    vec8<MT> ta[PA], tb[PB];
    split8<MT, PA>(va, ta);
    split8<MT, PB>(vb, tb);
    if (a_k_unit) {
      const int mm = tid >> 2, kk = (tid & 3) * 8;
#pragma unroll
      for (int p = 0; p < PA; ++p) *reinterpret_cast<vec8<MT>*>(&As[p][mm * kGP + kk]) = ta[p];
    } else {
      const int kk = tid >> 3, mm = (tid & 7) * 8;
#pragma unroll
      for (int p = 0; p < PA; ++p) *reinterpret_cast<vec8<MT>*>(&As[p][kk * kTP + mm]) = ta[p];
      if (rows_sum) {
#pragma unroll
        for (int i = 0; i < 8; ++i) rs[i] += va[i];
      }
    }
    if (!b_n_unit) {
      const int nn = tid >> 2, kk = (tid & 3) * 8;
#pragma unroll
      for (int p = 0; p < PB; ++p) *reinterpret_cast<vec8<MT>*>(&Bs[p][nn * kGP + kk]) = tb[p];
    } else {
      const int kk = tid >> 3, nn = (tid & 7) * 8;
#pragma unroll
      for (int p = 0; p < PB; ++p) *reinterpret_cast<vec8<MT>*>(&Bs[p][kk * kTP + nn]) = tb[p];
    }
  };
  // Fragment i (rows 16 i .. of the wave's 32) of a plane stored as rows, or
  // half i of the 32-row pair of a plane stored [k][row].
  auto row_frag = [&](const MT* plane, int row0, int i) {
    return *reinterpret_cast<const vec8<MT>*>(&plane[(row0 + i * 16 + i16) * kGP + 8 * g4]);
  };
  auto tr_frag = [&](const MT* plane, int row0, int i) {
    const lds_v4s vl = (lds_v4s)&plane[(8 * g4 + (i16 >> 2)) * kTP + row0 + 8 * (i16 & 3)];
    return vt_frag<MT, kTP>(vl, 0, i);
  };
  if (k0 < k1) load(k0);
  for (int64_t kb = k0; kb < k1; kb += kGK) {
    stage();
    __syncthreads();
    if (kb + kGK < k1) load(kb + kGK);  // in flight during the products
    vec8<MT> af[PA][2], bf[PB][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int p = 0; p < PA; ++p)
        af[p][i] = a_k_unit ? row_frag(As[p], wm * 32, i) : tr_frag(As[p], wm * 32, i);
#pragma unroll
      for (int p = 0; p < PB; ++p)
        bf[p][i] = b_n_unit ? tr_frag(Bs[p], wn * 32, i) : row_frag(Bs[p], wn * 32, i);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (PB == 2) acc[i][j] = mma_16x16x32(af[0][i], bf[1][j], acc[i][j]);
        if constexpr (PA == 2) acc[i][j] = mma_16x16x32(af[1][i], bf[0][j], acc[i][j]);
        acc[i][j] = mma_16x16x32(af[0][i], bf[0][j], acc[i][j]);
      }
    __syncthreads();
  }
  if (rows_sum) {
    // Thread t staged rows 8 (t % 8) .. +7 at k = t / 8 of every step: the 8
    // lanes of a wave with the same t % 8 are summed by shuffles, then the 4
    // waves through LDS (the last barrier ended every read of As).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rs[i] += __shfl_xor(rs[i], 8);
      rs[i] += __shfl_xor(rs[i], 16);
      rs[i] += __shfl_xor(rs[i], 32);
    }
    float* red = reinterpret_cast<float*>(&As[0][0]);
    static_assert(sizeof(As) >= 4 * 64 * sizeof(float), "row-sum space");
    if (lane < 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave * 64 + lane * 8 + i] = rs[i];
    }
    __syncthreads();
    if (tid < 64 && m0 + tid < a.M)
      atomicAdd(a.rowsum + m0 + tid, red[tid] + red[64 + tid] + red[128 + tid] + red[192 + tid]);
  }
  // Lane l holds column l % 16 of rows 4 (l / 16) .. +3 of each 16 x 16 tile
  // (fragment rows and columns; a transposed operand's are permuted).
  TC* C = static_cast<TC*>(a.C);
  const bool add_bias = a.bias && (!ATOMIC || blockIdx.z == 0);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 32 + (b_n_unit ? 8 * (i16 >> 2) + 4 * j + (i16 & 3) : j * 16 + i16);
    if (n >= a.N) continue;
    const float bn = add_bias ? ld(static_cast<const TB*>(a.bias), n) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 32 + (a_k_unit ? i * 16 + 4 * g4 + r : 8 * g4 + 4 * i + r);
        if (m >= a.M) continue;
        const float v = acc[i][j][r] + bn;
        if constexpr (ATOMIC)
          atomicAdd(reinterpret_cast<float*>(C) + m * a.ldc + n, v);
        else
          C[m * a.ldc + n] = from_f32<TC>(v);
      }
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

// Per (window, head): recompute the attention and take its gradients, every
// product on the float32 matrix cores.  Phases:
//   1: row max m_i and sum l_i of exp(S_ij - m_i) over allowed keys;
//   2: P, O = P V (stored), then D_i = sum_j P_ij dP_ij as dO_i . O_i;
//   3: dS = P (dP - D); table (and V2 tau) gradients; dQ = dS K;
//   4: dV = P^T dO, dK = dS^T Q.
// S_ij = c (q_i . k_j) + table[rel(i, j)], c = scale (V1) or 1 / max(tau,
// tau_min) on unit q, k (V2); masked pairs get the logit kMasked, whose
// exponential underflows to exactly 0 (the pair (i, i) is always allowed).
// One workgroup of WV waves per (window, head); N is padded to NP (a multiple
// of 32) with zero rows whose label matches only other padding rows, so they
// stay finite and add nothing.  Wave w owns the TPW = NP / 16 / WV query tiles
// w TPW .. (16 rows each) for phases 1-3 and the same key tiles for phase 4.
// Products are 16 x 16 tiles (mma_16x16x32: lane l supplies row / column
// l % 16 and the K-slice 8 (l/16) .. +7; the result holds column l % 16 of
// rows 4 (l/16) .. +3):
//   S = Q K^T, dP = dO V^T (K-slice: head dims, fragments straight from rows);
//   O = P V, dQ = dS K (K-slice: keys; P and dS go through a per-wave LDS
//   tile to become row fragments, V and K are read as columns);
//   S^T = K Q^T, dP^T = V dO^T, dV = P^T dO, dK = dS^T Q (phase 4).
// LDS rows: K and V for phases 1-3, then Q and dO for phase 4, CH rows at a
// time (all NP when they fit: windows up to 16; window 24 passes them in two
// chunks per phase, the tiles' accumulators kept in registers across the
// chunks and their row statistics in LDS).
constexpr float kMasked = -1e30f;

template <int NP, int WV, int CH, bool V2>
__global__ __launch_bounds__(WV * 64) void attn_bwd_mfma_kernel(AttnBwd p) {
  constexpr int D = 32, LD = D + 4, NT = WV * 64;
  constexpr int TPW = NP / 16 / WV, NCH = NP / CH;
  static_assert(NP % 32 == 0 && (NP / 16) % WV == 0 && NP % CH == 0 && CH % 32 == 0, "split");
  constexpr int TMAX = NP <= 64 ? 15 * 15 : NP <= 256 ? 31 * 31 : 47 * 47;
  __shared__ __attribute__((aligned(16))) float b0[CH * LD];   // K, then Q
  __shared__ __attribute__((aligned(16))) float b1[CH * LD];   // V, then dO
  __shared__ __attribute__((aligned(16))) float stg[WV][16 * LD];
  __shared__ float rm[NP], rl[NP], rd[NP], nq[NP], nk[NP];
  __shared__ int lab[NP], ra[NP], rb[NP];
  __shared__ float tab[TMAX], dtab[TMAX];
  __shared__ float red[WV];

  const Geom& g = p.g;
  const int M = g.M, N = g.N, C = g.C, R = 2 * M - 1, R2 = R * R;
  const int item = blockIdx.x;
  const int w = item / g.heads, h = item - w * g.heads;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int64_t base = (int64_t)w * N;
  const float* qkv = p.qkv + h * D;
  const float* dout = p.dout + h * D;
  float c = p.scale, t_eff = 1.f;
  if constexpr (V2) {
    t_eff = fmaxf(p.tau[h], p.tau_min);
    c = 1.f / t_eff;
  }

  const int wl = w % g.nW;
  const int wy = wl / g.nWx, wx = wl - wy * g.nWx;
  const bool my = g.s > 0 && wy == g.H / M - 1;
  const bool mx = g.s > 0 && wx == g.nWx - 1;
  for (int e = t; e < R2; e += NT) {
    tab[e] = p.table[(int64_t)e * g.heads + h];
    dtab[e] = 0.f;
  }
  // V2 norm of a 32-float head slice.
  auto norm32 = [&](const float* src) {
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      const float4 a = *reinterpret_cast<const float4*>(src + e);
      sq = fmaf(a.x, a.x, fmaf(a.y, a.y, fmaf(a.z, a.z, fmaf(a.w, a.w, sq))));
    }
    return sqrtf(sq);
  };
  auto copy_row = [&](float* dst, const float* src, float mul) {
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      float4 a = src ? *reinterpret_cast<const float4*>(src + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      a.x *= mul; a.y *= mul; a.z *= mul; a.w *= mul;
      *reinterpret_cast<float4*>(dst + e) = a;
    }
  };
  // Row labels (region; padding 99), relative-index parts and V2 norms.
  for (int r = t; r < NP; r += NT) {
    const bool real = r < N;
    const int ty = real ? r / M : M - 1, tx = real ? r - (r / M) * M : M - 1;
    lab[r] = real ? (my && ty >= M - g.s ? 2 : 0) + (mx && tx >= M - g.s ? 1 : 0) : 99;
    ra[r] = (ty + M - 1) * R + tx + M - 1;
    rb[r] = ty * R + tx;
    const float* row = qkv + (base + r) * 3 * C;
    nq[r] = V2 && real ? norm32(row) : 0.f;
    nk[r] = V2 && real ? norm32(row + C) : 0.f;
  }
  __syncthreads();
  auto inv_norm = [&](float n) { return 1.f / fmaxf(n, p.eps); };
  // Rows c0 .. c0 + CH - 1 of K (unit rows in V2) and V, or of Q and dO.
  auto load_kv = [&](int c0) {
    for (int rr = t; rr < CH; rr += NT) {
      const int r = c0 + rr;
      const bool real = r < N;
      const float* row = qkv + (base + r) * 3 * C;
      copy_row(&b0[rr * LD], real ? row + C : nullptr, V2 && real ? inv_norm(nk[r]) : 1.f);
      copy_row(&b1[rr * LD], real ? row + 2 * C : nullptr, 1.f);
    }
  };
  auto load_qdo = [&](int c0) {
    for (int rr = t; rr < CH; rr += NT) {
      const int r = c0 + rr;
      const bool real = r < N;
      const float* row = qkv + (base + r) * 3 * C;
      copy_row(&b0[rr * LD], real ? row : nullptr, V2 && real ? inv_norm(nq[r]) : 1.f);
      copy_row(&b1[rr * LD], real ? dout + (base + r) * C : nullptr, 1.f);
    }
  };

  auto frag_row = [&](const float* r8) {  // 8 consecutive floats of an LDS row
    const float4 a = *reinterpret_cast<const float4*>(r8);
    const float4 b = *reinterpret_cast<const float4*>(r8 + 4);
    return vec8<float>{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  };
  auto frag_col = [&](const float* buf, int row0, int col) {  // rows row0 .. +7 of a column
    vec8<float> v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = buf[(row0 + e) * LD + col];
    return v;
  };
  // A fragment (row i16, K-slice 8 g4 .. +7) of a 32-float global row, scaled.
  auto frag_glob = [&](const float* src, bool real, float mul) {
    vec8<float> v = {};
    if (real) {
      const float4 a = *reinterpret_cast<const float4*>(src + 8 * g4);
      const float4 b = *reinterpret_cast<const float4*>(src + 8 * g4 + 4);
      v = vec8<float>{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= mul;
    }
    return v;
  };
  auto tidx = [&](int r) { return min(max(r, 0), R2 - 1); };
  float* sw = stg[wave];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // (query row, key) -> logit, or kMasked across regions.
  auto logit = [&](float sraw, int q, int key) {
    return lab[key] == lab[q] ? c * sraw + tab[tidx(ra[q] - rb[key])] : kMasked;
  };

  // ---- phases 1-3: the wave's query tiles ----
  // A fragments of the wave's query tile u (Q unit rows in V2, dO); reread
  // per chunk from L2 rather than held across chunks.
  auto q_frag = [&](int u) {
    const int qa = 16 * (wave * TPW + u) + i16;
    const bool real = qa < N;
    return frag_glob(qkv + (base + qa) * 3 * C, real, V2 && real ? inv_norm(nq[qa]) : 1.f);
  };
  auto do_frag = [&](int u) {
    const int qa = 16 * (wave * TPW + u) + i16;
    return frag_glob(dout + (base + qa) * C, qa < N, 1.f);
  };
  auto qrow_of = [&](int u, int r) { return 16 * (wave * TPW + u) + 4 * g4 + r; };
  float dtau_acc = 0.f;
  if constexpr (NCH == 1) {
    load_kv(0);
    __syncthreads();
  }
  // Phase 1: online max / sum per row over the lane's key columns, then
  // across the 16 lanes of the row group.
  float m[TPW][4], l[TPW][4];
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) { m[u][r] = kMasked; l[u][r] = 0.f; }
#pragma unroll 1
  for (int ch = 0; ch < NCH; ++ch) {
    if constexpr (NCH > 1) {
      __syncthreads();  // every wave is done with the previous chunk
      load_kv(ch * CH);
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const vec8<float> Qa = q_frag(u);
#pragma unroll 2
      for (int kt = 0; kt < CH / 16; ++kt) {
        const int kl = 16 * kt + i16, key = ch * CH + kl;
        const f32x4 S = mma_16x16x32(Qa, frag_row(&b0[kl * LD + 8 * g4]), zero4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sv = logit(S[r], qrow_of(u, r), key);
          const float mn = fmaxf(m[u][r], sv);
          l[u][r] = l[u][r] * __expf(m[u][r] - mn) + __expf(sv - mn);
          m[u][r] = mn;
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
#pragma unroll
    for (int d = 1; d < 16; d <<= 1)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mo = __shfl_xor(m[u][r], d), lo = __shfl_xor(l[u][r], d);
        const float mn = fmaxf(m[u][r], mo);
        l[u][r] = l[u][r] * __expf(m[u][r] - mn) + lo * __expf(mo - mn);
        m[u][r] = mn;
      }
    if (i16 == 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rm[qrow_of(u, r)] = m[u][r];
        rl[qrow_of(u, r)] = 1.f / l[u][r];
      }
  }
  __syncthreads();  // row max and inverse sum visible to the row group
  // Phase 2: P and O = P V; then D_i = sum_j P_ij dP_ij as dO_i . O_i (the
  // same sum, since dP_ij = dO_i . V_j), without forming dP.
  f32x4 o0[TPW], o1[TPW];  // the only per-row state held across chunks
#pragma unroll
  for (int u = 0; u < TPW; ++u) o0[u] = o1[u] = zero4;
#pragma unroll 1
  for (int ch = 0; ch < NCH; ++ch) {
    if constexpr (NCH > 1) {
      __syncthreads();
      load_kv(ch * CH);
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const vec8<float> Qa = q_frag(u);
      float mr[4], ilr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mr[r] = rm[qrow_of(u, r)];
        ilr[r] = rl[qrow_of(u, r)];
      }
#pragma unroll 1
      for (int kb = 0; kb < CH / 32; ++kb) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int kl = 32 * kb + 16 * tt + i16, key = ch * CH + kl;
          const f32x4 S = mma_16x16x32(Qa, frag_row(&b0[kl * LD + 8 * g4]), zero4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pv = __expf(logit(S[r], qrow_of(u, r), key) - mr[r]) * ilr[r];
            sw[(4 * g4 + r) * LD + 16 * tt + i16] = pv;
          }
        }
        asm volatile("" ::: "memory");
        const vec8<float> Pa = frag_row(&sw[i16 * LD + 8 * g4]);
        o0[u] = mma_16x16x32(Pa, frag_col(b1, 32 * kb + 8 * g4, i16), o0[u]);
        o1[u] = mma_16x16x32(Pa, frag_col(b1, 32 * kb + 8 * g4, 16 + i16), o1[u]);
        asm volatile("" ::: "memory");
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    // Lane: dims i16 and 16 + i16 of rows 4 g4 + r; D over the 16 lanes.
    float dd[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = qrow_of(u, r);
      const float* dr = dout + (base + (q < N ? q : 0)) * C;
      dd[r] = q < N ? fmaf(dr[i16], o0[u][r], dr[16 + i16] * o1[u][r]) : 0.f;
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1)
#pragma unroll
      for (int r = 0; r < 4; ++r) dd[r] += __shfl_xor(dd[r], d);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = qrow_of(u, r);
      if (i16 == 0) rd[q] = dd[r];
      if (q < N) {
        float* og = p.o + (base + q) * C + h * D;
        og[i16] = o0[u][r];
        og[16 + i16] = o1[u][r];
      }
    }
  }
  __syncthreads();  // D visible to the row group
  // Phase 3: dS = P (dP - D); table (and tau) gradients; dQ = dS K.
  f32x4 dq0[TPW], dq1[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) dq0[u] = dq1[u] = zero4;
  // dq of tile u (lane: dims i16 and 16 + i16 of the tile's rows 4 g4 + r).
  auto store_dq = [&](int u, f32x4 d0, f32x4 d1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = qrow_of(u, r);
      float a0 = c * d0[r], a1 = c * d1[r];
      if constexpr (V2) {
        // Through q_hat = q / max(|q|, eps): (dq_hat - q_hat (q_hat . dq_hat)) / |q|.
        const bool real = q < N;
        const float* qr = qkv + (base + (real ? q : 0)) * 3 * C;
        const float inv = inv_norm(nq[q]);
        const float h0 = real ? qr[i16] * inv : 0.f, h1 = real ? qr[16 + i16] * inv : 0.f;
        float pr = h0 * a0 + h1 * a1;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) pr += __shfl_xor(pr, d);
        const bool big = nq[q] > p.eps;
        a0 = (big ? a0 - h0 * pr : a0) * inv;
        a1 = (big ? a1 - h1 * pr : a1) * inv;
      }
      if (q < N) {
        float* dg = p.dqkv + (base + q) * 3 * C + h * D;
        dg[i16] = a0;
        dg[16 + i16] = a1;
      }
    }
  };
#pragma unroll 1
  for (int ch = 0; ch < NCH; ++ch) {
    if constexpr (NCH > 1) {
      __syncthreads();
      load_kv(ch * CH);
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const vec8<float> Qa = q_frag(u), DOa = do_frag(u);
      float mr[4], ilr[4], dr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mr[r] = rm[qrow_of(u, r)];
        ilr[r] = rl[qrow_of(u, r)];
        dr[r] = rd[qrow_of(u, r)];
      }
#pragma unroll 1
      for (int kb = 0; kb < CH / 32; ++kb) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int kl = 32 * kb + 16 * tt + i16, key = ch * CH + kl;
          const f32x4 S = mma_16x16x32(Qa, frag_row(&b0[kl * LD + 8 * g4]), zero4);
          const f32x4 dP = mma_16x16x32(DOa, frag_row(&b1[kl * LD + 8 * g4]), zero4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = qrow_of(u, r);
            const bool ok = lab[key] == lab[q];
            const int ti = tidx(ra[q] - rb[key]);
            const float pv = ok ? __expf(c * S[r] + tab[ti] - mr[r]) * ilr[r] : 0.f;
            const float ds = pv * (dP[r] - dr[r]);
            if (ok) atomicAdd(&dtab[ti], ds);
            if constexpr (V2) dtau_acc = fmaf(ds, S[r], dtau_acc);
            sw[(4 * g4 + r) * LD + 16 * tt + i16] = ds;
          }
        }
        asm volatile("" ::: "memory");
        const vec8<float> Sa = frag_row(&sw[i16 * LD + 8 * g4]);
        dq0[u] = mma_16x16x32(Sa, frag_col(b0, 32 * kb + 8 * g4, i16), dq0[u]);
        dq1[u] = mma_16x16x32(Sa, frag_col(b0, 32 * kb + 8 * g4, 16 + i16), dq1[u]);
        asm volatile("" ::: "memory");
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) store_dq(u, dq0[u], dq1[u]);
  __syncthreads();  // K, V no longer read; row statistics complete
  if constexpr (NCH == 1) {
    load_qdo(0);
    __syncthreads();
  }

  // ---- phase 4: the wave's key tiles ----
  f32x4 dk0[TPW], dk1[TPW], dv0[TPW], dv1[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) dk0[u] = dk1[u] = dv0[u] = dv1[u] = zero4;
  // dk, dv of key tile u.
  auto store_dkv = [&](int u, f32x4 k0, f32x4 k1, f32x4 v0, f32x4 v1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = qrow_of(u, r);
      float a0 = c * k0[r], a1 = c * k1[r];
      if constexpr (V2) {
        const bool real = k < N;
        const float* kr = qkv + (base + (real ? k : 0)) * 3 * C + C;
        const float inv = inv_norm(nk[k]);
        const float h0 = real ? kr[i16] * inv : 0.f, h1 = real ? kr[16 + i16] * inv : 0.f;
        float pr = h0 * a0 + h1 * a1;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) pr += __shfl_xor(pr, d);
        const bool big = nk[k] > p.eps;
        a0 = (big ? a0 - h0 * pr : a0) * inv;
        a1 = (big ? a1 - h1 * pr : a1) * inv;
      }
      if (k < N) {
        float* dg = p.dqkv + (base + k) * 3 * C + C + h * D;
        dg[i16] = a0;
        dg[16 + i16] = a1;
        dg[C + i16] = v0[r];
        dg[C + 16 + i16] = v1[r];
      }
    }
  };
#pragma unroll 1
  for (int ch = 0; ch < NCH; ++ch) {
    if constexpr (NCH > 1) {
      __syncthreads();
      load_qdo(ch * CH);
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int ka = 16 * (wave * TPW + u) + i16;
      const bool ka_real = ka < N;
      const float* krow = qkv + (base + ka) * 3 * C;
      const vec8<float> Ka = frag_glob(krow + C, ka_real, V2 && ka_real ? inv_norm(nk[ka]) : 1.f);
      const vec8<float> Va = frag_glob(krow + 2 * C, ka_real, 1.f);
#pragma unroll 1
      for (int qb = 0; qb < CH / 32; ++qb) {
        float pst[2][4], dst[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int ql = 32 * qb + 16 * tt + i16, q = ch * CH + ql;  // this lane's query column
          const f32x4 ST = mma_16x16x32(Ka, frag_row(&b0[ql * LD + 8 * g4]), zero4);
          const f32x4 dPT = mma_16x16x32(Va, frag_row(&b1[ql * LD + 8 * g4]), zero4);
          const float mq = rm[q], ilq = rl[q], dq_ = rd[q];
          const int labq = lab[q], raq = ra[q];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int k = qrow_of(u, r);
            const bool ok = labq == lab[k];
            const float pv = ok ? __expf(c * ST[r] + tab[tidx(raq - rb[k])] - mq) * ilq : 0.f;
            pst[tt][r] = pv;
            dst[tt][r] = pv * (dPT[r] - dq_);
          }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sw[(4 * g4 + r) * LD + 16 * tt + i16] = pst[tt][r];
        asm volatile("" ::: "memory");
        const vec8<float> Pa = frag_row(&sw[i16 * LD + 8 * g4]);
        dv0[u] = mma_16x16x32(Pa, frag_col(b1, 32 * qb + 8 * g4, i16), dv0[u]);
        dv1[u] = mma_16x16x32(Pa, frag_col(b1, 32 * qb + 8 * g4, 16 + i16), dv1[u]);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sw[(4 * g4 + r) * LD + 16 * tt + i16] = dst[tt][r];
        asm volatile("" ::: "memory");
        const vec8<float> Sa = frag_row(&sw[i16 * LD + 8 * g4]);
        dk0[u] = mma_16x16x32(Sa, frag_col(b0, 32 * qb + 8 * g4, i16), dk0[u]);
        dk1[u] = mma_16x16x32(Sa, frag_col(b0, 32 * qb + 8 * g4, 16 + i16), dk1[u]);
        asm volatile("" ::: "memory");
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) store_dkv(u, dk0[u], dk1[u], dv0[u], dv1[u]);
  __syncthreads();  // every wave's table-gradient adds are in dtab
  for (int e = t; e < R2; e += NT) atomicAdd(p.dtable + (int64_t)e * g.heads + h, dtab[e]);
  if constexpr (V2) {
    float v = dtau_acc;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    if (t == 0 && p.tau[h] > p.tau_min) {
      float sum = 0.f;
      for (int k = 0; k < WV; ++k) sum += red[k];
      atomicAdd(p.dtau + h, -sum / (t_eff * t_eff));
    }
  }
}

template <int NP, int WV, int CH>
void attn_bwd_launch(const AttnBwd& p, bool v2, int items, hipStream_t st) {
  if (v2)
    hipLaunchKernelGGL((attn_bwd_mfma_kernel<NP, WV, CH, true>), dim3(items), dim3(64 * WV), 0, st,
                       p);
  else
    hipLaunchKernelGGL((attn_bwd_mfma_kernel<NP, WV, CH, false>), dim3(items), dim3(64 * WV), 0,
                       st, p);
}

template <typename TA, typename TB, typename TC, bool ATOMIC>
hipError_t gemm_launch(const BwdGemm& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return hipSuccess;
  // Staging reads runs of 8 along a unit stride of each operand.
  if ((a.sak != 1 && a.sam != 1) || (a.sbn != 1 && a.sbk != 1)) return hipErrorInvalidValue;
  if ((a.sak == 1 ? a.sam : a.sak) % 8 || (a.sbn == 1 ? a.sbk : a.sbn) % 8)
    return hipErrorInvalidValue;
  BwdGemm b = a;
  int splits = 1;
  if (ATOMIC) {
    // Split the reduction so that the grid fills the chip (about 2048 groups).
    const int64_t tiles = ((a.M + kGT - 1) / kGT) * (int64_t)((a.N + kGT - 1) / kGT);
    int64_t want = 2048 / (tiles > 0 ? tiles : 1);
    if (want < 1) want = 1;
    int64_t kc = (a.K + want - 1) / want;
    kc = (kc + kGK - 1) / kGK * kGK;
    b.kc = kc;
    splits = (int)((a.K + kc - 1) / kc);
  } else {
    b.kc = a.K;
  }
  const dim3 grid((a.N + kGT - 1) / kGT, (unsigned)((a.M + kGT - 1) / kGT), splits);
  hipLaunchKernelGGL((bwd_gemm_kernel<TA, TB, TC, ATOMIC>), grid, dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

#define TRY(x)                        \
  do {                                \
    hipError_t e_ = (x);              \
    if (e_ != hipSuccess) return e_;  \
  } while (0)

template <typename T>
hipError_t backward(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int C = g.C;
  const int64_t T_ = (int64_t)g.B * g.H * g.W;
  const int eb = (int)sizeof(T);
  const int R2 = (2 * g.M - 1) * (2 * g.M - 1);
  // Gradients that are accumulated start at zero.
  TRY(zero(a.dw_qkv, 3LL * C * C, st));
  TRY(zero(a.db_qkv, 3LL * C, st));
  TRY(zero(a.dw_proj, (int64_t)C * C, st));
  TRY(zero(a.db_proj, C, st));
  TRY(zero(a.dtable, (int64_t)R2 * g.heads, st));
  if (a.v2) TRY(zero(a.dtau, g.heads, st));
  if (T_ == 0) return hipSuccess;
  // Window order of x and dy.
  TRY(launch_partition_shift(a.x, a.xw, g, eb, st));
  TRY(launch_partition_shift(a.dy, a.dyw, g, eb, st));
  // qkv = xw Wqkv^T + bqkv   [T, 3C]
  BwdGemm q{};
  q.M = T_; q.N = 3 * C; q.K = C;
  q.A = a.xw; q.sam = C; q.sak = 1;
  q.B = a.w_qkv; q.sbk = 1; q.sbn = C;
  q.bias = a.b_qkv; q.C = a.qkv; q.ldc = 3 * C;
  TRY((gemm_launch<T, T, float, false>(q, st)));
  // do = dyw Wp   [T, C]   (y = o Wp^T + bp)
  BwdGemm d{};
  d.M = T_; d.N = C; d.K = C;
  d.A = a.dyw; d.sam = C; d.sak = 1;
  d.B = a.w_proj; d.sbk = C; d.sbn = 1;
  d.C = a.dout; d.ldc = C;
  TRY((gemm_launch<T, T, float, false>(d, st)));
  // Attention backward per (window, head).
  AttnBwd p{};
  p.g = g; p.scale = a.scale; p.tau_min = a.tau_min; p.eps = a.eps;
  p.qkv = a.qkv; p.dout = a.dout; p.table = a.table; p.tau = a.tau;
  p.o = a.o; p.dqkv = a.dqkv; p.dtable = a.dtable; p.dtau = a.dtau;
  const int items = g.B * g.nW * g.heads;
  if (g.N <= 32) attn_bwd_launch<32, 2, 32>(p, a.v2, items, st);
  else if (g.N <= 64) attn_bwd_launch<64, 4, 64>(p, a.v2, items, st);
  else if (g.N <= 128) attn_bwd_launch<128, 8, 128>(p, a.v2, items, st);
  else if (g.N <= 256) attn_bwd_launch<256, 16, 256>(p, a.v2, items, st);
  else attn_bwd_launch<576, 12, 288>(p, a.v2, items, st);  // windows up to 24
  TRY(hipGetLastError());
  // dWp = dyw^T o   [C, C];  dbp = column sums of dyw
  BwdGemm wp{};
  wp.M = C; wp.N = C; wp.K = T_;
  wp.A = a.dyw; wp.sam = 1; wp.sak = C;
  wp.B = a.o; wp.sbk = C; wp.sbn = 1;
  wp.C = a.dw_proj; wp.ldc = C;
  wp.rowsum = a.db_proj;  // dbp = column sums of dyw
  TRY((gemm_launch<T, float, float, true>(wp, st)));
  // dWqkv = dqkv^T xw   [3C, C];  dbqkv = column sums of dqkv
  BwdGemm wq{};
  wq.M = 3 * C; wq.N = C; wq.K = T_;
  wq.A = a.dqkv; wq.sam = 1; wq.sak = 3 * C;
  wq.B = a.xw; wq.sbk = C; wq.sbn = 1;
  wq.C = a.dw_qkv; wq.ldc = C;
  wq.rowsum = a.db_qkv;  // dbqkv = column sums of dqkv
  TRY((gemm_launch<float, T, float, true>(wq, st)));
  // dxw = dqkv Wqkv   [T, C], then back to image order.
  BwdGemm dx{};
  dx.M = T_; dx.N = C; dx.K = 3 * C;
  dx.A = a.dqkv; dx.sam = 3 * C; dx.sak = 1;
  dx.B = a.w_qkv; dx.sbk = C; dx.sbn = 1;
  dx.C = a.dxw; dx.ldc = C;
  TRY((gemm_launch<float, T, T, false>(dx, st)));
  TRY(launch_reverse_unshift(a.dxw, a.dx, g, eb, st));
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t st) {
  // The attention kernel pads a window to at most 576 tokens (window 24).
  if (a.g.M > 24 || a.g.C != 32 * a.g.heads) return hipErrorInvalidValue;
  if (a.io == kF32) return backward<float>(a, st);
  if (a.io == kF16) return backward<h16>(a, st);
  return backward<b16>(a, st);
}

}  // namespace swin
