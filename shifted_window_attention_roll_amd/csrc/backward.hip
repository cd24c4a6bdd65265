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
//   dbp, dbqkv = column sums of dyw, dqkv                         (colsum)
//   dxw = dqkv Wqkv, dx = reverse+unshift(dxw)                    (bwd_gemm,
//                                                                   index map)
// The inverse of a permutation is its adjoint, so the index maps of the
// forward carry the gradients between the image and window orders.
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

// C[m][n] (+)= sum_k A(m, k) B(k, n) (+ bias[n]) with element strides, float32
// on the matrix cores (16x16x4 float32 products, eight per 32-deep step).
// 64 x 64 tile per workgroup of 4 waves, 32 x 32 per wave; K in steps of 32
// through LDS, both operands stored [row][k] (k contiguous) so that a lane's
// fragment is two 16-byte reads; blockIdx.z takes the K range [z*kc,
// (z+1)*kc).  ATOMIC adds the tile into C (float) instead of storing it; then
// only z = 0 adds bias.
constexpr int kGT = 64, kGK = 32, kGP = kGK + 4;

template <typename TA, typename TB, typename TC, bool ATOMIC>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(BwdGemm a) {
  __shared__ __attribute__((aligned(16))) float As[kGT * kGP];  // [m][k]
  __shared__ __attribute__((aligned(16))) float Bs[kGT * kGP];  // [n][k]
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
  for (int64_t kb = k0; kb < k1; kb += kGK) {
    // Each thread stages one run of 8 elements of each operand along its
    // unit-stride dimension (k, or the row dimension m / n).
    {
      float v[8];
      if (a_k_unit) {
        const int mm = tid >> 2, kk = (tid & 3) * 8;
        const int64_t m = m0 + mm, k = kb + kk;
        load_run8(A, m * a.sam + k, m < a.M ? (int)min<int64_t>(k1 - k, 8) : 0, v);
        store_row8(&As[mm * kGP + kk], v);
      } else {
        const int kk = tid >> 3, mm = (tid & 7) * 8;
        const int64_t m = m0 + mm, k = kb + kk;
        load_run8(A, m + k * a.sak, k < k1 ? (int)min<int64_t>(a.M - m, 8) : 0, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) As[(mm + i) * kGP + kk] = v[i];
      }
      if (!b_n_unit) {
        const int nn = tid >> 2, kk = (tid & 3) * 8;
        const int n = n0 + nn;
        const int64_t k = kb + kk;
        load_run8(B, (int64_t)n * a.sbn + k, n < a.N ? (int)min<int64_t>(k1 - k, 8) : 0, v);
        store_row8(&Bs[nn * kGP + kk], v);
      } else {
        const int kk = tid >> 3, nn = (tid & 7) * 8;
        const int n = n0 + nn;
        const int64_t k = kb + kk;
        load_run8(B, n + k * a.sbk, k < k1 ? (int)min<int64_t>(a.N - n, 8) : 0, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) Bs[(nn + i) * kGP + kk] = v[i];
      }
    }
    __syncthreads();
    vec8<float> af[2], bf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float* pa = &As[(wm * 32 + i * 16 + i16) * kGP + 8 * g4];
      const float* pb = &Bs[(wn * 32 + i * 16 + i16) * kGP + 8 * g4];
      const float4 a0 = *reinterpret_cast<const float4*>(pa);
      const float4 a1 = *reinterpret_cast<const float4*>(pa + 4);
      const float4 b0 = *reinterpret_cast<const float4*>(pb);
      const float4 b1 = *reinterpret_cast<const float4*>(pb + 4);
      af[i] = vec8<float>{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      bf[i] = vec8<float>{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mma_16x16x32(af[i], bf[j], acc[i][j]);
    __syncthreads();
  }
  // Lane l holds column l % 16 of rows 4 (l / 16) .. +3 of each 16 x 16 tile.
  TC* C = static_cast<TC*>(a.C);
  const bool add_bias = a.bias && (!ATOMIC || blockIdx.z == 0);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 32 + j * 16 + i16;
    if (n >= a.N) continue;
    const float bn = add_bias ? ld(static_cast<const TB*>(a.bias), n) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 32 + i * 16 + 4 * g4 + r;
        if (m >= a.M) continue;
        const float v = acc[i][j][r] + bn;
        if constexpr (ATOMIC)
          atomicAdd(reinterpret_cast<float*>(C) + m * a.ldc + n, v);
        else
          C[m * a.ldc + n] = from_f32<TC>(v);
      }
  }
}

// out[c] += sum over rows [z*rc, (z+1)*rc) of src[r*ld + c]; one column per thread.
template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(const T* src, int64_t rows, int cols,
                                                     int64_t ld, int64_t rc, float* out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * rc;
  const int64_t r1 = r0 + rc < rows ? r0 + rc : rows;
  float s = 0.f;
  for (int64_t r = r0; r < r1; ++r) s += (float)src[r * ld + c];
  atomicAdd(out + c, s);
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

// Per (window, head): recompute the attention and take its gradients.  One
// workgroup per item; thread t owns query row t (phases 1-3) and key row t
// (phase 4), and keeps that row's q, dO (then k, v) in registers.  Two LDS
// row buffers of 32 floats per token: K and V for phases 1-3, then Q and dO
// for phase 4 (the loops over the other index read one row per step, the same
// for every lane: a broadcast).
//   phase 0: V2 normalises q and k (keeps the norms);
//   phase 1: row max m_i and sum l_i of exp(S_ij - m_i) over allowed keys;
//   phase 2: O_i = sum_j P_ij v_j (stored), D_i = dO_i . O_i;
//   phase 3: dS_ij = P_ij (dO_i . v_j - D_i); dq_i; table and tau gradients;
//   phase 4: dv_j = sum_i P_ij dO_i, dk_j = sum_i dS_ij q_i.
// S_ij = c (q_i . k_j) + table[rel(i, j)], c = scale (V1) or 1 / max(tau,
// tau_min) on unit q, k (V2).  Masked pairs (labels differ) are skipped: their
// weight and gradient are zero.
constexpr float kMasked = -1e30f;

template <int NMAX, bool V2>
__global__ __launch_bounds__(NMAX) __attribute__((amdgpu_waves_per_eu(3))) void attn_bwd_kernel(AttnBwd p) {
  constexpr int D = 32;
  constexpr int TMAX = NMAX <= 64 ? 15 * 15 : 31 * 31;  // (2M-1)^2 for M <= 8, 16
  __shared__ __attribute__((aligned(16))) float b0[NMAX][D];  // K, then Q
  __shared__ __attribute__((aligned(16))) float b1[NMAX][D];  // V, then dO
  __shared__ float rm[NMAX], rl[NMAX], rd[NMAX];
  __shared__ int lab[NMAX];
  // rel(i, j) = ra[i] - rb[j]: ra = (y + M-1) R + x + M-1, rb = y R + x.
  __shared__ int ra[NMAX], rb[NMAX];
  __shared__ float tab[TMAX], dtab[TMAX];
  __shared__ float red[NMAX / 64];

  const Geom& g = p.g;
  const int M = g.M, N = g.N, C = g.C, R = 2 * M - 1;
  const int item = blockIdx.x;
  const int w = item / g.heads, h = item - w * g.heads;
  const int t = threadIdx.x;
  const bool row = t < N;
  const int64_t base = (int64_t)w * N;  // first window-order row of the window

  // Region labels: only the last window row / column of the grid mixes two
  // slices of the shifted frame, split at M - s.
  const int wl = w % g.nW;
  const int wy = wl / g.nWx, wx = wl - wy * g.nWx;
  const bool my = g.s > 0 && wy == g.H / M - 1;
  const bool mx = g.s > 0 && wx == g.nWx - 1;
  const int ty = t / M, tx = t - (t / M) * M;
  if (row) {
    lab[t] = (my && ty >= M - g.s ? 2 : 0) + (mx && tx >= M - g.s ? 1 : 0);
    ra[t] = (ty + M - 1) * R + tx + M - 1;
    rb[t] = ty * R + tx;
  }
  for (int e = t; e < R * R; e += NMAX) {
    tab[e] = p.table[(int64_t)e * g.heads + h];
    dtab[e] = 0.f;
  }
  // Own rows: q_t and dO_t in registers for phases 1-3; k_t and v_t go to LDS
  // (and are read again from memory for phase 4).
  float qi[D], doi[D];
  float c = p.scale, t_eff = 1.f, nq = 0.f;
  if constexpr (V2) {
    t_eff = fmaxf(p.tau[h], p.tau_min);
    c = 1.f / t_eff;
  }
  const float* src = p.qkv + (base + t) * 3 * C + h * D;
  // Row r of a 32-float head slice: 8 float4 loads into a register array.
  auto load_row = [&](const float* g_, float (&v)[D]) {
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      const float4 a = *reinterpret_cast<const float4*>(g_ + e);
      v[e] = a.x; v[e + 1] = a.y; v[e + 2] = a.z; v[e + 3] = a.w;
    }
  };
  // V2: v / max(|v|, eps) in place; returns |v|.
  auto unit = [&](float (&v)[D]) {
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) sq = fmaf(v[e], v[e], sq);
    const float n = sqrtf(sq), inv = 1.f / fmaxf(n, p.eps);
#pragma unroll
    for (int e = 0; e < D; ++e) v[e] *= inv;
    return n;
  };
  auto store_row = [&](float* l_, const float (&v)[D]) {
#pragma unroll
    for (int e = 0; e < D; e += 4)
      *reinterpret_cast<float4*>(l_ + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
  };
  if (row) {
    {
      float kv[D];
      load_row(src + C, kv);
      if constexpr (V2) unit(kv);
      store_row(b0[t], kv);
      load_row(src + 2 * C, kv);
      store_row(b1[t], kv);
    }
    load_row(src, qi);
    load_row(p.dout + (base + t) * C + h * D, doi);
    if constexpr (V2) nq = unit(qi);
  }
  __syncthreads();

  // a . b for a row b in LDS (16-byte reads).
  auto dot = [&](const float (&a)[D], const float* b) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      const float4 bv = *reinterpret_cast<const float4*>(b + e);
      s = fmaf(a[e], bv.x, s);
      s = fmaf(a[e + 1], bv.y, s);
      s = fmaf(a[e + 2], bv.z, s);
      s = fmaf(a[e + 3], bv.w, s);
    }
    return s;
  };
  // acc += f * b for a row b in LDS.
  auto axpy = [&](float (&acc)[D], float f, const float* b) {
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      const float4 bv = *reinterpret_cast<const float4*>(b + e);
      acc[e] = fmaf(f, bv.x, acc[e]);
      acc[e + 1] = fmaf(f, bv.y, acc[e + 1]);
      acc[e + 2] = fmaf(f, bv.z, acc[e + 2]);
      acc[e + 3] = fmaf(f, bv.w, acc[e + 3]);
    }
  };

  float dtau_acc = 0.f;
  if (row) {
    const int i = t;
    const int li = lab[i];
    const int ai = ra[i];
    // Phase 1.
    // Masked pairs get the logit kMasked: exp underflows to exactly 0, so
    // they add nothing, and the loops need no branch (the pair (i, i) is
    // always allowed, so the row max is a real logit).
    float m = kMasked, l = 0.f;
#pragma unroll 2
    for (int j = 0; j < N; ++j) {
      const float sij = lab[j] != li ? kMasked : c * dot(qi, b0[j]) + tab[ai - rb[j]];
      const float mn = fmaxf(m, sij);
      l = l * __expf(m - mn) + __expf(sij - mn);
      m = mn;
    }
    const float il = 1.f / l;
    // Phase 2.
    float o[D] = {};
#pragma unroll 2
    for (int j = 0; j < N; ++j) {
      const float sij = lab[j] != li ? kMasked : c * dot(qi, b0[j]) + tab[ai - rb[j]];
      const float pij = __expf(sij - m) * il;
      axpy(o, pij, b1[j]);
    }
    float di = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) di = fmaf(doi[e], o[e], di);
    float* og = p.o + (base + i) * C + h * D;
#pragma unroll
    for (int e = 0; e < D; e += 4)
      *reinterpret_cast<float4*>(og + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
    rm[i] = m;
    rl[i] = il;
    rd[i] = di;
    // Phase 3.
    float dq[D] = {};
#pragma unroll 2
    for (int j = 0; j < N; ++j) {
      const float sim = dot(qi, b0[j]);
      const int r = ai - rb[j];
      const float pij = lab[j] != li ? 0.f : __expf(c * sim + tab[r] - m) * il;
      const float dsij = pij * (dot(doi, b1[j]) - di);
      asm volatile("" ::: "memory");  // read the K row again: fewer live registers
      axpy(dq, dsij, b0[j]);
      atomicAdd(&dtab[r], dsij);  // distinct i give distinct r for one j
      if constexpr (V2) dtau_acc = fmaf(dsij, sim, dtau_acc);
    }
    float* dqg = p.dqkv + (base + i) * 3 * C + h * D;
    if constexpr (V2) {
      // dq_hat = c sum dS k_hat; through q_hat = q / max(|q|, eps).
      float pr = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        dq[e] *= c;
        pr = fmaf(qi[e], dq[e], pr);
      }
      const bool big = nq > p.eps;
      const float inv = 1.f / fmaxf(nq, p.eps);
#pragma unroll
      for (int e = 0; e < D; ++e) dq[e] = (big ? dq[e] - qi[e] * pr : dq[e]) * inv;
    } else {
#pragma unroll
      for (int e = 0; e < D; ++e) dq[e] *= c;
    }
#pragma unroll
    for (int e = 0; e < D; e += 4)
      *reinterpret_cast<float4*>(dqg + e) = make_float4(dq[e], dq[e + 1], dq[e + 2], dq[e + 3]);
  }
  __syncthreads();  // every read of K, V done; row statistics complete
  if (row) {
    store_row(b0[t], qi);
    store_row(b1[t], doi);
  }
  __syncthreads();

  if (row) {
    // Phase 4, thread t owns key row j = t.
    const int j = t;
    float ki[D], vi[D], nk = 0.f;
    load_row(src + C, ki);
    load_row(src + 2 * C, vi);
    if constexpr (V2) nk = unit(ki);
    const int lj = lab[j];
    const int bj = rb[j];
    float dk[D] = {}, dv[D] = {};
#pragma unroll 2
    for (int i = 0; i < N; ++i) {
      const float sij = c * dot(ki, b0[i]) + tab[ra[i] - bj];
      const float pij = lab[i] != lj ? 0.f : __expf(sij - rm[i]) * rl[i];
      const float dsij = pij * (dot(vi, b1[i]) - rd[i]);
      asm volatile("" ::: "memory");  // read the rows again: fewer live registers
      axpy(dv, pij, b1[i]);
      axpy(dk, dsij, b0[i]);
    }
    if constexpr (V2) {
      float pr = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        dk[e] *= c;
        pr = fmaf(ki[e], dk[e], pr);
      }
      const bool big = nk > p.eps;
      const float inv = 1.f / fmaxf(nk, p.eps);
#pragma unroll
      for (int e = 0; e < D; ++e) dk[e] = (big ? dk[e] - ki[e] * pr : dk[e]) * inv;
    } else {
#pragma unroll
      for (int e = 0; e < D; ++e) dk[e] *= c;
    }
    float* dkg = p.dqkv + (base + j) * 3 * C + C + h * D;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      *reinterpret_cast<float4*>(dkg + e) = make_float4(dk[e], dk[e + 1], dk[e + 2], dk[e + 3]);
      *reinterpret_cast<float4*>(dkg + C + e) = make_float4(dv[e], dv[e + 1], dv[e + 2], dv[e + 3]);
    }
  }
  for (int e = t; e < R * R; e += NMAX) atomicAdd(p.dtable + (int64_t)e * g.heads + h, dtab[e]);
  if constexpr (V2) {
    // d(t_eff) = -sum dS cos / t_eff^2, passed to tau where tau > tau_min.
    float v = dtau_acc;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    if (t == 0 && p.tau[h] > p.tau_min) {
      float s = 0.f;
      for (int k = 0; k < NMAX / 64; ++k) s += red[k];
      atomicAdd(p.dtau + h, -s / (t_eff * t_eff));
    }
  }
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

template <typename T>
hipError_t colsum_launch(const T* src, int64_t rows, int cols, int64_t ld, float* out,
                         hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int cb = (cols + 255) / 256;
  int64_t splits = 2048 / cb;
  if (splits > rows) splits = rows;
  if (splits < 1) splits = 1;
  const int64_t rc = (rows + splits - 1) / splits;
  splits = (rows + rc - 1) / rc;
  hipLaunchKernelGGL((colsum_kernel<T>), dim3(cb, (unsigned)splits), dim3(256), 0, st, src, rows,
                     cols, ld, rc, out);
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
  if (g.N <= 64) {
    if (a.v2) hipLaunchKernelGGL((attn_bwd_kernel<64, true>), dim3(items), dim3(64), 0, st, p);
    else hipLaunchKernelGGL((attn_bwd_kernel<64, false>), dim3(items), dim3(64), 0, st, p);
  } else {
    if (a.v2) hipLaunchKernelGGL((attn_bwd_kernel<256, true>), dim3(items), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((attn_bwd_kernel<256, false>), dim3(items), dim3(256), 0, st, p);
  }
  TRY(hipGetLastError());
  // dWp = dyw^T o   [C, C];  dbp = colsum(dyw)
  BwdGemm wp{};
  wp.M = C; wp.N = C; wp.K = T_;
  wp.A = a.dyw; wp.sam = 1; wp.sak = C;
  wp.B = a.o; wp.sbk = C; wp.sbn = 1;
  wp.C = a.dw_proj; wp.ldc = C;
  TRY((gemm_launch<T, float, float, true>(wp, st)));
  TRY(colsum_launch<T>(static_cast<const T*>(a.dyw), T_, C, C, a.db_proj, st));
  // dWqkv = dqkv^T xw   [3C, C];  dbqkv = colsum(dqkv)
  BwdGemm wq{};
  wq.M = 3 * C; wq.N = C; wq.K = T_;
  wq.A = a.dqkv; wq.sam = 1; wq.sak = 3 * C;
  wq.B = a.xw; wq.sbk = C; wq.sbn = 1;
  wq.C = a.dw_qkv; wq.ldc = C;
  TRY((gemm_launch<float, T, float, true>(wq, st)));
  TRY(colsum_launch<float>(a.dqkv, T_, 3 * C, 3 * C, a.db_qkv, st));
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
  if (a.g.M > 16 || a.g.C != 32 * a.g.heads) return hipErrorInvalidValue;
  if (a.io == kF32) return backward<float>(a, st);
  if (a.io == kF16) return backward<h16>(a, st);
  return backward<b16>(a, st);
}

}  // namespace swin
