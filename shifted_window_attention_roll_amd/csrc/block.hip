// Full Swin block forward around the attention sub-layer: the two LayerNorms,
// the MLP (Linear + GELU, Linear) and the residual connections, in the V1
// pre-norm and the V2 post-norm arrangement.
//
// Pages: "Boost Vision Transformer with GPU-Friendly Sparsity and Quantization",
// Section 3.2 / Figure 3 (the Swin block is the standard transformer block with
// shifted-window attention in place of multi-head attention; the feed-forward
// layers are GEMMs) and Section 2.2 (GeLU as the activation); "Boosting Swin
// Transformer Speed", Training Optimization (LayerNorm is part of the block);
// "Swin Transformer V2" summary, How It Works (V1 normalises before each
// sub-layer, V2 normalises each residual branch before adding it back).
//
//   V1:  h = x + A(LN1(x)),   y = h + F(LN2(h))
//   V2:  h = x + LN1(A(x)),   y = h + LN2(F(h))
// with A = swin_wmsa_fwd and F(u) = GELU(u W1^T + b1) W2^T + b2 (exact GELU).
//
// Kernels: ln_kernel (one wave per token; the residual adds are fused into it
// or into the second GEMM) and the dense layers: the persistent tiled GEMM of
// gemm_tiled.hip (16-bit, N % 128 == 0, K in 256 .. 2048) or else dense_kernel
// (the general matrix-core tile of gemm_core.hpp), both with a bias / GELU /
// residual epilogue.
#include <string.h>

#include <type_traits>

#include "gemm_core.hpp"
#include "launch.hpp"
#include "swin_wmsa.h"

namespace swin {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

constexpr int kLnMaxC = 512;

// Sum over the LPR consecutive lanes that share a row (LPR a power of two).
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int d = LPR / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// v = a (+ b); u (if given) <- v; out <- LN(v) * gamma + beta (+ r).  LayerNorm
// over the C channels of a token, biased variance, in float32.  Each lane takes
// one 16-byte chunk (8 channels) of a row, LPR lanes a row (C <= 8 LPR), so a
// wave covers 64 / LPR rows with full-width loads and stores.
template <typename T, int LPR>
__global__ __launch_bounds__(256) void ln_kernel(const T* __restrict__ a, const T* __restrict__ b,
                                                 T* __restrict__ u, const T* __restrict__ gamma,
                                                 const T* __restrict__ beta,
                                                 const T* __restrict__ r, T* __restrict__ out,
                                                 int rows, int C, float eps) {
  static_assert(sizeof(T) == 2, "16-bit rows");
  constexpr int RPW = 64 / LPR;  // rows per wave
  const int lane = threadIdx.x & 63;
  const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int c0 = 8 * (lane % LPR);
  const bool live = row < rows && c0 < C;  // idle lanes still join the reductions
  const int64_t o = (int64_t)row * C + c0;
  float v[8];
  float s = 0.f;
  if (live) {
    const vec8<T> av = gload8(a + o);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)av[e];
    if (b) {
      const vec8<T> bv = gload8(b + o);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += (float)bv[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[e];
  }
  const float mean = group_sum<LPR>(s) / (float)C;
  float q = 0.f;
  if (live) {
#pragma unroll
    for (int e = 0; e < 8; ++e) q += (v[e] - mean) * (v[e] - mean);
  }
  const float rstd = 1.0f / sqrtf(group_sum<LPR>(q) / (float)C + eps);
  if (!live) return;
  if (u) {
    vec8<T> uv;
#pragma unroll
    for (int e = 0; e < 8; ++e) uv[e] = (T)v[e];
    gstore16(u + o, __builtin_bit_cast(uint4, uv));
  }
  const vec8<T> gv = gload8(gamma + c0), bev = gload8(beta + c0);
  float z[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (v[e] - mean) * rstd * (float)gv[e] + (float)bev[e];
  if (r) {
    const vec8<T> rv = gload8(r + o);
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] += (float)rv[e];
  }
  vec8<T> zv;
#pragma unroll
  for (int e = 0; e < 8; ++e) zv[e] = (T)z[e];
  gstore16(out + o, __builtin_bit_cast(uint4, zv));
}

// float32 rows: one wave per row, lane c, c + 64, ... (up to 8 per lane).
template <>
__global__ __launch_bounds__(256) void ln_kernel<float, 64>(
    const float* __restrict__ a, const float* __restrict__ b, float* __restrict__ u,
    const float* __restrict__ gamma, const float* __restrict__ beta, const float* __restrict__ r,
    float* __restrict__ out, int rows, int C, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = (int64_t)row * C;
  float v[8];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane + 64 * i;
    v[i] = 0.f;
    if (c < C) {
      v[i] = a[base + c] + (b ? b[base + c] : 0.f);
      s += v[i];
    }
  }
  const float mean = group_sum<64>(s) / (float)C;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane + 64 * i;
    if (c < C) q += (v[i] - mean) * (v[i] - mean);
  }
  const float rstd = 1.0f / sqrtf(group_sum<64>(q) / (float)C + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane + 64 * i;
    if (c >= C) continue;
    if (u) u[base + c] = v[i];
    float z = (v[i] - mean) * rstd * gamma[c] + beta[c];
    if (r) z += r[base + c];
    out[base + c] = z;
  }
}

// Y = act(A Wt^T + bias) (+ R): A [rows, K], Wt [N, K] (nn.Linear layout), bias
// [N] or null, R / Y [rows, N].  Workgroup tile 128 x BN (gemm_core.hpp); lane l
// of wave w holds column (l % 16) of rows 32w + 16i + 4(l/16) + r.
template <typename T, int BN, bool GELU, bool RES>
__global__ __launch_bounds__(kThreads) void dense_kernel(const T* __restrict__ A,
                                                         const T* __restrict__ Wt,
                                                         const T* __restrict__ bias,
                                                         const T* __restrict__ R,
                                                         T* __restrict__ Y, int rows, int N, int K) {
  __shared__ GemmSmem<T, BN> sm;
  const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * BN;
  f32x4 acc[2][BN / 16];
  gemm_tile<T, BN, false>(A, Geom{}, rows, m0, Wt, n0, K, sm, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < BN / 16; ++j) {
    const int col = n0 + j * 16 + (lane & 15);
    const float bj = bias ? (float)bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wave * 32 + i * 16 + (lane >> 4) * 4 + r;
        if (row >= rows) continue;
        float v = acc[i][j][r] + bj;
        // GELU(v) = v * Phi(v) = v (1 + erf(v / sqrt 2)) / 2.
        if constexpr (GELU) v = 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
        const int64_t o = (int64_t)row * N + col;
        if constexpr (RES) v += (float)R[o];
        Y[o] = (T)v;
      }
  }
}

template <typename T>
hipError_t launch_ln(const T* a, const T* b, T* u, const T* g, const T* be, const T* r, T* out,
                     int rows, int C, float eps, hipStream_t st) {
  if constexpr (sizeof(T) == 4) {
    hipLaunchKernelGGL((ln_kernel<float, 64>), dim3((rows + 3) / 4), dim3(256), 0, st, a, b, u, g,
                       be, r, out, rows, C, eps);
  } else {
    // Lanes per row: the next power of two of C / 8 (16-byte chunks per row).
    const int chunks = C / 8;
    auto go = [&](auto lpr) {
      constexpr int L = decltype(lpr)::value;
      const int per_wg = 4 * (64 / L);
      hipLaunchKernelGGL((ln_kernel<T, L>), dim3((rows + per_wg - 1) / per_wg), dim3(256), 0, st,
                         a, b, u, g, be, r, out, rows, C, eps);
    };
    if (chunks <= 4) go(std::integral_constant<int, 4>());
    else if (chunks <= 8) go(std::integral_constant<int, 8>());
    else if (chunks <= 16) go(std::integral_constant<int, 16>());
    else if (chunks <= 32) go(std::integral_constant<int, 32>());
    else go(std::integral_constant<int, 64>());
  }
  return hipGetLastError();
}

// The whole MLP sub-layer of a token row in one kernel, for 16-bit I/O and
// C <= 128, with the block's second LayerNorm and residual folded in:
//   V1 (pre-norm):  h = a + a2,  y = h + F(LN(h));
//   V2 (post-norm): h = a,       y = h + LN(F(h));
// F(u) = GELU(u W1^T + b1) W2^T + b2.  Each wave owns RT tiles of 16 rows.
// Their A fragments (row l % 16, channels 32 kk + 8 (l/16) .. +7) are loaded
// once (V1: h, its LayerNorm across the four lanes of a row, rounded to the
// I/O type as a stored LayerNorm output would be).  Per 32 hidden units: the
// hidden tile on the matrix cores (B = W1 rows), bias, exact GELU, rounded to
// the I/O type (the rounding an unfused MLP stores), through a per-wave LDS
// tile to become row fragments, then Y += H W2^T (B = W2 rows, contiguous in
// the hidden index).  Weights come from L2; each fragment serves the wave's
// RT row tiles.  The hidden layer never reaches HBM.
constexpr int kMlpRT = 2, kMlpLD = 40;

template <typename T>
struct MlpArgs {
  const T *a, *a2;     // h = a (+ a2)
  const T *g, *be;     // the second LayerNorm's gamma, beta
  const T *w1, *b1, *w2, *b2;
  T* y;
  int rows, hidden;
  float eps;
};

template <typename T, int C, bool V1>
__global__ __launch_bounds__(256) void mlp_fused_kernel(MlpArgs<T> p) {
  constexpr int KC = C / 32, CT = C / 16, RT = kMlpRT;
  // C = 128: the chunk's weights are staged in LDS for the 4 waves (measured
  // faster at SwinV2-B stage 1); smaller C keeps them in registers from L2
  // (more waves fit; measured faster at Swin-T stage 1).
  constexpr bool STAGE_W = C >= 128;
  __shared__ __attribute__((aligned(16))) T hs[4][RT][16 * kMlpLD];
  __shared__ __attribute__((aligned(16))) T w1s[STAGE_W ? 32 * (C + 8) : 8];
  __shared__ __attribute__((aligned(16))) T w2s[STAGE_W ? C * 40 : 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * 16 * RT;
  const int rows = p.rows, hidden = p.hidden;
  vec8<T> xa[RT][KC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t ra = r0 + 16 * rt + i16;
    const bool live = ra < rows;
    float v[KC][8];
    float sum = 0.f;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const int c0 = 32 * kk + 8 * g4;
      vec8<T> av = {}, bv = {};
      if (live) {
        av = gload8(p.a + ra * C + c0);
        if constexpr (V1) bv = gload8(p.a2 + ra * C + c0);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[kk][e] = (float)av[e] + (V1 ? (float)bv[e] : 0.f);
        sum += v[kk][e];
      }
    }
    if constexpr (V1) {
      // LayerNorm over the row's C channels, spread over lanes l, l^16, l^32, l^48.
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      const float mean = sum / (float)C;
      float q = 0.f;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) q += (v[kk][e] - mean) * (v[kk][e] - mean);
      q += __shfl_xor(q, 16);
      q += __shfl_xor(q, 32);
      const float rstd = 1.0f / sqrtf(q / (float)C + p.eps);
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const vec8<T> gv = gload8(p.g + 32 * kk + 8 * g4), be = gload8(p.be + 32 * kk + 8 * g4);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          xa[rt][kk][e] = from_f32<T>((v[kk][e] - mean) * rstd * (float)gv[e] + (float)be[e]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) xa[rt][kk][e] = from_f32<T>(v[kk][e]);
    }
  }
  f32x4 yacc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) yacc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (STAGE_W) {
  // The weights of a 32-unit hidden chunk (W1 rows hc .. +31, W2 columns hc ..
  // +31) go through LDS, shared by the 4 waves; the next chunk's 16-byte
  // pieces are loaded into registers during this chunk's products.
  constexpr int P1 = C + 8, P2 = 40;          // LDS row pitches (elements)
  constexpr int PER = (8 * C) / 256;          // 16-byte pieces per thread
  static_assert(PER * 256 == 8 * C, "chunk split");
  uint4 pre[PER];
  auto fetch_w = [&](int hc) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + 256 * i;
      if (e < 4 * C) {  // W1: 32 rows x C/8 pieces
        const int row = e / (C / 8), c8 = e - row * (C / 8);
        pre[i] = gload16(p.w1 + (int64_t)(hc + row) * C + 8 * c8);
      } else {          // W2: C rows x 4 pieces
        const int f = e - 4 * C, row = f >> 2, c8 = f & 3;
        pre[i] = gload16(p.w2 + (int64_t)row * hidden + hc + 8 * c8);
      }
    }
  };
  auto store_w = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + 256 * i;
      if (e < 4 * C) {
        const int row = e / (C / 8), c8 = e - row * (C / 8);
        *reinterpret_cast<uint4*>(&w1s[row * P1 + 8 * c8]) = pre[i];
      } else {
        const int f = e - 4 * C, row = f >> 2, c8 = f & 3;
        *reinterpret_cast<uint4*>(&w2s[row * P2 + 8 * c8]) = pre[i];
      }
    }
  };
  fetch_w(0);
  store_w();
  __syncthreads();
  for (int hc = 0; hc < hidden; hc += 32) {
    const bool more = hc + 32 < hidden;
    if (more) fetch_w(hc + 32);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int n = hc + 16 * t + i16;  // this lane's hidden unit (B column)
      vec8<T> wb[KC];
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) wb[kk] = load8(&w1s[(16 * t + i16) * P1 + 32 * kk + 8 * g4]);
      const float bn = p.b1 ? (float)p.b1[n] : 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 h = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) h = mma_16x16x32(xa[rt][kk], wb[kk], h);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = h[q] + bn;
          hs[wave][rt][(4 * g4 + q) * kMlpLD + 16 * t + i16] =
              from_f32<T>(0.5f * v * (1.0f + erff(v * 0.70710678118654752f)));
        }
      }
    }
    asm volatile("" ::: "memory");  // the wave's tile writes before its reads
    vec8<T> wb2[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) wb2[ct] = load8(&w2s[(16 * ct + i16) * P2 + 8 * g4]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const vec8<T> ha = load8(&hs[wave][rt][i16 * kMlpLD + 8 * g4]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) yacc[rt][ct] = mma_16x16x32(ha, wb2[ct], yacc[rt][ct]);
    }
    __syncthreads();  // every wave done with this chunk's weights (and its tile)
    if (more) {
      store_w();
      __syncthreads();
    }
  }
  } else {
  for (int hc = 0; hc < hidden; hc += 32) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int n = hc + 16 * t + i16;  // this lane's hidden unit (B column)
      vec8<T> wb[KC];
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) wb[kk] = gload8(p.w1 + (int64_t)n * C + 32 * kk + 8 * g4);
      const float bn = p.b1 ? (float)p.b1[n] : 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 h = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) h = mma_16x16x32(xa[rt][kk], wb[kk], h);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = h[q] + bn;
          hs[wave][rt][(4 * g4 + q) * kMlpLD + 16 * t + i16] =
              from_f32<T>(0.5f * v * (1.0f + erff(v * 0.70710678118654752f)));
        }
      }
    }
    asm volatile("" ::: "memory");  // the wave's tile writes before its reads
    vec8<T> wb2[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      wb2[ct] = gload8(p.w2 + (int64_t)(16 * ct + i16) * hidden + hc + 8 * g4);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const vec8<T> ha = load8(&hs[wave][rt][i16 * kMlpLD + 8 * g4]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) yacc[rt][ct] = mma_16x16x32(ha, wb2[ct], yacc[rt][ct]);
    }
    asm volatile("" ::: "memory");  // reads done before the next chunk's writes
  }
  }
  // Lane: channel 16 ct + i16 of rows 4 g4 + q of each row tile.
  float bc[CT], gc[CT], bec[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int c = 16 * ct + i16;
    bc[ct] = p.b2 ? (float)p.b2[c] : 0.f;
    gc[ct] = V1 ? 0.f : (float)p.g[c];
    bec[ct] = V1 ? 0.f : (float)p.be[c];
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = r0 + 16 * rt + 4 * g4 + q;
      float f[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) f[ct] = yacc[rt][ct][q] + bc[ct];
      if constexpr (!V1) {
        // LayerNorm of F over the row's C channels: CT per lane, 16 lanes.
        float sum = 0.f;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) sum += f[ct];
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) sum += __shfl_xor(sum, d);
        const float mean = sum / (float)C;
        float var = 0.f;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) var += (f[ct] - mean) * (f[ct] - mean);
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) var += __shfl_xor(var, d);
        const float rstd = 1.0f / sqrtf(var / (float)C + p.eps);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) f[ct] = (f[ct] - mean) * rstd * gc[ct] + bec[ct];
      }
      if (row >= rows) continue;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = 16 * ct + i16;
        float h = (float)p.a[row * C + c];
        if constexpr (V1) h += (float)p.a2[row * C + c];
        p.y[row * C + c] = from_f32<T>(h + f[ct]);
      }
    }
}

template <typename T>
hipError_t launch_mlp_fused(const MlpArgs<T>& a, int C, bool v1, hipStream_t st) {
  if constexpr (__is_same(T, float)) {
    return hipErrorInvalidValue;  // 16-bit operands only
  } else {
    const int per_wg = 4 * 16 * kMlpRT;
    const dim3 grid((a.rows + per_wg - 1) / per_wg), block(256);
    auto go = [&](auto cc) {
      constexpr int CC = decltype(cc)::value;
      if (v1)
        hipLaunchKernelGGL((mlp_fused_kernel<T, CC, true>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((mlp_fused_kernel<T, CC, false>), grid, block, 0, st, a);
    };
    switch (C) {
      case 32: go(std::integral_constant<int, 32>()); break;
      case 64: go(std::integral_constant<int, 64>()); break;
      case 96: go(std::integral_constant<int, 96>()); break;
      case 128: go(std::integral_constant<int, 128>()); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
}

bool mlp_fused_supported(int C, int io) {
  return io != kF32 && C % 32 == 0 && C <= 128;
}

template <typename T, bool GELU, bool RES>
hipError_t launch_dense(const T* A, const T* Wt, const T* bias, const T* R, T* Y, int rows, int N,
                        int K, hipStream_t st) {
  constexpr int io = __is_same(T, float) ? kF32 : __is_same(T, h16) ? kF16 : kBF16;
  if (dense_tiled_supported(rows, N, K, io)) {
    DenseParams d{io, rows, N, K, A, Wt, bias, RES ? R : nullptr, Y};
    return launch_dense_tiled(d, GELU, st);
  }
  const int gx = (rows + kBM - 1) / kBM;
  if (N % 128 == 0)
    hipLaunchKernelGGL((dense_kernel<T, 128, GELU, RES>), dim3(gx, N / 128), dim3(kThreads), 0,
                       st, A, Wt, bias, R, Y, rows, N, K);
  else if (N % 96 == 0)
    hipLaunchKernelGGL((dense_kernel<T, 96, GELU, RES>), dim3(gx, N / 96), dim3(kThreads), 0, st,
                       A, Wt, bias, R, Y, rows, N, K);
  else if (N % 64 == 0)
    hipLaunchKernelGGL((dense_kernel<T, 64, GELU, RES>), dim3(gx, N / 64), dim3(kThreads), 0, st,
                       A, Wt, bias, R, Y, rows, N, K);
  else
    hipLaunchKernelGGL((dense_kernel<T, 32, GELU, RES>), dim3(gx, N / 32), dim3(kThreads), 0, st,
                       A, Wt, bias, R, Y, rows, N, K);
  return hipGetLastError();
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

struct BlockLayout {
  size_t attn, a, b, h, u, total;
};

BlockLayout block_layout(const swin_block_desc* d) {
  const swin_wmsa_desc& at = d->attn;
  const size_t e = at.dtype == SWIN_F32 ? 4 : 2;
  const size_t T = (size_t)at.B * at.H * at.W;
  BlockLayout L;
  L.attn = 0;
  L.a = round256(swin_wmsa_workspace_size(&at));
  L.b = L.a + round256(T * at.C * e);
  L.h = L.b + round256(T * at.C * e);
  L.u = L.h + round256(T * at.C * e);
  L.total = L.u + round256(T * (size_t)d->hidden * e);
  return L;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }


template <typename T>
swin_status block_run(const swin_block_desc* d, const T* x, const swin_block_params* p, T* y,
                      char* ws, size_t ws_bytes, hipStream_t st) {
  const swin_wmsa_desc& at = d->attn;
  const BlockLayout L = block_layout(d);
  const int rows = at.B * at.H * at.W, C = at.C, hid = d->hidden;
  const float eps = d->ln_eps > 0.f ? d->ln_eps : 1e-5f;
  T* A = reinterpret_cast<T*>(ws + L.a);
  T* Bv = reinterpret_cast<T*>(ws + L.b);
  T* Hb = reinterpret_cast<T*>(ws + L.h);
  T* U = reinterpret_cast<T*>(ws + L.u);
  auto P = [](const void* q) { return static_cast<const T*>(q); };
  const size_t attn_ws = L.a;  // the attention's workspace is the first region
  constexpr int io = __is_same(T, float) ? kF32 : __is_same(T, h16) ? kF16 : kBF16;
  const bool fused_mlp = mlp_fused_supported(C, io);
  swin_status s;
  hipError_t e;
  if (at.mode == SWIN_V1) {
    e = launch_ln<T>(x, nullptr, nullptr, P(p->ln1_g), P(p->ln1_b), nullptr, A, rows, C, eps, st);
    if (e != hipSuccess) return hip_status(e);
    s = swin_wmsa_fwd(&at, A, p->w_qkv, p->b_qkv, p->w_proj, p->b_proj, p->bias_table, p->tau, Bv,
                      attn_ws ? ws : nullptr, attn_ws, st);
    if (s != SWIN_OK) return s;
    if (fused_mlp) {
      const MlpArgs<T> m{x, Bv, P(p->ln2_g), P(p->ln2_b), P(p->fc1_w), P(p->fc1_b),
                         P(p->fc2_w), P(p->fc2_b), y, rows, hid, eps};
      return hip_status(launch_mlp_fused<T>(m, C, true, st));
    }
    e = launch_ln<T>(x, Bv, Hb, P(p->ln2_g), P(p->ln2_b), nullptr, A, rows, C, eps, st);
    if (e == hipSuccess)
      e = launch_dense<T, true, false>(A, P(p->fc1_w), P(p->fc1_b), nullptr, U, rows, hid, C, st);
    if (e == hipSuccess)
      e = launch_dense<T, false, true>(U, P(p->fc2_w), P(p->fc2_b), Hb, y, rows, C, hid, st);
    return hip_status(e);
  }
  s = swin_wmsa_fwd(&at, x, p->w_qkv, p->b_qkv, p->w_proj, p->b_proj, p->bias_table, p->tau, Bv,
                    attn_ws ? ws : nullptr, attn_ws, st);
  if (s != SWIN_OK) return s;
  e = launch_ln<T>(Bv, nullptr, nullptr, P(p->ln1_g), P(p->ln1_b), x, Hb, rows, C, eps, st);
  if (e == hipSuccess && fused_mlp) {
    const MlpArgs<T> m{Hb, nullptr, P(p->ln2_g), P(p->ln2_b), P(p->fc1_w), P(p->fc1_b),
                       P(p->fc2_w), P(p->fc2_b), y, rows, hid, eps};
    return hip_status(launch_mlp_fused<T>(m, C, false, st));
  }
  if (e == hipSuccess)
    e = launch_dense<T, true, false>(Hb, P(p->fc1_w), P(p->fc1_b), nullptr, U, rows, hid, C, st);
  if (e == hipSuccess)
    e = launch_dense<T, false, false>(U, P(p->fc2_w), P(p->fc2_b), nullptr, A, rows, C, hid, st);
  if (e == hipSuccess)
    e = launch_ln<T>(A, nullptr, nullptr, P(p->ln2_g), P(p->ln2_b), Hb, y, rows, C, eps, st);
  (void)ws_bytes;
  return hip_status(e);
}

}  // namespace

}  // namespace swin

extern "C" {

size_t swin_block_workspace_size(const swin_block_desc* d) {
  if (!d || swin_wmsa_kernel_count(&d->attn) == 0) return 0;
  if (d->hidden < 32 || d->hidden % 32) return 0;
  return swin::block_layout(d).total;
}

swin_status swin_block_fwd(const swin_block_desc* d, const void* x, const swin_block_params* p,
                           void* y, void* workspace, size_t ws_bytes, void* stream) {
  using namespace swin;
  if (!d || !p) return SWIN_ERR_NULL;
  const swin_wmsa_desc& at = d->attn;
  if (at.B < 0) return SWIN_ERR_SHAPE;
  if (at.B == 0) return SWIN_OK;
  if (swin_wmsa_kernel_count(&at) == 0) return SWIN_ERR_SHAPE;  // invalid attention desc
  if (d->hidden < 32 || d->hidden % 32 || d->hidden > 16384) return SWIN_ERR_SHAPE;
  if (at.C > kLnMaxC) return SWIN_ERR_UNSUPPORTED;
  if (!x || !y || !workspace || !p->w_qkv || !p->w_proj || !p->bias_table || !p->ln1_g ||
      !p->ln1_b || !p->ln2_g || !p->ln2_b || !p->fc1_w || !p->fc2_w)
    return SWIN_ERR_NULL;
  if (at.mode == SWIN_V2 && !p->tau) return SWIN_ERR_NULL;
  const BlockLayout L = block_layout(d);
  if (ws_bytes < L.total) return SWIN_ERR_WORKSPACE;
  const size_t e = at.dtype == SWIN_F32 ? 4 : 2;
  const size_t act = (size_t)at.B * at.H * at.W * at.C * e;
  const size_t C = at.C, hid = d->hidden;
  const size_t R2 = (size_t)(2 * at.M - 1) * (2 * at.M - 1);
  // Neither the output nor the workspace may overlap any input, or each other.
  struct Span { const void* q; size_t n; };
  const Span ins[] = {{x, act}, {p->w_qkv, 3 * C * C * e}, {p->b_qkv, 3 * C * e},
                      {p->w_proj, C * C * e}, {p->b_proj, C * e},
                      {p->bias_table, R2 * at.heads * 4},
                      {at.mode == SWIN_V2 ? p->tau : nullptr, at.heads * 4u},
                      {p->ln1_g, C * e}, {p->ln1_b, C * e}, {p->ln2_g, C * e}, {p->ln2_b, C * e},
                      {p->fc1_w, hid * C * e}, {p->fc1_b, hid * e}, {p->fc2_w, hid * C * e},
                      {p->fc2_b, C * e}};
  for (const Span& in : ins)
    if (overlaps(y, act, in.q, in.n) || overlaps(workspace, L.total, in.q, in.n))
      return SWIN_ERR_ALIAS;
  if (overlaps(y, act, workspace, L.total)) return SWIN_ERR_ALIAS;
  if (!al16(x) || !al16(y) || !al16(workspace) || !al16(p->fc1_w) || !al16(p->fc2_w) ||
      !al16(p->w_qkv) || !al16(p->w_proj) || !al16(p->ln1_g) || !al16(p->ln1_b) ||
      !al16(p->ln2_g) || !al16(p->ln2_b))
    return SWIN_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  switch (at.dtype) {
    case SWIN_F32:
      return block_run<float>(d, static_cast<const float*>(x), p, static_cast<float*>(y), ws,
                              ws_bytes, st);
    case SWIN_F16:
      return block_run<h16>(d, static_cast<const h16*>(x), p, static_cast<h16*>(y), ws, ws_bytes,
                            st);
    case SWIN_BF16:
      return block_run<b16>(d, static_cast<const b16*>(x), p, static_cast<b16*>(y), ws, ws_bytes,
                            st);
    default:
      return SWIN_ERR_DTYPE;
  }
}

}  // extern "C"
