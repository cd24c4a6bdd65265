// 2:4 structured-sparse linear layers for the QKV and projection GEMMs on the
// gfx950 sparse matrix cores (16x16x64 products with 16-bit operands).
//
// Page: "Boost Vision Transformer with GPU-Friendly Sparsity and
// Quantization", Section 3.1 / Figure 1 (two of every four consecutive weights
// along the reduction dimension kept, stored as values plus positions, run on
// sparse matrix cores) and Section 3.2 / Figure 3 (applied to the QKV,
// projection and feed-forward GEMMs).
//
// Compressed weight of w [N, K]: values [N, K/2] (two per group of four along
// K, the lower position first) and codes [N, K/4] bytes (positions p0 | p1 << 2).
// Pruning keeps the two largest magnitudes of each group (ties: the lower
// position).
#include "launch.hpp"

namespace swin {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void prune24_kernel(const T* __restrict__ w, int64_t groups,
                                                      T* __restrict__ vals,
                                                      uint8_t* __restrict__ codes) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= groups) return;
  float a[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = fabsf((float)w[4 * g + e]);
  // First and second largest magnitude, the lower position on ties.
  int i1 = 0;
#pragma unroll
  for (int e = 1; e < 4; ++e) if (a[e] > a[i1]) i1 = e;
  int i2 = i1 == 0 ? 1 : 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) if (e != i1 && a[e] > a[i2]) i2 = e;
  const int p0 = min(i1, i2), p1 = max(i1, i2);
  vals[2 * g] = w[4 * g + p0];
  vals[2 * g + 1] = w[4 * g + p1];
  codes[g] = (uint8_t)(p0 | (p1 << 2));
}

// Y[t][n] = sum_k x[t][k] wp[n][k] + bias[n].  The sparse operand is the
// weight: each product is a 16 (output channels) x 16 (tokens) tile over 64
// values of K.  Lane l of the weight fragment: channel l % 16, the 8 kept
// values of groups 4 (l/16) .. +3 of the 64-block and their positions (4 bits
// per group); lane l of the token fragment: token l % 16, k = 8 (l/16) .. +7
// and 32 + 8 (l/16) .. +7 of the block -- the pairing of the sparse products
// (k = 16 G + 4 q + position for weight lane group G, group q).  64 x 64 tile
// per workgroup of 4 waves, 32 x 32 per wave, fragments straight from memory.
template <typename T>
__global__ __launch_bounds__(256) void sparse24_linear_kernel(Sparse24Linear p) {
  typedef T v8 __attribute__((ext_vector_type(8)));
  typedef T v16 __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int n0 = blockIdx.x * 64 + (wave >> 1) * 32;           // output channels
  const int64_t t0 = (int64_t)blockIdx.y * 64 + (wave & 1) * 32;  // tokens
  const T* x = static_cast<const T*>(p.x);
  const T* vals = static_cast<const T*>(p.vals);
  const int K = p.K;
  int nr[2];
  int64_t tr[2];
  bool nok[2], tok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    nr[i] = n0 + 16 * i + i16;
    tr[i] = t0 + 16 * i + i16;
    nok[i] = nr[i] < p.N;
    tok[i] = tr[i] < p.rows;
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < K; kb += 64) {
    v8 wv[2];
    int wi[2];
    v16 xf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (nok[i]) {
        const int64_t vo = (int64_t)nr[i] * (K / 2) + kb / 2 + 8 * g4;
        wv[i] = *reinterpret_cast<const v8*>(vals + vo);
        const uint32_t c4 =
            *reinterpret_cast<const uint32_t*>(p.codes + (int64_t)nr[i] * (K / 4) + kb / 4 + 4 * g4);
        wi[i] = (int)((c4 & 0xFu) | ((c4 >> 4) & 0xF0u) | ((c4 >> 8) & 0xF00u) |
                      ((c4 >> 12) & 0xF000u));
      } else {
        wv[i] = v8{};
        wi[i] = 0x4444;  // positions (0, 1) in every group; the values are zero
      }
      if (tok[i]) {
        const T* xr = x + tr[i] * K + kb + 8 * g4;
        const v8 lo = *reinterpret_cast<const v8*>(xr);
        const v8 hi = *reinterpret_cast<const v8*>(xr + 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xf[i][e] = lo[e];
          xf[i][8 + e] = hi[e];
        }
      } else {
        xf[i] = v16{};
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (__is_same(T, h16))
          acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(wv[i], xf[j], acc[i][j], wi[i], 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(wv[i], xf[j], acc[i][j], wi[i], 0, 0);
      }
  }
  // Lane l holds token l % 16 (column) of channels 4 (l/16) .. +3 (rows).
  T* y = static_cast<T*>(p.y);
  const T* bias = static_cast<const T*>(p.bias);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t t = tr[j];
      if (t >= p.rows) continue;
      const int nb = n0 + 16 * i + 4 * g4;
      T v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        v[r] = from_f32<T>(acc[i][j][r] + ((bias && nb + r < p.N) ? (float)bias[nb + r] : 0.f));
      T* dst = y + t * p.N + nb;
      if (nb + 4 <= p.N && (reinterpret_cast<uintptr_t>(dst) & 7) == 0) {
        *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, v);  // 4 channels at once
      } else {
        for (int r = 0; r < 4 && nb + r < p.N; ++r) dst[r] = v[r];
      }
    }
}

// The same product with 128 x 128 tiles (channels x tokens) of 4 waves (64 x
// 64 each, 16 accumulator tiles), K in steps of 64 staged through LDS from
// registers loaded a step ahead: per step the tile's kept values (64 bytes a
// channel), positions (16 bytes a channel) and token rows (128 bytes a
// token).  Needs K % 64 == 0 and N % 4 == 0.
constexpr int kSpT = 128, kSpVP = 80, kSpXP = 144;

template <typename T>
__global__ __launch_bounds__(256) void sparse24_tiled_kernel(Sparse24Linear p) {
  typedef T v8 __attribute__((ext_vector_type(8)));
  typedef T v16 __attribute__((ext_vector_type(16)));
  __shared__ __attribute__((aligned(16))) uint8_t vl[kSpT * kSpVP];
  __shared__ __attribute__((aligned(16))) uint8_t cl[kSpT * 16];
  __shared__ __attribute__((aligned(16))) uint8_t xl[kSpT * kSpXP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int wn = (wave >> 1) * 64, wt = (wave & 1) * 64;
  const int n0 = blockIdx.x * kSpT;
  const int64_t t0 = (int64_t)blockIdx.y * kSpT;
  const int K = p.K;
  const uint8_t* vals = static_cast<const uint8_t*>(p.vals);
  const uint8_t* xs = static_cast<const uint8_t*>(p.x);
  uint4 rv[2], rx[4], rc = {0u, 0u, 0u, 0u};
  auto fetch = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // values: 128 channels x 4 chunks
      const int c = tid + 256 * i, row = c >> 2, cc = c & 3;
      const int n = n0 + row;
      rv[i] = n < p.N ? *reinterpret_cast<const uint4*>(vals + ((int64_t)n * (K / 2) + kb / 2) * 2 + 16 * cc)
                      : uint4{0u, 0u, 0u, 0u};
    }
    if (tid < kSpT) {  // positions: 16 bytes a channel
      const int n = n0 + tid;
      rc = n < p.N ? *reinterpret_cast<const uint4*>(p.codes + (int64_t)n * (K / 4) + kb / 4)
                   : uint4{0x44444444u, 0x44444444u, 0x44444444u, 0x44444444u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // tokens: 128 rows x 8 chunks
      const int c = tid + 256 * i, row = c >> 3, cc = c & 7;
      const int64_t t = t0 + row;
      rx[i] = t < p.rows ? *reinterpret_cast<const uint4*>(xs + (t * K + kb) * 2 + 16 * cc)
                         : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 2, cc = c & 3;
      *reinterpret_cast<uint4*>(&vl[row * kSpVP + 16 * cc]) = rv[i];
    }
    if (tid < kSpT) *reinterpret_cast<uint4*>(&cl[tid * 16]) = rc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, cc = c & 7;
      *reinterpret_cast<uint4*>(&xl[row * kSpXP + 16 * cc]) = rx[i];
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  stage();
  __syncthreads();
  for (int kb = 0; kb < K; kb += 64) {
    const bool more = kb + 64 < K;
    if (more) fetch(kb + 64);
    v8 wv[4];
    int wi[4];
    v16 xf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int ch = wn + 16 * t + i16;
      wv[t] = *reinterpret_cast<const v8*>(&vl[ch * kSpVP + 16 * g4]);
      const uint32_t c4 = *reinterpret_cast<const uint32_t*>(&cl[ch * 16 + 4 * g4]);
      wi[t] = (int)((c4 & 0xFu) | ((c4 >> 4) & 0xF0u) | ((c4 >> 8) & 0xF00u) |
                    ((c4 >> 12) & 0xF000u));
      const int tk = wt + 16 * t + i16;
      const v8 lo = *reinterpret_cast<const v8*>(&xl[tk * kSpXP + 16 * g4]);
      const v8 hi = *reinterpret_cast<const v8*>(&xl[tk * kSpXP + 64 + 16 * g4]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xf[t][e] = lo[e];
        xf[t][8 + e] = hi[e];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (__is_same(T, h16))
          acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(wv[i], xf[j], acc[i][j], wi[i], 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(wv[i], xf[j], acc[i][j], wi[i], 0, 0);
      }
    __syncthreads();  // every wave done reading this step
    if (more) {
      stage();
      __syncthreads();
    }
  }
  T* y = static_cast<T*>(p.y);
  const T* bias = static_cast<const T*>(p.bias);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nb = n0 + wn + 16 * i + 4 * g4;
    if (nb >= p.N) continue;
    float bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) bv[r] = bias ? (float)bias[nb + r] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + wt + 16 * j + i16;
      if (t >= p.rows) continue;
      T v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = from_f32<T>(acc[i][j][r] + bv[r]);
      *reinterpret_cast<uint2*>(y + t * p.N + nb) = __builtin_bit_cast(uint2, v);
    }
  }
}

}  // namespace

hipError_t launch_prune24(const void* w, int io, int N, int K, void* vals, uint8_t* codes,
                          hipStream_t st) {
  const int64_t groups = (int64_t)N * K / 4;
  if (groups <= 0) return hipSuccess;
  const dim3 grid((unsigned)((groups + 255) / 256)), block(256);
  if (io == kF16)
    hipLaunchKernelGGL(prune24_kernel<h16>, grid, block, 0, st, static_cast<const h16*>(w), groups,
                       static_cast<h16*>(vals), codes);
  else if (io == kBF16)
    hipLaunchKernelGGL(prune24_kernel<b16>, grid, block, 0, st, static_cast<const b16*>(w), groups,
                       static_cast<b16*>(vals), codes);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_sparse24_linear(const Sparse24Linear& p, int io, hipStream_t st) {
  if (p.rows <= 0) return hipSuccess;
  if (p.K % 64) return hipErrorInvalidValue;
  if (sparse24_tiled2_supported(p, io)) return launch_sparse24_tiled2(p, io, st);
  if (p.N % 4 == 0 && (reinterpret_cast<uintptr_t>(p.y) & 7) == 0 &&
      (reinterpret_cast<uintptr_t>(p.codes) & 15) == 0 && (p.K / 4) % 16 == 0) {
    const dim3 grid((p.N + kSpT - 1) / kSpT, (unsigned)((p.rows + kSpT - 1) / kSpT)), block(256);
    if (io == kF16)
      hipLaunchKernelGGL(sparse24_tiled_kernel<h16>, grid, block, 0, st, p);
    else if (io == kBF16)
      hipLaunchKernelGGL(sparse24_tiled_kernel<b16>, grid, block, 0, st, p);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const dim3 grid((p.N + 63) / 64, (unsigned)((p.rows + 63) / 64)), block(256);
  if (io == kF16)
    hipLaunchKernelGGL(sparse24_linear_kernel<h16>, grid, block, 0, st, p);
  else if (io == kBF16)
    hipLaunchKernelGGL(sparse24_linear_kernel<b16>, grid, block, 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace swin
