// Cyclic shift + window partition and its inverse as standalone copy kernels
// ("Boosting Swin Transformer Speed: Profiling, Mixed Precision, and Kernel Fusion
// Secrets", Training Optimization: partition / shift / reverse are index maps).
// They move bits only, so the result is an exact permutation for any element
// type.  The attention forward never calls them: it folds the same map into the
// projection GEMMs' row addressing.
#include "common.hpp"
#include "launch.hpp"

namespace swin {

// One thread per CH-byte chunk of a token row, grid-stride over all chunks.
// dst row r (window order) <- src row src_token(r) (partition) or the reverse.
template <int CH, bool REVERSE>
__global__ __launch_bounds__(256) void index_map_kernel(const uint8_t* __restrict__ in,
                                                        uint8_t* __restrict__ out, Geom g,
                                                        int chunks_per_row, int64_t total) {
  using V = typename std::conditional<CH == 16, uint4,
            typename std::conditional<CH == 8, uint2,
            typename std::conditional<CH == 4, uint32_t, uint16_t>::type>::type>::type;
  const int64_t row_bytes = (int64_t)chunks_per_row * CH;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int r = (int)(i / chunks_per_row);
    int c = (int)(i - (int64_t)r * chunks_per_row);
    int64_t src = src_token(g, r);
    int64_t win_off = (int64_t)r * row_bytes + (int64_t)c * CH;
    int64_t img_off = src * row_bytes + (int64_t)c * CH;
    if (!REVERSE)
      *reinterpret_cast<V*>(out + win_off) = *reinterpret_cast<const V*>(in + img_off);
    else
      *reinterpret_cast<V*>(out + img_off) = *reinterpret_cast<const V*>(in + win_off);
  }
}

template <bool REVERSE>
static hipError_t launch_index_map(const void* in, void* out, const Geom& g, int elem_bytes,
                                   hipStream_t st) {
  int64_t row_bytes = (int64_t)g.C * elem_bytes;
  int64_t rows = (int64_t)g.B * g.H * g.W;
  int ch = (row_bytes % 16 == 0) ? 16 : (row_bytes % 8 == 0) ? 8 : (row_bytes % 4 == 0) ? 4 : 2;
  int cpr = (int)(row_bytes / ch);
  int64_t total = rows * cpr;
  int64_t blocks64 = (total + 255) / 256;
  int blocks = (int)(blocks64 < 65536 ? blocks64 : 65536);
  auto i8 = static_cast<const uint8_t*>(in);
  auto o8 = static_cast<uint8_t*>(out);
  switch (ch) {
    case 16: hipLaunchKernelGGL((index_map_kernel<16, REVERSE>), dim3(blocks), dim3(256), 0, st, i8, o8, g, cpr, total); break;
    case 8: hipLaunchKernelGGL((index_map_kernel<8, REVERSE>), dim3(blocks), dim3(256), 0, st, i8, o8, g, cpr, total); break;
    case 4: hipLaunchKernelGGL((index_map_kernel<4, REVERSE>), dim3(blocks), dim3(256), 0, st, i8, o8, g, cpr, total); break;
    default: hipLaunchKernelGGL((index_map_kernel<2, REVERSE>), dim3(blocks), dim3(256), 0, st, i8, o8, g, cpr, total); break;
  }
  return hipGetLastError();
}

hipError_t launch_partition_shift(const void* x, void* xw, const Geom& g, int elem_bytes,
                                  hipStream_t st) {
  return launch_index_map<false>(x, xw, g, elem_bytes, st);
}

hipError_t launch_reverse_unshift(const void* xw, void* x, const Geom& g, int elem_bytes,
                                  hipStream_t st) {
  return launch_index_map<true>(xw, x, g, elem_bytes, st);
}

// ---------------------------------------------------------------------------
// V2 continuous position bias table ("Swin Transformer V2" summary, How It
// Works: a meta-network on log-spaced relative coordinates outputs the bias).
// One block per relative offset row; the hidden layer goes through LDS and each
// wave reduces whole heads.
// ---------------------------------------------------------------------------
// Log-spaced meta-network input of table row `row`: u = coord_scale * (dy,
// dx), g(u) = sign(u) log2(1 + |u|) / log2(8) per component.
__device__ __forceinline__ void cpb_coords(int row, int M, float coord_scale, float& gy,
                                           float& gx) {
  const int n = 2 * M - 1;
  const float dy = (float)(row / n - (M - 1)) * coord_scale;
  const float dx = (float)(row % n - (M - 1)) * coord_scale;
  gy = copysignf(log2f(1.0f + fabsf(dy)) * (1.0f / 3.0f), dy);
  gx = copysignf(log2f(1.0f + fabsf(dx)) * (1.0f / 3.0f), dx);
}

__global__ __launch_bounds__(256) void cpb_table_kernel(const float* __restrict__ w1,
                                                        const float* __restrict__ b1,
                                                        const float* __restrict__ w2,
                                                        const float* __restrict__ b2, int hidden,
                                                        int heads, int M, float coord_scale,
                                                        float* __restrict__ table) {
  extern __shared__ float hid[];
  const int row = blockIdx.x;
  float gy, gx;
  cpb_coords(row, M, coord_scale, gy, gx);
  for (int i = threadIdx.x; i < hidden; i += blockDim.x) {
    float h = fmaf(w1[2 * i], gy, fmaf(w1[2 * i + 1], gx, b1[i]));
    hid[i] = h > 0.0f ? h : 0.0f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int hd = wave; hd < heads; hd += blockDim.x >> 6) {
    float acc = 0.0f;
    for (int i = lane; i < hidden; i += 64) acc = fmaf(w2[(int64_t)hd * hidden + i], hid[i], acc);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
      float o = acc + (b2 ? b2[hd] : 0.0f);
      table[(int64_t)row * heads + hd] = 16.0f / (1.0f + expf(-o));
    }
  }
}

// Backward of the meta-network.  Pass 1, one workgroup per table row r:
// dO[r, h] = dtable[r, h] * 16 sigmoid'(o[r, h]) (o the pre-sigmoid output).
__global__ __launch_bounds__(256) void cpb_bwd_out_kernel(const float* __restrict__ w1,
                                                          const float* __restrict__ b1,
                                                          const float* __restrict__ w2,
                                                          const float* __restrict__ b2,
                                                          int hidden, int heads, int M,
                                                          float coord_scale,
                                                          const float* __restrict__ dtable,
                                                          float* __restrict__ dout) {
  extern __shared__ float hid[];
  const int row = blockIdx.x;
  float gy, gx;
  cpb_coords(row, M, coord_scale, gy, gx);
  for (int i = threadIdx.x; i < hidden; i += blockDim.x) {
    const float h = fmaf(w1[2 * i], gy, fmaf(w1[2 * i + 1], gx, b1[i]));
    hid[i] = h > 0.0f ? h : 0.0f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int hd = wave; hd < heads; hd += blockDim.x >> 6) {
    float acc = 0.0f;
    for (int i = lane; i < hidden; i += 64) acc = fmaf(w2[(int64_t)hd * hidden + i], hid[i], acc);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
      const float sg = 1.0f / (1.0f + expf(-(acc + (b2 ? b2[hd] : 0.0f))));
      dout[(int64_t)row * heads + hd] = dtable[(int64_t)row * heads + hd] * 16.0f * sg * (1.0f - sg);
    }
  }
}

// Pass 2, one thread per hidden unit i (rows r in LDS chunks of dO):
//   dw2[h, i] = sum_r dO[r, h] relu(pre[r, i]);
//   dpre[r, i] = (sum_h dO[r, h] w2[h, i]) [pre[r, i] > 0];
//   dw1[i, :] = sum_r dpre[r, i] g[r],  db1[i] = sum_r dpre[r, i];
// and thread h < heads also db2[h] = sum_r dO[r, h].  Every output element is
// written by one thread (no accumulation across calls).
constexpr int kCpbHeads = 64, kCpbChunk = 64;

__global__ __launch_bounds__(256) void cpb_bwd_param_kernel(const float* __restrict__ w1,
                                                            const float* __restrict__ b1,
                                                            const float* __restrict__ w2,
                                                            int hidden, int heads, int M,
                                                            float coord_scale,
                                                            const float* __restrict__ dout,
                                                            float* __restrict__ dw1,
                                                            float* __restrict__ db1,
                                                            float* __restrict__ dw2,
                                                            float* __restrict__ db2) {
  __shared__ float dsh[kCpbChunk][kCpbHeads];
  __shared__ float gsh[kCpbChunk][2];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const bool live = i < hidden;
  const int rows = (2 * M - 1) * (2 * M - 1);
  float wa = 0.f, wb = 0.f, bb = 0.f, w2c[kCpbHeads];
#pragma unroll
  for (int hd = 0; hd < kCpbHeads; ++hd) w2c[hd] = (live && hd < heads) ? w2[(int64_t)hd * hidden + i] : 0.f;
  if (live) {
    wa = w1[2 * i];
    wb = w1[2 * i + 1];
    bb = b1[i];
  }
  float a2[kCpbHeads] = {};
  float g0 = 0.f, g1 = 0.f, gb = 0.f, d2 = 0.f;
  for (int r0 = 0; r0 < rows; r0 += kCpbChunk) {
    const int nr = min(kCpbChunk, rows - r0);
    __syncthreads();
    for (int e = threadIdx.x; e < nr * kCpbHeads; e += 256) {
      const int rr = e / kCpbHeads, hd = e - rr * kCpbHeads;
      dsh[rr][hd] = hd < heads ? dout[(int64_t)(r0 + rr) * heads + hd] : 0.f;
    }
    for (int rr = threadIdx.x; rr < nr; rr += 256) cpb_coords(r0 + rr, M, coord_scale, gsh[rr][0], gsh[rr][1]);
    __syncthreads();
    for (int rr = 0; rr < nr; ++rr) {
      const float gy = gsh[rr][0], gx = gsh[rr][1];
      const float pre = fmaf(wa, gy, fmaf(wb, gx, bb));
      const float hv = pre > 0.f ? pre : 0.f;
      float dp = 0.f;
#pragma unroll
      for (int hd = 0; hd < kCpbHeads; ++hd) {
        const float d = dsh[rr][hd];
        a2[hd] = fmaf(d, hv, a2[hd]);
        dp = fmaf(d, w2c[hd], dp);
      }
      if (pre > 0.f) {
        g0 = fmaf(dp, gy, g0);
        g1 = fmaf(dp, gx, g1);
        gb += dp;
      }
      if (threadIdx.x + blockIdx.x * 256 < heads) d2 += dsh[rr][threadIdx.x];
    }
  }
  if (live) {
#pragma unroll
    for (int hd = 0; hd < kCpbHeads; ++hd)
      if (hd < heads) dw2[(int64_t)hd * hidden + i] = a2[hd];
    dw1[2 * i] = g0;
    dw1[2 * i + 1] = g1;
    db1[i] = gb;
  }
  if (db2 && blockIdx.x == 0 && threadIdx.x < heads) db2[threadIdx.x] = d2;
}

hipError_t launch_cpb_bwd(const float* w1, const float* b1, const float* w2, const float* b2,
                          int hidden, int heads, int M, float coord_scale, const float* dtable,
                          float* dw1, float* db1, float* dw2, float* db2, float* dout,
                          hipStream_t st) {
  if (heads > kCpbHeads) return hipErrorInvalidValue;
  const int rows = (2 * M - 1) * (2 * M - 1);
  hipLaunchKernelGGL(cpb_bwd_out_kernel, dim3(rows), dim3(256), hidden * sizeof(float), st, w1,
                     b1, w2, b2, hidden, heads, M, coord_scale, dtable, dout);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cpb_bwd_param_kernel, dim3((hidden + 255) / 256), dim3(256), 0, st, w1, b1,
                     w2, hidden, heads, M, coord_scale, dout, dw1, db1, dw2, db2);
  return hipGetLastError();
}

hipError_t launch_cpb_table(const float* w1, const float* b1, const float* w2, const float* b2,
                            int hidden, int heads, int M, float coord_scale, float* table,
                            hipStream_t st) {
  int rows = (2 * M - 1) * (2 * M - 1);
  hipLaunchKernelGGL(cpb_table_kernel, dim3(rows), dim3(256), hidden * sizeof(float), st, w1, b1,
                     w2, b2, hidden, heads, M, coord_scale, table);
  return hipGetLastError();
}

}  // namespace swin
