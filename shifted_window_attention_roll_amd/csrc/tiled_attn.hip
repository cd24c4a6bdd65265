// Attention for windows whose side M is a multiple of 8 (SwinV2 windows of 8,
// 16, 24), 16-bit I/O, one workgroup per (window, head), between the QKV and
// projection GEMMs: q, k, v per (window, head) as [N][32] (q scaled so that
// the logits are in base 2) in, O as [window slot][C] out.  The core (bias,
// mask, lazy-max softmax, both products) is attn_tiles in attn_core.hpp.
#include "attn_core.hpp"
#include "launch.hpp"

namespace swin {

namespace {

template <typename QT, typename VT, int M, int QTL, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void tiled_attn_kernel(FwdParams p) {
  constexpr int D = 32;
  constexpr int N = M * M;
  constexpr int LDK = kAttnLD;
  static_assert(M % 8 == 0 && N / 16 == QTL * WAVES, "tile split");
  constexpr int TS = table_stride<M>();
  __shared__ __attribute__((aligned(16))) QT ks[N * LDK];
  __shared__ __attribute__((aligned(16))) VT vs[N * LDK];
  __shared__ __attribute__((aligned(16))) float rt4[4 * TS];
  __shared__ __attribute__((aligned(16))) float ninf[8];

  const Geom& g = p.g;
  const int item = blockIdx.x;  // window * heads + head
  const int w = item / g.heads, h = item - w * g.heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NT = 64 * WAVES;

  const QT* kg = static_cast<const QT*>(p.buf.k) + (int64_t)item * N * D;
  const VT* vg = static_cast<const VT*>(p.buf.v) + (int64_t)item * N * D;
  for (int i = tid; i < N * D / 8; i += NT) {
    const int r = i >> 2, c = i & 3;
    *reinterpret_cast<uint4*>(&ks[r * LDK + c * 8]) = gload16(kg + i * 8);
    *reinterpret_cast<uint4*>(&vs[r * LDK + c * 8]) = gload16(vg + i * 8);
  }
  fill_bias_copies<M>(rt4, p.table, g.heads, h, tid, NT);
  if (tid < 8) ninf[tid] = -__builtin_inff();

  const QT* qg = static_cast<const QT*>(p.buf.q) + (int64_t)item * N * D;
  const int g4 = lane >> 4, i16 = lane & 15;
  vec8<QT> qf[QTL];
  int tile[QTL];
#pragma unroll
  for (int j = 0; j < QTL; ++j) {
    tile[j] = wave * QTL + j;
    qf[j] = gload8(qg + (tile[j] * 16 + i16) * D + g4 * 8);
  }
  __syncthreads();

  const int wl = w % g.nW;
  const int wy = wl / g.nWx, wx = wl - (wl / g.nWx) * g.nWx;
  const bool my = g.s > 0 && wy == g.H / M - 1;
  const bool mx = g.s > 0 && wx == g.nWx - 1;
  float o[QTL][8];
  if (my || mx)
    attn_tiles<QT, VT, M, QTL, true>(qf, tile, ks, vs, rt4, ninf, lane, M - g.s, my, mx, o);
  else
    attn_tiles<QT, VT, M, QTL, false>(qf, tile, ks, vs, rt4, ninf, lane, M - g.s, false, false, o);

  // O rows in slot order, columns h*32 + d: the lane's 8 dims, one store.
  VT* og = static_cast<VT*>(p.buf.o);
#pragma unroll
  for (int j = 0; j < QTL; ++j) {
    vec8<VT> v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = from_f32<VT>(o[j][e]);
    gstore16(og + ((int64_t)w * N + tile[j] * 16 + i16) * g.C + h * D + 8 * g4,
             __builtin_bit_cast(uint4, v));
  }
}

template <typename QT, typename VT>
hipError_t tiled_dispatch(const FwdParams& p, hipStream_t st) {
  const dim3 grid(p.g.B * p.g.nW * p.g.heads);
  switch (p.g.M) {
    case 8: hipLaunchKernelGGL((tiled_attn_kernel<QT, VT, 8, 1, 4>), grid, dim3(256), 0, st, p); break;
    case 16: hipLaunchKernelGGL((tiled_attn_kernel<QT, VT, 16, 2, 8>), grid, dim3(512), 0, st, p); break;
    case 24: hipLaunchKernelGGL((tiled_attn_kernel<QT, VT, 24, 3, 12>), grid, dim3(768), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool tiled_attn_supported(int M, int io) { return io != kF32 && (M == 8 || M == 16 || M == 24); }

hipError_t launch_tiled_attn(const FwdParams& p, hipStream_t st) {
  if (!tiled_attn_supported(p.g.M, p.io) || !p.g.chunked) return hipErrorInvalidValue;
  if (p.io == kF16) return tiled_dispatch<h16, h16>(p, st);
  if (p.qk == kF16) return tiled_dispatch<h16, b16>(p, st);
  return tiled_dispatch<b16, b16>(p, st);
}

}  // namespace swin
