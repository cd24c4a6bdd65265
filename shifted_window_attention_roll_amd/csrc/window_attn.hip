// Per-window attention core: logits with relative position bias and the
// shifted-window region mask, softmax, and the AV product, for one (window, head)
// per workgroup.
//
// Pages: "Boosting Swin Transformer Speed", Training Optimization (fused MHA:
// the softmax is fused with the products) and Inference Optimization (invariant
// data pre-processed once: the bias table is precomputed, the mask is pure index
// arithmetic); "Swin Transformer V2" summary, How It Works (logit = similarity +
// relative position bias B_ij; V2 similarity = cosine / tau, folded into q by
// the QKV projection).
//
// Layout in registers.  A wave owns 16 queries.  It computes S^T = K Q^T on the
// matrix cores so that lane l ends up with query (l % 16) and 8 consecutive keys
// 8*(l/16) .. +7 of each 32-key block: the K rows fed to the two 16-key MFMAs
// are permuted so that the output rows land on those keys.  That register
// layout is exactly the B operand of O^T = V^T P^T, so the probabilities never
// leave registers, and the softmax row state (max, sum) lives in the lane that
// owns the query.  The bias (pre-scaled by log2 e, with -inf for masked and
// padded keys) is the accumulator's initial value, so adding it costs nothing.
#include "common.hpp"
#include "launch.hpp"

namespace swin {

template <typename QT, typename VT, int MMAX>
__global__ __launch_bounds__(256) void window_attn_kernel(FwdParams p) {
  constexpr int D = 32;
  constexpr int NPMAX = ((MMAX * MMAX + 31) / 32) * 32;
  constexpr int LDK = D + 16 / (int)sizeof(QT);
  constexpr int LDV = NPMAX + 16 / (int)sizeof(VT);
  constexpr int TABMAX = (2 * MMAX - 1) * (2 * MMAX - 1);
  __shared__ QT ks[NPMAX * LDK];
  __shared__ VT vt[D * LDV];
  __shared__ float tab[TABMAX];

  const Geom g = p.g;
  const int N = g.N, M = g.M;
  const int NP = (N + 31) & ~31;
  const int wh = blockIdx.x;  // window * heads + head
  const int w = wh / g.heads;
  const int h = wh - w * g.heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = (int64_t)wh * N * D;
  const QT* qg = static_cast<const QT*>(p.buf.q) + base;
  const QT* kg = static_cast<const QT*>(p.buf.k) + base;
  const VT* vg = static_cast<const VT*>(p.buf.v) + base;

  // Stage K (row-major, zero rows past N) and V^T into LDS.
  constexpr int KE = 16 / (int)sizeof(QT);
  constexpr int KCPR = D / KE;
  for (int i = tid; i < NP * KCPR; i += 256) {
    int r = i / KCPR, c = i - (i / KCPR) * KCPR;
    uint4 v = r < N ? *reinterpret_cast<const uint4*>(kg + r * D + c * KE) : uint4{0, 0, 0, 0};
    *reinterpret_cast<uint4*>(&ks[r * LDK + c * KE]) = v;
  }
  constexpr int VE = 16 / (int)sizeof(VT);
  constexpr int VCPR = D / VE;
  for (int i = tid; i < NP * VCPR; i += 256) {
    int r = i / VCPR, c = i - (i / VCPR) * VCPR;
    uint4 u = r < N ? *reinterpret_cast<const uint4*>(vg + r * D + c * VE) : uint4{0, 0, 0, 0};
    struct E { VT e[VE]; };
    E ev = __builtin_bit_cast(E, u);
#pragma unroll
    for (int e = 0; e < VE; ++e) vt[(c * VE + e) * LDV + r] = ev.e[e];
  }
  const int nrel = (2 * M - 1) * (2 * M - 1);
  for (int i = tid; i < nrel; i += 256) tab[i] = p.table[(int64_t)i * g.heads + h] * kLog2e;
  __syncthreads();

  const int wl = w % g.nW;
  const int wy = wl / g.nWx, wx = wl - (wl / g.nWx) * g.nWx;
  // Only the last window row / column mixes slices of the shifted frame.
  const bool masked = g.s > 0 && (wy == g.H / M - 1 || wx == g.nWx - 1);
  const float NEG_INF = -__builtin_inff();
  const int g4 = lane >> 4;
  const int i16 = lane & 15;

  for (int qt = wave; qt < NP / 16; qt += 4) {
    const int qi = qt * 16 + i16;
    const int qic = qi < N ? qi : N - 1;
    const vec8<QT> qf = load8(qg + qic * D + g4 * 8);
    const int tyq = qic / M, txq = qic - (qic / M) * M;
    const int regq = masked ? 3 * axis_slice(wy * M + tyq, g.H, M, g.s) +
                                  axis_slice(wx * M + txq, g.W, M, g.s)
                            : 0;
    float m = NEG_INF, lsum = 0.0f;
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < NP; kb += 32) {
      f32x4 s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb + 8 * g4 + 4 * t + r;
          float b = NEG_INF;
          if (key < N) {
            const int tyk = key / M, txk = key - (key / M) * M;
            b = tab[(tyq - tyk + M - 1) * (2 * M - 1) + (txq - txk + M - 1)];
            if (masked) {
              int regk = 3 * axis_slice(wy * M + tyk, g.H, M, g.s) +
                         axis_slice(wx * M + txk, g.W, M, g.s);
              if (regk != regq) b = NEG_INF;
            }
          }
          s[t][r] = b;
        }
      // K rows for output rows 4*g'+r' of 16-key MFMA t: key 8*g' + 4*t + r'.
      const int krow = kb + 8 * (i16 >> 2) + (i16 & 3);
      const vec8<QT> kf0 = load8(&ks[krow * LDK + g4 * 8]);
      const vec8<QT> kf1 = load8(&ks[(krow + 4) * LDK + g4 * 8]);
      s[0] = mma_16x16x32(kf0, qf, s[0]);
      s[1] = mma_16x16x32(kf1, qf, s[1]);

      float mloc = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float mnew = fmaxf(m, mloc);
      const float mref = mnew == NEG_INF ? 0.0f : mnew;
      const float alpha = fast_exp2(m - mref);
      vec8<VT> pf;
      float psum = 0.0f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float e = fast_exp2(s[t][r] - mref);
          psum += e;
          pf[4 * t + r] = from_f32<VT>(e);
        }
      lsum = lsum * alpha + psum;
      o0 *= alpha;
      o1 *= alpha;
      const vec8<VT> vf0 = load8(&vt[i16 * LDV + kb + g4 * 8]);
      const vec8<VT> vf1 = load8(&vt[(16 + i16) * LDV + kb + g4 * 8]);
      o0 = mma_16x16x32(vf0, pf, o0);
      o1 = mma_16x16x32(vf1, pf, o1);
      m = mnew;
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const float inv = 1.0f / lsum;
    if (qi < N) {
      VT* og = static_cast<VT*>(p.buf.o) + ((int64_t)w * N + qi) * g.C + h * D + 4 * g4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        og[r] = from_f32<VT>(o0[r] * inv);
        og[16 + r] = from_f32<VT>(o1[r] * inv);
      }
    }
  }
}

template <typename QT, typename VT>
static hipError_t attn_dispatch(const FwdParams& p, hipStream_t st) {
  dim3 grid(p.g.B * p.g.nW * p.g.heads);
  if (p.g.M <= 8)
    hipLaunchKernelGGL((window_attn_kernel<QT, VT, 8>), grid, dim3(256), 0, st, p);
  else if (p.g.M <= 16)
    hipLaunchKernelGGL((window_attn_kernel<QT, VT, 16>), grid, dim3(256), 0, st, p);
  else if constexpr (sizeof(QT) == 2 && sizeof(VT) == 2)
    hipLaunchKernelGGL((window_attn_kernel<QT, VT, 24>), grid, dim3(256), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_window_attn(const FwdParams& p, hipStream_t st) {
  if (p.io == kF32) return attn_dispatch<float, float>(p, st);
  if (p.io == kF16) return attn_dispatch<h16, h16>(p, st);
  if (p.qk == kF16) return attn_dispatch<h16, b16>(p, st);
  return attn_dispatch<b16, b16>(p, st);
}

}  // namespace swin
