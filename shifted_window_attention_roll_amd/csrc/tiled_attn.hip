// Attention core for windows whose side M is a multiple of 8 (SwinV2 windows of
// 8, 16, 24), 16-bit I/O: logits with the relative position bias and the
// shifted-window region mask, softmax and the AV product, one workgroup per
// (window, head).
//
// Pages: "Boosting Swin Transformer Speed", Training Optimization (fused MHA:
// softmax fused with the two products) and Inference Optimization (the bias
// table is prepared once; the mask is index arithmetic); "Swin Transformer V2"
// summary, How It Works (logit = similarity + relative position bias; the V2
// similarity is the cosine over tau, folded into q by the QKV projection).
//
// Slots are chunked (see Geom): 16 consecutive slots are a 2 x 8 patch of the
// window and 32 consecutive slots a 4 x 8 patch.  Inputs per (window, head):
// q, k, v as [N][32], q already scaled so that the logits are in base 2; v is
// transposed into V^T while it is staged in LDS.
//
// Register layout.  A wave owns QTL tiles of 16 queries.  S^T = K Q^T on the
// matrix cores, with the K rows of each 32-key block permuted so that lane l
// receives query (l % 16) and the 8 keys 8*(l/16) .. +7 of the block: one
// window row, 8 consecutive columns.  The relative position index of those 8
// keys then walks one row of the table backwards, so with the rows of the
// table stored reversed in LDS the lane reads its 8 biases from 8 consecutive
// floats; they are the MFMA's initial accumulator.  P stays in registers as the
// B operand of O^T = V^T P^T, and its row sums come from one more MFMA (ones x
// P^T), i.e. from exactly the rounded P that multiplies V.
//
// Softmax.  Base 2, online, with a lazy running max: a block only rescales when
// some lane sees a logit more than 8 above the row's current reference, so the
// exponentials stay below 2^8 and the common path is max-test, subtract, exp2.
//
// Shifted windows.  Only the last window row (column) of the grid mixes two
// slices of the shifted frame, split at M - s; a pair is allowed when query and
// key are on the same side in both directions.  Blocks where no lane of a
// query tile has an allowed key are skipped; otherwise the bias of a fully
// masked key group is read from a row of -inf, and a group that straddles the
// split gets -inf per key.
#include "common.hpp"
#include "launch.hpp"

namespace swin {

namespace {

template <typename QT, typename VT, int M, int QTL, bool MASKED>
__device__ __forceinline__ void tiled_attn_body(const FwdParams& p, const QT* ks, const VT* vts,
                                                const float* rt, int item, int wave, int lane,
                                                bool my, bool mx) {
  constexpr int D = 32;
  constexpr int N = M * M;
  constexpr int R = 2 * M - 1;
  constexpr int LDK = D + 8;
  constexpr int LDV = N + 8;
  constexpr int CH = M / 8;   // column chunks
  constexpr int TPC = M / 2;  // 16-query tiles per chunk
  constexpr int BPC = M / 4;  // 32-key blocks per chunk
  const Geom& g = p.g;
  const int g4 = lane >> 4, i16 = lane & 15;
  const int bnd = M - g.s;  // slice split inside a masked window
  const float NEG_INF = -__builtin_inff();

  const QT* qg = static_cast<const QT*>(p.buf.q) + (int64_t)item * N * D;
  vec8<QT> qf[QTL];
  int qy[QTL], qx[QTL], a0[QTL];
  f32x4 o0[QTL], o1[QTL], ls[QTL];
  float m[QTL];
#pragma unroll
  for (int j = 0; j < QTL; ++j) {
    const int T = wave * QTL + j;
    const int cq = T / TPC, rp = T - cq * TPC;
    qy[j] = 2 * rp + (i16 >> 3);
    qx[j] = 8 * cq + (i16 & 7);
    qf[j] = gload8(qg + (T * 16 + i16) * D + g4 * 8);
    // Table row of (qy, key row 4b + g4) is qy - 4b - g4 + M - 1; reversed
    // column of key column 8c is 8c - qx + M - 1.  a0 is the index at b = BPC-1,
    // c = 0 (the smallest), so every block adds a non-negative constant.
    a0[j] = (qy[j] - 4 * (BPC - 1) - g4 + M - 1) * R + (M - 1 - qx[j]);
    o0[j] = o1[j] = ls[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[j] = -1e30f;
  }
  vec8<VT> ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = from_f32<VT>(1.0f);

  for (int ck = 0; ck < CH; ++ck) {
    // Allowed key columns of this chunk for the lane's query (masked windows).
    unsigned xbits[QTL];
    bool straddle = false;
    if constexpr (MASKED) {
      const int left = min(max(bnd - 8 * ck, 0), 8);
      const unsigned lm = (1u << left) - 1u;
      straddle = mx && left > 0 && left < 8;
#pragma unroll
      for (int j = 0; j < QTL; ++j)
        xbits[j] = !mx ? 0xffu : (qx[j] < bnd ? lm : (~lm & 0xffu));
    }
#pragma unroll
    for (int b = 0; b < BPC; ++b) {
      const int kb = ck * 8 * M + 32 * b;
      const int krow = kb + 8 * (i16 >> 2) + (i16 & 3);
      const vec8<QT> kf0 = load8(&ks[krow * LDK + g4 * 8]);
      const vec8<QT> kf1 = load8(&ks[(krow + 4) * LDK + g4 * 8]);
      const vec8<VT> vf0 = load8(&vts[i16 * LDV + kb + g4 * 8]);
      const vec8<VT> vf1 = load8(&vts[(16 + i16) * LDV + kb + g4 * 8]);
      const int boff = 8 * ck + 4 * R * (BPC - 1 - b);
#pragma unroll
      for (int j = 0; j < QTL; ++j) {
        const float* bp = rt + a0[j] + boff;
        unsigned bits = 0xffu;
        if constexpr (MASKED) {
          const int ky = 4 * b + g4;
          const bool yok = !my || ((ky < bnd) == (qy[j] < bnd));
          bits = yok ? xbits[j] : 0u;
          if (!__any(bits != 0u)) continue;  // whole tile masked in this block
          if (bits == 0u) bp = rt + R * R;  // a row of -inf
        }
        f32x4 s0, s1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s0[r] = bp[r];
          s1[r] = bp[4 + r];
        }
        if constexpr (MASKED) {
          if (straddle) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (!((bits >> r) & 1u)) s0[r] = NEG_INF;
              if (!((bits >> (4 + r)) & 1u)) s1[r] = NEG_INF;
            }
          }
        }
        s0 = mma_16x16x32(kf0, qf[j], s0);
        s1 = mma_16x16x32(kf1, qf[j], s1);
        const float bm = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                               fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        if (__any(bm > m[j] + 8.0f)) {
          const float rm = xor32_max(xor16_max(bm));
          const float mn = fmaxf(m[j], rm);
          const float alpha = fast_exp2(m[j] - mn);
          o0[j] *= alpha;
          o1[j] *= alpha;
          ls[j] *= alpha;
          m[j] = mn;
        }
        vec8<VT> pf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pf[r] = from_f32<VT>(fast_exp2(s0[r] - m[j]));
          pf[4 + r] = from_f32<VT>(fast_exp2(s1[r] - m[j]));
        }
        o0[j] = mma_16x16x32(vf0, pf, o0[j]);
        o1[j] = mma_16x16x32(vf1, pf, o1[j]);
        ls[j] = mma_16x16x32(ones, pf, ls[j]);
      }
    }
  }

  // O rows in slot order, columns h*32 + d; lane holds d = 4*g4 + r (+16).
  const int w = item / g.heads, h = item - w * g.heads;
  VT* og = static_cast<VT*>(p.buf.o);
#pragma unroll
  for (int j = 0; j < QTL; ++j) {
    const float inv = __builtin_amdgcn_rcpf(ls[j][0]);
    const int slot = (wave * QTL + j) * 16 + i16;
    VT* dst = og + ((int64_t)w * N + slot) * g.C + h * D + 4 * g4;
    typedef VT v4 __attribute__((ext_vector_type(4)));
    v4 a = {from_f32<VT>(o0[j][0] * inv), from_f32<VT>(o0[j][1] * inv),
            from_f32<VT>(o0[j][2] * inv), from_f32<VT>(o0[j][3] * inv)};
    v4 c = {from_f32<VT>(o1[j][0] * inv), from_f32<VT>(o1[j][1] * inv),
            from_f32<VT>(o1[j][2] * inv), from_f32<VT>(o1[j][3] * inv)};
    *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, a);
    *reinterpret_cast<uint2*>(dst + 16) = __builtin_bit_cast(uint2, c);
  }
}

template <typename QT, typename VT, int M, int QTL, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void tiled_attn_kernel(FwdParams p) {
  constexpr int D = 32;
  constexpr int N = M * M;
  constexpr int R = 2 * M - 1;
  constexpr int LDK = D + 8;
  constexpr int LDV = N + 8;
  static_assert(M % 8 == 0 && N / 16 == QTL * WAVES, "tile split");
  __shared__ __attribute__((aligned(16))) QT ks[N * LDK];
  __shared__ __attribute__((aligned(16))) VT vts[D * LDV];
  __shared__ float rt[R * R + 8];

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
  }
  // V arrives as [N][32]; it is transposed into V^T on the way into LDS.
  for (int i = tid; i < N * D / 8; i += NT) {
    const int r = i >> 2, c = i & 3;
    const vec8<VT> v = __builtin_bit_cast(vec8<VT>, gload16(vg + i * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) vts[(c * 8 + e) * LDV + r] = v[e];
  }
  // Table rows stored reversed, times log2(e); then 8 x -inf.
  for (int i = tid; i < R * R + 8; i += NT) {
    float v = -__builtin_inff();
    if (i < R * R) {
      const int r = i / R, c = i - r * R;
      v = p.table[(int64_t)(r * R + (R - 1 - c)) * g.heads + h] * kLog2e;
    }
    rt[i] = v;
  }
  __syncthreads();

  const int wl = w % g.nW;
  const int wy = wl / g.nWx, wx = wl - (wl / g.nWx) * g.nWx;
  const bool my = g.s > 0 && wy == g.H / M - 1;
  const bool mx = g.s > 0 && wx == g.nWx - 1;
  if (my || mx)
    tiled_attn_body<QT, VT, M, QTL, true>(p, ks, vts, rt, item, wave, lane, my, mx);
  else
    tiled_attn_body<QT, VT, M, QTL, false>(p, ks, vts, rt, item, wave, lane, false, false);
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
