// Attention core for windows of side 7 or 8 laid out on an 8 x 8 slot grid
// (slot = 8 * ty + tx; for side 7 the last row and column are padding), one
// wave per (window, head): its 4 query tiles against the 64 keys in two
// 32-key blocks, with an exact row max.
//
// Pages: "Boosting Swin Transformer Speed", Training Optimization (fused MHA:
// softmax fused with both products) and Inference Optimization (the bias table
// prepared once; the mask is index arithmetic); "Swin Transformer V2" summary,
// How It Works (logit = similarity + relative position bias B_ij).
//
// S^T = K Q^T on the matrix cores with the K rows permuted so that lane l
// holds query l%16 of a tile and the 8 keys 8(l/16) .. +7 of a block (one row
// of 8 columns); the bias (times log2 e) is the accumulator's initial value,
// read from a reversed per-head table at an immediate offset from one lane
// base.  P stays in registers as the B operand of O^T = V^T P^T; row sums come
// from a ones x P^T product.
#pragma once

#include "kv_frag.hpp"

namespace swin {

// Reversed bias table per head: entry [a][c] (rows of 16 floats) is the bias
// (times log2 e) of dy = a - 7, dx = 7 - c; -inf outside the window's range
// and in the kPadInf entries after the 15 rows (read by padded key rows).
constexpr int kTabRows = 15 * 16;
constexpr int kPadInf = 3 * 32 + 8;
constexpr int kTab = kTabRows + kPadInf;

typedef __attribute__((address_space(3))) const float* lds_f;

// ZERO: the softmax reference is 0 instead of the exact row max (no max
// reductions); returns false when some real query's row sum left the safe
// range (every tile has been stored all the same), and the caller then redoes
// the item with ZERO = false, which overwrites every store and returns true.
template <typename QT, typename T, int MV, bool MASKED, bool ZERO, class Store>
__device__ __forceinline__ bool w8_attend(const vec8<QT> (&qf)[4], const vec8<QT> (&kf)[2][2],
                                          const vec8<T> (&vf)[2][2], lds_f tb0,
                                          lds_f tb1, int qy0, int qx, int g4, int bnd,
                                          bool my, bool mx, Store store) {
  const float NEG_INF = -__builtin_inff();
  vec8<T> ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = from_f32<T>(1.0f);
  // Shifted windows: allowed key columns of the lane's query column.
  unsigned xbits = 0xffu;
  if (MASKED && mx) {
    const unsigned lm = (1u << bnd) - 1u;
    xbits = qx < bnd ? lm : (~lm & 0xffu);
  }
  // Safe range of a row sum with the zero reference: float16 P below 2^15
  // (its largest finite value is 65504) and a row sum of at least 1 (the
  // largest P >= 1/64, so P too small for a normal float16 hardly matters);
  // bfloat16 P between 2^-60 and 2^64.
  constexpr bool H16 = __is_same(T, h16);
  constexpr float kLo = H16 ? 1.0f : 8.673617379884035e-19f;
  constexpr float kHi = H16 ? 32768.0f : 18446744073709551616.0f;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // Logits of the lane's query (slot 16j + l%16) against keys 32b + 8g + e:
    // key row 4b + g, column e.  Bias = initial accumulator.
    f32x4 s[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const lds_f tb = (b ? tb1 : tb0) + 32 * j;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[b][t][r] = tb[4 * t + r];
    }
    if constexpr (MASKED) {
      const int qy = 2 * j + qy0;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int ky = 4 * b + g4;
        const bool yok = !my || ((qy < bnd) == (ky < bnd));
        const unsigned bits = yok ? xbits : 0u;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!((bits >> (4 * t + r)) & 1u)) s[b][t][r] = NEG_INF;
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < 2; ++t) s[b][t] = mma_16x16x32(kf[b][t], qf[j], s[b][t]);
    // Exact row max over the 64 keys (column 7 is padding for side 7).
    float m = 0.f;
    if constexpr (!ZERO) {
      m = NEG_INF;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < MV) m = fmaxf(m, s[b][e >> 2][e & 3]);
      m = xor32_max(xor16_max(m));
      if constexpr (MASKED) m = m == NEG_INF ? 0.f : m;  // padded query with no allowed key
    }
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0, l = o0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      vec8<T> pf;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[e] = e < MV ? from_f32<T>(fast_exp2(s[b][e >> 2][e & 3] - m)) : from_f32<T>(0.f);
      o0 = mma_16x16x32(vf[b][0], pf, o0);
      o1 = mma_16x16x32(vf[b][1], pf, o1);
      l = mma_16x16x32(ones, pf, l);
    }
    // Only the window's real queries count (padding slots are not stored).
    if constexpr (ZERO) bad = bad || (2 * j + qy0 < MV && qx < MV && !(l[0] >= kLo && l[0] < kHi));
    const float inv = __builtin_amdgcn_rcpf(l[0]);
    vec8<T> of;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      of[r] = from_f32<T>(o0[r] * inv);
      of[4 + r] = from_f32<T>(o1[r] * inv);
    }
    // O of the lane's query (slot 16j + l%16), dims 8g .. 8g+7.
    store(j, of);
  }
  return !(ZERO && __builtin_amdgcn_ballot_w64(bad));
}


// Fills one head's reversed table (times log2 e) in the w8_attend layout from
// the [(2MV-1)^2, heads] float table.
template <int MV>
__device__ __forceinline__ void fill_w8_table(float* tab, const float* table, int heads, int h,
                                              int tid, int nthreads) {
  constexpr int R = 2 * MV - 1;
  for (int e = tid; e < kTab; e += nthreads) {
    const int dy = (e >> 4) - 7, dx = 7 - (e & 15);
    float v = -__builtin_inff();
    if (e < kTabRows && dy > -MV && dy < MV && dx > -MV && dx < MV)
      v = table[(int64_t)((dy + MV - 1) * R + dx + MV - 1) * heads + h] * kLog2e;
    tab[e] = v;
  }
}

}  // namespace swin
