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
// q, k, v as [N][32], q already scaled so that the logits are in base 2; K and
// V are staged in LDS as they are, and V^T fragments are read with the
// transposing LDS loads of gfx950.
//
// Register layout.  A wave owns QTL tiles of 16 queries.  S^T = K Q^T on the
// matrix cores, with the K rows of each 32-key block permuted so that lane l
// receives query (l % 16) and the 8 keys 8*(l/16) .. +7 of the block: one
// window row, 8 consecutive columns.  The relative position index of those 8
// keys then walks one row of the table backwards, so with the rows of the
// table stored reversed in LDS the lane reads its 8 biases from 8 consecutive
// floats (from one of four shifted copies of the table, so that the read is
// two aligned 16-byte loads); they are the MFMA's initial accumulator.  P stays in registers as the
// B operand of O^T = V^T P^T, and its row sums come from one more MFMA (ones x
// P^T), i.e. from exactly the rounded P that multiplies V.
//
// Softmax.  Base 2, online, with a lazy running max: a block only rescales when
// some lane sees a logit more than G above the row's current reference, so the
// exponentials stay below 2^G and the common path is max-test, subtract, exp2
// (G = 64 with bfloat16 P, whose exponent range is that of float; 8 with
// float16 P).
// Each key block runs in three phases over all of the wave's query tiles
// (logits, the rare rescale, exponentials and products), so that the common
// path is one straight block in which the tiles' chains interleave.
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

// V^T fragment (rows d0 .. d0+15, keys kb .. kb+31) from V stored as [key][d]
// rows of LD elements, by two transposing LDS reads (ds_read_b64_tr_b16).
// Within each 16-lane group g, lane (4a + b) of the read receives element b of
// the 8-byte chunk addressed by lane 4e + a, for e = 0..3; with lane s of
// group g addressing V[kb + 8g + 4h + s/4][d0 + 4(s%4)], lane i of group g gets
// V[kb + 8g + 4h + e][d0 + i]: column d0 + i of V^T, keys 8g + 4h + e, which is
// the A-operand slice of the 16x16x32 product.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s;

// vl: this lane's V address for kb = 0, d0 = 0 (lane s of group g:
// V[8g + s/4][4(s%4)]).
template <typename VT, int LD>
__device__ __forceinline__ vec8<VT> vt_frag(lds_v4s vl, int kb, int d0) {
  const lds_v4s p0 = vl + (kb * LD + d0) / 4;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0 + LD);
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(vec8<VT>, both);
}

// Floats per copy of the reversed bias table (+ room so that every copy can
// be read 8 floats past any start index it is used with).
template <int M>
constexpr int table_stride() { return ((2 * M - 1) * (2 * M - 1) + 8 + 3) / 4 * 4; }

template <typename QT, typename VT, int M, int QTL, bool MASKED>
__device__ __forceinline__ void tiled_attn_body(const FwdParams& p, const QT* ks, const VT* vs,
                                                const float* rt4, const float* ninf, int item,
                                                int wave, int lane, bool my, bool mx) {
  typedef __attribute__((address_space(3))) const vec8<QT>* lds_q8;
  typedef __attribute__((address_space(3))) const f32x4* lds_f4;
  constexpr int D = 32;
  constexpr int N = M * M;
  constexpr int R = 2 * M - 1;
  constexpr int LDK = D + 8;
  constexpr int CH = M / 8;   // column chunks
  constexpr int TPC = M / 2;  // 16-query tiles per chunk
  constexpr int BPC = M / 4;  // 32-key blocks per chunk
  constexpr int TS = table_stride<M>();
  const Geom& g = p.g;
  const int g4 = lane >> 4, i16 = lane & 15;
  const int bnd = M - g.s;  // slice split inside a masked window
  const float NEG_INF = -__builtin_inff();

  // Lazy-rescale headroom (base 2): P may reach 2^kGrow before the reference
  // moves.  bfloat16 P has the float exponent range; float16 P tops out at
  // 65504, so it keeps a margin of 8.
  constexpr float kGrow = sizeof(VT) == 2 && !__is_same(VT, h16) ? 64.0f : 8.0f;
  const QT* qg = static_cast<const QT*>(p.buf.q) + (int64_t)item * N * D;
  vec8<QT> qf[QTL];
  int qy[QTL], qx[QTL];
  lds_f4 tb[QTL];
  f32x4 o0[QTL], o1[QTL], ls[QTL];
  float m[QTL], mt[QTL];  // reference max and reference + kGrow
#pragma unroll
  for (int j = 0; j < QTL; ++j) {
    const int T = wave * QTL + j;
    const int cq = T / TPC, rp = T - cq * TPC;
    qy[j] = 2 * rp + (i16 >> 3);
    qx[j] = 8 * cq + (i16 & 7);
    qf[j] = gload8(qg + (T * 16 + i16) * D + g4 * 8);
    // Table row of (qy, key row 4b + g4) is qy - 4b - g4 + M - 1; reversed
    // column of key column 8c is 8c - qx + M - 1.  a0 is the index at b = BPC-1,
    // c = 0 (the smallest), so every block adds a non-negative multiple of 4.
    // Copy (a0 % 4) of the table is shifted so that the lane's 8 floats start
    // on a 16-byte boundary: two 16-byte reads with immediate offsets.
    const int a0 = (qy[j] - 4 * (BPC - 1) - g4 + M - 1) * R + (M - 1 - qx[j]);
    tb[j] = (lds_f4)(rt4 + (a0 & 3) * TS + (a0 & ~3));
    o0[j] = o1[j] = ls[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[j] = -1e30f;
    mt[j] = -1e30f;
  }
  vec8<VT> ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = from_f32<VT>(1.0f);
  // Per-lane LDS bases: K rows of the block permutation, V for the
  // transposing reads, the bias.  Opaque, so that every per-block address is
  // this base plus an immediate (the static LDS offsets of the arrays are not
  // folded into the immediates, which would overflow their 16 bits), and so
  // that the ones operand stays in vector registers.
  lds_q8 kl = (lds_q8)&ks[(8 * (i16 >> 2) + (i16 & 3)) * LDK + g4 * 8];
  lds_v4s vl = (lds_v4s)&vs[(8 * g4 + (i16 >> 2)) * LDK + 4 * (i16 & 3)];
  asm volatile("" : "+v"(kl), "+v"(vl), "+v"(ones));
#pragma unroll
  for (int j = 0; j < QTL; ++j) asm volatile("" : "+v"(tb[j]));
  lds_f4 ninf4 = (lds_f4)ninf;

  // Key blocks of 32: block kbi is chunk kbi / BPC, rows 4b .. 4b+3 with
  // b = kbi % BPC.  Fully unrolled, with the LDS operands of the next block
  // (K and V fragments, the tiles' biases) loaded while this one is computed.
  constexpr int NB = N / 32;
  struct Ops {
    vec8<QT> k0, k1;
    vec8<VT> v0, v1;
    f32x4 b0[QTL], b1[QTL];
    bool act[QTL];      // tile has an allowed key in this block (masked windows)
    unsigned bits[QTL];  // allowed keys of the lane's group (masked windows)
  };
  auto load = [&](int kbi, Ops& o) {
    const int ck = kbi / BPC, b = kbi - ck * BPC;
    const int kb = 32 * kbi;
    o.k0 = kl[kb * LDK / 8];
    o.k1 = kl[(kb + 4) * LDK / 8];
    o.v0 = vt_frag<VT, LDK>(vl, kb, 0);
    o.v1 = vt_frag<VT, LDK>(vl, kb, 16);
    const int boff = 8 * ck + 4 * R * (BPC - 1 - b);
#pragma unroll
    for (int j = 0; j < QTL; ++j) {
      lds_f4 bp = tb[j] + boff / 4;
      o.act[j] = true;
      o.bits[j] = 0xffu;
      if constexpr (MASKED) {
        // Allowed key columns of this chunk for the lane's query, and rows.
        const int left = min(max(bnd - 8 * ck, 0), 8);
        const unsigned lm = (1u << left) - 1u;
        const unsigned xb = !mx ? 0xffu : (qx[j] < bnd ? lm : (~lm & 0xffu));
        const int ky = 4 * b + g4;
        const bool yok = !my || ((ky < bnd) == (qy[j] < bnd));
        o.bits[j] = yok ? xb : 0u;
        o.act[j] = __any(o.bits[j] != 0u);  // else the tile is masked in this block
        if (o.bits[j] == 0u) bp = ninf4;
      }
      o.b0[j] = bp[0];
      o.b1[j] = bp[1];
    }
  };

  Ops cur;
  load(0, cur);
#pragma unroll
  for (int kbi = 0; kbi < NB; ++kbi) {
    Ops nxt;
    if (kbi + 1 < NB) load(kbi + 1, nxt);
    const int ck = kbi / BPC;
    bool straddle = false;
    if constexpr (MASKED) {
      const int left = min(max(bnd - 8 * ck, 0), 8);
      straddle = mx && left > 0 && left < 8;
    }
    // Phase 1, every tile: S^T = K Q^T on top of the bias, block max.
    f32x4 s0[QTL], s1[QTL];
    float bm[QTL];
#pragma unroll
    for (int j = 0; j < QTL; ++j) {
      s0[j] = cur.b0[j];
      s1[j] = cur.b1[j];
      if constexpr (MASKED) {
        if (straddle) {
          const unsigned bits = cur.bits[j];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (!((bits >> r) & 1u)) s0[j][r] = NEG_INF;
            if (!((bits >> (4 + r)) & 1u)) s1[j][r] = NEG_INF;
          }
        }
        if (!cur.act[j]) {
          bm[j] = NEG_INF;
          continue;
        }
      }
      s0[j] = mma_16x16x32(cur.k0, qf[j], s0[j]);
      s1[j] = mma_16x16x32(cur.k1, qf[j], s1[j]);
      bm[j] = fmaxf(fmaxf(fmaxf(s0[j][0], s0[j][1]), fmaxf(s0[j][2], s0[j][3])),
                    fmaxf(fmaxf(s1[j][0], s1[j][1]), fmaxf(s1[j][2], s1[j][3])));
    }
    // Phase 2, rare: some lane of some tile saw a logit more than kGrow above
    // its reference; move every tile's reference to its row max.
    uint64_t grow = 0;
#pragma unroll
    for (int j = 0; j < QTL; ++j) grow |= __builtin_amdgcn_ballot_w64(bm[j] > mt[j]);
    if (grow) {
#pragma unroll
      for (int j = 0; j < QTL; ++j) {
        const float rm = xor32_max(xor16_max(bm[j]));
        const float mn = fmaxf(m[j], rm);
        const float alpha = fast_exp2(m[j] - mn);
        o0[j] *= alpha;
        o1[j] *= alpha;
        ls[j] *= alpha;
        m[j] = mn;
        mt[j] = mn + kGrow;
      }
    }
    // Phase 3, every tile: P = exp2(S - m), O^T += V^T P^T, row sums.
#pragma unroll
    for (int j = 0; j < QTL; ++j) {
      if constexpr (MASKED) {
        if (!cur.act[j]) continue;
      }
      vec8<VT> pf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pf[r] = from_f32<VT>(fast_exp2(s0[j][r] - m[j]));
        pf[4 + r] = from_f32<VT>(fast_exp2(s1[j][r] - m[j]));
      }
      o0[j] = mma_16x16x32(cur.v0, pf, o0[j]);
      o1[j] = mma_16x16x32(cur.v1, pf, o1[j]);
      ls[j] = mma_16x16x32(ones, pf, ls[j]);
    }
    if (kbi + 1 < NB) cur = nxt;
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
  }
  for (int i = tid; i < N * D / 8; i += NT) {
    const int r = i >> 2, c = i & 3;
    *reinterpret_cast<uint4*>(&vs[r * LDK + c * 8]) = gload16(vg + i * 8);
  }
  // Table rows stored reversed, times log2(e), in 4 copies: copy c holds
  // element i + c at position i (past the end: -inf).
  for (int i = tid; i < 4 * TS; i += NT) {
    const int c = i / TS, e = i - c * TS + c;
    float v = -__builtin_inff();
    if (e < R * R) {
      const int r = e / R, cc = e - r * R;
      v = p.table[(int64_t)(r * R + (R - 1 - cc)) * g.heads + h] * kLog2e;
    }
    rt4[i] = v;
  }
  if (tid < 8) ninf[tid] = -__builtin_inff();
  __syncthreads();

  const int wl = w % g.nW;
  const int wy = wl / g.nWx, wx = wl - (wl / g.nWx) * g.nWx;
  const bool my = g.s > 0 && wy == g.H / M - 1;
  const bool mx = g.s > 0 && wx == g.nWx - 1;
  if (my || mx)
    tiled_attn_body<QT, VT, M, QTL, true>(p, ks, vs, rt4, ninf, item, wave, lane, my, mx);
  else
    tiled_attn_body<QT, VT, M, QTL, false>(p, ks, vs, rt4, ninf, item, wave, lane, false, false);
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
