// Attention core shared by the kernels whose window side M is a multiple of 8:
// QTL tiles of 16 queries of one (window, head) against the window's N = M*M
// keys, with K and V staged in LDS as [key][d] rows.
//
// Pages: "Boosting Swin Transformer Speed", Training Optimization (fused MHA:
// softmax fused with the two products) and Inference Optimization (the bias
// table is prepared once; the mask is index arithmetic); "Swin Transformer V2"
// summary, How It Works (logit = similarity + relative position bias B_ij).
//
// Slots are chunked (see Geom): 16 consecutive slots are a 2 x 8 patch of the
// window and 32 consecutive slots a 4 x 8 patch; tile T holds slots 16T..16T+15.
//
// Register layout.  S^T = K Q^T on the matrix cores, with the K rows of each
// 32-key block permuted so that lane l receives query (l % 16) and the 8 keys
// 8*(l/16) .. +7 of the block: one window row, 8 consecutive columns.  The
// relative position index of those 8 keys then walks one row of the table
// backwards, so with the rows of the table stored reversed the lane reads its
// 8 biases from 8 consecutive floats (from one of four shifted copies of the
// table, so that the read is two aligned 16-byte loads); they are the MFMA's
// initial accumulator.  P stays in registers as the B operand of
// O^T = V^T P^T; the V^T fragments come from transposing LDS reads
// (ds_read_b64_tr_b16) with the head dims of each 16-row fragment pair
// interleaved, so that lane l ends with O^T for d = 8*(l/16) .. +7 of its
// query -- the B-operand slice of a following product with O, or one 16-byte
// store.  Row sums come from one more MFMA (ones x P^T), i.e. from exactly the
// rounded P that multiplies V.
//
// Softmax.  Base 2, online, with a lazy running max: a block only rescales when
// some lane sees a logit more than G above the row's current reference, so the
// exponentials stay below 2^G (G = 64 with bfloat16 P, whose exponent range is
// that of float; 8 with float16 P).  Each key block runs in three phases over
// all query tiles (logits, the rare rescale, exponentials and products), with
// the next block's LDS operands loaded while the current one is computed.
//
// Shifted windows.  Only the last window row (column) of the grid mixes two
// slices of the shifted frame, split at M - s; a pair is allowed when query and
// key are on the same side in both directions.  A tile whose lanes have no
// allowed key in a block skips it; otherwise the bias of a fully masked key
// group is read from a row of -inf, and a group that straddles the split gets
// -inf per key.
#pragma once

#include "kv_frag.hpp"

namespace swin {

// Bias-table modes: kTable4 = four shifted copies (fill_bias_copies; two
// aligned 16-byte reads per lane and block), kTable1 = one copy
// (fill_bias_table; eight 4-byte reads).
enum class TableMode { kTable4, kTable1 };

// The single reversed copy keeps its 2M-1 rows at a pitch of 8 x odd floats
// (24, 40, 56 for M = 8, 16, 24): a wave's bias read touches 5 consecutive
// rows, 8 consecutive floats each, and at that pitch they fall on distinct
// banks (row pitch 2M-1 made them collide two ways).  Every lane reads 8
// floats inside one row.
template <int M>
constexpr int table1_pitch() { return ((2 * M - 1 + 7) / 8) % 2 ? (2 * M - 1 + 7) / 8 * 8 : (2 * M - 1 + 7) / 8 * 8 + 8; }
template <int M>
constexpr int table1_size() { return (2 * M - 1) * table1_pitch<M>(); }

template <int M>
__device__ __forceinline__ void fill_bias_table(float* rt, const float* table, int heads, int h,
                                                int tid, int nthreads) {
  constexpr int R = 2 * M - 1, P = table1_pitch<M>();
  for (int e = tid; e < table1_size<M>(); e += nthreads) {
    const int r = e / P, cc = e - r * P;
    float v = -__builtin_inff();
    if (cc < R) v = table[(int64_t)(r * R + (R - 1 - cc)) * heads + h] * kLog2e;
    rt[e] = v;
  }
}

// Softmax reference:
//   kLazy   -- moves lazily, one compare and ballot per key block;
//   kBlock0 -- block 0's row max, fixed (unmasked windows only: a masked row
//              may have no allowed key in block 0; masked windows then run
//              kLazy);
//   kZero   -- 0, fixed (bfloat16 P only; masked windows too): the caller has
//              shifted the head's bias table by a constant so that no logit
//              (base 2) exceeds kZeroTop; no max and no subtraction at all;
//   kOwn    -- fixed, per tile the row max over the tile's own key block (the
//              32 slots that hold its 16 queries: every row has its own token
//              there, always allowed, so the reference is a logit of the row
//              and every row sum is at least 1); masked windows too, at the
//              cost of two more products per tile.
// The fixed schemes check the row sums once at the end (the fallback of all
// of them is the lazy pass).
enum class RefMode { kLazy, kBlock0, kZero, kOwn };
constexpr float kZeroTop = 64.0f;

struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// Floats per copy of the reversed bias table (+ room so that every copy can
// be read 8 floats past any start index it is used with).
template <int M>
constexpr int table_stride() { return ((2 * M - 1) * (2 * M - 1) + 8 + 3) / 4 * 4; }

// Fills the 4 shifted copies of the head's reversed bias table (times log2 e):
// copy c holds element i + c at position i, -inf past the end; table is
// [(2M-1)^2, heads] float.
template <int M>
__device__ __forceinline__ void fill_bias_copies(float* rt4, const float* table, int heads, int h,
                                                 int tid, int nthreads) {
  constexpr int R = 2 * M - 1;
  constexpr int TS = table_stride<M>();
  for (int i = tid; i < 4 * TS; i += nthreads) {
    const int c = i / TS, e = i - c * TS + c;
    float v = -__builtin_inff();
    if (e < R * R) {
      const int r = e / R, cc = e - r * R;
      v = table[(int64_t)(r * R + (R - 1 - cc)) * heads + h] * kLog2e;
    }
    rt4[i] = v;
  }
}

// Attention of query tiles tile[0..QTL) (q fragments qf: lane l holds query
// 16*tile + l%16, d = 8*(l/16) .. +7, pre-scaled to base-2 logits) against all
// N keys.  ks, vs: K and V as [N][kAttnLD]; rt4: the 4 bias copies; ninf: 8 x
// -inf (16-byte aligned); bnd = M - s; my / mx: the window is in the last
// row / column of the grid (shift > 0).  On return o[j] holds the normalised
// O for the lane's query and d = 8*(l/16) + e, e = 0..7.  LAYOUT / TABLE pick
// the K, V layout and the bias-table mode; hook(kbi) runs at the start of key
// block kbi (the caller's work to interleave, e.g. staging the next item).
// With a fixed reference (kZero, kOwn, or kBlock0 and !MASKED), returns false
// (o undefined) when the row sums show that some P left the safe range; the
// caller then runs the MASKED kLazy instance (with the window's my / mx),
// which is exact for any logits.  Otherwise returns true.
template <typename QT, typename VT, int M, int QTL, bool MASKED,
          KvLayout LAYOUT = KvLayout::kPadded, TableMode TABLE = TableMode::kTable4,
          RefMode REF = RefMode::kBlock0, class Hook = NoHook>
__device__ __forceinline__ bool attn_tiles(const vec8<QT> (&qf)[QTL], const int (&tile)[QTL],
                                           const QT* ks, const VT* vs, const float* rt4,
                                           const float* ninf, int lane, int bnd, bool my, bool mx,
                                           float (&o)[QTL][8], Hook hook = Hook()) {
  typedef __attribute__((address_space(3))) const vec8<QT>* lds_q8;
  typedef __attribute__((address_space(3))) const f32x4* lds_f4;
  constexpr int N = M * M;
  constexpr int R = 2 * M - 1;
  static_assert(REF != RefMode::kZero || !__is_same(VT, h16), "zero reference needs bfloat16 P");
  constexpr bool SWZ = LAYOUT == KvLayout::kSwizzled;
  constexpr bool T1 = TABLE == TableMode::kTable1;
  constexpr int LDK = SWZ ? 32 : kAttnLD;
  typedef __attribute__((address_space(3))) const float* lds_f;
  constexpr int TPC = M / 2;  // 16-query tiles per chunk
  constexpr int BPC = M / 4;  // 32-key blocks per chunk
  constexpr int TS = table_stride<M>();
  constexpr int P1 = table1_pitch<M>();
  const int g4 = lane >> 4, i16 = lane & 15;
  const float NEG_INF = -__builtin_inff();
  // Lazy-rescale headroom (base 2): P may reach 2^kGrow before the reference
  // moves.  bfloat16 P has the float exponent range; float16 P tops out at
  // 65504, so it keeps a margin of 8.
  constexpr float kGrow = __is_same(VT, h16) ? 8.0f : 64.0f;

  int qy[QTL], qx[QTL];
  lds_f4 tb[QTL];   // TABLE == kTable4
  lds_f tbf[QTL];   // TABLE == kTable1
  f32x4 o0[QTL], o1[QTL], ls[QTL];
  float m[QTL], mt[QTL];  // reference max and reference + kGrow
#pragma unroll
  for (int j = 0; j < QTL; ++j) {
    const int T = tile[j];
    const int cq = T / TPC, rp = T - cq * TPC;
    qy[j] = 2 * rp + (i16 >> 3);
    qx[j] = 8 * cq + (i16 & 7);
    // Table row of (qy, key row 4b + g4) is qy - 4b - g4 + M - 1; reversed
    // column of key column 8c is 8c - qx + M - 1.  a0 is the index at b = BPC-1,
    // c = 0 (the smallest), so every block adds a non-negative multiple of 4.
    // Copy (a0 % 4) of the table is shifted so that the lane's 8 floats start
    // on a 16-byte boundary.
    const int a0 = (qy[j] - 4 * (BPC - 1) - g4 + M - 1) * (T1 ? P1 : R) + (M - 1 - qx[j]);
    if constexpr (T1)
      tbf[j] = (lds_f)(rt4 + a0);
    else
      tb[j] = (lds_f4)(rt4 + (a0 & 3) * TS + (a0 & ~3));
    o0[j] = o1[j] = ls[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[j] = REF == RefMode::kZero ? 0.0f : -1e30f;
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
  // Swizzled rows: for the K reads (row/8) % 4 = l%16 / 4, for the V reads
  // (row/8) % 4 = l/16, whatever the block.
  lds_q8 kl = SWZ ? (lds_q8)&ks[(8 * (i16 >> 2) + (i16 & 3)) * LDK + ((g4 ^ (i16 >> 2)) << 3)]
                  : (lds_q8)&ks[(8 * (i16 >> 2) + (i16 & 3)) * LDK + g4 * 8];
  lds_v4s vl = SWZ ? (lds_v4s)&vs[(8 * g4 + (i16 >> 2)) * LDK + (((i16 & 3) ^ g4) << 3)]
                   : (lds_v4s)&vs[(8 * g4 + (i16 >> 2)) * LDK + 8 * (i16 & 3)];
  asm volatile("" : "+v"(kl), "+v"(vl), "+v"(ones));
#pragma unroll
  for (int j = 0; j < QTL; ++j) {
    if constexpr (T1)
      asm volatile("" : "+v"(tbf[j]));
    else
      asm volatile("" : "+v"(tb[j]));
  }
  lds_f4 ninf4 = (lds_f4)ninf;

  // Key blocks of 32: block kbi is chunk kbi / BPC, rows 4b .. 4b+3 with
  // b = kbi % BPC.  Fully unrolled, with the LDS operands of the next block
  // (K and V fragments; with four table copies also the tiles' biases) loaded
  // while this one is computed; with one table copy the biases are read at
  // the block's start (fewer registers).
  constexpr int NB = N / 32;
  struct Ops {
    vec8<QT> k0, k1;
    vec8<VT> v0, v1;
    f32x4 b0[QTL], b1[QTL];
    bool act[QTL];       // tile has an allowed key in this block (masked windows)
    unsigned bits[QTL];  // allowed keys of the lane's group (masked windows)
  };
  auto load_kv = [&](int kbi, Ops& op) {
    const int kb = 32 * kbi;
    op.k0 = kl[kb * LDK / 8];
    op.k1 = kl[(kb + 4) * LDK / 8];
    op.v0 = vt_frag<VT, LDK>(vl, kb, 0);
    op.v1 = vt_frag<VT, LDK>(vl, kb, 1);
  };
  auto load_bias = [&](int kbi, Ops& op) {
    const int ck = kbi / BPC, b = kbi - ck * BPC;
    const int boff = 8 * ck + 4 * (T1 ? P1 : R) * (BPC - 1 - b);
#pragma unroll
    for (int j = 0; j < QTL; ++j) {
      lds_f4 bp = tb[j] + boff / 4;
      lds_f bpf = tbf[j] + boff;
      op.act[j] = true;
      op.bits[j] = 0xffu;
      if constexpr (MASKED) {
        // Allowed key columns of this chunk for the lane's query, and rows.
        const int left = min(max(bnd - 8 * ck, 0), 8);
        const unsigned lm = (1u << left) - 1u;
        const unsigned xb = !mx ? 0xffu : (qx[j] < bnd ? lm : (~lm & 0xffu));
        const int ky = 4 * b + g4;
        const bool yok = !my || ((ky < bnd) == (qy[j] < bnd));
        op.bits[j] = yok ? xb : 0u;
        op.act[j] = __any(op.bits[j] != 0u);  // else the tile is masked in this block
        if (op.bits[j] == 0u) {
          bp = ninf4;
          bpf = (lds_f)ninf4;
        }
      }
      if constexpr (T1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          op.b0[j][r] = bpf[r];
          op.b1[j][r] = bpf[4 + r];
        }
      } else {
        op.b0[j] = bp[0];
        op.b1[j] = bp[1];
      }
    }
  };

  if constexpr (REF == RefMode::kOwn) {
#pragma unroll
    for (int j = 0; j < QTL; ++j) {
      const int kbo = tile[j] >> 1;  // the key block holding the tile's slots
      Ops op;
      load_kv(kbo, op);
      load_bias(kbo, op);
      f32x4 s0 = op.b0[j], s1 = op.b1[j];
      if constexpr (MASKED) {
        const int left = min(max(bnd - 8 * (kbo / BPC), 0), 8);
        if (mx && left > 0 && left < 8) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (!((op.bits[j] >> r) & 1u)) s0[r] = NEG_INF;
            if (!((op.bits[j] >> (4 + r)) & 1u)) s1[r] = NEG_INF;
          }
        }
      }
      s0 = mma_16x16x32(op.k0, qf[j], s0);
      s1 = mma_16x16x32(op.k1, qf[j], s1);
      const float bm = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                             fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
      m[j] = xor32_max(xor16_max(bm));
    }
  }

  Ops cur;
  load_kv(0, cur);
  if constexpr (!T1) load_bias(0, cur);
#pragma unroll
  for (int kbi = 0; kbi < NB; ++kbi) {
    hook(kbi);
    if constexpr (T1) load_bias(kbi, cur);
    Ops nxt;
    if (kbi + 1 < NB) {
      load_kv(kbi + 1, nxt);
      if constexpr (!T1) load_bias(kbi + 1, nxt);
    }
    const int ck = kbi / BPC;
    bool straddle = false;
    if constexpr (MASKED) {
      const int left = min(max(bnd - 8 * ck, 0), 8);
      straddle = mx && left > 0 && left < 8;
      // Skip the block when every tile is masked in it.  Otherwise every tile
      // is computed: a masked tile's logits are -inf (its bias reads the -inf
      // strip), so its P is 0 and it adds nothing.  The wave's tiles share
      // a column chunk and usually a row region, so they are masked together.
      bool any = false;
#pragma unroll
      for (int j = 0; j < QTL; ++j) any = any || cur.act[j];
      if (!any) {
        if (kbi + 1 < NB) cur = nxt;
        continue;
      }
    }
    // Phase 1, every tile: S^T = K Q^T on top of the bias, block max (with
    // the fixed reference, only in block 0).
    constexpr bool FIXED = REF == RefMode::kZero || REF == RefMode::kOwn ||
                           (REF == RefMode::kBlock0 && !MASKED);
    constexpr bool BLOCK0 = FIXED && REF == RefMode::kBlock0;
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
      }
      s0[j] = mma_16x16x32(cur.k0, qf[j], s0[j]);
      s1[j] = mma_16x16x32(cur.k1, qf[j], s1[j]);
      if (!FIXED || (BLOCK0 && kbi == 0))
        bm[j] = fmaxf(fmaxf(fmaxf(s0[j][0], s0[j][1]), fmaxf(s0[j][2], s0[j][3])),
                      fmaxf(fmaxf(s1[j][0], s1[j][1]), fmaxf(s1[j][2], s1[j][3])));
    }
    // Phase 2.  Unmasked windows with a fixed reference (block 0's row max,
    // or 0): it never moves -- no per-block max, compare or branch; the row
    // sums are checked once at the end.  Otherwise (masked windows, where a
    // row may have no allowed key in block 0, the fallback, and kLazy) lazy:
    // when some lane of some tile saw a logit more than kGrow above its
    // reference, every tile's reference moves to its row max.
    if constexpr (BLOCK0) {
      if (kbi == 0) {
#pragma unroll
        for (int j = 0; j < QTL; ++j) m[j] = xor32_max(xor16_max(bm[j]));
      }
    }
    uint64_t grow = 0;
    if constexpr (!FIXED) {
#pragma unroll
      for (int j = 0; j < QTL; ++j) grow |= __builtin_amdgcn_ballot_w64(bm[j] > mt[j]);
    }
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

  if constexpr (REF == RefMode::kZero || REF == RefMode::kOwn ||
                (REF == RefMode::kBlock0 && !MASKED)) {
    // Every P is at most its row sum.  A row sum below kFixedLimit (also
    // false for inf / NaN) means no P went past it: bfloat16 P stays far
    // from its overflow, float16 P below 65504.  With block 0's max as the
    // reference the largest P is >= 1; with the zero reference a row sum of
    // at least 2^-60 keeps every P that matters a normal number.  Otherwise
    // the caller redoes the item on the lazy path.
    constexpr float kFixedLimit = __is_same(VT, h16) ? 32768.0f : 18446744073709551616.0f;
    constexpr float kZeroFloor = 8.673617379884035e-19f;  // 2^-60
    bool far = false;
#pragma unroll
    for (int j = 0; j < QTL; ++j) {
      far = far || !(ls[j][0] < kFixedLimit);
      if constexpr (REF == RefMode::kZero) far = far || !(ls[j][0] >= kZeroFloor);
    }
    if (__builtin_amdgcn_ballot_w64(far)) return false;
  }
  // Fragment pair t row 4*g4 + r is head dim 8*g4 + 4t + r.
#pragma unroll
  for (int j = 0; j < QTL; ++j) {
    const float inv = __builtin_amdgcn_rcpf(ls[j][0]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      o[j][r] = o0[j][r] * inv;
      o[j][4 + r] = o1[j][r] * inv;
    }
  }
  return true;
}

}  // namespace swin
