// Whole block forward in one kernel for window side 16 (N = 256 tokens) and
// up to 4 heads (C = 32 * heads <= 128), 16-bit I/O: one workgroup of 8 waves
// per window, nothing but x, the weights and y touch HBM.
//
// Pages: "Boosting Swin Transformer Speed: Profiling, Mixed Precision, and
// Kernel Fusion Secrets" -- Training Optimization (the index maps fused away;
// QKV, bias and softmax fused) and Inference Optimization (GEMMs carry their
// biases, no separate transposes); "Boost Vision Transformer with
// GPU-Friendly Sparsity and Quantization", Section 3.2 / Figure 3 (Q/K/V and
// output projections are GEMMs); "Swin Transformer V2" summary, How It Works
// (cosine attention over tau, continuous position bias).
//
// Per window: the 256 token rows are gathered from x through the cyclic shift
// into LDS (chunked slot order, see Geom).  Then for each head:
//   1. its 96 rows of W_qkv and its bias-table copies go to LDS;
//   2. wave w computes q, k, v of its 32 tokens (tiles 2w, 2w+1) as C^T
//      products (weight rows of each 16-channel tile pair interleaved, so a
//      lane holds 8 consecutive dims of a token): q, normalised and scaled,
//      stays in registers as the B operand of S^T = K Q^T; k and v go to LDS;
//   3. attention of the wave's 2 query tiles against the 256 keys
//      (attn_core.hpp), leaving O_h with 8 consecutive dims per lane -- the B
//      operand of the output projection;
//   4. Y^T += Wp[:, head] O_h^T, accumulated over heads in registers.
// Finally the projection bias is added and each token's row is stored at its
// un-shifted position (window reverse + inverse shift).
#include "attn_core.hpp"
#include "launch.hpp"

namespace swin {

namespace {

constexpr int kW16Waves = 8;

template <typename T>
__device__ __forceinline__ vec8<T> to_vec8(const float (&v)[8], float mult) {
  vec8<T> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(v[e] * mult);
  return o;
}

template <typename T, typename QT, int HEADS, bool V2>
__global__ __launch_bounds__(64 * kW16Waves, 1) void fused_w16_kernel(FwdParams p) {
  constexpr int M = 16, N = 256, D = 32;
  constexpr int C = 32 * HEADS;
  constexpr int LDX = C + 8;  // x rows (16-byte padded)
  constexpr int TS = table_stride<M>();
  constexpr int QTL = 2;      // 16-token tiles per wave
  constexpr int NT = 64 * kW16Waves;
  constexpr int CT = C / 16;  // output channel tiles
  __shared__ __attribute__((aligned(16))) T xs[N * LDX];
  __shared__ __attribute__((aligned(16))) T ws[96 * LDX];
  __shared__ __attribute__((aligned(16))) QT ks[N * 32];  // swizzled rows (attn_core.hpp)
  __shared__ __attribute__((aligned(16))) T vs[N * 32];
  __shared__ __attribute__((aligned(16))) float rt4[4 * TS];
  __shared__ __attribute__((aligned(16))) float ninf[8];
  // The head's projection columns Wp[:, h*32 .. +31] in fragment order:
  // fragment c (output channel tile) is 64 lanes x 16 bytes, lane l holding
  // row 32(c/2) + 8(l%16 / 4) + 4(c%2) + l%4, columns h*32 + 8(l/16) .. +7.
  __shared__ __attribute__((aligned(16))) T wps[C / 16 * 512];
  __shared__ float bqs[3 * C], bps[C];  // linear biases

  const Geom& g = p.g;
  const int n_windows = g.B * g.nW;
  int w = blockIdx.x;  // window (persistent: then w + gridDim.x, ...)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, i16 = lane & 15;
  const T* x = static_cast<const T*>(p.x);
  const T* wq = static_cast<const T*>(p.w_qkv);
  const T* wp = static_cast<const T*>(p.w_proj);
  const T* bq = static_cast<const T*>(p.b_qkv);
  const T* bp = static_cast<const T*>(p.b_proj);

  constexpr int XCH = C / 8;  // 16-byte chunks per row
  if (tid < 8) ninf[tid] = -__builtin_inff();
  for (int i = tid; i < 4 * C; i += NT) {
    if (i < 3 * C)
      bqs[i] = bq ? (float)bq[i] : 0.f;
    else
      bps[i - 3 * C] = bp ? (float)bp[i - 3 * C] : 0.f;
  }

  int tile[QTL];
#pragma unroll
  for (int j = 0; j < QTL; ++j) tile[j] = QTL * wave + j;
  const float eps2 = p.eps * p.eps;
  f32x4 yacc[QTL][CT];

  // Weight-row permutation inside a 32-row pair of 16-row tiles: fragment t's
  // row i16 is row 8*(i16/4) + 4t + i16%4, so that output lanes hold 8
  // consecutive channels.
  const int prow0 = 8 * (i16 >> 2) + (i16 & 3);

  // A head's q, k, v weight rows, projection columns and bias-table entries go
  // through registers (loaded during the previous head, stored to LDS at the
  // head's start).
  constexpr int WPT = (96 * XCH + NT - 1) / NT;   // 16-byte weight chunks per thread
  constexpr int PPT = (CT * 64 + NT - 1) / NT;    // 16-byte projection chunks per thread
  // Copy c of the table holds element p + c at position p, so elements
  // 0 .. TS + 2 cover all four: each is loaded once and stored up to 4 times.
  constexpr int TE = TS + 3;
  constexpr int TPT = (TE + NT - 1) / NT;         // table elements per thread
  constexpr int R = 2 * M - 1;
  uint4 wreg[WPT], preg[PPT];
  float treg[TPT];
  auto fetch_head = [&](int hh) {
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int i = tid + k * NT;
      if (i < 96 * XCH) {
        const int r = i / XCH, c = i - r * XCH;
        wreg[k] = gload16(wq + (int64_t)((r >> 5) * C + hh * D + (r & 31)) * C + 8 * c);
      }
    }
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int q = tid + k * NT;
      if (q < CT * 64) {
        const int c = q >> 6, l = q & 63;
        const int row = 32 * (c >> 1) + 8 * ((l & 15) >> 2) + (l & 3) + 4 * (c & 1);
        preg[k] = gload16(wp + (int64_t)row * C + hh * D + 8 * (l >> 4));
      }
    }
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int e = tid + k * NT;
      treg[k] = e < R * R ? p.table[(int64_t)((e / R) * R + (R - 1 - e % R)) * HEADS + hh] * kLog2e
                          : -__builtin_inff();
    }
  };
  auto store_head = [&]() {
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int i = tid + k * NT;
      if (i < 96 * XCH) {
        const int r = i / XCH, c = i - r * XCH;
        *reinterpret_cast<uint4*>(&ws[r * LDX + 8 * c]) = wreg[k];
      }
    }
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int q = tid + k * NT;
      if (q < CT * 64) *reinterpret_cast<uint4*>(&wps[q * 8]) = preg[k];
    }
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int e = tid + k * NT;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (e - c >= 0 && e - c < TS) rt4[c * TS + e - c] = treg[k];
    }
  };
  // Shift + partition map.  A window's origin (uniform): its image's first
  // token and its first row and column in the shifted frame.  Slot t (chunks
  // of 8 columns x 16 rows) is row (t % 128) / 8, column 8 (t / 128) + t % 8
  // of the window; rows and columns past the image wrap around.
  struct Origin {
    int64_t base;
    int y0, x0;
  };
  auto origin = [&](int win) {
    const int b = (int)fdiv((uint32_t)win, g.dnW);
    const int wl = win - b * g.nW;
    const int wy = (int)fdiv((uint32_t)wl, g.dnWx);
    return Origin{(int64_t)b * g.H * g.W, wy * M + g.s, (wl - wy * g.nWx) * M + g.s};
  };
  auto token = [&](const Origin& o, int t) -> int64_t {
    int yy = o.y0 + ((t & 127) >> 3);
    if (yy >= g.H) yy -= g.H;
    int xx = o.x0 + ((t >> 7) << 3) + (t & 7);
    if (xx >= g.W) xx -= g.W;
    return o.base + (int64_t)__umul24(yy, g.W) + xx;
  };
  // Window rows: chunk c of this thread is row (tid + c*NT) / XCH, 16-byte
  // column (tid + c*NT) % XCH.
  constexpr int CHX = N * XCH / NT;
  static_assert(CHX * NT == N * XCH, "gather split");
  auto x_src = [&](const Origin& o, int c) {
    int i = tid + c * NT;
    asm volatile("" : "+v"(i));  // address computed where it is used, not kept live
    const int r = i / XCH;
    return x + token(o, r) * C + 8 * (i - r * XCH);
  };
  auto x_dst = [&](int c) {
    const int i = tid + c * NT, r = i / XCH;
    return &xs[r * LDX + 8 * (i - r * XCH)];
  };
  fetch_head(0);  // in flight together with the window rows
#pragma unroll
  for (int c = 0; c < CHX; ++c)
    *reinterpret_cast<uint4*>(x_dst(c)) = gload16(x_src(origin(w), c));

  for (; w < n_windows; w += gridDim.x) {
  const int nxt = w + gridDim.x;
  const bool more = nxt < n_windows;
  const Origin org = origin(w), org_n = origin(nxt);
  const int wl = w % g.nW;
  const int wy = wl / g.nWx, wx = wl - (wl / g.nWx) * g.nWx;
  const bool my = g.s > 0 && wy == g.H / M - 1;
  const bool mx = g.s > 0 && wx == g.nWx - 1;
#pragma unroll
  for (int j = 0; j < QTL; ++j)
#pragma unroll
    for (int c = 0; c < CT; ++c) yacc[j][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int h = 0; h < HEADS; ++h) {
    // Every wave is done with the previous head's weights and table (and, at
    // a window's first head, the previous window's rows are all in LDS).
    __syncthreads();
    // 1. This head's q, k, v weight rows and bias-table copies; the next
    //    head's are fetched while this one is computed.
    store_head();
    __syncthreads();

    // 2. q, k, v of the wave's tokens: acc[j][part][t].
    f32x4 acc[QTL][3][2];
#pragma unroll
    for (int j = 0; j < QTL; ++j)
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) acc[j][pt][0] = acc[j][pt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C / 32; ++kk) {
      vec8<T> xf[QTL], wf[3][2];
#pragma unroll
      for (int j = 0; j < QTL; ++j)
        xf[j] = load8(&xs[(16 * tile[j] + i16) * LDX + 32 * kk + 8 * g4]);
#pragma unroll
      for (int pt = 0; pt < 3; ++pt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          wf[pt][t] = load8(&ws[(32 * pt + prow0 + 4 * t) * LDX + 32 * kk + 8 * g4]);
#pragma unroll
      for (int j = 0; j < QTL; ++j)
#pragma unroll
        for (int pt = 0; pt < 3; ++pt)
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[j][pt][t] = mma_16x16x32(wf[pt][t], xf[j], acc[j][pt][t]);
    }
    // Lane: token 16*tile + i16, dims 8*g4 + e of q / k / v.
    float qmult = p.q_mult;
    if constexpr (V2) qmult = kLog2e / fmaxf(p.tau[h], p.tau_min);
    float bias[3][8];
#pragma unroll
    for (int pt = 0; pt < 3; ++pt)
#pragma unroll
      for (int e = 0; e < 8; ++e) bias[pt][e] = bqs[pt * C + h * D + 8 * g4 + e];
    vec8<QT> qf[QTL];
#pragma unroll
    for (int j = 0; j < QTL; ++j) {
      const int row = 16 * tile[j] + i16;
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[j][pt][0][r] + bias[pt][r];
          v[4 + r] = acc[j][pt][1][r] + bias[pt][4 + r];
        }
        float mult = pt == 0 ? qmult : 1.0f;
        if (V2 && pt < 2) {
          // "Swin Transformer V2" summary, How It Works: cosine similarity;
          // 1 / max(|v|, eps) = rsqrt(max(|v|^2, eps^2)).
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
          ss = xor32_sum(xor16_sum(ss));
          mult *= __builtin_amdgcn_rsqf(fmaxf(ss, eps2));
        }
        if (pt == 0)
          qf[j] = to_vec8<QT>(v, mult);
        else if (pt == 1)
          *reinterpret_cast<vec8<QT>*>(&ks[kv_swz(row, g4)]) = to_vec8<QT>(v, mult);
        else
          *reinterpret_cast<vec8<T>*>(&vs[kv_swz(row, g4)]) = to_vec8<T>(v, 1.0f);
      }
    }
    __syncthreads();

    // The next head's (or the next window's first head's) weights and table
    // are fetched while this one's attention runs.
    const bool last = h + 1 == HEADS;
    if (!last)
      fetch_head(h + 1);
    else if (more)
      fetch_head(0);

    // 3. Attention of the wave's two query tiles.  During the window's last
    //    head (every wave is past its last read of the rows) the next
    //    window's rows go into LDS, one 16-byte chunk per key block or two:
    //    chunk c is loaded at block (c * NB) / CHX and stored when the next
    //    one is loaded.
    constexpr int NB = N / 32;
    uint4 pend = {0, 0, 0, 0};
    auto hook = [&](int kbi) {
      if (!(last && more)) return;
#pragma unroll
      for (int c = 0; c < CHX; ++c) {
        if ((c * NB) / CHX == kbi) {
          // Keep each chunk's load in its own key block (not hoisted together).
          __builtin_amdgcn_sched_barrier(0);
          if (c > 0) *reinterpret_cast<uint4*>(x_dst(c - 1)) = pend;
          pend = gload16(x_src(org_n, c));
        }
      }
    };
    float o[QTL][8];
    // Opaque here, so that the per-block mask values derived from it are
    // computed in the blocks rather than hoisted out of the loops (which
    // runs out of scalar registers).
    int bnd = M - g.s;
    asm volatile("" : "+s"(bnd));
    // Unmasked windows take the fixed-reference pass; masked ones, and the
    // rare item whose row sums outgrow it, the exact lazy one (running the
    // hook twice stores the same rows twice).
    bool done = false;
    if (!(my || mx))
      done = attn_tiles<QT, T, M, QTL, false, KvLayout::kSwizzled>(qf, tile, ks, vs, rt4, ninf,
                                                                   lane, bnd, false, false, o, hook);
    if (!done)
      attn_tiles<QT, T, M, QTL, true, KvLayout::kSwizzled>(qf, tile, ks, vs, rt4, ninf, lane, bnd,
                                                           my, mx, o, hook);
    if (last && more) *reinterpret_cast<uint4*>(x_dst(CHX - 1)) = pend;

    // 4. Y^T += Wp[:, h*32 .. +31] O_h^T (fragments from LDS); the Wp rows of
    //    each channel-tile pair are interleaved like the QKV weight rows.
    vec8<T> of[QTL];
#pragma unroll
    for (int j = 0; j < QTL; ++j) of[j] = to_vec8<T>(o[j], 1.0f);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const vec8<T> wpf = load8(&wps[(c * 64 + lane) * 8]);
#pragma unroll
      for (int j = 0; j < QTL; ++j) yacc[j][c] = mma_16x16x32(wpf, of[j], yacc[j][c]);
    }
  }

  // Projection bias; each token row to its un-shifted position.
  T* y = static_cast<T*>(p.y);
#pragma unroll
  for (int j = 0; j < QTL; ++j) {
    const int64_t dst = token(org, 16 * tile[j] + i16) * C;
#pragma unroll
    for (int cp = 0; cp < CT / 2; ++cp) {
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c0 = 32 * cp + 8 * g4;
        v[r] = yacc[j][2 * cp][r] + bps[c0 + r];
        v[4 + r] = yacc[j][2 * cp + 1][r] + bps[c0 + 4 + r];
      }
      gstore16(y + dst + 32 * cp + 8 * g4, __builtin_bit_cast(uint4, to_vec8<T>(v, 1.0f)));
    }
  }
  }  // windows
}

template <typename T, typename QT, bool V2>
hipError_t w16_heads(const FwdParams& p, hipStream_t st) {
  // Persistent: one workgroup per CU (the LDS holds one), each walking
  // windows with the grid as stride.
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int n = p.g.B * p.g.nW;
  const dim3 grid(n < cus ? n : cus), block(64 * kW16Waves);
  switch (p.g.heads) {
    case 1: hipLaunchKernelGGL((fused_w16_kernel<T, QT, 1, V2>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((fused_w16_kernel<T, QT, 2, V2>), grid, block, 0, st, p); break;
    case 3: hipLaunchKernelGGL((fused_w16_kernel<T, QT, 3, V2>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((fused_w16_kernel<T, QT, 4, V2>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool fused_w16_supported(int M, int C, int heads, int io) {
  return io != kF32 && M == 16 && heads >= 1 && heads <= 4 && C == 32 * heads;
}

hipError_t launch_fused_w16(const FwdParams& p, hipStream_t st) {
  if (!fused_w16_supported(p.g.M, p.g.C, p.g.heads, p.io) || !p.g.chunked)
    return hipErrorInvalidValue;
  if (p.io == kF16) return p.v2 ? w16_heads<h16, h16, true>(p, st) : w16_heads<h16, h16, false>(p, st);
  if (p.v2) return w16_heads<b16, h16, true>(p, st);  // V2: q, k in float16
  return w16_heads<b16, b16, false>(p, st);
}

}  // namespace swin
