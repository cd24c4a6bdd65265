// Whole block forward in one kernel for window side 16 (N = 256 tokens) and up
// to 4 heads (C = 32 * heads <= 128), 16-bit I/O: nothing but x, the weights
// and y touch HBM.
//
// Pages: "Boosting Swin Transformer Speed: Profiling, Mixed Precision, and
// Kernel Fusion Secrets" -- Training Optimization (the index maps fused away;
// QKV, bias and softmax fused) and Inference Optimization (GEMMs carry their
// biases, no separate transposes); "Boost Vision Transformer with
// GPU-Friendly Sparsity and Quantization", Section 3.2 / Figure 3 (Q/K/V and
// output projections are GEMMs); "Swin Transformer V2" summary, How It Works
// (cosine attention over tau, continuous position bias).
//
// Persistent workgroups (as many per CU as the LDS holds) walk the windows;
// the heads run side by side, 2 waves each.  Wave w serves head w / 2 and the
// query tiles 8 (w % 2) .. +7 (16 window slots each, chunked slot order, see
// Geom):
//   1. the window's token rows, gathered through the cyclic shift, go to LDS
//      (coalesced 16-byte loads, every thread a share);
//   2. k, v, then q of its head for its 128 slots as C^T products: W_qkv
//      fragments from global memory (the weight rows of each 16-channel tile
//      pair interleaved, so a lane holds 8 consecutive head dims of a token),
//      x fragments from LDS; k and v go to the head's LDS rows (over the x
//      rows, after a barrier), q (normalised and scaled in V2) stays in
//      registers;
//   3. attention of its query tiles, two at a time (attn_core.hpp), against
//      the head's 256 keys;
//   4. O of every head goes to LDS as [slot][C] rows, W_proj next to it; each
//      wave projects whole slots (Y^T = W_proj O^T over all C channels) and
//      stores each token's row at its un-shifted position.
// The softmax reference is fixed (see attn_core.hpp); a wave whose row-sum
// check fails flags the window (one flag per wave, always written) and the
// redo launch recomputes the flagged windows on the exact lazy pass.
#include "attn_core.hpp"
#include "launch.hpp"

namespace swin {

namespace {

template <typename T>
__device__ __forceinline__ vec8<T> to_vec8(const float (&v)[8], float mult) {
  vec8<T> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(v[e] * mult);
  return o;
}

constexpr int kW16WPH = 2;             // waves per head
constexpr int kW16TPW = 16 / kW16WPH;  // query tiles per wave

// Workgroups that fit on one CU (LDS: K and V plus the bias table per head).
template <int HEADS>
constexpr int w16_per_cu() {
  constexpr int lds = HEADS * (2 * 256 * 32 * 2 + table1_size<16>() * 4) + 2048;
  return 160 * 1024 / lds > 0 ? 160 * 1024 / lds : 1;
}

template <typename T, typename QT, int HEADS, bool V2, bool REDO>
__device__ __forceinline__ void w16_body(const FwdParams& p, int* flags) {
  constexpr int M = 16, N = 256, D = 32;
  constexpr int C = 32 * HEADS, WAVES = kW16WPH * HEADS, NT = 64 * WAVES;
  constexpr int TSZ = table1_size<M>();
  constexpr int KS = C / 32;      // 32-channel steps of the products over C
  constexpr int LDO = C + 8;      // O / W_proj row pitch in LDS (16-byte padded)
  constexpr int AQ = 2;  // query tiles per attention pass
  constexpr bool ZREF = V2 && !__is_same(T, h16);  // zero softmax reference
  // K and V of each head (QT / T rows of 32, swizzled, kv_frag.hpp); after
  // the attention, O [N][LDO] and W_proj [C][LDO] in the same bytes.
  __shared__ __attribute__((aligned(16))) char kv[HEADS * 2 * N * D * 2];
  __shared__ __attribute__((aligned(16))) float rt[HEADS][TSZ];
  __shared__ __attribute__((aligned(16))) float ninf[8];
  __shared__ float red[WAVES];
  __shared__ __attribute__((aligned(16))) float bqs[3 * C], bps[C];  // linear biases
  static_assert((N + C) * LDO * 2 <= HEADS * 2 * N * D * 2 || HEADS == 1, "O + W_proj fit");
  static_assert(N * LDO * 2 <= HEADS * 2 * N * D * 2, "x rows fit");
  T* xs = reinterpret_cast<T*>(kv);  // the window's x rows [N][LDO], phase 1 only
  T* os = reinterpret_cast<T*>(kv);
  T* wps = reinterpret_cast<T*>(kv + N * LDO * 2);
  constexpr int LDX = LDO;
  constexpr int XCH = C / 8;         // 16-byte chunks per x row
  constexpr int XPT = N * XCH / NT;  // of them per thread
  static_assert(N * XCH % NT == 0, "x staging split");

  const Geom& g = p.g;
  const int n_windows = g.B * g.nW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = wave / kW16WPH;  // this wave's head
  int tile[kW16TPW];
#pragma unroll
  for (int j = 0; j < kW16TPW; ++j) tile[j] = kW16TPW * (wave % kW16WPH) + j;
  const T* x = static_cast<const T*>(p.x);
  const T* wq = static_cast<const T*>(p.w_qkv);
  const T* wp = static_cast<const T*>(p.w_proj);
  const T* bq = static_cast<const T*>(p.b_qkv);
  const T* bp = static_cast<const T*>(p.b_proj);
  T* y = static_cast<T*>(p.y);
  const float eps2 = p.eps * p.eps;

  if constexpr (REDO) {
    // Nothing to do unless one of this workgroup's windows is flagged.
    int any = 0;
    const int mine = (n_windows - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;
    for (int i = threadIdx.x; i < mine * WAVES; i += NT)
      any |= flags[(blockIdx.x + (i / WAVES) * gridDim.x) * WAVES + i % WAVES];
    if (!__syncthreads_or(any)) return;
  }
  // Every head's reversed bias table (cosine attention with bfloat16 P: each
  // shifted by its logit bound minus kZeroTop, see attn_core.hpp).
  if (threadIdx.x < 8) ninf[threadIdx.x] = -__builtin_inff();
  for (int i = threadIdx.x; i < 4 * C; i += NT) {
    if (i < 3 * C)
      bqs[i] = bq ? (float)bq[i] : 0.f;
    else
      bps[i - 3 * C] = bp ? (float)bp[i - 3 * C] : 0.f;
  }
  for (int h = 0; h < HEADS; ++h) fill_bias_table<M>(rt[h], p.table, HEADS, h, threadIdx.x, NT);
  if constexpr (ZREF) {
    __syncthreads();
    const int lane = threadIdx.x & 63;
    for (int h = 0; h < HEADS; ++h) {
      float bmax = -__builtin_inff();
      for (int e = threadIdx.x; e < TSZ; e += NT) bmax = fmaxf(bmax, rt[h][e]);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, d));
      if (lane == 0) red[wave] = bmax;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < WAVES; ++w) bmax = fmaxf(bmax, red[w]);
      const float qm = kLog2e / fmaxf(p.tau[h], p.tau_min);
      const float shift = qm * (1.0f + 1.0f / 256.0f) + bmax - kZeroTop;
      __syncthreads();
      for (int e = threadIdx.x; e < TSZ; e += NT) rt[h][e] -= shift;
    }
  }

  for (int win = blockIdx.x; win < n_windows; win += gridDim.x) {
    if constexpr (REDO) {
      int any = 0;
      for (int w = 0; w < WAVES; ++w) any |= flags[win * WAVES + w];
      if (__builtin_amdgcn_readfirstlane(any) == 0) continue;
    }
    // Per-lane values derived anew per window from an opaque thread index, so
    // that they are not kept live through the attention.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, g4 = lane >> 4, i16 = lane & 15;
    const int bi = (int)fdiv((uint32_t)win, g.dnW);
    const int wl = win - bi * g.nW;
    const int wy = (int)fdiv((uint32_t)wl, g.dnWx);
    const int wx = wl - wy * g.nWx;
    const bool my = g.s > 0 && wy == g.H / M - 1;
    const bool mx = g.s > 0 && wx == g.nWx - 1;
    // Token of slot t: window row (t % 128) / 8, column 8 (t / 128) + t % 8,
    // through the cyclic shift.
    auto token = [&](int t) -> uint32_t {
      int yy = wy * M + g.s + ((t & 127) >> 3);
      if (yy >= g.H) yy -= g.H;
      int xx = wx * M + g.s + ((t >> 7) << 3) + (t & 7);
      if (xx >= g.W) xx -= g.W;
      return (uint32_t)((bi * g.H + yy) * g.W + xx);
    };
    // Weight-row permutation inside a 32-row pair of 16-row fragments:
    // fragment t's row i16 is row 8 (i16 / 4) + 4t + i16 % 4, so output lanes
    // hold 8 consecutive channels.
    const int prow0 = 8 * (i16 >> 2) + (i16 & 3);
    auto wrow = [&](int pt, int t) {  // W_qkv row of part pt, fragment t
      return wq + (size_t)(pt * C + hh * D + prow0 + 4 * t) * C + 8 * g4;
    };
    // A part's weight fragments for all KS steps, in flight together.
    vec8<T> wf[KS][2];
    auto load_w = [&](int pt) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int t = 0; t < 2; ++t) wf[kk][t] = gload8(wrow(pt, t) + 32 * kk);
    };
    // Every wave is past its last read of the previous window's LDS.
    __syncthreads();

    // 1. The window's token rows, gathered through the cyclic shift, into LDS
    // (in the bytes that K and V take later): row t of xs is slot t.
    {
      uint4 xr[XPT];
#pragma unroll
      for (int k = 0; k < XPT; ++k) {
        const int i = tid + k * NT, t = i / XCH, c = i - t * XCH;
        xr[k] = gload16(x + (size_t)token(t) * C + 8 * c);
      }
      load_w(1);
#pragma unroll
      for (int k = 0; k < XPT; ++k) {
        const int i = tid + k * NT, t = i / XCH, c = i - t * XCH;
        *reinterpret_cast<uint4*>(&xs[t * LDX + 8 * c]) = xr[k];
      }
    }
    __syncthreads();

    // 2. k, v, then q of head hh for the wave's query tiles as C^T products
    // (weights from global memory, x fragments from LDS), with the bias; k
    // (and q) normalised in V2, q scaled.
    // Products of tiles j0, j0 + 1 with the loaded part, plus its bias.
    auto part2 = [&](int pt, int j0, float (&v)[2][8]) {
      f32x4 acc[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const vec8<T> xf = *reinterpret_cast<const vec8<T>*>(
              &xs[(16 * tile[j0 + j] + i16) * LDX + 32 * kk + 8 * g4]);
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[j][t] = mma_16x16x32(wf[kk][t], xf, acc[j][t]);
        }
      float bias[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) bias[e] = bqs[pt * C + hh * D + 8 * g4 + e];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[j][r] = acc[j][0][r] + bias[r];
          v[j][4 + r] = acc[j][1][r] + bias[4 + r];
        }
    };
    // "Swin Transformer V2" summary, How It Works: cosine similarity;
    // 1 / max(|v|, eps) = rsqrt(max(|v|^2, eps^2)) over the head's 32 dims
    // (8 per lane, 4 lanes).
    auto inv_norm = [&](const float (&v)[8]) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
      ss = xor32_sum(xor16_sum(ss));
      return __builtin_amdgcn_rsqf(fmaxf(ss, eps2));
    };
    float qmult = p.q_mult;
    if constexpr (V2) qmult = kLog2e / fmaxf(p.tau[hh], p.tau_min);
    vec8<QT> kf[kW16TPW], qf[kW16TPW];
    vec8<T> vf[kW16TPW];
#pragma unroll
    for (int pt = 1; pt < 4; ++pt) {  // k, v, q (part 0 last)
      const int part = pt & 3 ? pt : 0;
      if (pt > 1) load_w(part == 3 ? 0 : part);
#pragma unroll
      for (int j0 = 0; j0 < kW16TPW; j0 += 2) {
        float v[2][8];
        part2(part == 3 ? 0 : part, j0, v);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (pt == 1) kf[j0 + j] = to_vec8<QT>(v[j], V2 ? inv_norm(v[j]) : 1.0f);
          if (pt == 2) vf[j0 + j] = to_vec8<T>(v[j], 1.0f);
          if (pt == 3) qf[j0 + j] = to_vec8<QT>(v[j], V2 ? qmult * inv_norm(v[j]) : qmult);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // every wave is done with x
    {
      QT* ks = reinterpret_cast<QT*>(kv + hh * 2 * N * D * 2);
      T* vs = reinterpret_cast<T*>(kv + hh * 2 * N * D * 2 + N * D * 2);
#pragma unroll
      for (int j = 0; j < kW16TPW; ++j) {
        const int row = 16 * tile[j] + i16;
        *reinterpret_cast<vec8<QT>*>(&ks[kv_swz(row, g4)]) = kf[j];
        *reinterpret_cast<vec8<T>*>(&vs[kv_swz(row, g4)]) = vf[j];
      }
    }
    __syncthreads();  // every head's K and V complete

    // 3. Attention, AQ query tiles at a time, on a fixed reference (the zero
    // reference with cosine attention and bfloat16 P, else block 0's row max
    // for unmasked windows and each tile's own-block row max for masked ones);
    // REDO: the exact lazy pass.
    const QT* ksh = reinterpret_cast<const QT*>(kv + hh * 2 * N * D * 2);
    const T* vsh = reinterpret_cast<const T*>(kv + hh * 2 * N * D * 2 + N * D * 2);
    vec8<T> ov[kW16TPW];
    bool done = true;
#pragma unroll
    for (int pr = 0; pr < kW16TPW / AQ; ++pr) {
      vec8<QT> q2[AQ];
      int t2[AQ];
#pragma unroll
      for (int j = 0; j < AQ; ++j) {
        q2[j] = qf[AQ * pr + j];
        t2[j] = tile[AQ * pr + j];
      }
      float o[AQ][8];
      bool ok = true;
      if constexpr (REDO) {
        attn_tiles<QT, T, M, AQ, true, KvLayout::kSwizzled, TableMode::kTable1, RefMode::kLazy>(
            q2, t2, ksh, vsh, rt[hh], ninf, lane, M - g.s, my, mx, o);
      } else if (!(my || mx)) {
        ok = attn_tiles<QT, T, M, AQ, false, KvLayout::kSwizzled, TableMode::kTable1,
                        ZREF ? RefMode::kZero : RefMode::kBlock0>(q2, t2, ksh, vsh, rt[hh], ninf,
                                                                  lane, M - g.s, false, false, o);
      } else {
        ok = attn_tiles<QT, T, M, AQ, true, KvLayout::kSwizzled, TableMode::kTable1,
                        ZREF ? RefMode::kZero : RefMode::kOwn>(q2, t2, ksh, vsh, rt[hh], ninf,
                                                               lane, M - g.s, my, mx, o);
      }
      done = done && ok;
#pragma unroll
      for (int j = 0; j < AQ; ++j) ov[AQ * pr + j] = to_vec8<T>(o[j], 1.0f);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!REDO) {
      // One flag per wave, always written.
      if (lane == 0) flags[win * WAVES + wave] = done ? 0 : 1;
    }
    __syncthreads();  // every wave is done with K and V

    // 4. O rows (the lane's 8 dims of head hh) and W_proj into LDS, then the
    // projection of whole slot tiles: wave w takes tiles w, w + WAVES, ...
#pragma unroll
    for (int j = 0; j < kW16TPW; ++j)
      *reinterpret_cast<vec8<T>*>(&os[(16 * tile[j] + i16) * LDO + hh * D + 8 * g4]) = ov[j];
    for (int e = tid; e < C * C / 8; e += NT) {
      const int r = e / (C / 8), c8 = e - r * (C / 8);
      *reinterpret_cast<uint4*>(&wps[r * LDO + 8 * c8]) = gload16(wp + (size_t)r * C + 8 * c8);
    }
    __syncthreads();
    constexpr int CT = C / 16;  // output channel tiles
    for (int yt = wave; yt < 16; yt += WAVES) {
      f32x4 acc[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const vec8<T> of = *reinterpret_cast<const vec8<T>*>(&os[(16 * yt + i16) * LDO + 32 * kk + 8 * g4]);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          // Rows of each channel-tile pair interleaved like the QKV weights.
          const int row = 32 * (c >> 1) + prow0 + 4 * (c & 1);
          const vec8<T> wf = *reinterpret_cast<const vec8<T>*>(&wps[row * LDO + 32 * kk + 8 * g4]);
          acc[c] = mma_16x16x32(wf, of, acc[c]);
        }
      }
      // Projection bias; the token row at its un-shifted position.
      const size_t dst = (size_t)token(16 * yt + i16) * C;
#pragma unroll
      for (int cp = 0; cp < CT / 2; ++cp) {
        const int c0 = 32 * cp + 8 * g4;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bps[c0 + e];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] += acc[2 * cp][r];
          v[4 + r] += acc[2 * cp + 1][r];
        }
        gstore16(y + dst + c0, __builtin_bit_cast(uint4, to_vec8<T>(v, 1.0f)));
      }
    }
  }
}

template <typename T, typename QT, int HEADS, bool V2>
__global__ __launch_bounds__(64 * kW16WPH * HEADS)
__attribute__((amdgpu_waves_per_eu((kW16WPH * HEADS + 3) / 4, (kW16WPH * HEADS + 3) / 4)))
void fused_w16_kernel(FwdParams p, int* flags) {
  w16_body<T, QT, HEADS, V2, false>(p, flags);
}

template <typename T, typename QT, int HEADS, bool V2>
__global__ __launch_bounds__(64 * kW16WPH * HEADS)
__attribute__((amdgpu_waves_per_eu((kW16WPH * HEADS + 3) / 4, (kW16WPH * HEADS + 3) / 4)))
void fused_w16_redo_kernel(FwdParams p, int* flags) {
  w16_body<T, QT, HEADS, V2, true>(p, flags);
}

template <typename T, typename QT, bool V2, int HEADS>
hipError_t w16_launch(const FwdParams& p, int* flags, bool redo, hipStream_t st) {
  // Persistent: as many workgroups per CU as its LDS holds, each walking the
  // windows with the grid as stride.
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int n = p.g.B * p.g.nW, slots = cus * w16_per_cu<HEADS>();
  const dim3 grid(n < slots ? n : slots), block(64 * kW16WPH * HEADS);
  if (redo)
    hipLaunchKernelGGL((fused_w16_redo_kernel<T, QT, HEADS, V2>), grid, block, 0, st, p, flags);
  else
    hipLaunchKernelGGL((fused_w16_kernel<T, QT, HEADS, V2>), grid, block, 0, st, p, flags);
  return hipGetLastError();
}

template <typename T, typename QT, bool V2>
hipError_t w16_heads(const FwdParams& p, int* flags, bool redo, hipStream_t st) {
  switch (p.g.heads) {
    case 1: return w16_launch<T, QT, V2, 1>(p, flags, redo, st);
    case 2: return w16_launch<T, QT, V2, 2>(p, flags, redo, st);
    case 3: return w16_launch<T, QT, V2, 3>(p, flags, redo, st);
    case 4: return w16_launch<T, QT, V2, 4>(p, flags, redo, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool fused_w16_supported(int64_t tokens, int M, int C, int heads, int io) {
  // Token rows are addressed with 32-bit element offsets.
  return io != kF32 && M == 16 && heads >= 1 && heads <= 4 && C == 32 * heads &&
         tokens * C < ((int64_t)1 << 31);
}

int64_t fused_w16_flag_count(int heads, int64_t windows) { return windows * kW16WPH * heads; }

hipError_t launch_fused_w16(const FwdParams& p, int* flags, bool redo, hipStream_t st) {
  const int64_t tokens = (int64_t)p.g.B * p.g.H * p.g.W;
  if (!fused_w16_supported(tokens, p.g.M, p.g.C, p.g.heads, p.io) || !p.g.chunked || !flags)
    return hipErrorInvalidValue;
  if (p.io == kF16)
    return p.v2 ? w16_heads<h16, h16, true>(p, flags, redo, st)
                : w16_heads<h16, h16, false>(p, flags, redo, st);
  if (p.v2) return w16_heads<b16, h16, true>(p, flags, redo, st);  // V2: q, k in float16
  return w16_heads<b16, b16, false>(p, flags, redo, st);
}

}  // namespace swin
