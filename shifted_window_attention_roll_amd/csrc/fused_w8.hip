// Whole block forward in one kernel for window sides 7 and 8 with
// C = 32 * heads, heads <= 4, 16-bit I/O.  The window is laid out on an 8 x 8
// grid of slots (slot = 8 * ty + tx; for side 7 the last row and column are
// padding), so that every 16-slot tile is two window rows and the 8 keys a
// lane holds in the attention are one row of 8 columns.
//
// Pages: "Boosting Swin Transformer Speed: Profiling, Mixed Precision, and
// Kernel Fusion Secrets" -- Training Optimization (index maps fused away; QKV,
// bias and softmax fused) and Inference Optimization (the bias table prepared
// once; GEMMs carry their biases; no separate transposes); "Boost Vision
// Transformer with GPU-Friendly Sparsity and Quantization", Section 3.2 /
// Figure 3 (Q/K/V and output projections are GEMMs); "Swin Transformer V2"
// summary, How It Works (cosine attention over tau; relative position bias).
//
// Persistent: a workgroup of `heads` waves walks a strided list of windows.
// Wave h owns head h:
//   1. q, k, v of head h for the 64 slots, as C^T products with the weight rows
//      of each 16-channel tile pair interleaved (a lane ends with 8 consecutive
//      head dims of one slot).  q (normalised and scaled) stays in registers as
//      the B operand of S^T = K Q^T; k and v go to the wave's own LDS rows.
//   2. attention of its 4 query tiles against the 64 keys: two 32-key blocks,
//      an exact max (no online rescale), P in registers as the B operand of
//      O^T = V^T P^T (V^T fragments by transposing LDS reads), row sums from a
//      ones x P^T product.  O overwrites the wave's K rows.
//   -- workgroup barrier: every head's O is in LDS --
//   3. output channels 32h .. 32h+31 of the projection for the 64 slots, plus
//      bias, stored straight to the un-shifted token rows (16 bytes a lane).
// With up to 3 heads a wave keeps its weights (its head's q, k, v rows and its
// 32 projection rows) in registers for the whole kernel and loads the next
// window's token rows right after its attention; with 4 heads it reloads
// weights and rows per window.  A second barrier (after the next window's q)
// keeps the K stores behind every wave's projection reads.
#include "launch.hpp"
#include "w8_core.hpp"

namespace swin {

namespace {

// Waves per SIMD the kernel is compiled for: with up to 3 heads the wave keeps
// all of its weights in registers across windows (2 waves per SIMD at 2 and 3
// heads); with 4 it reloads them per window.
template <int HEADS>
constexpr bool w8_resident() { return HEADS <= 3; }
template <int HEADS>
constexpr int w8_waves_per_simd() { return HEADS == 2 || HEADS == 3 ? 2 : 3; }

template <typename T, typename QT, int HEADS, int MV, bool V2>
__global__ __launch_bounds__(64 * HEADS) __attribute__((amdgpu_waves_per_eu(w8_waves_per_simd<HEADS>())))
void fused_w8_kernel(FwdParams p, int n_windows) {
  constexpr bool RES = w8_resident<HEADS>();
  constexpr int C = 32 * HEADS, D = 32, LDK = kAttnLD;
  constexpr int NT = 64 * HEADS;
  static_assert(MV == 7 || MV == 8, "window side");
  static_assert(sizeof(QT) == sizeof(T), "O reuses the K rows");
  __shared__ __attribute__((aligned(16))) QT ks[HEADS][64 * LDK];  // K, then O (T bits)
  __shared__ __attribute__((aligned(16))) T vs[HEADS][64 * LDK];
  __shared__ __attribute__((aligned(16))) float tabs[HEADS][kTab];
  __shared__ __attribute__((aligned(16))) float lb[4 * C];  // b_q, b_k, b_v, b_proj

  const Geom& g = p.g;
  int w = blockIdx.x;
  if (w >= n_windows) return;  // uniform per workgroup
  const int tid = threadIdx.x, lane = tid & 63;
  const int h = __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's head
  const int g4 = lane >> 4, i16 = lane & 15;
  const T* x = static_cast<const T*>(p.x);
  T* y = static_cast<T*>(p.y);
  const float NEG_INF = -__builtin_inff();

  for (int hh = 0; hh < HEADS; ++hh) fill_w8_table<MV>(tabs[hh], p.table, HEADS, hh, tid, NT);
  {
    const T* bq = static_cast<const T*>(p.b_qkv);
    const T* bp = static_cast<const T*>(p.b_proj);
    for (int i = tid; i < 4 * C; i += NT)
      lb[i] = i < 3 * C ? (bq ? (float)bq[i] : 0.f) : (bp ? (float)bp[i - 3 * C] : 0.f);
  }

  // Lane constants.  Slot 16j + l%16 is window row 2j + qy0, column qx.
  const int qx = i16 & 7, qy0 = i16 >> 3;
  // Interleaved row inside a 32-row pair of 16-row tiles (fragment t adds 4):
  // output lanes then hold 8 consecutive channels.
  const int prow = 8 * (i16 >> 2) + (i16 & 3);
  // Bias of (query tile j, key block b, key column e) = tb_b[32j + e]: row
  // qy - ky + 7, column e - qx + 7 of the reversed table.  With side 7 the key
  // row 7 (block 1, lane group 3) reads the -inf entries.
  lds_f tb0 = (lds_f)&tabs[h][((qy0 - g4 + 7) << 4) + 7 - qx];
  lds_f tb1 = (MV < 8 && g4 == 3) ? (lds_f)&tabs[h][kTabRows] : tb0 - 64;
  // K rows permuted so that lane l receives keys 8(l/16) .. +7 of a block (see
  // attn_core.hpp); V read through transposing loads.
  typedef __attribute__((address_space(3))) const vec8<QT>* lds_q8;
  lds_q8 kl = (lds_q8)&ks[h][prow * LDK + 8 * g4];
  lds_v4s vl = (lds_v4s)&vs[h][(8 * g4 + (i16 >> 2)) * LDK + 8 * (i16 & 3)];
  asm volatile("" : "+v"(tb0), "+v"(tb1), "+v"(kl), "+v"(vl));

  gptr<T> wq = (gptr<T>)p.w_qkv;
  gptr<T> wp = (gptr<T>)p.w_proj;
  auto wq_frags = [&](int pt, vec8<T> (&f)[2][HEADS]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kk = 0; kk < HEADS; ++kk)
        f[t][kk] = gload8(wq + (uint32_t)((pt * C + h * D + prow + 4 * t) * C + 32 * kk + 8 * g4));
  };

  // Source token row of the lane's slot in tile j (cyclic shift + partition).
  // A padding slot (side 7) takes the row of the nearest real slot: its q, k, v
  // are then finite, its keys get weight 0 and its output is not stored.
  auto locate = [&](int win, int (&row)[4]) {
    const int b = (int)fdiv((uint32_t)win, g.dnW);
    const int wl = win - b * g.nW;
    const int wy = (int)fdiv((uint32_t)wl, g.dnWx);
    const int wx = wl - wy * g.nWx;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ty = 2 * j + qy0 < MV ? 2 * j + qy0 : MV - 1;
      const int tx = qx < MV ? qx : MV - 1;
      int yy = wy * MV + ty + g.s;
      if (yy >= g.H) yy -= g.H;
      int xx = wx * MV + tx + g.s;
      if (xx >= g.W) xx -= g.W;
      row[j] = (b * g.H + yy) * g.W + xx;
    }
  };
  vec8<T> xf[4][HEADS];
  auto fetch_x = [&](const int (&row)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int kk = 0; kk < HEADS; ++kk)
        xf[j][kk] = gload8(x + (int64_t)row[j] * C + 32 * kk + 8 * g4);
  };

  auto wp_frags = [&](vec8<T> (&f)[2][HEADS]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kk = 0; kk < HEADS; ++kk)
        f[t][kk] = gload8(wp + (uint32_t)((h * D + prow + 4 * t) * C + 32 * kk + 8 * g4));
  };

  int row[4];
  // Resident weights: q, k, v rows of head h and projection rows 32h .. 32h+31.
  vec8<T> wres[3][2][HEADS], wpres[2][HEADS];
  if constexpr (RES) {
#pragma unroll
    for (int pt = 0; pt < 3; ++pt) wq_frags(pt, wres[pt]);
    wp_frags(wpres);
    locate(w, row);
    fetch_x(row);
  }
  __syncthreads();  // tables and biases

  const float eps2 = p.eps * p.eps;
  float qmult = p.q_mult;
  if constexpr (V2) qmult = kLog2e / fmaxf(p.tau[h], p.tau_min);
  const int bnd = MV - g.s;

  for (; w < n_windows; w += gridDim.x) {
    const int wl = w - (int)fdiv((uint32_t)w, g.dnW) * g.nW;
    const int wy = (int)fdiv((uint32_t)wl, g.dnWx);
    const bool my = g.s > 0 && wy == g.H / MV - 1;
    const bool mx = g.s > 0 && wl - wy * g.nWx == g.nWx - 1;
    if constexpr (!RES) {
      // The weights do not fit in registers across windows: keep their loads
      // inside the loop.
      asm volatile("" : "+s"(wq), "+s"(wp));
      locate(w, row);
      fetch_x(row);
    }

    // ---- 1. q, k, v of head h -----------------------------------------------
    vec8<QT> qf[4];
#pragma unroll
    for (int pt = 0; pt < 3; ++pt) {
      vec8<T> wf[2][HEADS];
      if constexpr (RES) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int kk = 0; kk < HEADS; ++kk) wf[t][kk] = wres[pt][t][kk];
      } else {
        wq_frags(pt, wf);
      }
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(&lb[pt * C + h * D + 8 * g4]);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(&lb[pt * C + h * D + 8 * g4 + 4]);
      f32x4 acc[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[0][j] = b0;
        acc[1][j] = b1;
      }
#pragma unroll
      for (int kk = 0; kk < HEADS; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[t][j] = mma_16x16x32(wf[t][kk], xf[j][kk], acc[t][j]);
      // Lane: slot 16j + l%16, head dims 8g + e (e = 4t + r).
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float mult = pt == 0 ? qmult : 1.0f;
        if (V2 && pt < 2) {
          // "Swin Transformer V2" summary, How It Works: cosine similarity;
          // 1 / max(|v|, eps) = rsqrt(max(|v|^2, eps^2)).
          float ss = 0.f;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) ss = fmaf(acc[t][j][r], acc[t][j][r], ss);
          ss = xor32_sum(xor16_sum(ss));
          mult *= __builtin_amdgcn_rsqf(fmaxf(ss, eps2));
        }
        if (pt == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[j][e] = from_f32<QT>(acc[e >> 2][j][e & 3] * mult);
        } else {
          vec8<T> v;
          vec8<QT> k;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            k[e] = from_f32<QT>(acc[e >> 2][j][e & 3] * mult);
            v[e] = from_f32<T>(acc[e >> 2][j][e & 3]);
          }
          if (pt == 1)
            store8(&ks[h][(16 * j + i16) * LDK + 8 * g4], k);
          else
            store8(&vs[h][(16 * j + i16) * LDK + 8 * g4], v);
        }
      }
      // Every wave's projection has read the previous window's O (which lives
      // in the K rows) before any K row is overwritten.
      if (pt == 0) __syncthreads();
    }
    // The wave reads back only rows it wrote itself (LDS is in order per wave).
    asm volatile("" ::: "memory");

    // ---- 2. attention of head h ---------------------------------------------
    vec8<QT> kf[2][2];
    vec8<T> vf[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        kf[b][t] = kl[(32 * b + 4 * t) * LDK / 8];
        vf[b][t] = vt_frag<T>(vl, 32 * b, t);
      }
    // O of query tile j into the wave's K rows (their fragments are all in
    // registers already).
    T* os = reinterpret_cast<T*>(ks[h]) + i16 * LDK + 8 * g4;
    auto store_o = [&](int j, const vec8<T>& of) { store8(os + 16 * j * LDK, of); };
    if (my || mx)
      w8_attend<QT, T, MV, true, false>(qf, kf, vf, tb0, tb1, qy0, qx, g4, bnd, my, mx, store_o);
    else if (!w8_attend<QT, T, MV, false, true>(qf, kf, vf, tb0, tb1, qy0, qx, g4, bnd, false,
                                                  false, store_o))
      // Some row outgrew the zero reference: redo with exact row maxima.
      w8_attend<QT, T, MV, false, false>(qf, kf, vf, tb0, tb1, qy0, qx, g4, bnd, false, false,
                                           store_o);
    // The next window's token rows, in flight across the barrier and the
    // projection.
    int cur[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cur[j] = row[j];
    if constexpr (RES) {
      const int nxt = w + gridDim.x;
      if (nxt < n_windows) {
        locate(nxt, row);
        fetch_x(row);
      }
    }
    // Projection weights of output channels 32h .. 32h+31 (reloaded: in flight
    // across the barrier).
    vec8<T> wpf[2][HEADS];
    if constexpr (RES) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kk = 0; kk < HEADS; ++kk) wpf[t][kk] = wpres[t][kk];
    } else {
      wp_frags(wpf);
    }
    __syncthreads();  // every head's O in LDS

    // ---- 3. projection, output channels 32h .. 32h+31 ------------------------
    const f32x4 pb0 = *reinterpret_cast<const f32x4*>(&lb[3 * C + h * D + 8 * g4]);
    const f32x4 pb1 = *reinterpret_cast<const f32x4*>(&lb[3 * C + h * D + 8 * g4 + 4]);
    f32x4 ya[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ya[0][j] = pb0;
      ya[1][j] = pb1;
    }
#pragma unroll
    for (int kk = 0; kk < HEADS; ++kk) {
      const T* ok = reinterpret_cast<const T*>(ks[kk]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const vec8<T> o8 = load8(&ok[(16 * j + i16) * LDK + 8 * g4]);
#pragma unroll
        for (int t = 0; t < 2; ++t) ya[t][j] = mma_16x16x32(wpf[t][kk], o8, ya[t][j]);
      }
    }
    // Lane: channels 32h + 8g + e of slot 16j + l%16, to its un-shifted row.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (2 * j + qy0 >= MV || qx >= MV) continue;  // padding slot
      vec8<T> v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = from_f32<T>(ya[e >> 2][j][e & 3]);
      gstore16(y + (int64_t)cur[j] * C + h * D + 8 * g4, __builtin_bit_cast(uint4, v));
    }
  }
}

template <typename T, typename QT, int MV, bool V2>
hipError_t w8_heads(const FwdParams& p, int cus, hipStream_t st) {
  const int n = p.g.B * p.g.nW;
  const int heads = p.g.heads;
  // Resident workgroups per CU: LDS (K, V, table per head + biases), and at
  // most 12 waves.
  const int lds = heads * (2 * 64 * kAttnLD * 2 + kTab * 4) + 16 * 32 * heads;
  int per_cu = (160 * 1024) / lds;
  const int wave_cap = 4 * (heads == 2 || heads == 3 ? 2 : 3) / heads;  // w8_waves_per_simd
  per_cu = per_cu > wave_cap ? wave_cap : (per_cu < 1 ? 1 : per_cu);
  const int grid = n < cus * per_cu ? n : cus * per_cu;
  const dim3 block(64 * heads);
  switch (heads) {
    case 1: hipLaunchKernelGGL((fused_w8_kernel<T, QT, 1, MV, V2>), dim3(grid), block, 0, st, p, n); break;
    case 2: hipLaunchKernelGGL((fused_w8_kernel<T, QT, 2, MV, V2>), dim3(grid), block, 0, st, p, n); break;
    case 3: hipLaunchKernelGGL((fused_w8_kernel<T, QT, 3, MV, V2>), dim3(grid), block, 0, st, p, n); break;
    case 4: hipLaunchKernelGGL((fused_w8_kernel<T, QT, 4, MV, V2>), dim3(grid), block, 0, st, p, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, typename QT, bool V2>
hipError_t w8_side(const FwdParams& p, int cus, hipStream_t st) {
  return p.g.M == 7 ? w8_heads<T, QT, 7, V2>(p, cus, st) : w8_heads<T, QT, 8, V2>(p, cus, st);
}

}  // namespace

bool fused_w8_supported(int M, int C, int heads, int io) {
  return io != kF32 && (M == 7 || M == 8) && heads >= 1 && heads <= 4 && C == 32 * heads;
}

hipError_t launch_fused_w8(const FwdParams& p, hipStream_t st) {
  if (!fused_w8_supported(p.g.M, p.g.C, p.g.heads, p.io)) return hipErrorInvalidValue;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (p.io == kF16) return p.v2 ? w8_side<h16, h16, true>(p, cus, st) : w8_side<h16, h16, false>(p, cus, st);
  if (p.v2) return w8_side<b16, h16, true>(p, cus, st);  // V2: q, k in float16
  return w8_side<b16, b16, false>(p, cus, st);
}

}  // namespace swin
