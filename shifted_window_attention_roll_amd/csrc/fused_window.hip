// Whole forward in one kernel for small windows (N = M*M <= 64) and few heads
// (C = 32 * HEADS, HEADS <= 4).  Persistent: each workgroup walks a strided list
// of windows; per window it runs three phases separated by workgroup barriers.
//
// Pages: "Boosting Swin Transformer Speed: Profiling, Mixed Precision, and Kernel
// Fusion Secrets" -- Training Optimization (the index maps fused away to save
// launches and global traffic; QKV GEMM + bias + softmax fused) and Inference
// Optimization (invariant data pre-processed once; no separate transposes);
// "Boost Vision Transformer with GPU-Friendly Sparsity and Quantization",
// Section 3.2 / Figure 3 (Q/K/V and output projections are GEMMs); "Swin
// Transformer V2" summary, How It Works (relative position bias; cosine / tau).
//
// All products are 16x16x32 matrix-core steps (lane l supplies row / column l%16
// and the K-slice 8*(l/16)..+7; results land as column l%16, rows 4*(l/16)..+3).
//   Phase 1, QKV.  The window's token rows are gathered straight from x through
//     the cyclic shift into registers (fetched during the previous window's
//     phase 3).  Work items are (q|k|v, head) blocks of 32 channels.  q and k
//     are computed transposed (W X^T), so a lane holds 4 consecutive head dims
//     of one token: V2 normalises them with a 4-lane-group reduction, and they
//     are stored as 8-byte rows of Q / K.  v is computed as X W^T and stored as
//     8-byte runs of tokens of V^T.  Accumulators start from the linear biases.
//   Phase 2, attention.  Work items are (head, 16-query tile).  S^T = K Q^T with
//     the K rows permuted so that lane l ends up with query l%16 and the 8
//     consecutive keys 8*(l/16)..+7 of each 32-key block; the relative position
//     bias (times log2 e; -inf for padded keys, from the table's upper half; -inf
//     across shifted-window regions) is the accumulator's initial value.  The
//     base-2 softmax stays in that lane, P is the B operand of O^T = V^T P^T, and
//     one more MFMA (ones times P) gives the row sums of exactly the rounded P.
//     O overwrites the Q slots the item read.
//   Phase 3, output projection Y^T = Wp O^T per 16-channel tile, plus bias,
//     staged in LDS as token rows and written with 16-byte stores to the
//     un-shifted positions (window reverse + inverse shift).
#include "common.hpp"
#include "launch.hpp"

namespace swin {

namespace {

constexpr int kD = 32;
constexpr int kTabSmall = 15 * 15;  // (2M-1)^2 for M <= 8

// Four consecutive elements of T at p (8 bytes for 16-bit types, 16 for float).
template <typename T>
__device__ __forceinline__ void store4(T* p, const f32x4& v, float scale) {
  if constexpr (sizeof(T) == 2) {
    typedef T v4 __attribute__((ext_vector_type(4)));
    v4 o = {from_f32<T>(v[0] * scale), from_f32<T>(v[1] * scale), from_f32<T>(v[2] * scale),
            from_f32<T>(v[3] * scale)};
    *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, o);
  } else {
    *reinterpret_cast<f32x4*>(p) = v * scale;
  }
}

template <int HEADS>
constexpr int waves_for() { return HEADS == 3 ? 3 : 4; }

template <typename T, typename QT, int HEADS, int KT, bool V2>
__global__ __launch_bounds__(64 * waves_for<HEADS>(), 3)
void fused_window_kernel(FwdParams p, int n_windows) {
  constexpr int WAVES = waves_for<HEADS>();
  constexpr int NT = 64 * WAVES;
  constexpr int C = 32 * HEADS;
  constexpr int NP = 16 * KT;                       // padded window tokens (32 or 64)
  constexpr int LDQ = C + 16 / (int)sizeof(T);      // row pitch of Q / K / O / Y (elements)
  constexpr int LDV = NP + 16 / (int)sizeof(T);     // row pitch of V^T
  constexpr int EPC = 16 / (int)sizeof(T);          // elements per 16-byte chunk
  constexpr int CPR = C / EPC;                      // chunks per token row
  constexpr int PF = (NP * CPR + NT - 1) / NT;      // y-store chunks per thread
  static_assert(sizeof(QT) == sizeof(T), "q/k and v storage share a pitch");
  __shared__ T qs[NP * LDQ];                        // Q (QT bits), then O
  __shared__ T ks[NP * LDQ];                        // K (QT bits), then Y staging
  __shared__ T vt[C * LDV];                         // V^T
  __shared__ float tab[HEADS][2 * kTabSmall];       // bias * log2(e), then -inf
  __shared__ float lb[4 * C];                       // b_q, b_k, b_v, b_proj
  __shared__ int koff_s[4][NP];                     // see koffb below

  const Geom g = p.g;
  const int N = g.N, M = g.M;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int g4 = lane >> 4, i16 = lane & 15;
  const int n2 = 2 * M - 1;
  const int nrel = n2 * n2;
  const T* x = static_cast<const T*>(p.x);
  T* y = static_cast<T*>(p.y);
  const T* wq = static_cast<const T*>(p.w_qkv);
  const T* wp = static_cast<const T*>(p.w_proj);
  const float NEG_INF = -__builtin_inff();

  // Window w -> image and shifted-frame origin (uniform per workgroup).
  struct WinPos { int b, y0, x0; };
  auto win_pos = [&](int w) {
    const int b = w / g.nW;
    const int wl = w - b * g.nW;
    const int wy = wl / g.nWx;
    return WinPos{b, wy * M, (wl - wy * g.nWx) * M};
  };
  // Original-frame row of token (ty, tx) (packed ty << 8 | tx) of a window:
  // the cyclic shift reads ((y0+ty+s) mod H, (x0+tx+s) mod W).
  auto src_row = [&](const WinPos& wpos, int yx) -> int64_t {
    int yy = wpos.y0 + (yx >> 8) + g.s;
    if (yy >= g.H) yy -= g.H;
    int xx = wpos.x0 + (yx & 255) + g.s;
    if (xx >= g.W) xx -= g.W;
    return ((int64_t)wpos.b * g.H + yy) * g.W + xx;
  };
  auto pack_yx = [&](int t) { return t < N ? ((t / M) << 8) | (t - (t / M) * M) : -1; };

  // X fragments of this lane: token 16j + (l%16), channels 32ks + 8g .. +7.
  int tok_yx[KT];
#pragma unroll
  for (int j = 0; j < KT; ++j) tok_yx[j] = pack_yx(16 * j + i16);
  vec8<T> xf[KT][HEADS];
  auto fetch_x = [&](int w) {
    const WinPos wpos = win_pos(w);
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const bool ok = tok_yx[j] >= 0;
      const T* row = x + (ok ? src_row(wpos, tok_yx[j]) * C : 0) + g4 * 8;
#pragma unroll
      for (int k = 0; k < HEADS; ++k) {
        xf[j][k] = ok ? gload8(row + k * 32) : vec8<T>{};
      }
    }
  };
  // y-store slots of this thread (chunk tid + k*NT of the NP x CPR tile).
  int slot_yx[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int i = tid + k * NT;
    slot_yx[k] = i < NP * CPR ? pack_yx(i / CPR) : -1;
  }

  int w = blockIdx.x;
  if (w >= n_windows) return;  // uniform per workgroup
  fetch_x(w);
  for (int i = tid; i < HEADS * 2 * kTabSmall; i += NT) {
    const int hh = i / (2 * kTabSmall), r = i - hh * (2 * kTabSmall);
    tab[hh][r] = r < nrel ? p.table[(int64_t)r * HEADS + hh] * kLog2e : NEG_INF;
  }
  {
    const T* bq = static_cast<const T*>(p.b_qkv);
    const T* bp = static_cast<const T*>(p.b_proj);
    for (int i = tid; i < 4 * C; i += NT)
      lb[i] = i < 3 * C ? (bq ? (float)bq[i] : 0.0f) : (bp ? (float)bp[i - 3 * C] : 0.0f);
  }
  // Per-lane constants of phase 2: table byte offsets (negated) of this lane's
  // keys 32kb + 8g + e (e = 4t + r); padded keys land in the -inf half.  Bit
  // 8kb + e of key_lo_y / key_lo_x: that key's ty / tx lies before the slice
  // boundary M - s of the last window row / column.
  // The offsets depend only on the lane's 16-lane group g, so they live in LDS:
  // koff_s[g][8kb + e].
  unsigned key_lo_y = 0, key_lo_x = 0;
#pragma unroll
  for (int kb = 0; kb < KT / 2; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = 32 * kb + 8 * g4 + e;
      const int ty = key / M, tx = key - (key / M) * M;
      if (i16 == 0) koff_s[g4][8 * kb + e] = 4 * (key < N ? ty * n2 + tx : -nrel);
      key_lo_y |= (unsigned)(ty < M - g.s) << (8 * kb + e);
      key_lo_x |= (unsigned)(tx < M - g.s) << (8 * kb + e);
    }
  __syncthreads();

  auto wfrag = [&](gptr<T> base, int row, int k) {
    return gload8(base + (uint32_t)(row * C + k * 32 + g4 * 8));
  };

  for (; w < n_windows; w += gridDim.x) {
    const WinPos wpos = win_pos(w);
    gptr<T> wqi = (gptr<T>)wq;
    gptr<T> wpi = (gptr<T>)wp;
    asm volatile("" : "+s"(wqi), "+s"(wpi));  // keep the weight loads in the loop

    // ---- phase 1: QKV blocks (p, h) = (q|k|v, head) -----------------------------
#pragma unroll 1
    for (int blk = wave; blk < 3 * HEADS; blk += WAVES) {
      const int part = blk / HEADS, h = blk - part * HEADS;
      const int row0 = part * C + h * kD;  // weight rows = output channels
      vec8<T> wf[2][HEADS];
#pragma unroll
      for (int k = 0; k < HEADS; ++k)
#pragma unroll
        for (int t = 0; t < 2; ++t) wf[t][k] = wfrag(wqi, row0 + 16 * t + i16, k);
      if (part < 2) {
        // Transposed: acc[t][j] lane l = channel 16t + 4g + r of token 16j + (l%16).
        f32x4 acc[2][KT];
        f32x4 b[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) b[t] = *reinterpret_cast<const f32x4*>(&lb[row0 + 16 * t + 4 * g4]);
#pragma unroll
        for (int k = 0; k < HEADS; ++k)
#pragma unroll
          for (int j = 0; j < KT; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t)
              acc[t][j] = mma_16x16x32(wf[t][k], xf[j][k], k == 0 ? b[t] : acc[t][j]);
        const float mult = part == 0 ? (V2 ? kLog2e / fmaxf(p.tau[h], p.tau_min) : p.q_mult) : 1.0f;
        QT* dst = reinterpret_cast<QT*>(part == 0 ? qs : ks);
#pragma unroll
        for (int j = 0; j < KT; ++j) {
          float sc = mult;
          if constexpr (V2) {
            float ss = 0.f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int r = 0; r < 4; ++r) ss = fmaf(acc[t][j][r], acc[t][j][r], ss);
            ss = xor32_sum(xor16_sum(ss));
            sc = mult * __builtin_amdgcn_rsqf(fmaxf(ss, p.eps * p.eps));
          }
#pragma unroll
          for (int t = 0; t < 2; ++t)
            store4<QT>(&dst[(16 * j + i16) * LDQ + h * kD + 16 * t + 4 * g4], acc[t][j], sc);
        }
      } else {
        // acc[j][t] lane l = channel 16t + (l%16) of tokens 16j + 4g + r.
        f32x4 acc[KT][2];
        f32x4 b[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float bv = lb[row0 + 16 * t + i16];
          b[t] = f32x4{bv, bv, bv, bv};
        }
#pragma unroll
        for (int k = 0; k < HEADS; ++k)
#pragma unroll
          for (int j = 0; j < KT; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t)
              acc[j][t] = mma_16x16x32(xf[j][k], wf[t][k], k == 0 ? b[t] : acc[j][t]);
#pragma unroll
        for (int j = 0; j < KT; ++j)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            store4<T>(&vt[(h * kD + 16 * t + i16) * LDV + 16 * j + 4 * g4], acc[j][t], 1.0f);
      }
    }
    __syncthreads();  // Q, K, V^T complete

    // ---- phase 2: attention items (head, query tile) ----------------------------
    const bool last_row = g.s > 0 && wpos.y0 == g.H - M;
    const bool last_col = g.s > 0 && wpos.x0 == g.W - M;
    vec8<T> ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = from_f32<T>(1.0f);
#pragma unroll 1
    for (int it = wave; it < HEADS * KT; it += WAVES) {
      const int h = it / KT, i = it - h * KT;
      const QT* qsq = reinterpret_cast<const QT*>(qs);
      const QT* ksq = reinterpret_cast<const QT*>(ks);
      const int q = 16 * i + i16;
      const vec8<QT> qf = load8(&qsq[q * LDQ + h * kD + 8 * g4]);
      const int qc = q < N ? q : N - 1;
      const int tyq = qc / M, txq = qc - (qc / M) * M;
      const char* tq = reinterpret_cast<const char*>(tab[h]) + 4 * ((tyq + M - 1) * n2 + txq + M - 1);
      unsigned allow = ~0u;
      if (last_row) allow &= (tyq < M - g.s) ? key_lo_y : ~key_lo_y;
      if (last_col) allow &= (txq < M - g.s) ? key_lo_x : ~key_lo_x;
      f32x4 s[KT / 2][2];
#pragma unroll
      for (int kb = 0; kb < KT / 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int4 ko = *reinterpret_cast<const int4*>(&koff_s[g4][8 * kb + 4 * t]);
          s[kb][t][0] = *reinterpret_cast<const float*>(tq - ko.x);
          s[kb][t][1] = *reinterpret_cast<const float*>(tq - ko.y);
          s[kb][t][2] = *reinterpret_cast<const float*>(tq - ko.z);
          s[kb][t][3] = *reinterpret_cast<const float*>(tq - ko.w);
          if (last_row || last_col) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (!((allow >> (8 * kb + 4 * t + r)) & 1u)) s[kb][t][r] = NEG_INF;
          }
          // K rows for S^T rows 4g'+r' of this 16-key MFMA: key 32kb + 8g' + 4t + r'.
          const int krow = 32 * kb + 8 * (i16 >> 2) + 4 * t + (i16 & 3);
          s[kb][t] = mma_16x16x32(load8(&ksq[krow * LDQ + h * kD + 8 * g4]), qf, s[kb][t]);
        }
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < KT / 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          mx = fmaxf(fmaxf(mx, fmaxf(s[kb][t][0], s[kb][t][1])), fmaxf(s[kb][t][2], s[kb][t][3]));
      mx = xor32_max(xor16_max(mx));
      f32x4 o[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 l = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KT / 2; ++kb) {
        vec8<T> pf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) pf[4 * t + r] = from_f32<T>(fast_exp2(s[kb][t][r] - mx));
#pragma unroll
        for (int n = 0; n < 2; ++n)
          o[n] = mma_16x16x32(load8(&vt[(h * kD + 16 * n + i16) * LDV + 32 * kb + 8 * g4]), pf, o[n]);
        l = mma_16x16x32(ones, pf, l);
      }
      const float inv = __builtin_amdgcn_rcpf(l[0]);
      // O^T: lane l holds head dims 16n + 4g + r of query q; O replaces Q there.
#pragma unroll
      for (int n = 0; n < 2; ++n) store4<T>(&qs[q * LDQ + h * kD + 16 * n + 4 * g4], o[n], inv);
    }
    __syncthreads();  // O complete; K no longer needed

    // ---- phase 3: output projection, one 16-channel tile per item ---------------
    const int nxt = w + gridDim.x;
    if (nxt < n_windows) fetch_x(nxt);  // next window's tokens, in flight
#pragma unroll 1
    for (int ct = wave; ct < 2 * HEADS; ct += WAVES) {
      vec8<T> wf[HEADS];
#pragma unroll
      for (int k = 0; k < HEADS; ++k) wf[k] = wfrag(wpi, 16 * ct + i16, k);
      const f32x4 b = *reinterpret_cast<const f32x4*>(&lb[3 * C + 16 * ct + 4 * g4]);
      f32x4 acc[KT];
#pragma unroll
      for (int k = 0; k < HEADS; ++k)
#pragma unroll
        for (int j = 0; j < KT; ++j)
          acc[j] = mma_16x16x32(wf[k], load8(&qs[(16 * j + i16) * LDQ + 32 * k + 8 * g4]),
                                k == 0 ? b : acc[j]);
      // Y^T: lane l holds channels 16ct + 4g + r of token 16j + (l%16).
#pragma unroll
      for (int j = 0; j < KT; ++j) store4<T>(&ks[(16 * j + i16) * LDQ + 16 * ct + 4 * g4], acc[j], 1.0f);
    }
    __syncthreads();  // Y staged

#pragma unroll
    for (int k = 0; k < PF; ++k) {
      if (slot_yx[k] < 0) continue;
      const int i = tid + k * NT;
      const int c = i % CPR;
      gstore16(y + src_row(wpos, slot_yx[k]) * C + c * EPC,
               *reinterpret_cast<const uint4*>(&ks[(i / CPR) * LDQ + c * EPC]));
    }
    __syncthreads();  // staging read before the next window's phase 1 writes K
  }
}

template <typename T, typename QT, int HEADS, bool V2>
hipError_t launch_heads(const FwdParams& p, int per_cu, int cus, hipStream_t st) {
  const int n = p.g.B * p.g.nW;
  const int grid = n < cus * per_cu ? n : cus * per_cu;
  dim3 block(64 * waves_for<HEADS>());
  if (p.g.N <= 32)
    hipLaunchKernelGGL((fused_window_kernel<T, QT, HEADS, 2, V2>), dim3(grid), block, 0, st, p, n);
  else
    hipLaunchKernelGGL((fused_window_kernel<T, QT, HEADS, 4, V2>), dim3(grid), block, 0, st, p, n);
  return hipGetLastError();
}

template <typename T, typename QT, bool V2>
hipError_t launch_type(const FwdParams& p, int cus, hipStream_t st) {
  // Resident workgroups per CU: what the 160 KB of LDS holds, at most 3.
  const int C = 32 * p.g.heads, NP = p.g.N <= 32 ? 32 : 64, e = (int)sizeof(T);
  const int lds = 2 * NP * (C + 16 / e) * e + C * (NP + 16 / e) * e + p.g.heads * 2 * 225 * 4 +
                  16 * C + 16 * NP;
  int per_cu = (160 * 1024) / lds;
  per_cu = per_cu < 1 ? 1 : (per_cu > 3 ? 3 : per_cu);
  switch (p.g.heads) {
    case 1: return launch_heads<T, QT, 1, V2>(p, per_cu, cus, st);
    case 2: return launch_heads<T, QT, 2, V2>(p, per_cu, cus, st);
    case 3: return launch_heads<T, QT, 3, V2>(p, per_cu, cus, st);
    default: return launch_heads<T, QT, 4, V2>(p, per_cu, cus, st);
  }
}

template <bool V2>
hipError_t launch_mode(const FwdParams& p, int cus, hipStream_t st) {
  if (p.io == kF32) return launch_type<float, float, V2>(p, cus, st);
  if (p.io == kF16) return launch_type<h16, h16, V2>(p, cus, st);
  if (p.qk == kF16) return launch_type<b16, h16, V2>(p, cus, st);
  return launch_type<b16, b16, V2>(p, cus, st);
}

}  // namespace

hipError_t launch_fused_window(const FwdParams& p, hipStream_t st) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return p.v2 ? launch_mode<true>(p, cus, st) : launch_mode<false>(p, cus, st);
}

}  // namespace swin
