// QKV projection fused into the window attention, for window sides 16 and 24
// and C a multiple of 32 with 16-bit I/O: q, k and v never reach HBM.
//
// Pages: "Boosting Swin Transformer Speed: Profiling, Mixed Precision, and
// Kernel Fusion Secrets" -- Training Optimization (the fused MHA computes the
// QKV GEMM with its bias and the softmax in one kernel; shift / partition are
// index maps) and Inference Optimization (no separate transposes); "Swin
// Transformer V2" summary, How It Works (cosine attention over tau, continuous
// position bias); "Boost Vision Transformer with GPU-Friendly Sparsity and
// Quantization", Section 3.2 / Figure 3 (the Q/K/V projections are GEMMs).
//
// Persistent workgroups walk (window, head) items.  Item mapping: workgroup b
// runs on XCD b % 8 (workgroups reach the XCDs round-robin); XCD x owns the
// windows x, x + 8, ..., and its workgroups take that list's (window, head)
// items in turn, so the workgroups running together on one XCD work on the
// same one or two windows and read their token rows from that XCD's L2 (x is
// read from HBM about once), and -- when the XCD's workgroup count is a
// multiple of the head count -- each workgroup keeps one head (its bias table
// is staged once).
//
// Per item, phase 1 (QKV) is a GEMM of the window's N token rows (gathered
// from x through the shift + partition map) with the head's 96 rows of W_qkv,
// in steps of 32 channels: both operands go global -> LDS by direct-to-LDS
// buffer loads into three buffers (the token rows partly in the LDS that K
// and V take in phase 2), two steps' loads in flight while one is
// multiplied.  Wave w owns the query tiles w*QTL .. w*QTL+QTL-1 (16 window
// slots each, chunked slot order, see Geom) and forms q, k, v of its slots as
// C^T products; the weight rows of each 16-channel tile pair are read
// interleaved, so a lane ends with 8 consecutive head dims of its token: q
// (scaled, or normalised and scaled in V2) stays in registers as the B operand
// of S^T = K Q^T, k and v go to LDS.  Phase 2: the attention core
// (attn_core.hpp) against all N keys; O of the head goes to the workspace in
// window-slot order for the projection GEMM.
#include "attn_core.hpp"
#include "launch.hpp"

namespace swin {

namespace {

template <int M>
struct FqaCfg;
template <>
struct FqaCfg<16> {
  static constexpr int WAVES = 8, QTL = 2, PER_CU = 2, WPE = 4;  // WPE: waves per SIMD
};
template <>
struct FqaCfg<24> {
  static constexpr int WAVES = 12, QTL = 3, PER_CU = 1, WPE = 3;
};

// One phase-1 step: 32 channels, i.e. 64-byte rows of four 16-byte chunks.
// Chunk q of LDS row r sits at position q ^ sw(r), sw(r) = (r/2 ^ r/4 ^ r/16)
// % 4: for the 16 consecutive rows of a fragment read, any 8, 16 or 32
// consecutive lanes then touch distinct 16-byte bank slots modulo 128, 256 and
// 512 bytes.  Weight rows are stored permuted inside each 32-row part (LDS
// row 16t + 4a + b holds row 8a + 4t + b), so that the 16 rows 8a + 4t + b of
// a fragment (a, b in 0..3) are 16 consecutive LDS rows too.
__device__ __forceinline__ int sw(int r) { return ((r >> 1) ^ (r >> 2) ^ (r >> 4)) & 3; }
__device__ __forceinline__ int xsw(int r, int q) { return r * 32 + ((q ^ sw(r)) << 3); }
// Weight row r (part r / 32, interleaved fragment order) -> its LDS row, and back.
__device__ __forceinline__ int wrow_lds(int r) {
  return (r & ~31) | (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
}
__device__ __forceinline__ int wrow_of_lds(int l) {
  return (l & ~31) | (((l >> 2) & 3) << 3) | (((l >> 4) & 1) << 2) | (l & 3);
}

// s_waitcnt vmcnt(N) only: all but the last N vector-memory operations of this
// wave have completed (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4]
// left at 7, lgkmcnt [11:8] left at 15).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// The same for a wave-uniform count 0 .. 15 (larger counts wait for everything).
__device__ __forceinline__ void wait_vm_rt(int n) {
  switch (n) {
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;
    case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break;
    case 11: wait_vm<11>(); break;
    case 12: wait_vm<12>(); break;
    case 13: wait_vm<13>(); break;
    case 14: wait_vm<14>(); break;
    case 15: wait_vm<15>(); break;
    default: wait_vm<0>(); break;
  }
}

constexpr int kStages = 3;  // phase-1 buffers: the loads of step s+2 fly during step s

template <typename T>
__device__ __forceinline__ vec8<T> cvt8(const float (&v)[8], float mult) {
  vec8<T> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(v[e] * mult);
  return o;
}

// The kernel body.  !REDO: every (window, head) item of the launch; a wave
// whose fixed-reference row sums leave the safe range (attn_core.hpp) sets
// flags[(win * heads + h) * WAVES + wave] = 1 (else 0) and leaves its O to the
// redo launch.  REDO: only the items with a flag set, every tile, on the
// exact lazy pass.
template <typename T, typename QT, int M, bool V2, bool REDO>
__device__ __forceinline__ void fqa_body(const FwdParams& p, int* flags) {
  using Cf = FqaCfg<M>;
  constexpr int N = M * M, D = 32, WAVES = Cf::WAVES, QTL = Cf::QTL, NT = 64 * WAVES;
  constexpr int TSZ = table1_size<M>();  // one reversed bias-table copy (attn_core.hpp)
  static_assert(N / 16 == QTL * WAVES, "tile split");
  constexpr int XI = N / 16;              // 1 KB load instructions per step: token rows
  constexpr int WI = 96 / 16;             // ... weight rows
  constexpr int XU = XI / WAVES;          // token-row instructions per wave
  static_assert(XI % WAVES == 0 && WI <= WAVES, "load split");
  // Zero softmax reference: cosine attention with bfloat16 P.
  constexpr bool ZREF = V2 && !__is_same(T, h16);
  // Phase 1: kStages buffers of the token rows' 32-channel step (N * 64 bytes
  // each); phase 2: K and V in the first 2 * N * 64 bytes.
  __shared__ __attribute__((aligned(1024))) char kvx[kStages * N * 64];
  __shared__ __attribute__((aligned(1024))) T wsm[kStages][96 * 32];
  __shared__ __attribute__((aligned(16))) float rt[TSZ];
  __shared__ __attribute__((aligned(16))) float ninf[8];
  __shared__ float red[WAVES];
  __shared__ __attribute__((aligned(16))) float bqs[96];  // the head's q, k, v biases
  QT* ks = reinterpret_cast<QT*>(kvx);  // swizzled rows (kv_frag.hpp)
  T* vs = reinterpret_cast<T*>(kvx + N * D * 2);

  const Geom& g = p.g;
  const int C = g.C, heads = g.heads;
  const int NS = C / 32;  // phase-1 steps
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const T* bq = static_cast<const T*>(p.b_qkv);
  T* og = static_cast<T*>(p.buf.o);

  // Items of this workgroup (see the header comment).  The redo launch walks
  // every item id = window * heads + head and takes the flagged ones.
  const int G = gridDim.x, b = blockIdx.x;
  const int nx = G < 8 ? G : 8;
  const int xcd = b % nx;
  const int n_win = g.B * g.nW;
  const int j0 = REDO ? b : b / nx;
  const int wpx = REDO ? G : (G - xcd + nx - 1) / nx;
  const int n_it = REDO ? n_win * heads : ((n_win - xcd + nx - 1) / nx) * heads;
  if (j0 >= n_it) return;

  if (threadIdx.x < 8) ninf[threadIdx.x] = -__builtin_inff();
  int tile[QTL];
#pragma unroll
  for (int j = 0; j < QTL; ++j) tile[j] = wave * QTL + j;
  const float eps2 = p.eps * p.eps;

  // Buffer resources (bounds: the whole tensor; x below 2 GiB, see the plan
  // choice): 32-bit lane offsets, the step's offset a scalar.
  const i32x4 rx = make_rsrc(p.x, (uint32_t)((int64_t)g.B * g.H * g.W * C * (int)sizeof(T)));
  const i32x4 rw = make_rsrc(p.w_qkv, (uint32_t)(3 * C * C * (int)sizeof(T)));
  const uint32_t kvx_a = lds_addr(kvx), wsm_a = lds_addr(&wsm[0][0]);

  // Redo launch: the items with a flag set, found with one load per thread
  // (bit i of `todo`: the workgroup's i-th item).
  __shared__ unsigned todo_lds[2];
  uint64_t todo = ~0ull;
  if constexpr (REDO) {
    if (threadIdx.x < 2) todo_lds[threadIdx.x] = 0u;
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * WAVES; e += NT) {
      const int kk = j0 + wpx * (e / WAVES);
      if (kk < n_it && flags[kk * WAVES + e % WAVES])
        atomicOr(&todo_lds[(e / WAVES) >> 5], 1u << ((e / WAVES) & 31));
    }
    __syncthreads();
    todo = ((uint64_t)todo_lds[1] << 32) | todo_lds[0];
    if (todo == 0) return;
  }

  // Item k: window and head.
  auto item_win = [&](int kk) { return REDO ? kk / heads : xcd + nx * (kk / heads); };
  auto item_head = [&](int kk) { return kk - (kk / heads) * heads; };
  // Token index of slot r (chunked order) of window win: the shift + partition map.
  auto slot_token = [&](int win, int r) -> uint32_t {
    const int bi = (int)fdiv((uint32_t)win, g.dnW);
    const int wl = win - bi * g.nW;
    const int wy = (int)fdiv((uint32_t)wl, g.dnWx);
    const int wx = wl - wy * g.nWx;
    const int cx = r / (8 * M), rem = r - cx * 8 * M;
    int yy = wy * M + g.s + (rem >> 3);
    if (yy >= g.H) yy -= g.H;
    int xx = wx * M + g.s + 8 * cx + (rem & 7);
    if (xx >= g.W) xx -= g.W;
    return (uint32_t)((bi * g.H + yy) * g.W + xx);
  };
  // Load instructions of one step: token-row instruction i (< XI) fills rows
  // 16i .. 16i+15 of the step's token buffer, weight-row instruction i (< WI)
  // rows 16i .. 16i+15 of its weight buffer; lane L lands at row 16i + L/4,
  // 16-byte slot L%4, and fetches the chunk the swizzle puts there.  Wave w
  // issues token-row instructions w + WAVES u (u < XU) and, if w < WI,
  // weight-row instruction w.  off[u], off[XU]: this lane's byte offsets
  // (step 0).
  auto item_offsets = [&](int win, int h, int lane, uint32_t (&off)[XU + 1]) {
    const int slot = lane & 3;
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int r = 16 * (wave + WAVES * u) + (lane >> 2);
      off[u] = slot_token(win, r) * (uint32_t)(C * (int)sizeof(T)) +
               (uint32_t)((slot ^ sw(r)) << 4);
    }
    const int l = 16 * wave + (lane >> 2);  // LDS weight row (wave < WI)
    const int r = wrow_of_lds(l);
    const uint32_t row = (uint32_t)((r >> 5) * C + h * D + (r & 31));
    off[XU] = row * (uint32_t)(C * (int)sizeof(T)) + (uint32_t)((slot ^ sw(l)) << 4);
  };
  // Step s of an item into buffer (s + 2) % 3: step 0 lands in the buffer
  // past K and V, so that it can be loaded during the previous item's
  // attention.
  auto issue_step = [&](const uint32_t (&off)[XU + 1], int s) {
    const int soff = s * 64, bi = (s + 2) % kStages;
#pragma unroll
    for (int u = 0; u < XU; ++u)
      lds_dma16(rx, kvx_a + bi * N * 64 + (wave + WAVES * u) * 1024, off[u], soff);
    if (wave < WI) lds_dma16(rw, wsm_a + bi * 96 * 64 + wave * 1024, off[XU], soff);
  };
  // Load instructions this wave issues per step (uniform).
  const int nld = XU + (wave < WI ? 1 : 0);

  // Vector-memory operations are counted in issue order per wave.  Per item:
  // step 0 (during the previous item's attention, or at the item's start for
  // the first one), then steps 1 and 2 (after the previous attention), then
  // the previous item's O stores (nst of them), then step s + 2 at the start
  // of step s >= 1.
  int k = j0;
  if constexpr (REDO) {
    while (!((todo >> ((k - j0) / wpx)) & 1)) k += wpx;
  }
  int win = item_win(k), h = item_head(k);
  {
    uint32_t off0[XU + 1];
    item_offsets(win, h, threadIdx.x & 63, off0);
#pragma unroll
    for (int s0 = 0; s0 < 3; ++s0)
      if (s0 < NS) issue_step(off0, s0);
  }
  int nst = 0;  // O stores issued after this item's steps 1 and 2
  int cur_head = -1;
  while (true) {
    // Per-lane values are derived from the thread index anew in every item
    // (opaque to the compiler), so that they are not hoisted out of the item
    // loop and kept live through the attention, which needs every register.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, g4 = lane >> 4, i16 = lane & 15;
    const int wl = win - (int)fdiv((uint32_t)win, g.dnW) * g.nW;
    const int wy = (int)fdiv((uint32_t)wl, g.dnWx);
    const bool my = g.s > 0 && wy == g.H / M - 1;
    const bool mx = g.s > 0 && wl - wy * g.nWx == g.nWx - 1;

    if (h != cur_head) {
      // Every wave is past its last read of the previous head's table.
      __syncthreads();
      fill_bias_table<M>(rt, p.table, heads, h, tid, NT);
      for (int e = tid; e < 96; e += NT)
        bqs[e] = bq ? (float)bq[(e >> 5) * C + h * D + (e & 31)] : 0.f;
      if constexpr (ZREF) {
        // |q . k| <= log2(e) / max(tau, tau_min) (q carries that factor, both
        // are unit vectors; 2^-8 covers their float16 rounding), so no logit
        // exceeds that plus the table's largest entry; a constant shift of the
        // head's table (the softmax does not see it) puts that bound at
        // kZeroTop.
        __syncthreads();
        float bmax = -__builtin_inff();
        for (int e = tid; e < TSZ; e += NT) bmax = fmaxf(bmax, rt[e]);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, d));
        if (lane == 0) red[wave] = bmax;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < WAVES; ++w) bmax = fmaxf(bmax, red[w]);
        const float qm = kLog2e / fmaxf(p.tau[h], p.tau_min);
        const float shift = qm * (1.0f + 1.0f / 256.0f) + bmax - kZeroTop;
        for (int e = tid; e < TSZ; e += NT) rt[e] -= shift;
      }
      cur_head = h;
    }
    // Step 0 landed: only steps 1, 2 and the O stores may still fly.
    wait_vm_rt(nld * (NS > 2 ? 2 : NS - 1) + nst);
    __syncthreads();  // step 0 (and the table) published

    // Phase 1: q, k, v of the wave's slots, acc[j][part][t].
    // Weight-row permutation inside a 32-row pair of 16-row fragments: fragment
    // t's row i16 is row 8 (i16 / 4) + 4t + i16 % 4, so output lanes hold 8
    // consecutive channels.
    const int prow0 = 8 * (i16 >> 2) + (i16 & 3);
    // (The load offsets are recomputed where they are used rather than kept
    // through the attention, which has no register to spare for them.)
    uint32_t off[XU + 1];
    item_offsets(win, h, lane, off);
    f32x4 acc[QTL][3][2];
#pragma unroll
    for (int j = 0; j < QTL; ++j)
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) acc[j][pt][0] = acc[j][pt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < NS; ++s) {
      // Buffer (s + 4) % 3 was last read in step s - 1, before the barrier
      // that ended it.
      if (s >= 1 && s + 2 < NS) issue_step(off, s + 2);
      const int bi = (s + 2) % kStages;
      const T* xb = reinterpret_cast<const T*>(kvx + bi * N * 64);
      const T* wb = wsm[bi];
      vec8<T> xf[QTL], wf[3][2];
#pragma unroll
      for (int j = 0; j < QTL; ++j)
        xf[j] = *reinterpret_cast<const vec8<T>*>(&xb[xsw(16 * tile[j] + i16, g4)]);
#pragma unroll
      for (int pt = 0; pt < 3; ++pt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          wf[pt][t] = *reinterpret_cast<const vec8<T>*>(&wb[xsw(wrow_lds(32 * pt + prow0 + 4 * t), g4)]);
      // Every fragment read of the step goes out before its products.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < QTL; ++j)
#pragma unroll
        for (int pt = 0; pt < 3; ++pt)
#pragma unroll
          for (int t = 0; t < 2; ++t) acc[j][pt][t] = mma_16x16x32(wf[pt][t], xf[j], acc[j][pt][t]);
      if (s + 1 < NS) {
        // Step s + 1 landed: after it come step s + 2 and, while s + 1 <= 2,
        // the previous item's O stores.
        wait_vm_rt((s + 2 < NS ? nld : 0) + (s <= 1 ? nst : 0));
      }
      __syncthreads();  // for every wave; and buffer (s + 2) % 3 is free
    }

    // The next item.
    int kn = k + wpx;
    if constexpr (REDO) {
      while (kn < n_it && !((todo >> ((kn - j0) / wpx)) & 1)) kn += wpx;
    }
    const bool more = kn < n_it;
    const int win_n = more ? item_win(kn) : win, h_n = more ? item_head(kn) : h;

    // Epilogue: bias; V2 unit vectors (1 / max(|v|, eps) = rsqrt(max(|v|^2,
    // eps^2))) with log2(e) / max(tau, tau_min) folded into q; V1 q times
    // scale * log2(e).  Lane: slot 16 tile + i16, dims 8 g4 .. +7.
    float qmult = p.q_mult;
    if constexpr (V2) qmult = kLog2e / fmaxf(p.tau[h], p.tau_min);
    float bias[3][8];
#pragma unroll
    for (int pt = 0; pt < 3; ++pt)
#pragma unroll
      for (int e = 0; e < 8; ++e) bias[pt][e] = bqs[32 * pt + 8 * g4 + e];
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
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
          ss = xor32_sum(xor16_sum(ss));
          mult *= __builtin_amdgcn_rsqf(fmaxf(ss, eps2));
        }
        if (pt == 0)
          qf[j] = cvt8<QT>(v, mult);
        else if (pt == 1)
          *reinterpret_cast<vec8<QT>*>(&ks[kv_swz(row, g4)]) = cvt8<QT>(v, mult);
        else
          *reinterpret_cast<vec8<T>*>(&vs[kv_swz(row, g4)]) = cvt8<T>(v, 1.0f);
      }
    }
    __syncthreads();  // K and V of the item complete

    // During the attention: the next item's step 0 (into the buffer past K
    // and V), and its window's token rows touched into L2 -- each head's
    // workgroup one share of the rows, so that the workgroups of a window
    // cover it once (lines of 128 bytes).
    unsigned touched = 0;
    if (more && !REDO) {
      uint32_t off_n[XU + 1];
      item_offsets(win_n, h_n, lane, off_n);
      issue_step(off_n, 0);
      const int r0 = (h_n * N) / heads, r1 = ((h_n + 1) * N) / heads;
      const int lines = C * (int)sizeof(T) / 128;
      const T* xg = static_cast<const T*>(p.x);
      for (int e = tid; e < (r1 - r0) * lines; e += NT) {
        const int r = r0 + e / lines, ln = e - (e / lines) * lines;
        touched ^= *reinterpret_cast<const unsigned*>(
            xg + (size_t)slot_token(win_n, r) * C + ln * (128 / (int)sizeof(T)));
      }
    }

    // Phase 2: attention of the wave's query tiles on a fixed reference: the
    // zero reference with cosine attention and bfloat16 P, else block 0's row
    // max (unmasked windows) or each tile's own-block row max (masked ones).
    // The rare item whose logits outgrow it is flagged for the redo launch,
    // which runs the exact lazy pass.
    float o[QTL][8];
    bool done = true;
    if constexpr (REDO) {
      attn_tiles<QT, T, M, QTL, true, KvLayout::kSwizzled, TableMode::kTable1, RefMode::kLazy>(
          qf, tile, ks, vs, rt, ninf, lane, M - g.s, my, mx, o);
    } else {
      if (!(my || mx))
        done = attn_tiles<QT, T, M, QTL, false, KvLayout::kSwizzled, TableMode::kTable1,
                          ZREF ? RefMode::kZero : RefMode::kBlock0>(qf, tile, ks, vs, rt, ninf,
                                                                    lane, M - g.s, false, false, o);
      else
        done = attn_tiles<QT, T, M, QTL, true, KvLayout::kSwizzled, TableMode::kTable1,
                          ZREF ? RefMode::kZero : RefMode::kOwn>(qf, tile, ks, vs, rt, ninf, lane,
                                                                 M - g.s, my, mx, o);
      // One flag per wave (each wave decides for its own tiles), always
      // written, so the array needs no clearing.
      if (lane == 0) flags[(win * heads + h) * WAVES + wave] = done ? 0 : 1;
    }
    asm volatile("" ::"v"(touched));  // the touches are consumed (and waited for) here
    // Every wave is done with K and V of this item: the next item's steps 1
    // and 2 go where they were.
    __syncthreads();
    if (more) {
      int tid2 = threadIdx.x;
      asm volatile("" : "+v"(tid2));
      uint32_t off_n[XU + 1];
      item_offsets(win_n, h_n, tid2 & 63, off_n);
      if (REDO) issue_step(off_n, 0);
#pragma unroll
      for (int s1 = 1; s1 < 3; ++s1)
        if (s1 < NS) issue_step(off_n, s1);
    }
    // O rows in window-slot order, columns h*32 + d: the lane's 8 dims (a wave
    // whose fixed reference failed leaves them to the redo launch).
    nst = 0;
    if (done) {
#pragma unroll
      for (int j = 0; j < QTL; ++j)
        gstore16(og + ((int64_t)win * N + 16 * tile[j] + i16) * C + h * D + 8 * g4,
                 __builtin_bit_cast(uint4, cvt8<T>(o[j], 1.0f)));
      nst = QTL;
    }
    if (!more) break;
    k = kn;
    win = win_n;
    h = h_n;
  }
}

template <typename T, typename QT, int M, bool V2>
__global__ __launch_bounds__(64 * FqaCfg<M>::WAVES)
__attribute__((amdgpu_waves_per_eu(FqaCfg<M>::WPE, FqaCfg<M>::WPE)))
void fused_qkv_attn_kernel(FwdParams p, int* flags) {
  fqa_body<T, QT, M, V2, false>(p, flags);
}

template <typename T, typename QT, int M, bool V2>
__global__ __launch_bounds__(64 * FqaCfg<M>::WAVES)
__attribute__((amdgpu_waves_per_eu(FqaCfg<M>::WPE, FqaCfg<M>::WPE)))
void fused_qkv_attn_redo_kernel(FwdParams p, int* flags) {
  fqa_body<T, QT, M, V2, true>(p, flags);
}

template <typename T, typename QT, int M, bool V2>
hipError_t fqa_launch(const FwdParams& p, int* flags, bool redo, hipStream_t st) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int n = p.g.B * p.g.nW * p.g.heads;
  int grid = cus * FqaCfg<M>::PER_CU;
  if (grid > n) grid = n;
  const dim3 block(64 * FqaCfg<M>::WAVES);
  if (redo)
    hipLaunchKernelGGL((fused_qkv_attn_redo_kernel<T, QT, M, V2>), dim3(grid), block, 0, st, p,
                       flags);
  else
    hipLaunchKernelGGL((fused_qkv_attn_kernel<T, QT, M, V2>), dim3(grid), block, 0, st, p, flags);
  return hipGetLastError();
}

template <typename T, typename QT>
hipError_t fqa_dispatch(const FwdParams& p, int* flags, bool redo, hipStream_t st) {
  switch (p.g.M) {
    case 16:
      return p.v2 ? fqa_launch<T, QT, 16, true>(p, flags, redo, st)
                  : fqa_launch<T, QT, 16, false>(p, flags, redo, st);
    case 24:
      return p.v2 ? fqa_launch<T, QT, 24, true>(p, flags, redo, st)
                  : fqa_launch<T, QT, 24, false>(p, flags, redo, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool fused_qkv_attn_supported(int64_t tokens, int M, int C, int heads, int io) {
  // x and W_qkv are addressed through buffer resources with 32-bit bounds.
  return io != kF32 && (M == 16 || M == 24) && C == 32 * heads && C <= 1024 &&
         tokens * C * 2 < ((int64_t)1 << 31);
}

int64_t fused_qkv_attn_flag_count(int M, int64_t items) {
  return items * (M == 16 ? FqaCfg<16>::WAVES : FqaCfg<24>::WAVES);
}

hipError_t launch_fused_qkv_attn(const FwdParams& p, int* flags, bool redo, hipStream_t st) {
  const int64_t tokens = (int64_t)p.g.B * p.g.H * p.g.W;
  if (!fused_qkv_attn_supported(tokens, p.g.M, p.g.C, p.g.heads, p.io) || !p.g.chunked || !flags)
    return hipErrorInvalidValue;
  if (p.io == kF16) return fqa_dispatch<h16, h16>(p, flags, redo, st);
  if (p.v2) return fqa_dispatch<b16, h16>(p, flags, redo, st);  // V2: q, k in float16
  return fqa_dispatch<b16, b16>(p, flags, redo, st);
}

}  // namespace swin
