// Attention for windows whose side M is a multiple of 8 (SwinV2 windows of 8,
// 16, 24), 16-bit I/O, between the QKV and projection GEMMs: q, k, v per
// (window, head) as [N][32] (q scaled so that the logits are in base 2) in, O
// as [window slot][C] out.  The core (bias, mask, lazy-max softmax, both
// products) is attn_tiles in attn_core.hpp.
//
// Persistent workgroups walk the (window, head) items with a stride that is a
// multiple of the head count, so a workgroup keeps one head and stages that
// head's bias table once.  K and V of an item sit in one of two LDS buffers
// (swizzled rows, no padding); while an item is computed, every thread copies
// its share of the next item's K and V into the other buffer, one 16-byte
// chunk per few key blocks (a chunk's global load is issued a few blocks
// before its LDS store), so consecutive items do not wait for their staging.
#include "attn_core.hpp"
#include "launch.hpp"

namespace swin {

namespace {

// Waves per SIMD the launch below keeps resident (workgroups per CU x WAVES / 4).
template <int M>
constexpr int tiled_waves_per_simd() { return M == 24 ? 3 : 4; }

template <typename QT, typename VT, int M, int QTL, int WAVES, bool V2>
__global__ __launch_bounds__(64 * WAVES)
__attribute__((amdgpu_waves_per_eu(tiled_waves_per_simd<M>())))
void tiled_attn_kernel(FwdParams p, int n_items) {
  constexpr int D = 32;
  constexpr int N = M * M;
  static_assert(M % 8 == 0 && N / 16 == QTL * WAVES, "tile split");
  constexpr int NT = 64 * WAVES;
  constexpr int CPT = N * D / 8 / NT;      // 16-byte chunks of K (and of V) per thread
  static_assert(CPT * NT * 8 == N * D, "staging split");
  constexpr int NB = N / 32;               // key blocks
  constexpr int CH = 2 * CPT;              // chunks staged per thread and item
  __shared__ __attribute__((aligned(16))) QT ks[2][N * 32];
  __shared__ __attribute__((aligned(16))) VT vs[2][N * 32];
  __shared__ __attribute__((aligned(16))) float rt[table1_size<M>()];
  __shared__ __attribute__((aligned(16))) float ninf[8];
  __shared__ float red[WAVES];  // per-wave partial maxima

  const Geom& g = p.g;
  int item = blockIdx.x;  // window * heads + head; the head stays fixed
  if (item >= n_items) return;
  const int h = item % g.heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, i16 = lane & 15;

  // Chunk c of this thread: K for c < CPT, V after; element offset
  // tid * 8 + (c % CPT) * NT * 8 of the item's [N][32] tensor, i.e. row
  // tid / 4 + (c % CPT) * NT / 4, 16-byte column tid % 4.  NT / 4 is a
  // multiple of 32 rows, so the row's swizzle does not depend on c.
  static_assert((NT / 4) % 32 == 0, "swizzle independent of the chunk");
  const uint32_t src_off = (uint32_t)tid * 8;
  const int dst_off = kv_swz(tid >> 2, tid & 3);
  auto chunk_src = [&](int it, int c) -> const void* {
    const uint32_t off = src_off + (uint32_t)((c % CPT) * NT * 8);
    if (c < CPT) return (const void*)((gptr<QT>)p.buf.k + (size_t)it * N * D + off);
    return (const void*)((gptr<VT>)p.buf.v + (size_t)it * N * D + off);
  };
  auto chunk_dst = [&](int buf, int c) -> void* {
    const int off = dst_off + (c % CPT) * (NT / 4) * 32;
    return c < CPT ? (void*)&ks[buf][off] : (void*)&vs[buf][off];
  };

#pragma unroll
  for (int c = 0; c < CH; ++c)
    *reinterpret_cast<uint4*>(chunk_dst(0, c)) = gload16(chunk_src(item, c));
  fill_bias_table<M>(rt, p.table, g.heads, h, tid, NT);
  if (tid < 8) ninf[tid] = -__builtin_inff();
  // Zero reference: cosine attention with bfloat16 P.
  constexpr bool ZREF = V2 && !__is_same(VT, h16);
  if constexpr (ZREF) {
    // Cosine attention: |q . k| <= log2(e) / max(tau, tau_min) (q carries that
    // factor, both are unit vectors; 2^-8 covers their 16-bit rounding), so
    // every logit is at most that plus the table's largest entry.  Shifting
    // the head's table by that bound minus kZeroTop (a constant per head
    // leaves the softmax unchanged) lets the unmasked windows use the zero
    // reference.
    float bmax = -__builtin_inff();
    for (int e = tid; e < table1_size<M>(); e += NT) bmax = fmaxf(bmax, rt[e]);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, d));
    if (lane == 0) red[wave] = bmax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WAVES; ++w) bmax = fmaxf(bmax, red[w]);
    const float qmult = kLog2e / fmaxf(p.tau[h], p.tau_min);
    const float shift = qmult * (1.0f + 1.0f / 256.0f) + bmax - kZeroTop;
    for (int e = tid; e < table1_size<M>(); e += NT) rt[e] -= shift;
  }

  int tile[QTL];
#pragma unroll
  for (int j = 0; j < QTL; ++j) tile[j] = wave * QTL + j;
  auto load_q = [&](int it, vec8<QT> (&qf)[QTL]) {
    const QT* qg = static_cast<const QT*>(p.buf.q) + (int64_t)it * N * D;
#pragma unroll
    for (int j = 0; j < QTL; ++j) qf[j] = gload8(qg + (tile[j] * 16 + i16) * D + g4 * 8);
  };
  vec8<QT> qf[QTL];
  load_q(item, qf);
  __syncthreads();

  for (int buf = 0; item < n_items; item += gridDim.x, buf ^= 1) {
    const int w = item / g.heads;
    const int nxt = item + gridDim.x;
    const bool more = nxt < n_items;
    const int wl = w % g.nW;
    const int wy = wl / g.nWx, wx = wl - (wl / g.nWx) * g.nWx;
    const bool my = g.s > 0 && wy == g.H / M - 1;
    const bool mx = g.s > 0 && wx == g.nWx - 1;

    // The next item's K and V into the other buffer: chunk c is loaded at key
    // block (c * NB) / CH and stored when the next chunk is loaded (the last
    // one after the blocks).
    uint4 pend = {0, 0, 0, 0};
    auto hook = [&](int kbi) {
      if (!more) return;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if ((c * NB) / CH == kbi) {
          if (c > 0) *reinterpret_cast<uint4*>(chunk_dst(buf ^ 1, c - 1)) = pend;
          pend = gload16(chunk_src(nxt, c));
        }
      }
    };

    // Unmasked windows take the fast path, and so do masked ones with the
    // zero reference (cosine attention, bfloat16 P); the rest, and the rare
    // item whose logits outgrow the fixed reference, the exact lazy one
    // (running the hook twice stages the same chunks twice).
    float o[QTL][8];
    bool done = false;
    if (!(my || mx))
      done = attn_tiles<QT, VT, M, QTL, false, KvLayout::kSwizzled, TableMode::kTable1,
                        ZREF ? RefMode::kZero : RefMode::kBlock0>(
          qf, tile, ks[buf], vs[buf], rt, ninf, lane, M - g.s, false, false, o, hook);
    else if constexpr (ZREF)
      done = attn_tiles<QT, VT, M, QTL, true, KvLayout::kSwizzled, TableMode::kTable1,
                        RefMode::kZero>(qf, tile, ks[buf], vs[buf], rt, ninf, lane, M - g.s, my,
                                        mx, o, hook);
    if (!done)
      attn_tiles<QT, VT, M, QTL, true, KvLayout::kSwizzled, TableMode::kTable1, RefMode::kLazy>(
          qf, tile, ks[buf], vs[buf], rt, ninf, lane, M - g.s, my, mx, o, hook);

    // O rows in slot order, columns h*32 + d: the lane's 8 dims, one store.
    VT* og = static_cast<VT*>(p.buf.o);
#pragma unroll
    for (int j = 0; j < QTL; ++j) {
      vec8<VT> v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = from_f32<VT>(o[j][e]);
      gstore16(og + ((int64_t)w * N + tile[j] * 16 + i16) * g.C + h * D + 8 * g4,
               __builtin_bit_cast(uint4, v));
    }
    if (more) {
      *reinterpret_cast<uint4*>(chunk_dst(buf ^ 1, CH - 1)) = pend;
      load_q(nxt, qf);
    }
    // Every wave is done with this buffer, and the other one is complete.
    __syncthreads();
  }
}

template <typename QT, typename VT, int M, int QTL, int WAVES>
hipError_t tiled_launch(const FwdParams& p, int per_cu, hipStream_t st) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int n = p.g.B * p.g.nW * p.g.heads;
  // A multiple of the head count, so that each workgroup keeps one head.
  int grid = cus * per_cu;
  if (grid > n) grid = n;
  grid = grid / p.g.heads * p.g.heads;
  if (grid < p.g.heads) grid = p.g.heads;
  if (p.v2)
    hipLaunchKernelGGL((tiled_attn_kernel<QT, VT, M, QTL, WAVES, true>), dim3(grid),
                       dim3(64 * WAVES), 0, st, p, n);
  else
    hipLaunchKernelGGL((tiled_attn_kernel<QT, VT, M, QTL, WAVES, false>), dim3(grid),
                       dim3(64 * WAVES), 0, st, p, n);
  return hipGetLastError();
}

template <typename QT, typename VT>
hipError_t tiled_dispatch(const FwdParams& p, hipStream_t st) {
  // Workgroups per CU: what the LDS holds (two K, V buffers + the table).
  switch (p.g.M) {
    case 8: return tiled_launch<QT, VT, 8, 1, 4>(p, 4, st);
    case 16: return tiled_launch<QT, VT, 16, 2, 8>(p, 2, st);
    case 24: return tiled_launch<QT, VT, 24, 3, 12>(p, 1, st);
    default: return hipErrorInvalidValue;
  }
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
