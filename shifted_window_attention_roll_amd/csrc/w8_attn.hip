// Attention for window side 7 (16-bit I/O) between the QKV and projection
// GEMMs: q, k, v per (window, head) as [49][32] in row-major slot order
// (q scaled so that the logits are in base 2) in, O as [window slot][C] out.
//
// Pages: "Boosting Swin Transformer Speed", Training Optimization (fused MHA);
// "Swin Transformer V2" summary, How It Works (logit = similarity + relative
// position bias B_ij).
//
// Each wave works alone on whole (window, head) items: no workgroup barrier.
// The waves walk the items with a stride that is a multiple of the head count,
// so a wave keeps one head and fills that head's bias table once.  Per item
// the wave places q (registers), K and V (its own LDS rows) on the 8 x 8 slot
// grid of w8_core.hpp -- a padding slot takes the row of the nearest real
// slot, so everything stays finite -- runs w8_attend and writes O of the real
// slots.  The next item's q, K, V are loaded into registers during the
// current item's attention.
#include "launch.hpp"
#include "w8_core.hpp"

namespace swin {

namespace {

constexpr int kW8AttnWaves = 4;

template <typename QT, typename VT, int MV>
__global__ __launch_bounds__(64 * kW8AttnWaves) __attribute__((amdgpu_waves_per_eu(3)))
void w8_attn_kernel(FwdParams p, int n_items) {
  constexpr int D = 32, N = MV * MV;
  static_assert(sizeof(QT) == 2 && sizeof(VT) == 2, "16-bit q, k, v");
  __shared__ __attribute__((aligned(16))) QT ks[kW8AttnWaves][64 * 32];  // swizzled rows
  __shared__ __attribute__((aligned(16))) VT vs[kW8AttnWaves][64 * 32];
  __shared__ __attribute__((aligned(16))) float tabs[kW8AttnWaves][kTab];

  const Geom& g = p.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stride = gridDim.x * kW8AttnWaves;  // a multiple of the head count
  int item = blockIdx.x * kW8AttnWaves + wave;   // window * heads + head
  if (item >= n_items) return;                    // no barriers below
  const int h = item % g.heads;
  const int g4 = lane >> 4, i16 = lane & 15;
  const int qx = i16 & 7, qy0 = i16 >> 3;

  fill_w8_table<MV>(tabs[wave], p.table, g.heads, h, lane, 64);

  // Row (in the item's row-major slots) of grid slot 16j + l%16 and of the
  // K / V chunk rows this lane stages (grid slot 16c + l/4, chunk l%4).
  auto src_row = [&](int ty, int tx) {
    return (ty < MV ? ty : MV - 1) * MV + (tx < MV ? tx : MV - 1);
  };
  int qrow[4], krow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qrow[j] = src_row(2 * j + qy0, qx);
    const int s = 16 * j + (lane >> 2);
    krow[j] = src_row(s >> 3, s & 7);
  }
  const int kc = lane & 3;
  gptr<QT> qg = (gptr<QT>)p.buf.q;
  gptr<QT> kg = (gptr<QT>)p.buf.k;
  gptr<VT> vg = (gptr<VT>)p.buf.v;
  vec8<QT> qf[4];
  uint4 kr[4], vr[4];
  auto fetch = [&](int it) {
    const size_t base = (size_t)it * N * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qf[j] = gload8(qg + base + (uint32_t)(qrow[j] * D + 8 * g4));
      kr[j] = __builtin_bit_cast(uint4, *(cg16)(kg + base + (uint32_t)(krow[j] * D + 8 * kc)));
      vr[j] = __builtin_bit_cast(uint4, *(cg16)(vg + base + (uint32_t)(krow[j] * D + 8 * kc)));
    }
  };

  // LDS addresses (see w8_core.hpp and the swizzle of attn_core.hpp).
  QT* kst = &ks[wave][0];
  VT* vst = &vs[wave][0];
  typedef __attribute__((address_space(3))) const vec8<QT>* lds_q8;
  const int prow = 8 * (i16 >> 2) + (i16 & 3);
  lds_q8 kl = (lds_q8)&ks[wave][prow * 32 + ((g4 ^ (i16 >> 2)) << 3)];
  lds_v4s vl = (lds_v4s)&vs[wave][(8 * g4 + (i16 >> 2)) * 32 + (((i16 & 3) ^ g4) << 3)];
  lds_f tb0 = (lds_f)&tabs[wave][((qy0 - g4 + 7) << 4) + 7 - qx];
  lds_f tb1 = (MV < 8 && g4 == 3) ? (lds_f)&tabs[wave][kTabRows] : tb0 - 64;
  const int bnd = MV - g.s;

  fetch(item);
  for (; item < n_items; item += stride) {
    const int w = item / g.heads;
    // This item's K and V rows into the wave's LDS (row 16c + l/4 of the
    // grid, chunk l%4); the wave reads back only rows it wrote itself.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int s = 16 * c + (lane >> 2);
      *reinterpret_cast<uint4*>(&kst[kv_swz(s, kc)]) = kr[c];
      *reinterpret_cast<uint4*>(&vst[kv_swz(s, kc)]) = vr[c];
    }
    asm volatile("" ::: "memory");
    vec8<QT> qc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) qc[j] = qf[j];
    vec8<QT> kf[2][2];
    vec8<VT> vf[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        kf[b][t] = kl[(32 * b + 4 * t) * 32 / 8];
        vf[b][t] = vt_frag<VT, 32>(vl, 32 * b, t);
      }
    if (item + stride < n_items) fetch(item + stride);  // in flight during the attention

    const int wl = w % g.nW;
    const int wy = wl / g.nWx, wx = wl - (wl / g.nWx) * g.nWx;
    const bool my = g.s > 0 && wy == g.H / MV - 1;
    const bool mx = g.s > 0 && wx == g.nWx - 1;
    VT* og = static_cast<VT*>(p.buf.o) + (int64_t)w * N * g.C + h * D + 8 * g4;
    auto store_o = [&](int j, const vec8<VT>& of) {
      if (2 * j + qy0 < MV && qx < MV)
        gstore16(og + (int64_t)((2 * j + qy0) * MV + qx) * g.C, __builtin_bit_cast(uint4, of));
    };
    if (my || mx)
      w8_attend<QT, VT, MV, true, false>(qc, kf, vf, tb0, tb1, qy0, qx, g4, bnd, my, mx, store_o);
    else  // exact row maxima: a zero-reference pass would need more registers here
      w8_attend<QT, VT, MV, false, false>(qc, kf, vf, tb0, tb1, qy0, qx, g4, bnd, false, false,
                                          store_o);
    // The next item's K / V stores must not pass this item's fragment reads.
    asm volatile("" ::: "memory");
  }
}

template <typename QT, typename VT>
hipError_t w8_attn_launch(const FwdParams& p, hipStream_t st) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int n = p.g.B * p.g.nW * p.g.heads;
  // Waves: a multiple of the head count (each wave keeps one head), at most
  // 12 per CU, at most one per item rounded up to whole heads.
  int waves = cus * 12;
  const int cap = (n + p.g.heads - 1) / p.g.heads * p.g.heads;
  if (waves > cap) waves = cap;
  waves = waves / p.g.heads * p.g.heads;
  if (waves < p.g.heads) waves = p.g.heads;
  // Whole workgroups: the wave count is also a multiple of kW8AttnWaves.
  int unit = p.g.heads;
  while (unit % kW8AttnWaves) unit += p.g.heads;
  waves = (waves + unit - 1) / unit * unit;
  hipLaunchKernelGGL((w8_attn_kernel<QT, VT, 7>), dim3(waves / kW8AttnWaves),
                     dim3(64 * kW8AttnWaves), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace

bool w8_attn_supported(int M, int io) { return io != kF32 && M == 7; }

hipError_t launch_w8_attn(const FwdParams& p, hipStream_t st) {
  if (!w8_attn_supported(p.g.M, p.io) || p.g.chunked) return hipErrorInvalidValue;
  if (p.io == kF16) return w8_attn_launch<h16, h16>(p, st);
  if (p.qk == kF16) return w8_attn_launch<h16, b16>(p, st);
  return w8_attn_launch<b16, b16>(p, st);
}

}  // namespace swin
