// Shared device helpers for the gfx950 shifted-window attention kernels:
// element types, 16-byte fragment loads, the 16x16x32 matrix-core step and the
// window geometry (cyclic shift + window partition as pure index arithmetic).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swin {

typedef _Float16 h16;
typedef __bf16 b16;

typedef float f32x4 __attribute__((ext_vector_type(4)));
template <typename T>
using vec8 = T __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// Eight consecutive elements (one lane's K-slice of a 16x16x32 operand).
template <typename T>
__device__ __forceinline__ vec8<T> load8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(vec8<T>, u);
  } else {
    uint4 u0 = reinterpret_cast<const uint4*>(p)[0];
    uint4 u1 = reinterpret_cast<const uint4*>(p)[1];
    struct P { uint4 a, b; } pr{u0, u1};
    return __builtin_bit_cast(vec8<T>, pr);
  }
}

// Global-memory (address space 1) 16-byte loads / stores.  Pointers that travel
// through a kernel-argument struct or inline-asm laundering lose their address
// space, and the generic (flat) instructions the compiler then emits also count
// against the LDS wait counter; these keep them on the global path.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;
typedef const __attribute__((address_space(1))) u32x4* cg16;
typedef __attribute__((address_space(1))) u32x4* g16;

__device__ __forceinline__ uint4 gload16(const void* p) {
  return __builtin_bit_cast(uint4, *(cg16)(p));
}
__device__ __forceinline__ void gstore16(void* p, uint4 v) {
  *(g16)(p) = __builtin_bit_cast(u32x4, v);
}

template <typename T>
__device__ __forceinline__ vec8<T> gload8(gptr<T> p) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(vec8<T>, *(cg16)p);
  } else {
    struct P { u32x4 a, b; } pr{*(cg16)p, *(cg16)(p + 4)};
    return __builtin_bit_cast(vec8<T>, pr);
  }
}

template <typename T>
__device__ __forceinline__ vec8<T> gload8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(vec8<T>, gload16(p));
  } else {
    struct P { uint4 a, b; } pr{gload16(p), gload16(p + 4)};
    return __builtin_bit_cast(vec8<T>, pr);
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const vec8<T>& v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
  } else {
    struct P { uint4 a, b; };
    P pr = __builtin_bit_cast(P, v);
    reinterpret_cast<uint4*>(p)[0] = pr.a;
    reinterpret_cast<uint4*>(p)[1] = pr.b;
  }
}

// acc += A(16x32) * B(32x16) on the matrix cores.  Lane l supplies row / column
// (l % 16) and the K-slice 8*(l/16) .. 8*(l/16)+7 of each operand; the result
// tile holds, in lane l, column (l % 16) of rows 4*(l/16) .. 4*(l/16)+3.
// For float32 the slice is fed as eight 16x16x4 steps; A and B pair their K
// indices identically, so the sum covers the same 32 products.
__device__ __forceinline__ f32x4 mma_16x16x32(const vec8<h16>& a, const vec8<h16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_16x16x32(const vec8<b16>& a, const vec8<b16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_16x16x32(const vec8<float>& a, const vec8<float>& b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

template <typename T>
__device__ __forceinline__ T from_f32(float v) { return (T)v; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Butterfly steps across the four 16-lane rows of a wave on the VALU
// (v_permlane16_swap / v_permlane32_swap): each call returns, in every lane, the
// sum or max of the lane's value and that of lane l^16 (resp. l^32); both
// partners get the identical result.
__device__ __forceinline__ float xor16_sum(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// Window geometry.  Window w = b*nW + wy*nWx + wx; slot t of the window holds
// window-local (ty, tx), i.e. shifted-frame (wy*M+ty, wx*M+tx), i.e. original
// position ((wy*M+ty+s) mod H, (wx*M+tx+s) mod W).  Slots are row-major
// (t = ty*M + tx) unless `chunked`: for M % 8 == 0 the window is cut into
// column chunks 8 tokens wide, and t = cx*8M + ty*8 + (tx - 8cx) with cx = tx/8,
// so that every 8 consecutive slots are 8 consecutive tokens of one window row
// and every 16 consecutive slots are a 2 x 8 patch.  Attention does not depend
// on the order of the tokens inside a window; the order only has to be the
// same where the slots are written and where they are read back.
// Division of 32-bit unsigned n by a divisor d fixed at launch: one high
// multiply, a subtract, an add and two shifts (round-up multiplier method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d)
// + 1, n / d = (t + ((n - t) >> 1)) >> (l - 1) where t = umulhi(m, n), exact
// for every n < 2^32.
struct FastDiv {
  uint32_t d, m, s1, s2;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  f.s1 = l > 0 ? 1 : 0;
  f.s2 = l > 0 ? l - 1 : 0;
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint32_t t = __umulhi(n, f.m);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

struct Geom {
  int B, H, W, C, M, s, nWx, nW, N, heads;
  int chunked;
  FastDiv dN, dnW, dnWx, dM, dChunk;  // N, nW, nWx, M, 8M
};

__device__ __forceinline__ void slot_yx(const Geom& g, int t, int& ty, int& tx) {
  if (g.chunked) {
    const int cx = (int)fdiv((uint32_t)t, g.dChunk);
    const int rem = t - cx * 8 * g.M;
    ty = rem >> 3;
    tx = 8 * cx + (rem & 7);
  } else {
    ty = (int)fdiv((uint32_t)t, g.dM);
    tx = t - ty * g.M;
  }
}

// Window w and slot t of window-order row r.
__device__ __forceinline__ void row_wt(const Geom& g, int r, int& w, int& t) {
  w = (int)fdiv((uint32_t)r, g.dN);
  t = r - w * g.N;
}

__device__ __forceinline__ int64_t src_token(const Geom& g, int r) {
  int w, t;
  row_wt(g, r, w, t);
  int b = (int)fdiv((uint32_t)w, g.dnW);
  int wl = w - b * g.nW;
  int wy = (int)fdiv((uint32_t)wl, g.dnWx);
  int wx = wl - wy * g.nWx;
  int ty, tx;
  slot_yx(g, t, ty, tx);
  int y = wy * g.M + ty + g.s;
  if (y >= g.H) y -= g.H;
  int x = wx * g.M + tx + g.s;
  if (x >= g.W) x -= g.W;
  return ((int64_t)b * g.H + y) * g.W + x;
}

// Slice of a shifted-frame coordinate v on an axis of length L (region mask).
__device__ __forceinline__ int axis_slice(int v, int L, int M, int s) {
  return v < L - M ? 0 : (v < L - s ? 1 : 2);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (32-bit byte bound) as four scalar dwords.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// LDS byte address of a __shared__ object.
template <typename P>
__device__ __forceinline__ uint32_t lds_addr(P* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)p);
}

// One 16-byte direct-to-LDS load per lane: lane L's bytes voff + soff of the
// buffer land at LDS byte lds + 16 L.  Written as inline assembly so that the
// compiler does not see the LDS write: it would otherwise wait for every such
// load before any later LDS read, including the loads meant to fly two steps
// ahead; the waits are explicit instead (wait_vm, then a barrier).  There is
// no output register.
__device__ __forceinline__ void lds_dma16(const i32x4& rs, uint32_t lds, uint32_t voff,
                                          uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}

// The same for one 4-byte load per lane (lane L's bytes land at lds + 4 L).
__device__ __forceinline__ void lds_dma4(const i32x4& rs, uint32_t lds, uint32_t voff,
                                         uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}

}  // namespace swin
