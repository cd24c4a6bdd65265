// K and V of one (window, head) staged in LDS as [key][d] rows, and the
// transposing read that turns V into the A operand of O^T = V^T P^T; shared by
// the attention cores (attn_core.hpp, w8_core.hpp).
//
// Pages: "Boosting Swin Transformer Speed", Training Optimization (fused MHA:
// softmax fused with both products).
#pragma once

#include "common.hpp"

namespace swin {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s;

constexpr int kAttnLD = 40;  // LDS row pitch (elements) of staged K and V, padded layout

// Second K / V layout (KvLayout::kSwizzled): rows of 32 elements, the 16-byte
// chunk c of row r stored at chunk c ^ ((r / 8) % 4) -- no padding, and the
// fragment reads of the attention cores stay free of bank conflicts.
enum class KvLayout { kPadded, kSwizzled };
__device__ __forceinline__ int kv_swz(int r, int c) { return r * 32 + ((c ^ ((r >> 3) & 3)) << 3); }

// V^T fragment pair t (t = 0, 1) of keys kb .. kb+31 from V stored as [key][d]
// rows of kAttnLD elements, by two transposing LDS reads.  Within each 16-lane
// group g, lane (4a + b) of the read receives element b of the 8-byte chunk
// addressed by lane 4e + a, for e = 0..3; lane s of group g addresses
// V[kb + 8g + 4h + s/4][8(s%4) + 4t] (h = read 0 or 1), so lane i = 4a + b gets
// V[kb + 8g + 4h + e][8a + 4t + b]: row i of fragment t is head dim
// 8a + 4t + b, its k-slice the keys 8g .. 8g+7.
// vl: this lane's address for kb = 0, t = 0, h = 0.
template <typename VT, int LD = kAttnLD>
__device__ __forceinline__ vec8<VT> vt_frag(lds_v4s vl, int kb, int t) {
  const lds_v4s p0 = vl + (kb * LD + 4 * t) / 4;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0 + LD);  // 4 rows on
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(vec8<VT>, both);
}

}  // namespace swin
