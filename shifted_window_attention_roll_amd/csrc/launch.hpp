// Host-side launchers of the device kernels (one definition per .hip file).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "swin_wmsa.h"

namespace swin {

// The calling thread's last HIP error that an entry point returned as
// SWIN_ERR_HIP (hipSuccess until one does).
inline hipError_t& last_hip_error() {
  static thread_local hipError_t e = hipSuccess;
  return e;
}

// SWIN_OK for hipSuccess, else SWIN_ERR_HIP with the error recorded.
inline swin_status hip_status(hipError_t e) {
  if (e == hipSuccess) return SWIN_OK;
  last_hip_error() = e;
  return SWIN_ERR_HIP;
}

// Element type of x / y / weights: 0 = float32, 1 = float16, 2 = bfloat16.
enum IoType { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Per-window intermediates written by the QKV projection and read by the
// window attention.  Layout of q, k, v: [B*nW, heads, N, 32] (one window-head
// block contiguous, token-major, head dim fastest); o: [B*nW*N, C] window order.
struct QkvBuffers {
  void* q;  // qk_type
  void* k;  // qk_type
  void* v;  // io type
  void* o;  // io type
};

struct FwdParams {
  Geom g;
  int io;          // IoType of x, y, weights, linear biases
  int qk;          // IoType of the stored q and k
  bool v2;         // scaled cosine attention
  float q_mult;    // V1: scale * log2(e) folded into q
  float tau_min;   // V2 clip
  float eps;       // V2 norm clamp
  const void* x;
  const void* w_qkv;
  const void* b_qkv;   // may be null
  const void* w_proj;
  const void* b_proj;  // may be null
  const float* table;  // [(2M-1)^2, heads]
  const float* tau;    // [heads] (V2)
  void* y;
  QkvBuffers buf;
};

hipError_t launch_partition_shift(const void* x, void* xw, const Geom& g, int elem_bytes,
                                  hipStream_t st);
hipError_t launch_reverse_unshift(const void* xw, void* x, const Geom& g, int elem_bytes,
                                  hipStream_t st);
hipError_t launch_cpb_table(const float* w1, const float* b1, const float* w2, const float* b2,
                            int hidden, int heads, int M, float coord_scale, float* table,
                            hipStream_t st);
hipError_t launch_cpb_bwd(const float* w1, const float* b1, const float* w2, const float* b2,
                          int hidden, int heads, int M, float coord_scale, const float* dtable,
                          float* dw1, float* db1, float* dw2, float* db2, float* dout,
                          hipStream_t st);
hipError_t launch_qkv_gemm(const FwdParams& p, hipStream_t st);
hipError_t launch_window_attn(const FwdParams& p, hipStream_t st);
hipError_t launch_proj_gemm(const FwdParams& p, hipStream_t st);
// Attention for window sides 8, 16, 24 with 16-bit I/O; needs chunked slots
// (see Geom).
bool tiled_attn_supported(int M, int io);
hipError_t launch_tiled_attn(const FwdParams& p, hipStream_t st);
// QKV / projection GEMMs for 16-bit I/O and C in {256, 512} (32-bit offsets:
// tokens * C * 2 must stay below 2^31).
// Dense layer of the block's MLP on the tiled GEMM: y = act(a w^T + bias) (+ res);
// a [rows, K], w [N, K], res / y [rows, N]; 16-bit, N % 128 == 0, K in {256,
// 512, 1024, 2048}.
struct DenseParams {
  int io, rows, N, K;
  const void* a;
  const void* w;
  const void* bias;  // [N] or null
  const void* res;   // [rows, N] or null
  void* y;
};
// rows * K * 2 must stay below 2^31 (32-bit buffer offsets); else the general kernel.
bool dense_tiled_supported(int64_t rows, int N, int K, int io);
hipError_t launch_dense_tiled(const DenseParams& d, bool gelu, hipStream_t st);

bool tiled_gemm_supported(int C, int io);
hipError_t launch_qkv_tiled(const FwdParams& p, hipStream_t st);
hipError_t launch_proj_tiled(const FwdParams& p, hipStream_t st);
// Single-kernel forward for window side 16 with C = 32 * heads, heads <= 4,
// 16-bit I/O, x below 2^31 elements (needs chunked slots).  flags: one int per
// (window, wave) -- fused_w16_flag_count -- written by the main launch
// (!redo); the redo launch recomputes the flagged windows exactly.
bool fused_w16_supported(int64_t tokens, int M, int C, int heads, int io);
int64_t fused_w16_flag_count(int heads, int64_t windows);
hipError_t launch_fused_w16(const FwdParams& p, int* flags, bool redo, hipStream_t st);
// QKV projection + attention in one kernel for window sides 16 and 24, C = 32
// x heads up to 1024, 16-bit I/O, x below 2 GiB (needs chunked slots); O goes
// to buf.o in window-slot order for the projection GEMM.  flags: one int per
// (window, head, wave) -- fused_qkv_attn_flag_count -- written by the main
// launch (!redo); the redo launch recomputes the flagged items exactly.
bool fused_qkv_attn_supported(int64_t tokens, int M, int C, int heads, int io);
int64_t fused_qkv_attn_flag_count(int M, int64_t items);
hipError_t launch_fused_qkv_attn(const FwdParams& p, int* flags, bool redo, hipStream_t st);
// Attention for window side 7 with 16-bit I/O between the GEMMs (row-major
// slots).
bool w8_attn_supported(int M, int io);
hipError_t launch_w8_attn(const FwdParams& p, hipStream_t st);
// Single-kernel forward for window sides 7 and 8 with C = 32 * heads,
// heads <= 4, 16-bit I/O (its own 8 x 8 slot layout).
bool fused_w8_supported(int M, int C, int heads, int io);
hipError_t launch_fused_w8(const FwdParams& p, hipStream_t st);
// Single-kernel forward for N <= 64 and C = 32 * heads with heads <= 4.
hipError_t launch_fused_window(const FwdParams& p, hipStream_t st);

// Largest window side the attention kernel stages in LDS for an element size.
// Backward pass (backward.hip).  Element-strided GEMM C = A B (+ bias):
// A(m, k) = A[m*sam + k*sak], B(k, n) = B[k*sbk + n*sbn], C row pitch ldc;
// one stride of each operand is 1 and the other a multiple of 8.
struct BwdGemm {
  int64_t M, N, K, kc;
  const void* A;
  int64_t sam, sak;
  const void* B;
  int64_t sbk, sbn;
  const void* bias;  // [N], B's element type, or null
  void* C;
  int64_t ldc;
  float* rowsum;     // ATOMIC with sam == 1 only: += sum_k A(m, k), or null
};
struct AttnBwd {
  Geom g;
  float scale, tau_min, eps;
  const float* qkv;    // [T, 3C] window order, linear bias included
  const float* dout;   // [T, C] gradient of the attention output
  const float* table;  // [(2M-1)^2, heads]
  const float* tau;    // [heads] (V2)
  float* o;            // [T, C] recomputed attention output
  float* dqkv;         // [T, 3C]
  float* dtable;       // accumulated
  float* dtau;         // accumulated (V2)
};
struct BwdArgs {
  Geom g;
  int io;
  bool v2;
  float scale, tau_min, eps;
  const void *x, *dy, *w_qkv, *b_qkv, *w_proj;
  const float *table, *tau;
  void* dx;
  float *dw_qkv, *db_qkv, *dw_proj, *db_proj, *dtable, *dtau;
  // workspace
  void *xw, *dyw, *dxw;
  float *qkv, *dout, *o, *dqkv;
};
hipError_t launch_backward(const BwdArgs& a, hipStream_t st);

// FP8 linear layers (fp8.hip).
struct Fp8Linear {
  const uint8_t* a;   // [rows, K] E4M3 codes
  const float* sa;    // [rows]
  const uint8_t* w;   // [N, K] E4M3 codes
  const float* sw;    // [N]
  const void* bias;   // [N] of bias_type, or null
  int bias_type;
  void* y;            // [rows, N]
  int64_t rows;
  int N, K;
};
__device__ __forceinline__ float ld_any(const void* p, int type, int i) {
  if (type == kF32) return static_cast<const float*>(p)[i];
  if (type == kF16) return (float)static_cast<const h16*>(p)[i];
  return (float)static_cast<const b16*>(p)[i];
}
hipError_t launch_fp8_quant(const void* x, int io, int rows, int K, uint8_t* codes, float* scales,
                            hipStream_t st);
hipError_t launch_fp8_linear(const Fp8Linear& p, int out_io, hipStream_t st);
// The persistent tiled FP8 product (gemm_tiled.hip) where it applies.
bool fp8_tiled_supported(const Fp8Linear& p);
hipError_t launch_fp8_tiled(const Fp8Linear& p, int out_io, hipStream_t st);

// 2:4 sparse linear layers (sparse.hip).
struct Sparse24Linear {
  const void* x;         // [rows, K]
  const void* vals;      // [N, K/2]
  const uint8_t* codes;  // [N, K/4]
  const void* bias;      // [N] or null
  void* y;               // [rows, N]
  int64_t rows;
  int N, K;
};
hipError_t launch_prune24(const void* w, int io, int N, int K, void* vals, uint8_t* codes,
                          hipStream_t st);
hipError_t launch_sparse24_linear(const Sparse24Linear& p, int io, hipStream_t st);
// The persistent tiled sparse product (gemm_tiled.hip) where it applies.
bool sparse24_tiled2_supported(const Sparse24Linear& p, int io);
hipError_t launch_sparse24_tiled2(const Sparse24Linear& p, int io, hipStream_t st);

inline int max_window(int io_bytes) { return io_bytes == 4 ? 16 : 24; }

}  // namespace swin
