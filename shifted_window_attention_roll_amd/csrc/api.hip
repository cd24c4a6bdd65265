// C ABI: argument validation, workspace layout and kernel dispatch.
// Declarations and the contract of every entry point are in include/swin_wmsa.h.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "swin_wmsa.h"
#include "launch.hpp"

using namespace swin;

namespace {

constexpr int kHeadDim = 32;

int elem_bytes(int dt) { return dt == SWIN_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

swin_status check_geometry(int B, int H, int W, int C, int M, int s) {
  // A window holds at least 2 x 2 tokens.
  if (B < 0 || H < 1 || W < 1 || C < 1 || M < 2) return SWIN_ERR_SHAPE;
  if (H % M || W % M) return SWIN_ERR_SHAPE;
  if (s < 0 || s >= M) return SWIN_ERR_SHAPE;
  if ((int64_t)B * H * W > INT32_MAX) return SWIN_ERR_UNSUPPORTED;
  return SWIN_OK;
}

Geom make_geom(int B, int H, int W, int C, int M, int s, int heads) {
  Geom g;
  g.B = B; g.H = H; g.W = W; g.C = C; g.M = M; g.s = s;
  g.nWx = W / M;
  g.nW = (H / M) * (W / M);
  g.N = M * M;
  g.heads = heads;
  g.chunked = 0;
  g.dN = make_fastdiv(g.N);
  g.dnW = make_fastdiv(g.nW);
  g.dnWx = make_fastdiv(g.nWx);
  g.dM = make_fastdiv(M);
  g.dChunk = make_fastdiv(8 * M);
  return g;
}

swin_status from_hip(hipError_t e) { return hip_status(e); }

// Storage type of q and k: V2 with 16-bit I/O keeps the normalised, 1/tau-scaled
// q and k in float16 (|q| <= log2(e)/0.01, |k| <= 1), whose 11-bit significand
// keeps the cosine logits accurate when 1/tau reaches 100.
int qk_type(const swin_wmsa_desc* d) {
  if (d->dtype == SWIN_F32) return kF32;
  if (d->mode == SWIN_V2) return kF16;
  return d->dtype == SWIN_F16 ? kF16 : kBF16;
}

// Kernel plan: one fused kernel for small windows with few heads (a dedicated
// one for window sides 7 and 8 with 16-bit I/O), and for window side 16 with
// few heads and 16-bit I/O; else the QKV GEMM -> window
// attention -> projection GEMM sequence through the workspace, with the tiled
// attention (chunked slots) for 16-bit I/O and window sides 8, 16, 24.
enum Plan {
  kPlanFusedSmall = 0,
  kPlanThree = 1,
  kPlanTiled = 2,
  kPlanFusedW16 = 3,
  kPlanFusedW8 = 4,
  kPlanFusedQkv = 5  // QKV + attention in one kernel, then the projection GEMM
};

int io_type(const swin_wmsa_desc* d) {
  return d->dtype == SWIN_F32 ? kF32 : d->dtype == SWIN_F16 ? kF16 : kBF16;
}

Plan choose_plan(const swin_wmsa_desc* d) {
  const int heads = d->heads;
  if (fused_w8_supported(d->M, d->C, heads, io_type(d))) return kPlanFusedW8;
  if (d->M * d->M <= 64 && heads <= 4 && d->C == kHeadDim * heads) return kPlanFusedSmall;
  if (fused_w16_supported((int64_t)d->B * d->H * d->W, d->M, d->C, heads, io_type(d)))
    return kPlanFusedW16;
  if (fused_qkv_attn_supported((int64_t)d->B * d->H * d->W, d->M, d->C, heads, io_type(d)))
    return kPlanFusedQkv;
  if (tiled_attn_supported(d->M, io_type(d))) return kPlanTiled;
  return kPlanThree;
}

bool use_tiled_gemm(const swin_wmsa_desc* d) {
  const size_t bytes = (size_t)d->B * d->H * d->W * d->C * elem_bytes(d->dtype);
  return tiled_gemm_supported(d->C, io_type(d)) && bytes < ((size_t)1 << 31);
}

struct WsLayout {
  size_t q, k, v, o, total;
};

WsLayout ws_layout(const swin_wmsa_desc* d) {
  const Plan plan = choose_plan(d);
  if (plan == kPlanFusedSmall || plan == kPlanFusedW8) return WsLayout{0, 0, 0, 0, 0};
  if (plan == kPlanFusedW16) {  // the redo flags only (at offset 0)
    const size_t windows = (size_t)d->B * (d->H / d->M) * (d->W / d->M);
    return WsLayout{0, 0, 0, 0,
                    round_up((size_t)fused_w16_flag_count(d->heads, windows) * 4, 256)};
  }
  const size_t tokens = (size_t)d->B * d->H * d->W;
  const size_t e = elem_bytes(d->dtype);
  const size_t eq = qk_type(d) == kF32 ? 4 : 2;
  if (plan == kPlanFusedQkv) {  // O, then the redo flags (L.q marks their offset)
    const size_t o = round_up(tokens * d->C * e, 256);
    const size_t items = (size_t)d->B * (d->H / d->M) * (d->W / d->M) * d->heads;
    return WsLayout{o, 0, 0, 0,
                    o + round_up((size_t)fused_qkv_attn_flag_count(d->M, items) * 4, 256)};
  }
  WsLayout L;
  L.q = 0;
  L.k = round_up(L.q + tokens * d->C * eq, 256);
  L.v = round_up(L.k + tokens * d->C * eq, 256);
  L.o = round_up(L.v + tokens * d->C * e, 256);
  L.total = round_up(L.o + tokens * d->C * e, 256);
  return L;
}

// Largest window of the backward: its attention kernel pads a window to at most
// 576 tokens, whatever the I/O type (it computes in float32).
constexpr int kBwdMaxWindow = 24;

// Descriptor checks shared by the forward and the backward; max_m is the
// largest window the caller's kernels take for this descriptor.
swin_status validate_desc_upto(const swin_wmsa_desc* d, int max_m) {
  if (!d) return SWIN_ERR_NULL;
  if (d->mode != SWIN_V1 && d->mode != SWIN_V2) return SWIN_ERR_DTYPE;
  if (d->dtype != SWIN_F32 && d->dtype != SWIN_F16 && d->dtype != SWIN_BF16) return SWIN_ERR_DTYPE;
  swin_status st = check_geometry(d->B, d->H, d->W, d->C, d->M, d->s);
  if (st != SWIN_OK) return st;
  if (d->heads < 1 || d->C % d->heads) return SWIN_ERR_SHAPE;
  if (d->C / d->heads != kHeadDim) return SWIN_ERR_UNSUPPORTED;
  if (d->M > max_m) return SWIN_ERR_UNSUPPORTED;
  return SWIN_OK;
}

swin_status validate_desc(const swin_wmsa_desc* d) {
  if (!d) return SWIN_ERR_NULL;
  return validate_desc_upto(d, max_window(elem_bytes(d->dtype)));
}

}  // namespace

extern "C" {

const char* swin_status_str(swin_status s) {
  switch (s) {
    case SWIN_OK: return "SWIN_OK";
    case SWIN_ERR_NULL: return "SWIN_ERR_NULL: a required pointer is NULL";
    case SWIN_ERR_SHAPE: return "SWIN_ERR_SHAPE: inconsistent sizes (H % M, W % M, shift range, C % heads)";
    case SWIN_ERR_DTYPE: return "SWIN_ERR_DTYPE: unknown dtype or mode";
    case SWIN_ERR_UNSUPPORTED: return "SWIN_ERR_UNSUPPORTED: head dim must be 32, window side within the kernel limit";
    case SWIN_ERR_ALIAS: return "SWIN_ERR_ALIAS: an output overlaps an input or the workspace";
    case SWIN_ERR_WORKSPACE: return "SWIN_ERR_WORKSPACE: workspace too small";
    case SWIN_ERR_ALIGN: return "SWIN_ERR_ALIGN: pointer not 16-byte aligned";
    case SWIN_ERR_HIP: return "SWIN_ERR_HIP: the HIP runtime reported an error";
    case SWIN_ERR_SCRATCH:
      return "SWIN_ERR_SCRATCH: the call needs more than the no-alloc entry point's fixed "
             "scratch (SWIN_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown swin_status";
}

int swin_abi_version(void) { return SWIN_WMSA_ABI_VERSION; }

const char* swin_last_hip_error(void) { return hipGetErrorString(last_hip_error()); }

static swin_status index_map_common(const void* in, void* out, int B, int H, int W, int C, int M,
                                    int s, swin_dtype dt, void* stream, bool reverse) {
  if (dt != SWIN_F32 && dt != SWIN_F16 && dt != SWIN_BF16) return SWIN_ERR_DTYPE;
  swin_status st = check_geometry(B, H, W, C, M, s);
  if (st != SWIN_OK) return st;
  if (B == 0) return SWIN_OK;
  if (!in || !out) return SWIN_ERR_NULL;
  const size_t bytes = (size_t)B * H * W * C * elem_bytes(dt);
  if (overlap(in, bytes, out, bytes)) return SWIN_ERR_ALIAS;
  if (!aligned16(in) || !aligned16(out)) return SWIN_ERR_ALIGN;
  Geom g = make_geom(B, H, W, C, M, s, 1);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = reverse ? launch_reverse_unshift(in, out, g, elem_bytes(dt), hs)
                         : launch_partition_shift(in, out, g, elem_bytes(dt), hs);
  return from_hip(e);
}

swin_status swin_partition_shift(const void* x, void* xw, int B, int H, int W, int C, int M, int s,
                                 swin_dtype dt, void* stream) {
  return index_map_common(x, xw, B, H, W, C, M, s, dt, stream, false);
}

swin_status swin_reverse_unshift(const void* xw, void* x, int B, int H, int W, int C, int M,
                                 int s, swin_dtype dt, void* stream) {
  return index_map_common(xw, x, B, H, W, C, M, s, dt, stream, true);
}

swin_status swin_cpb_table(const float* w1, const float* b1, const float* w2, const float* b2,
                           int hidden, int heads, int M, float coord_scale, float* table,
                           void* stream) {
  if (!w1 || !b1 || !w2 || !table) return SWIN_ERR_NULL;
  if (hidden < 1 || hidden > 4096 || heads < 1 || heads > 64 || M < 2 || M > 32)
    return SWIN_ERR_SHAPE;
  const size_t tbytes = (size_t)(2 * M - 1) * (2 * M - 1) * heads * sizeof(float);
  if (overlap(table, tbytes, w1, (size_t)hidden * 2 * 4) || overlap(table, tbytes, b1, hidden * 4u) ||
      overlap(table, tbytes, w2, (size_t)heads * hidden * 4) ||
      (b2 && overlap(table, tbytes, b2, heads * 4u)))
    return SWIN_ERR_ALIAS;
  if (!(coord_scale > 0.0f)) coord_scale = M > 1 ? 8.0f / (float)(M - 1) : 1.0f;
  return from_hip(launch_cpb_table(w1, b1, w2, b2, hidden, heads, M, coord_scale, table,
                                   static_cast<hipStream_t>(stream)));
}

size_t swin_wmsa_workspace_size(const swin_wmsa_desc* d) {
  if (validate_desc(d) != SWIN_OK || d->B == 0) return 0;
  return ws_layout(d).total;
}

static const int kPlanCount[6] = {1, 3, 3, 2, 1, 3};

static const char* stage_name(const swin_wmsa_desc* d, int i) {
  const Plan plan = choose_plan(d);
  if (plan == kPlanFusedSmall) return "fused_window_kernel";
  if (plan == kPlanFusedW16) return i == 0 ? "fused_w16_kernel" : "fused_w16_redo_kernel";
  if (plan == kPlanFusedW8) return "fused_w8_kernel";
  const bool tg = use_tiled_gemm(d);
  if (plan == kPlanFusedQkv)
    return i == 0   ? "fused_qkv_attn_kernel"
           : i == 1 ? "fused_qkv_attn_redo_kernel"
           : tg     ? "proj_tiled_kernel"
                    : "proj_gemm_kernel";
  if (i == 0) return tg ? "qkv_tiled_kernel" : "qkv_gemm_kernel";
  if (i == 1)
    return plan == kPlanTiled                         ? "tiled_attn_kernel"
           : w8_attn_supported(d->M, io_type(d)) ? "w8_attn_kernel"
                                                   : "window_attn_kernel";
  return tg ? "proj_tiled_kernel" : "proj_gemm_kernel";
}
constexpr int kMaxStages = 3;

int swin_wmsa_kernel_count(const swin_wmsa_desc* d) {
  if (validate_desc(d) != SWIN_OK || d->B == 0) return 0;
  return kPlanCount[choose_plan(d)];
}

const char* swin_wmsa_kernel_name(const swin_wmsa_desc* d, int i) {
  if (i < 0 || i >= swin_wmsa_kernel_count(d)) return nullptr;
  return stage_name(d, i);
}

static swin_status wmsa_forward(const swin_wmsa_desc* d, const void* x, const void* w_qkv,
                                const void* b_qkv, const void* w_proj, const void* b_proj,
                                const float* bias_table, const float* tau, void* y,
                                void* workspace, size_t ws_bytes, void* stream,
                                void* const* events, int n_events) {
  swin_status st = validate_desc(d);
  if (st != SWIN_OK) return st;
  if (d->B == 0) return SWIN_OK;
  const Plan plan = choose_plan(d);
  const int stages = kPlanCount[plan];
  const WsLayout L = ws_layout(d);
  if (!x || !w_qkv || !w_proj || !bias_table || !y) return SWIN_ERR_NULL;
  if (L.total > 0 && !workspace) return SWIN_ERR_NULL;
  if (d->mode == SWIN_V2 && !tau) return SWIN_ERR_NULL;
  if (events) {
    if (n_events < stages + 1) return SWIN_ERR_SHAPE;
    for (int i = 0; i <= stages; ++i)
      if (!events[i]) return SWIN_ERR_NULL;
  }
  if (ws_bytes < L.total) return SWIN_ERR_WORKSPACE;
  const size_t e = elem_bytes(d->dtype);
  const size_t act = (size_t)d->B * d->H * d->W * d->C * e;
  const size_t C = d->C;
  const size_t R2 = (size_t)(2 * d->M - 1) * (2 * d->M - 1);
  // Neither the output nor the workspace may overlap any input, or each other.
  struct Span { const void* p; size_t n; };
  const Span ins[] = {{x, act}, {w_qkv, 3 * C * C * e}, {b_qkv, 3 * C * e},
                      {w_proj, C * C * e}, {b_proj, C * e}, {bias_table, R2 * d->heads * 4},
                      {d->mode == SWIN_V2 ? tau : nullptr, d->heads * 4u}};
  for (const Span& in : ins)
    if (overlap(y, act, in.p, in.n) || overlap(workspace, L.total, in.p, in.n))
      return SWIN_ERR_ALIAS;
  if (overlap(y, act, workspace, L.total)) return SWIN_ERR_ALIAS;
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(w_proj) || !aligned16(y) ||
      (L.total > 0 && !aligned16(workspace)))
    return SWIN_ERR_ALIGN;

  FwdParams p;
  memset(&p, 0, sizeof(p));
  p.g = make_geom(d->B, d->H, d->W, d->C, d->M, d->s, d->heads);
  p.io = io_type(d);
  p.g.chunked = (plan == kPlanTiled || plan == kPlanFusedW16 || plan == kPlanFusedQkv) ? 1 : 0;
  p.qk = qk_type(d);
  p.v2 = d->mode == SWIN_V2;
  const float scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf((float)kHeadDim);
  p.q_mult = scale * kLog2e;
  p.tau_min = d->tau_min > 0.0f ? d->tau_min : 0.01f;
  p.eps = 1e-12f;
  p.x = x;
  p.w_qkv = w_qkv;
  p.b_qkv = b_qkv;
  p.w_proj = w_proj;
  p.b_proj = b_proj;
  p.table = bias_table;
  p.tau = tau;
  p.y = y;
  char* ws = static_cast<char*>(workspace);
  p.buf.q = ws + L.q;
  p.buf.k = ws + L.k;
  p.buf.v = ws + L.v;
  p.buf.o = ws + L.o;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), hs) : hipSuccess;
  };
  hipError_t err = mark(0);
  if (plan == kPlanFusedSmall || plan == kPlanFusedW8) {
    if (err == hipSuccess)
      err = plan == kPlanFusedSmall ? launch_fused_window(p, hs) : launch_fused_w8(p, hs);
    if (err == hipSuccess) err = mark(1);
    return from_hip(err);
  }
  if (plan == kPlanFusedW16) {
    int* flags = reinterpret_cast<int*>(ws);
    if (err == hipSuccess) err = launch_fused_w16(p, flags, false, hs);
    if (err == hipSuccess) err = mark(1);
    if (err == hipSuccess) err = launch_fused_w16(p, flags, true, hs);
    if (err == hipSuccess) err = mark(2);
    return from_hip(err);
  }
  const bool tg = use_tiled_gemm(d);
  if (plan == kPlanFusedQkv) {
    int* flags = reinterpret_cast<int*>(ws + L.q);
    p.buf.o = ws;
    if (err == hipSuccess) err = launch_fused_qkv_attn(p, flags, false, hs);
    if (err == hipSuccess) err = mark(1);
    if (err == hipSuccess) err = launch_fused_qkv_attn(p, flags, true, hs);
    if (err == hipSuccess) err = mark(2);
    if (err == hipSuccess) err = tg ? launch_proj_tiled(p, hs) : launch_proj_gemm(p, hs);
    if (err == hipSuccess) err = mark(3);
    return from_hip(err);
  }
  if (err == hipSuccess) err = tg ? launch_qkv_tiled(p, hs) : launch_qkv_gemm(p, hs);
  if (err == hipSuccess) err = mark(1);
  if (err == hipSuccess)
    err = plan == kPlanTiled                    ? launch_tiled_attn(p, hs)
          : w8_attn_supported(p.g.M, p.io) ? launch_w8_attn(p, hs)
                                           : launch_window_attn(p, hs);
  if (err == hipSuccess) err = mark(2);
  if (err == hipSuccess) err = tg ? launch_proj_tiled(p, hs) : launch_proj_gemm(p, hs);
  if (err == hipSuccess) err = mark(3);
  return from_hip(err);
}

swin_status swin_wmsa_fwd(const swin_wmsa_desc* d, const void* x, const void* w_qkv,
                          const void* b_qkv, const void* w_proj, const void* b_proj,
                          const float* bias_table, const float* tau, void* y, void* workspace,
                          size_t ws_bytes, void* stream) {
  return wmsa_forward(d, x, w_qkv, b_qkv, w_proj, b_proj, bias_table, tau, y, workspace,
                      ws_bytes, stream, nullptr, 0);
}

swin_status swin_wmsa_fwd_timed(const swin_wmsa_desc* d, const void* x, const void* w_qkv,
                                const void* b_qkv, const void* w_proj, const void* b_proj,
                                const float* bias_table, const float* tau, void* y,
                                void* workspace, size_t ws_bytes, void* stream,
                                void* const* events, int n_events) {
  if (!events) return SWIN_ERR_NULL;
  return wmsa_forward(d, x, w_qkv, b_qkv, w_proj, b_proj, bias_table, tau, y, workspace,
                      ws_bytes, stream, events, n_events);
}

// ---------------------------------------------------------------------------
// No-allocation forward: the workspace is this file-scope device array.  In
// host code `scratch` names a host-side stand-in, never its device address:
// kernels and copies only ever get the address hipGetSymbolAddress returns,
// kept per device.

static __device__ __attribute__((aligned(256))) unsigned char scratch[SWIN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up once per
// device, with that device current).
swin_status scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess) return hip_status(es);
    if (!p) return hip_status(hipErrorInvalidSymbol);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SWIN_OK;
}
}  // namespace

swin_status swin_wmsa_fwd_noalloc(const swin_wmsa_desc* d, const void* x, const void* w_qkv,
                                  const void* b_qkv, const void* w_proj, const void* b_proj,
                                  const float* bias_table, const float* tau, void* y,
                                  void* stream) {
  swin_status st = validate_desc(d);
  if (st != SWIN_OK) return st;
  if (d->B == 0) return SWIN_OK;
  const size_t need = ws_layout(d).total;
  if (need > SWIN_NOALLOC_SCRATCH_BYTES) return SWIN_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != SWIN_OK) return st;
  }
  return wmsa_forward(d, x, w_qkv, b_qkv, w_proj, b_proj, bias_table, tau, y, ws,
                      need > 0 ? (size_t)SWIN_NOALLOC_SCRATCH_BYTES : 0, stream, nullptr, 0);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward pass.

namespace {

struct BwdLayout {
  size_t xw, dyw, dxw, qkv, dout, o, dqkv, total;
};

BwdLayout bwd_layout(const swin_wmsa_desc* d) {
  BwdLayout L{};
  const size_t T = (size_t)d->B * d->H * d->W, C = d->C, e = elem_bytes(d->dtype);
  L.xw = 0;
  L.dyw = round_up(L.xw + T * C * e, 256);
  L.dxw = round_up(L.dyw + T * C * e, 256);
  L.qkv = round_up(L.dxw + T * C * e, 256);
  L.dout = round_up(L.qkv + T * 3 * C * 4, 256);
  L.o = round_up(L.dout + T * C * 4, 256);
  L.dqkv = round_up(L.o + T * C * 4, 256);
  L.total = round_up(L.dqkv + T * 3 * C * 4, 256);
  return L;
}

swin_status validate_bwd_desc(const swin_wmsa_desc* d) {
  return validate_desc_upto(d, kBwdMaxWindow);
}

}  // namespace

size_t swin_wmsa_bwd_workspace_size(const swin_wmsa_desc* d) {
  if (validate_bwd_desc(d) != SWIN_OK || d->B == 0) return 0;
  return bwd_layout(d).total;
}

swin_status swin_wmsa_bwd(const swin_wmsa_desc* d, const void* x, const void* w_qkv,
                          const void* b_qkv, const void* w_proj, const float* bias_table,
                          const float* tau, const void* dy, const swin_wmsa_grads* gr,
                          void* workspace, size_t ws_bytes, void* stream) {
  swin_status st = validate_bwd_desc(d);
  if (st != SWIN_OK) return st;
  const bool v2 = d->mode == SWIN_V2;
  if (!gr || !w_qkv || !w_proj || !bias_table || !gr->dw_qkv || !gr->db_qkv || !gr->dw_proj ||
      !gr->db_proj || !gr->dtable)
    return SWIN_ERR_NULL;
  if (d->B > 0 && (!x || !dy || !gr->dx)) return SWIN_ERR_NULL;
  if (v2 && (!tau || !gr->dtau)) return SWIN_ERR_NULL;
  const BwdLayout L = bwd_layout(d);
  if (d->B > 0 && !workspace) return SWIN_ERR_NULL;
  if (d->B > 0 && ws_bytes < L.total) return SWIN_ERR_WORKSPACE;
  const size_t e = elem_bytes(d->dtype), C = d->C;
  const size_t act = (size_t)d->B * d->H * d->W * C * e;
  const size_t R2 = (size_t)(2 * d->M - 1) * (2 * d->M - 1);
  const size_t ws = d->B > 0 ? L.total : 0;
  struct Span { const void* p; size_t n; };
  const Span outs[] = {{gr->dx, act}, {gr->dw_qkv, 3 * C * C * 4}, {gr->db_qkv, 3 * C * 4},
                       {gr->dw_proj, C * C * 4}, {gr->db_proj, C * 4},
                       {gr->dtable, R2 * d->heads * 4}, {v2 ? gr->dtau : nullptr, d->heads * 4u}};
  const Span ins[] = {{x, act}, {dy, act}, {w_qkv, 3 * C * C * e}, {b_qkv, 3 * C * e},
                      {w_proj, C * C * e}, {bias_table, R2 * d->heads * 4},
                      {v2 ? tau : nullptr, d->heads * 4u}, {workspace, ws}};
  const int no = sizeof(outs) / sizeof(outs[0]), ni = sizeof(ins) / sizeof(ins[0]);
  for (int i = 0; i < no; ++i) {
    for (int j = 0; j < ni; ++j)
      if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return SWIN_ERR_ALIAS;
    for (int j = i + 1; j < no; ++j)
      if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return SWIN_ERR_ALIAS;
  }
  if (overlap(x, act, workspace, ws) || overlap(dy, act, workspace, ws)) return SWIN_ERR_ALIAS;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(gr->dx) || !aligned16(w_qkv) ||
      !aligned16(w_proj) || (ws > 0 && !aligned16(workspace)))
    return SWIN_ERR_ALIGN;

  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.g = make_geom(d->B, d->H, d->W, d->C, d->M, d->s, d->heads);
  a.io = io_type(d);
  a.v2 = v2;
  a.scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf((float)kHeadDim);
  a.tau_min = d->tau_min > 0.0f ? d->tau_min : 0.01f;
  a.eps = 1e-12f;
  a.x = x; a.dy = dy; a.w_qkv = w_qkv; a.b_qkv = b_qkv; a.w_proj = w_proj;
  a.table = bias_table; a.tau = tau;
  a.dx = gr->dx; a.dw_qkv = gr->dw_qkv; a.db_qkv = gr->db_qkv; a.dw_proj = gr->dw_proj;
  a.db_proj = gr->db_proj; a.dtable = gr->dtable; a.dtau = v2 ? gr->dtau : nullptr;
  char* w = static_cast<char*>(workspace);
  if (d->B > 0) {
    a.xw = w + L.xw; a.dyw = w + L.dyw; a.dxw = w + L.dxw;
    a.qkv = reinterpret_cast<float*>(w + L.qkv);
    a.dout = reinterpret_cast<float*>(w + L.dout);
    a.o = reinterpret_cast<float*>(w + L.o);
    a.dqkv = reinterpret_cast<float*>(w + L.dqkv);
  }
  return from_hip(launch_backward(a, static_cast<hipStream_t>(stream)));
}

size_t swin_cpb_bwd_workspace_size(int hidden, int heads, int M) {
  if (hidden < 1 || hidden > 4096 || heads < 1 || heads > 64 || M < 1 || M > 32) return 0;
  return round_up((size_t)(2 * M - 1) * (2 * M - 1) * heads * sizeof(float), 256);
}

swin_status swin_cpb_bwd(const float* w1, const float* b1, const float* w2, const float* b2,
                         int hidden, int heads, int M, float coord_scale, const float* dtable,
                         float* dw1, float* db1, float* dw2, float* db2, void* workspace,
                         size_t ws_bytes, void* stream) {
  if (!w1 || !b1 || !w2 || !dtable || !dw1 || !db1 || !dw2 || !workspace) return SWIN_ERR_NULL;
  const size_t ws = swin_cpb_bwd_workspace_size(hidden, heads, M);
  if (ws == 0) return SWIN_ERR_SHAPE;
  if (ws_bytes < ws) return SWIN_ERR_WORKSPACE;
  const size_t tb = (size_t)(2 * M - 1) * (2 * M - 1) * heads * 4, hb = (size_t)hidden * 4;
  struct Span { const void* p; size_t n; };
  const Span outs[] = {{dw1, 2 * hb}, {db1, hb}, {dw2, heads * hb}, {db2, heads * 4u},
                       {workspace, ws}};
  const Span ins[] = {{w1, 2 * hb}, {b1, hb}, {w2, heads * hb}, {b2, heads * 4u}, {dtable, tb}};
  const int no = sizeof(outs) / sizeof(outs[0]), ni = sizeof(ins) / sizeof(ins[0]);
  for (int i = 0; i < no; ++i) {
    for (int j = 0; j < ni; ++j)
      if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return SWIN_ERR_ALIAS;
    for (int j = i + 1; j < no; ++j)
      if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return SWIN_ERR_ALIAS;
  }
  if (!(coord_scale > 0.0f)) coord_scale = M > 1 ? 8.0f / (float)(M - 1) : 1.0f;
  return from_hip(launch_cpb_bwd(w1, b1, w2, b2, hidden, heads, M, coord_scale, dtable, dw1, db1,
                                 dw2, db2, static_cast<float*>(workspace),
                                 static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// FP8 linear layers.

namespace {
bool valid_dt(int dt) { return dt == SWIN_F32 || dt == SWIN_F16 || dt == SWIN_BF16; }
int io_of(int dt) { return dt == SWIN_F32 ? kF32 : dt == SWIN_F16 ? kF16 : kBF16; }
}  // namespace

swin_status swin_fp8_quantize(const void* x, swin_dtype dt, int rows, int K,
                              unsigned char* codes, float* scales, void* stream) {
  if (!valid_dt(dt)) return SWIN_ERR_DTYPE;
  if (rows < 0 || K < 1 || K > 65536) return SWIN_ERR_SHAPE;
  if (rows == 0) return SWIN_OK;
  if (!x || !codes || !scales) return SWIN_ERR_NULL;
  const size_t xb = (size_t)rows * K * elem_bytes(dt), cb = (size_t)rows * K, sb = rows * 4u;
  if (overlap(codes, cb, x, xb) || overlap(scales, sb, x, xb) || overlap(codes, cb, scales, sb))
    return SWIN_ERR_ALIAS;
  if (!aligned16(x)) return SWIN_ERR_ALIGN;
  return from_hip(launch_fp8_quant(x, io_of(dt), rows, K, codes, scales,
                                   static_cast<hipStream_t>(stream)));
}

swin_status swin_fp8_linear(const unsigned char* a, const float* sa, const unsigned char* w,
                            const float* sw, const void* bias, swin_dtype bias_dt, void* y,
                            swin_dtype y_dt, int rows, int N, int K, void* stream) {
  if (!valid_dt(y_dt) || (bias && !valid_dt(bias_dt))) return SWIN_ERR_DTYPE;
  if (rows < 0 || N < 1 || K < 32 || K % 32 || K > 65536) return SWIN_ERR_SHAPE;
  if (rows == 0) return SWIN_OK;
  if (!a || !sa || !w || !sw || !y) return SWIN_ERR_NULL;
  const size_t yb = (size_t)rows * N * elem_bytes(y_dt);
  if (overlap(y, yb, a, (size_t)rows * K) || overlap(y, yb, w, (size_t)N * K) ||
      overlap(y, yb, sa, rows * 4u) || overlap(y, yb, sw, N * 4u) ||
      (bias && overlap(y, yb, bias, (size_t)N * elem_bytes(bias_dt))))
    return SWIN_ERR_ALIAS;
  if (!aligned16(a) || !aligned16(w)) return SWIN_ERR_ALIGN;
  Fp8Linear p{a, sa, w, sw, bias, bias ? io_of(bias_dt) : kF32, y, rows, N, K};
  return from_hip(launch_fp8_linear(p, io_of(y_dt), static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// 2:4 sparse linear layers.

swin_status swin_sparse24_compress(const void* w, swin_dtype dt, int N, int K, void* values,
                                   unsigned char* codes, void* stream) {
  if (dt != SWIN_F16 && dt != SWIN_BF16) return SWIN_ERR_DTYPE;
  if (N < 0 || K < 4 || K % 4) return SWIN_ERR_SHAPE;
  if (N == 0) return SWIN_OK;
  if (!w || !values || !codes) return SWIN_ERR_NULL;
  const size_t wb = (size_t)N * K * 2, vb = wb / 2, cb = (size_t)N * K / 4;
  if (overlap(values, vb, w, wb) || overlap(codes, cb, w, wb) || overlap(values, vb, codes, cb))
    return SWIN_ERR_ALIAS;
  return from_hip(launch_prune24(w, io_of(dt), N, K, values, codes,
                                 static_cast<hipStream_t>(stream)));
}

swin_status swin_sparse24_linear(const void* x, const void* values, const unsigned char* codes,
                                 const void* bias, void* y, swin_dtype dt, int rows, int N, int K,
                                 void* stream) {
  if (dt != SWIN_F16 && dt != SWIN_BF16) return SWIN_ERR_DTYPE;
  if (rows < 0 || N < 1 || K < 64 || K % 64) return SWIN_ERR_SHAPE;
  if (rows == 0) return SWIN_OK;
  if (!x || !values || !codes || !y) return SWIN_ERR_NULL;
  const size_t yb = (size_t)rows * N * 2;
  if (overlap(y, yb, x, (size_t)rows * K * 2) || overlap(y, yb, values, (size_t)N * K) ||
      overlap(y, yb, codes, (size_t)N * K / 4) || (bias && overlap(y, yb, bias, (size_t)N * 2)))
    return SWIN_ERR_ALIAS;
  // The tiled product reads the positions of 64 consecutive K with one
  // 16-byte load per output channel.
  if (!aligned16(x) || !aligned16(values) || !aligned16(codes)) return SWIN_ERR_ALIGN;
  Sparse24Linear p{x, values, codes, bias, y, rows, N, K};
  return from_hip(launch_sparse24_linear(p, io_of(dt), static_cast<hipStream_t>(stream)));
}
