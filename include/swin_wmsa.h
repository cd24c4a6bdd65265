/*
 * swin_wmsa.h -- C ABI of the gfx950 (MI355X) shifted-window multi-head
 * self-attention block forward (Swin V1 and V2).
 *
 * Every tensor pointer is a DEVICE pointer to a dense row-major array, unless
 * stated otherwise.  The caller owns every buffer (inputs, outputs and the
 * workspace); the library allocates no memory and keeps no state between calls,
 * so calls are reentrant and thread-safe.  `stream` is a hipStream_t passed as
 * void* (NULL = the null stream); every call only enqueues work on it and never
 * synchronises.  Arguments are validated on the host before anything is
 * launched: an invalid call returns its status code and enqueues nothing.  A
 * launch failure reported by the HIP runtime returns SWIN_ERR_HIP.  No C++
 * exception crosses this interface.
 *
 * Geometry used throughout:
 *   x    [B, H, W, C] tokens, channels last.
 *   M    window side, M >= 2; a window holds N = M*M tokens; nW = (H/M)*(W/M)
 *        windows per image.  Requires H % M == 0 and W % M == 0 (else
 *        SWIN_ERR_SHAPE).
 *   s    cyclic shift, 0 <= s < M.  Shifted-frame position (y', x') holds
 *        original position ((y'+s) mod H, (x'+s) mod W).
 *   Window w = b*nW + wy*(W/M) + wx; in-window token t = ty*M + tx; window
 *   slot (w, t) holds shifted-frame position (wy*M+ty, wx*M+tx).
 */
#ifndef SWIN_WMSA_H
#define SWIN_WMSA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWIN_WMSA_ABI_VERSION 1

typedef enum {
  SWIN_OK = 0,
  SWIN_ERR_NULL = 1,        /* a required pointer is NULL                          */
  SWIN_ERR_SHAPE = 2,       /* sizes inconsistent (H % M, W % M, s range, C % heads) */
  SWIN_ERR_DTYPE = 3,       /* unknown dtype or mode value                         */
  SWIN_ERR_UNSUPPORTED = 4, /* valid but not implemented (head dim != 32, large M) */
  SWIN_ERR_ALIAS = 5,       /* an output overlaps an input or the workspace        */
  SWIN_ERR_WORKSPACE = 6,   /* workspace smaller than swin_wmsa_workspace_size()   */
  SWIN_ERR_ALIGN = 7,       /* a pointer is not 16-byte aligned                    */
  SWIN_ERR_HIP = 8,         /* the HIP runtime reported an error at launch         */
  SWIN_ERR_SCRATCH = 9      /* swin_wmsa_fwd_noalloc: the call needs more scratch
                               than SWIN_NOALLOC_SCRATCH_BYTES                      */
} swin_status;

typedef enum { SWIN_F32 = 0, SWIN_F16 = 1, SWIN_BF16 = 2 } swin_dtype;
typedef enum { SWIN_V1 = 1, SWIN_V2 = 2 } swin_mode;

typedef struct {
  int B, H, W, C, heads, M, s;
  int mode;      /* swin_mode                                                  */
  int dtype;     /* swin_dtype of x, y, the weights and the linear biases      */
  float scale;   /* V1 logit multiplier; <= 0 selects (C/heads)^-1/2           */
  float tau_min; /* V2 lower clip of tau; <= 0 selects 0.01                    */
} swin_wmsa_desc;

/* Human-readable name of a status code (static string, never NULL). */
const char* swin_status_str(swin_status s);

/* SWIN_WMSA_ABI_VERSION of the built library. */
int swin_abi_version(void);

/* The HIP runtime's description of the last HIP error that an entry point
 * returned as SWIN_ERR_HIP on the calling thread ("no error" before any);
 * a static string, never NULL.  Kept per thread until the next such error. */
const char* swin_last_hip_error(void);

/*
 * Cyclic shift + window partition ("Boosting Swin Transformer Speed:
 * Profiling, Mixed Precision, and Kernel Fusion Secrets", Training Optimization:
 * window partition / shift are index-mapping operations).
 *   x  [B, H, W, C]        input, element type dt (only its size matters).
 *   xw [B*nW, M*M, C]      output; xw[w, t, :] = x[b, (wy*M+ty+s) mod H,
 *                          (wx*M+tx+s) mod W, :].  A bit-exact permutation.
 * xw must not overlap x (SWIN_ERR_ALIAS).  B == 0 is a no-op.
 */
swin_status swin_partition_shift(const void* x, void* xw, int B, int H, int W, int C,
                                 int M, int s, swin_dtype dt, void* stream);

/*
 * Window reverse + inverse shift, the exact inverse of swin_partition_shift
 * (same page and section).  xw [B*nW, M*M, C] -> x [B, H, W, C].
 */
swin_status swin_reverse_unshift(const void* xw, void* x, int B, int H, int W, int C,
                                 int M, int s, swin_dtype dt, void* stream);

/*
 * V2 continuous position bias table ("Swin Transformer V2" research summary,
 * How It Works: a meta-network on log-spaced relative coordinates outputs the
 * bias).  For every offset (dy, dx) in [-(M-1), M-1]^2, row r = (dy+M-1)*(2M-1)
 * + (dx+M-1):
 *   u = coord_scale * (dy, dx)          (coord_scale <= 0 selects 8/(M-1))
 *   g = sign(u) * log2(1 + |u|) / 3     (per component; log2(8) = 3)
 *   table[r, h] = 16 * sigmoid( w2[h, :] . relu(w1 g + b1) + b2[h] )
 *   w1 [hidden, 2] (columns dy, dx), b1 [hidden], w2 [heads, hidden],
 *   b2 [heads] or NULL (no second bias); table [(2M-1)^2, heads].  All float32.
 * hidden in 1..4096, heads in 1..64, M in 2..32 (else SWIN_ERR_SHAPE); table
 * must not overlap an input (SWIN_ERR_ALIAS).
 */
swin_status swin_cpb_table(const float* w1, const float* b1, const float* w2,
                           const float* b2, int hidden, int heads, int M,
                           float coord_scale, float* table, void* stream);

/*
 * Workspace bytes swin_wmsa_fwd needs for this descriptor (0 for an invalid
 * descriptor or B == 0).  The workspace holds per-window intermediates (Q, K,
 * V and the attention output), is overwritten by every call and must not be
 * shared by calls that may run concurrently.
 */
size_t swin_wmsa_workspace_size(const swin_wmsa_desc* d);

/*
 * Shifted-window multi-head self-attention block forward (attention sub-layer
 * only: no LayerNorm, residual or MLP).
 *   Pages: "Boosting Swin Transformer Speed" -- Introduction (windowed
 *   attention with shifted windows), Training / Inference Optimization (index
 *   maps, QKV GEMM + bias + softmax fused, no transposes); "Boost Vision
 *   Transformer with GPU-Friendly Sparsity and Quantization" -- Section 3.2 and
 *   Figure 3 (Q/K/V and output projections are GEMMs); "Swin Transformer V2"
 *   summary -- How It Works (V1 relative position bias, V2 scaled cosine
 *   attention with tau clipped at 0.01 plus bias B_ij).
 *
 *   x       [B, H, W, C]   input tokens, desc->dtype.
 *   w_qkv   [3C, C]        rows 0..C-1 = q, C..2C-1 = k, 2C..3C-1 = v (out x in);
 *                          head h uses rows h*d..h*d+d-1 of each block, d = C/heads.
 *   b_qkv   [3C] or NULL   (NULL = zeros).
 *   w_proj  [C, C], b_proj [C] or NULL.
 *   bias_table [(2M-1)^2, heads] float32: V1 learned table or V2 CPB table;
 *           query i, key j of a window read row (ty_i-ty_j+M-1)*(2M-1) +
 *           (tx_i-tx_j+M-1).
 *   tau     [heads] float32, V2 only (raw; max(tau, tau_min) is used); may be
 *           NULL in V1.
 *   y       [B, H, W, C]   output, desc->dtype.  Neither y nor the workspace may
 *           overlap any input (x, the weights, the biases, bias_table, tau) or
 *           each other (SWIN_ERR_ALIAS).
 *   workspace, ws_bytes    at least swin_wmsa_workspace_size(desc) bytes.
 * Per window, with q, k, v the projections of the window's tokens:
 *   V1: logit(i,j) = scale * q_h(i).k_h(j) + table[idx(i,j), h]
 *   V2: logit(i,j) = cos(q_h(i), k_h(j)) / max(tau_h, tau_min) + table[idx(i,j), h]
 *   with s > 0, pairs whose shifted-frame region labels differ get weight 0
 *   (along an axis of length L: slice 0 for v < L-M, 1 for v < L-s, else 2;
 *   label = 3*slice_y + slice_x); softmax over the remaining keys; head outputs
 *   concatenated, projected, and written back at the un-shifted position.
 * Computes in float32 for SWIN_F32; for SWIN_F16 / SWIN_BF16 the products run on
 * 16-bit matrix cores with float32 accumulation and float32 softmax.
 * Requires C/heads == 32 and M <= 24 (16-bit) or M <= 16 (float32), else
 * SWIN_ERR_UNSUPPORTED.
 */
swin_status swin_wmsa_fwd(const swin_wmsa_desc* desc, const void* x, const void* w_qkv,
                          const void* b_qkv, const void* w_proj, const void* b_proj,
                          const float* bias_table, const float* tau, void* y,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * Number of kernels swin_wmsa_fwd enqueues for this descriptor (0 if invalid or
 * B == 0), and the function name (no namespace or template arguments) of the
 * i-th one, as profilers print it inside the full name (NULL if out of range).
 * Lets a profiler match per-kernel traces to the stages of the forward.
 */
int swin_wmsa_kernel_count(const swin_wmsa_desc* d);
const char* swin_wmsa_kernel_name(const swin_wmsa_desc* d, int i);

/*
 * swin_wmsa_fwd plus per-kernel timing: records events[0] on `stream` before the
 * first kernel and events[i+1] right after the i-th kernel.  `events` holds
 * n_events caller-created hipEvent_t handles (passed as void*), n_events >=
 * swin_wmsa_kernel_count(desc) + 1, else SWIN_ERR_SHAPE.  Same arguments,
 * validation and results as swin_wmsa_fwd (page citations there).
 */
swin_status swin_wmsa_fwd_timed(const swin_wmsa_desc* desc, const void* x, const void* w_qkv,
                                const void* b_qkv, const void* w_proj, const void* b_proj,
                                const float* bias_table, const float* tau, void* y,
                                void* workspace, size_t ws_bytes, void* stream,
                                void* const* events, int n_events);

/*
 * swin_wmsa_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * workspace is the library's own fixed device array of
 * SWIN_NOALLOC_SCRATCH_BYTES per GPU (a file-scope static, held by every GPU the
 * library runs on until the process ends), instead of a caller buffer.  Same
 * arguments (minus workspace / ws_bytes), validation, kernels and results as
 * swin_wmsa_fwd; the caller still passes inputs and outputs.  A descriptor
 * whose swin_wmsa_workspace_size exceeds SWIN_NOALLOC_SCRATCH_BYTES returns
 * SWIN_ERR_SCRATCH and launches nothing.  Nothing here calls hipMalloc / hipFree
 * or an allocating library routine; the array's device address is looked up
 * (hipGetSymbolAddress) on the first call on each device, with that device
 * current.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind: calls that may overlap on one GPU (several streams or
 * threads) race and must be serialised by the caller.
 */
#define SWIN_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
swin_status swin_wmsa_fwd_noalloc(const swin_wmsa_desc* desc, const void* x, const void* w_qkv,
                                  const void* b_qkv, const void* w_proj, const void* b_proj,
                                  const float* bias_table, const float* tau, void* y,
                                  void* stream);

/*
 * Full block forward around the attention sub-layer.
 *   Pages: "Boost Vision Transformer with GPU-Friendly Sparsity and
 *   Quantization" -- Section 3.2 / Figure 3 (the Swin block is the standard
 *   transformer block with shifted-window attention in place of multi-head
 *   attention; the feed-forward layers are GEMMs) and Section 2.2 (GeLU);
 *   "Boosting Swin Transformer Speed", Training Optimization (LayerNorm in the
 *   block); "Swin Transformer V2" summary, How It Works (V1 pre-norm, V2
 *   residual post-norm).
 *   V1 (attn.mode == SWIN_V1):  h = x + A(LN1(x)),  y = h + F(LN2(h))
 *   V2 (attn.mode == SWIN_V2):  h = x + LN1(A(x)),  y = h + LN2(F(h))
 *   A = swin_wmsa_fwd with `attn` and the attention parameters below;
 *   LN(v) = (v - mean) / sqrt(var + ln_eps) * gamma + beta over the C channels
 *   of a token (biased variance); F(u) = GELU(u fc1_w^T + fc1_b) fc2_w^T + fc2_b
 *   with the exact GELU v * Phi(v).
 * Parameters (device pointers, attn.dtype unless noted): the attention's as in
 * swin_wmsa_fwd; ln1_g, ln1_b, ln2_g, ln2_b [C]; fc1_w [hidden, C], fc1_b
 * [hidden] or NULL; fc2_w [C, hidden], fc2_b [C] or NULL.
 *   x, y [B, H, W, C].  Neither y nor the workspace may overlap any input (x and
 *   every parameter pointer) or each other (SWIN_ERR_ALIAS).
 *   workspace, ws_bytes >= swin_block_workspace_size(desc): the attention's
 *   workspace plus four intermediates (three [B*H*W, C], one [B*H*W, hidden]).
 * Requires a valid attention descriptor, hidden a multiple of 32 (<= 16384),
 * C <= 512 (else SWIN_ERR_UNSUPPORTED), x, y, the workspace, the weights and the
 * LayerNorm parameters 16-byte aligned (else SWIN_ERR_ALIGN); LayerNorms and
 * GELU in float32; the intermediates are stored in attn.dtype.
 */
typedef struct {
  swin_wmsa_desc attn;
  int hidden;     /* MLP hidden width (4C in the usual block)                  */
  float ln_eps;   /* LayerNorm epsilon; <= 0 selects 1e-5                      */
} swin_block_desc;

typedef struct {
  const void *w_qkv, *b_qkv, *w_proj, *b_proj;
  const float *bias_table, *tau;
  const void *ln1_g, *ln1_b, *ln2_g, *ln2_b;
  const void *fc1_w, *fc1_b, *fc2_w, *fc2_b;
} swin_block_params;

/* Workspace bytes of swin_block_fwd (0 for an invalid descriptor or B == 0). */
size_t swin_block_workspace_size(const swin_block_desc* d);

swin_status swin_block_fwd(const swin_block_desc* d, const void* x, const swin_block_params* p,
                           void* y, void* workspace, size_t ws_bytes, void* stream);

/*
 * Backward pass of the attention sub-layer (training).
 *   Pages: "Boosting Swin Transformer Speed", Training Optimization (the fused
 *   MHA and the shift / partition kernels are training speed-ups, so the
 *   sub-layer is differentiated through the projection, both attention
 *   products, the softmax with bias and mask, the QKV projection and the index
 *   maps); "Swin Transformer V2" summary, How It Works (cosine logits over
 *   max(tau, 0.01) plus the position bias).
 * Given dy = dL/dy for y = swin_wmsa_fwd(desc, x, ...), writes the gradients of
 * x (desc->dtype, [B, H, W, C]) and, in float32, of w_qkv [3C, C], b_qkv [3C],
 * w_proj [C, C], b_proj [C], the bias table [(2M-1)^2, heads] (V2: the table
 * the forward consumes, i.e. the CPB output) and (V2) tau [heads]; the tau
 * gradient is 0 for a head whose tau <= tau_min (the clamp is flat there).
 * Every gradient output is overwritten (not accumulated into).  Inputs as in
 * swin_wmsa_fwd (b_qkv may be NULL = zero; b_proj does not enter the gradients).
 *   workspace, ws_bytes >= swin_wmsa_bwd_workspace_size(desc): x and dy in
 *   window order, the recomputed q | k | v and attention output and their
 *   gradients (float32); overwritten by every call.
 * Requires a descriptor valid as for swin_wmsa_fwd, except that M <= 24 for
 * every dtype (else SWIN_ERR_UNSUPPORTED);
 * x, dy, dx, w_qkv, w_proj and the workspace 16-byte aligned (SWIN_ERR_ALIGN);
 * no output overlapping an input, another output or the workspace
 * (SWIN_ERR_ALIAS); dtau non-NULL in V2.  Intermediates and sums in float32;
 * the GEMMs on 16-bit matrix cores with float32 accumulation (exact products
 * when both operands share a 16-bit type, else each operand as two bfloat16
 * terms, about 2^-16 relative per product); the attention on float32 products.
 */
typedef struct {
  void* dx;        /* [B, H, W, C], desc->dtype                      */
  float* dw_qkv;   /* [3C, C]                                        */
  float* db_qkv;   /* [3C]                                           */
  float* dw_proj;  /* [C, C]                                         */
  float* db_proj;  /* [C]                                            */
  float* dtable;   /* [(2M-1)^2, heads]                              */
  float* dtau;     /* [heads]; V2 only (ignored and may be NULL in V1) */
} swin_wmsa_grads;

/*
 * Backward of the V2 meta-network (same page and section as swin_cpb_table):
 * given dtable = dL/dtable [(2M-1)^2, heads] (e.g. from swin_wmsa_bwd), writes
 * dw1 [hidden, 2], db1 [hidden], dw2 [heads, hidden] and db2 [heads] (NULL
 * allowed: then not written) for the table of swin_cpb_table with the same
 * w1, b1, w2, b2, M and coord_scale.  Reading: ReLU'(0) = 0.  Every output is
 * overwritten.  All float32; hidden in 1..4096, heads in 1..64, M in 1..32
 * (else SWIN_ERR_SHAPE); workspace, ws_bytes >= swin_cpb_bwd_workspace_size
 * (the sigmoid-side gradient, (2M-1)^2 x heads floats); no output may overlap
 * an input, another output or the workspace (SWIN_ERR_ALIAS).
 */
size_t swin_cpb_bwd_workspace_size(int hidden, int heads, int M);

swin_status swin_cpb_bwd(const float* w1, const float* b1, const float* w2, const float* b2,
                         int hidden, int heads, int M, float coord_scale, const float* dtable,
                         float* dw1, float* db1, float* dw2, float* db2, void* workspace,
                         size_t ws_bytes, void* stream);

/*
 * FP8 linear layers for the QKV and projection GEMMs.
 *   Page: "Boosting Swin Transformer Speed", Inference Optimization (those GEMMs
 *   in 8 bits with per-channel scales; the MI355X's native 8-bit float takes
 *   the place of 8-bit integers).
 * Format: OCP FP8 E4M3 (exponent bias 7, 3 mantissa bits, largest finite 448,
 * subnormals k * 2^-9).
 *
 * swin_fp8_quantize: per row r of x [rows, K] (dtype dt): amax = max |x[r]|,
 * scales[r] = amax / 448 and inv = 448 / amax (1 and 1 when amax = 0), codes
 * [rows, K] = E4M3(x * inv) to nearest, ties to even, after clamping to
 * +-448, sign bit set when x * inv < 0; every step in float32.  For an
 * activation the rows are tokens; for a weight [out, in] the rows are output
 * channels.  rows >= 0, 1 <= K <= 65536 (else SWIN_ERR_SHAPE); x 16-byte
 * aligned (SWIN_ERR_ALIGN); codes, scales must not overlap x or each other
 * (SWIN_ERR_ALIAS).
 *
 * swin_fp8_linear: y [rows, N] (y_dt) = (dec(a) dec(w)^T) * sa[:, None] *
 * sw[None, :] + bias[None, :] with a [rows, K] and w [N, K] codes, sa [rows],
 * sw [N] from swin_fp8_quantize, bias [N] (bias_dt) or NULL; products
 * accumulate in float32.  K a multiple of 32, N >= 1, rows >= 0 (else
 * SWIN_ERR_SHAPE); a, w 16-byte aligned (SWIN_ERR_ALIGN); y must not overlap
 * an input (SWIN_ERR_ALIAS).
 */
swin_status swin_fp8_quantize(const void* x, swin_dtype dt, int rows, int K,
                              unsigned char* codes, float* scales, void* stream);

swin_status swin_fp8_linear(const unsigned char* a, const float* sa, const unsigned char* w,
                            const float* sw, const void* bias, swin_dtype bias_dt, void* y,
                            swin_dtype y_dt, int rows, int N, int K, void* stream);

/*
 * 2:4 structured-sparse linear layers for the QKV and projection GEMMs.
 *   Page: "Boost Vision Transformer with GPU-Friendly Sparsity and
 *   Quantization", Section 3.1 / Figure 1 (two of every four consecutive
 *   weights along the reduction dimension kept, stored as values plus
 *   positions, run on sparse matrix cores) and Section 3.2 / Figure 3 (the
 *   QKV, projection and feed-forward GEMMs).
 *
 * swin_sparse24_compress: w [N, K] (dt float16 or bfloat16) -> values [N, K/2]
 * (dt; the two kept weights of each group of four along K, the lower position
 * first) and codes [N, K/4] bytes (positions p0 | p1 << 2, p0 < p1).  Kept:
 * the two largest magnitudes of the group (ties: the lower position).  K a
 * multiple of 4, N >= 0 (SWIN_ERR_SHAPE); float32 is SWIN_ERR_DTYPE; outputs
 * must not overlap w or each other (SWIN_ERR_ALIAS).
 *
 * swin_sparse24_linear: y [rows, N] = x [rows, K] wp^T + bias (dt, float32
 * accumulation), wp the dense matrix the compressed form describes; bias [N]
 * or NULL.  K a multiple of 64, N >= 1, rows >= 0 (SWIN_ERR_SHAPE); x, values
 * and codes 16-byte aligned (SWIN_ERR_ALIGN); y must not overlap
 * an input (SWIN_ERR_ALIAS).
 */
swin_status swin_sparse24_compress(const void* w, swin_dtype dt, int N, int K, void* values,
                                   unsigned char* codes, void* stream);

swin_status swin_sparse24_linear(const void* x, const void* values, const unsigned char* codes,
                                 const void* bias, void* y, swin_dtype dt, int rows, int N, int K,
                                 void* stream);

/* Workspace bytes of swin_wmsa_bwd (0 for an invalid descriptor or B == 0). */
size_t swin_wmsa_bwd_workspace_size(const swin_wmsa_desc* desc);

swin_status swin_wmsa_bwd(const swin_wmsa_desc* desc, const void* x, const void* w_qkv,
                          const void* b_qkv, const void* w_proj, const float* bias_table,
                          const float* tau, const void* dy, const swin_wmsa_grads* grads,
                          void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIN_WMSA_H */
