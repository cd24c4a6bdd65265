// QKV and output projection GEMMs for 16-bit I/O and C a multiple of 128: large
// output tiles on the matrix cores, operands streamed global -> LDS by
// direct-to-LDS loads into a double buffer.
//
// "Boost Vision Transformer with GPU-Friendly Sparsity and Quantization",
// Section 3.2 / Figure 3: Q/K/V and the output projection are GEMMs.
// "Boosting Swin Transformer Speed", Inference Optimization (GEMM with its bias
// fused, no separate transposes) and Training Optimization (shift / partition /
// reverse folded into the neighbouring ops): the A rows of the QKV GEMM are
// gathered from x through the cyclic shift + window partition map, and the
// projection stores each row at its un-shifted token position.
//
// Tile BM x BN, K in stages of 64 (128 bytes per row).  Each wave instruction
// of `global_load_lds_dwordx4` fills 1 KB of LDS = 8 rows of a stage; lane L
// lands at row L/8, 16-byte slot L%8, and fetches source chunk
// (L%8) ^ (row%8), so that a stage row holds its eight chunks XOR-swizzled and
// the 16 rows of a matrix-core fragment read conflict-free.
//
// Persistent workgroups, one per CU, walk their tiles as one continuous
// sequence of stages, so the loads of the next tile's first stages overlap the
// current tile's last stages and its epilogue.  Two LDS buffers: the loads of
// stage s+2 go out mid-stage s (after the barrier that publishes stage s+1),
// and the A rows of stage s+4 are touched with a 4-byte load per row so that
// they are in L2 by the time their stage is loaded.  Workgroups reach the 8
// XCDs (each with its own L2) round-robin; every XCD walks a contiguous range
// of tiles, column tiles fastest, so the workgroups running together on one
// XCD share their A rows, and A is read from HBM about once.
//
// Orientation.  The products are formed as C^T (the weight fragment is the
// MFMA's A operand) with the weight rows of each pair of 16-channel tiles
// interleaved, so a lane holds 8 consecutive channels of one token: one
// 16-byte store, and V2 normalises a head with a 4-lane reduction.
#include "common.hpp"
#include "launch.hpp"

namespace swin {

namespace {

typedef __attribute__((address_space(3))) void* lds_vptr;

constexpr int kStageK = 64;
constexpr int kPrefetch = 4;  // stages ahead for the L2 touch of A

template <int BM, int BN, int WGM, int WGN>
struct Cfg {
  static constexpr int WAVES = WGM * WGN;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_INS = BM / 8 / WAVES;  // 1 KB wave instructions per stage
  static constexpr int B_INS = BN / 8 / WAVES;
  static constexpr int SMEM = 2 * STAGE + 4 * WAVES * 64;  // + touch-load sink
  static_assert(BM % (8 * WAVES) == 0 && BN % (8 * WAVES) == 0, "load split");
  static_assert(WM % 16 == 0 && WN % 32 == 0, "wave tile");
};

// vmcnt(n) and lgkmcnt(0): all but the last n global loads of this wave have
// landed, and so have all of its LDS reads (gfx9 encoding: vmcnt low bits
// [3:0] and high bits [15:14], expcnt [6:4] left at 7, lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Source byte offsets of one tile for this lane (stage 0): its A load rows
// (gathered: one offset per row; linear: row i adds i * 8 rows, folded into
// the scalar offset), its first B load row (the others follow linearly) and
// the A row it touches for L2.  Rows past the end of A read zeros (the buffer
// resource's bound).
template <int AI, bool LINEAR>
struct TileSrc {
  uint32_t a[LINEAR ? 1 : AI], b, touch;
};

// Row r of a stage is filled by wave instruction r / 8, lane 8*(r%8) + slot;
// the lane fetches chunk (L%8) ^ (L/8), i.e. (slot) ^ (row % 8).
template <int INS>
__device__ __forceinline__ int load_row(int i) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave * INS + i) * 8 + (lane >> 3);
}
__device__ __forceinline__ uint32_t load_chunk_bytes() {
  const int lane = threadIdx.x & 63;
  return (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
}

// Tiles of this workgroup: XCD x = id % 8 owns the contiguous range
// [x*per + min(x, rem), ...) of the row-major tile order; its workgroups take
// every (workgroups on x)-th tile of the range.
struct TileWalk {
  int first, stride, count;
};
__device__ __forceinline__ TileWalk tile_walk(int ntiles) {
  const int G = gridDim.x, id = blockIdx.x;
  const int nx = G < 8 ? G : 8;
  const int x = id % nx, j = id / nx;
  const int wpx = (G - x + nx - 1) / nx;  // workgroups on XCD x
  const int per = ntiles / nx, rem = ntiles % nx;
  const int start = x * per + min(x, rem), cnt = per + (x < rem ? 1 : 0);
  TileWalk t;
  t.first = start + j;
  t.stride = wpx;
  t.count = j < cnt ? (cnt - j + wpx - 1) / wpx : 0;
  return t;
}

// Tile count of the XCD's first workgroup (the largest).
__device__ __forceinline__ int tile_walk_first_count(int ntiles) {
  const int G = gridDim.x, id = blockIdx.x;
  const int nx = G < 8 ? G : 8;
  const int x = id % nx;
  const int wpx = (G - x + nx - 1) / nx;
  const int cnt = ntiles / nx + (x < ntiles % nx ? 1 : 0);
  return (cnt + wpx - 1) / wpx;
}

// The persistent main loop.  src(tile, TileSrc&) fills the source offsets of a
// tile, epi(tile, acc) consumes its accumulators.  With EPI_VM > 0, epi returns
// the number of vector-memory instructions it issued (stores only); when that
// is exactly EPI_VM, the next tile's first wait lets them stay in flight (they
// were issued after the loads it waits for), so the stores drain while stage 0
// is multiplied instead of stalling every workgroup at once.  acc[i][j] covers token tile
// i x channel tile j in C^T form; the weight rows of each pair of channel
// tiles are interleaved so that lane l holds token 16i + l%16 and channels
// 32(j/2) + 8(l/16) + 4(j%2) + r: 8 consecutive channels, one 16-byte store.
template <typename T, int BM, int BN, int WGM, int WGN, int NK, bool LINEAR, int EPI_VM = 0,
          class SrcFn, class EpiFn>
__device__ __forceinline__ void run_tiles(const char* __restrict__ A, uint32_t a_bytes,
                                          const char* __restrict__ Bw, uint32_t b_bytes,
                                          uint32_t rowbytes, char* smem, int ntiles, SrcFn src,
                                          EpiFn epi) {
  using G = Cfg<BM, BN, WGM, WGN>;
  using Src = TileSrc<G::A_INS, LINEAR>;
  static_assert(NK % 2 == 0 && NK >= kPrefetch, "stage parity and touch distance");
  static_assert(EPI_VM >= 0 && EPI_VM + 1 <= 63, "vmcnt range");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
  const TileWalk tw = tile_walk(ntiles);
  if (tw.count <= 0) return;
  if constexpr (EPI_VM > 0) {
    // Workgroups with one tile fewer than the first of their XCD start about
    // half a tile later (NK stages at about 2048 cycles each, halved; they
    // would wait at the end anyway): their epilogue stores then go out while
    // the others multiply, instead of every workgroup storing at once.
    if (tw.count < tile_walk_first_count(ntiles))
      for (int i = 0; i < NK / 2; ++i) __builtin_amdgcn_s_sleep(64);
  }

  // Buffer resources (raw, bounds = the whole tensor): the lane offset is a
  // 32-bit VGPR, the stage offset a scalar, so a load costs no vector ALU.
  // The loads are issued as inline assembly (common.hpp): the compiler, which
  // would see an LDS write, otherwise waits for each stage's loads right after
  // issuing them (before the next fragment reads), and the pipeline is gone.
  // Every wait is explicit (wait_vm, then a barrier).
  const i32x4 ra = make_rsrc(A, a_bytes);
  const i32x4 rbw = make_rsrc(Bw, b_bytes);
  const uint32_t smem_a = lds_addr(smem);
  auto dma = [&](const Src& sr, int buf, int k) {
    const uint32_t sa = smem_a + buf * G::STAGE;
    const uint32_t sb = sa + G::A_BYTES;
#pragma unroll
    for (int i = 0; i < G::A_INS; ++i)
      lds_dma16(ra, sa + (wave * G::A_INS + i) * 1024, sr.a[LINEAR ? 0 : i],
                k * (kStageK * 2) + (LINEAR ? i * 8 * rowbytes : 0));
#pragma unroll
    for (int i = 0; i < G::B_INS; ++i)
      lds_dma16(rbw, sb + (wave * G::B_INS + i) * 1024, sr.b, k * (kStageK * 2) + i * 8 * rowbytes);
  };
  // One 4-byte load per A row of stage k: the line lands in L2 (and a
  // throw-away LDS sink); nothing reads it.
  auto touch = [&](const Src& sr, int k) {
    lds_dma4(ra, smem_a + 2 * G::STAGE + wave * 256, sr.touch, k * (kStageK * 2));
  };

  // Fragment lane offsets inside a 32-row pair of tiles: row (t = tile parity)
  // 16t + l%16 for the token rows, 8(l%16 / 4) + 4t + l%4 for the weight rows
  // (they become the MFMA output rows); 16-byte chunk 4kk + l/16, swizzled by
  // row % 8.
  const int i16 = lane & 15, g4 = lane >> 4;
  auto lane_off = [&](bool perm, int t, int kk) -> uint32_t {
    const int row = perm ? 8 * (i16 >> 2) + 4 * t + (i16 & 3) : 16 * t + i16;
    return (uint32_t)row * 128 + ((uint32_t)((4 * kk + g4) ^ (row & 7)) << 4);
  };
  uint32_t offa[2][2], offb[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      offa[t][kk] = lane_off(false, t, kk);
      offb[t][kk] = lane_off(true, t, kk);
    }
  auto stage_a = [&](int buf) { return smem + buf * G::STAGE + wm * G::WM * 128; };
  auto stage_b = [&](int buf) { return smem + buf * G::STAGE + G::A_BYTES + wn * G::WN * 128; };
  auto read_frags = [&](int buf, int kk, vec8<T>(&af)[G::TM], vec8<T>(&bf)[G::TN]) {
    const char* sa = stage_a(buf);
    const char* sb = stage_b(buf);
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
      af[i] = *reinterpret_cast<const vec8<T>*>(sa + (i >> 1) * 4096 + offa[i & 1][kk]);
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
      bf[j] = *reinterpret_cast<const vec8<T>*>(sb + (j >> 1) * 4096 + offb[j & 1][kk]);
  };
  f32x4 acc[G::TM][G::TN];
  auto multiply = [&](const vec8<T>(&af)[G::TM], const vec8<T>(&bf)[G::TN]) {
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j) acc[i][j] = mma_16x16x32(bf[j], af[i], acc[i][j]);
  };

  Src cur, nxt;
  int tile = tw.first;
  src(tile, cur);
  src(tw.count > 1 ? tile + tw.stride : tile, nxt);
  // Prologue: stage 0 and the touches of stages 2, 3; then stage 1.  The wait
  // rule below (vmcnt(1)) relies on exactly one touch following every stage's
  // loads.
  dma(cur, 0, 0);
  touch(cur, 2);
  wait_vm<1>();
  __syncthreads();
  vec8<T> af0[G::TM], bf0[G::TN], af1[G::TM], bf1[G::TN];
  read_frags(0, 0, af0, bf0);
  read_frags(0, 1, af1, bf1);
  dma(cur, 1, 1);
  touch(cur, 3);

  int issued = -1;  // vector-memory instructions of the previous epilogue
  for (int it = 0; it < tw.count; ++it) {
    const bool more = it + 1 < tw.count;
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      __builtin_amdgcn_sched_barrier(0);
      multiply(af0, bf0);
      __builtin_amdgcn_sched_barrier(0);
      // This wave's loads of stage k+1 have landed (at k = 0 they are followed
      // by the touch and, possibly, the previous epilogue's EPI_VM stores).
      if (EPI_VM > 0 && k == 0 && issued == EPI_VM)
        wait_vm<1 + EPI_VM>();
      else
        wait_vm<1>();
      __syncthreads();  // ... everyone's; and buffer k%2 is free
      // Loads of stage k+2 (this tile or the next), touch of stage k+4.
      if (k + 2 < NK) dma(cur, k & 1, k + 2);
      else if (more) dma(nxt, k & 1, k + 2 - NK);
      if (k + kPrefetch < NK) touch(cur, k + kPrefetch);
      else touch(more ? nxt : cur, more ? k + kPrefetch - NK : NK - 1);
      if (k + 1 < NK) read_frags((k + 1) & 1, 0, af0, bf0);
      __builtin_amdgcn_sched_barrier(0);
      multiply(af1, bf1);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 1 < NK) read_frags((k + 1) & 1, 1, af1, bf1);
    }
    if constexpr (EPI_VM > 0)
      issued = epi(tile, acc);
    else
      epi(tile, acc);
    // The next tile's stage 0 (buffer 0) was published by the last barrier;
    // its fragments are read after the epilogue so that they do not occupy
    // registers during it (stale and unused after the last tile).
    __builtin_amdgcn_sched_barrier(0);
    read_frags(0, 0, af0, bf0);
    read_frags(0, 1, af1, bf1);
    tile += tw.stride;
    cur = nxt;
    if (it + 2 < tw.count) src(tile + tw.stride, nxt);
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8], float m) {
  vec8<T> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(v[e] * m);
  gstore16(p, __builtin_bit_cast(uint4, o));
}

// Eight consecutive linear-bias entries (element loads: the bias pointers
// carry no alignment promise beyond the element size).
template <typename T>
__device__ __forceinline__ void load_bias8(const T* b, int c, float (&o)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) o[r] = b ? (float)b[c + r] : 0.f;
}

// ---------------------------------------------------------------------------
// QKV projection: rows are window slots (gathered from x), columns 0..3C.
// ---------------------------------------------------------------------------
template <typename T, typename QT, int BM, int BN, int WGM, int WGN, int NK>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void qkv_tiled_kernel(FwdParams p) {
  using G = Cfg<BM, BN, WGM, WGN>;
  using Src = TileSrc<G::A_INS, false>;
  __shared__ __attribute__((aligned(1024))) char smem[G::SMEM];
  const Geom& g = p.g;
  const int rows = g.B * g.H * g.W;
  const int C = g.C;
  const int ncol = 3 * C / BN;
  const int ntiles = (rows + BM - 1) / BM * ncol;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
  const int g4 = lane >> 4, i16 = lane & 15;
  const uint32_t cb = load_chunk_bytes();
  const uint32_t rowbytes = (uint32_t)C * 2;

  auto src = [&](int tile, Src& sr) {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    const int m0 = rb * BM, n0 = cbk * BN;
#pragma unroll
    for (int i = 0; i < G::A_INS; ++i) {
      const int r = min(m0 + load_row<G::A_INS>(i), rows - 1);
      sr.a[i] = (uint32_t)src_token(g, r) * rowbytes + cb;
    }
    sr.b = (uint32_t)(n0 + load_row<G::B_INS>(0)) * rowbytes + cb;
    sr.touch = (uint32_t)src_token(g, min(m0 + (int)threadIdx.x % BM, rows - 1)) * rowbytes;
  };

  const T* bq = static_cast<const T*>(p.b_qkv);
  auto epi = [&](int tile, f32x4 (&acc)[G::TM][G::TN]) {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    const int m0 = rb * BM, n0 = cbk * BN;
    const int part = n0 / C;            // 0 = q, 1 = k, 2 = v (BN divides C)
    int c00 = n0 + wn * G::WN;  // first channel of this wave (a head start)
    int rbase = m0 + wm * G::WM;
    // Opaque here: keeps the epilogue's loads and row arithmetic from being
    // scheduled into the main loop, where they would hold registers.
    asm volatile("" : "+v"(rbase), "+s"(c00));
    const int h0 = (c00 - part * C) >> 5;
    constexpr int NH = G::TN / 2;
    // All loads first: under the in-order memory counter a load issued after
    // a store would make its wait cover that store too.
    float bias[NH][8], qm[NH];
#pragma unroll
    for (int jh = 0; jh < NH; ++jh) {
      load_bias8(bq, c00 + 32 * jh + 8 * g4, bias[jh]);
      qm[jh] = part != 0 ? 1.0f
                         : (p.v2 ? kLog2e / fmaxf(p.tau[h0 + jh], p.tau_min) : p.q_mult);
    }
    // lane: token 16i + i16; channels 32jh + 8 g4 + e of head h0 + jh.
    const bool norm = p.v2 && part < 2;
    const float eps2 = p.eps * p.eps;
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      const int row = rbase + 16 * i + i16;
      int w, t;
      row_wt(g, row, w, t);
      const bool ok = row < rows;
      // Element offset of (item = w*heads + h0, slot t, dim 8 g4) in a
      // [item][N][32] buffer; the next head adds N*32 (32-bit: tokens*C < 2^30).
      const uint32_t off = ((uint32_t)(w * g.heads + h0) * (uint32_t)g.N + (uint32_t)t) * 32u +
                           8u * (uint32_t)g4;
#pragma unroll
      for (int jh = 0; jh < NH; ++jh) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][2 * jh][r] + bias[jh][r];
          v[4 + r] = acc[i][2 * jh + 1][r] + bias[jh][4 + r];
        }
        float mult = qm[jh];
        if (norm) {
          // "Swin Transformer V2" summary, How It Works: cosine similarity over
          // tau (tau clipped at tau_min); 1/tau and log2(e) fold into q.
          // 1 / max(|v|, eps) = rsqrt(max(|v|^2, eps^2)).
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
          ss = xor32_sum(xor16_sum(ss));
          mult *= __builtin_amdgcn_rsqf(fmaxf(ss, eps2));
        }
        if (!ok) continue;
        const uint32_t o = off + (uint32_t)jh * (uint32_t)g.N * 32u;
        if (part < 2)
          store8(static_cast<QT*>(part == 0 ? p.buf.q : p.buf.k) + o, v, mult);
        else
          store8(static_cast<T*>(p.buf.v) + o, v, 1.0f);
      }
    }
  };
  run_tiles<T, BM, BN, WGM, WGN, NK, false>(static_cast<const char*>(p.x),
                                            (uint32_t)rows * rowbytes,
                                            static_cast<const char*>(p.w_qkv), 3 * C * rowbytes,
                                            rowbytes, smem, ntiles, src, epi);
}

// ---------------------------------------------------------------------------
// Output projection: rows are window slots of O, stored at their token in y.
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WGM, int WGN, int NK>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void proj_tiled_kernel(FwdParams p) {
  using G = Cfg<BM, BN, WGM, WGN>;
  using Src = TileSrc<G::A_INS, true>;
  constexpr int kMaxC = 512;  // tiled_gemm_supported
  __shared__ __attribute__((aligned(1024))) char smem[G::SMEM];
  __shared__ float bsm[kMaxC];  // the projection bias
  const Geom& g = p.g;
  const int rows = g.B * g.H * g.W;
  const int C = g.C;
  const int ncol = C / BN;
  const int ntiles = (rows + BM - 1) / BM * ncol;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
  const int g4 = lane >> 4, i16 = lane & 15;
  const uint32_t cb = load_chunk_bytes();
  const uint32_t rowbytes = (uint32_t)C * 2;

  auto src = [&](int tile, Src& sr) {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    const int m0 = rb * BM, n0 = cbk * BN;
    sr.a[0] = (uint32_t)(m0 + load_row<G::A_INS>(0)) * rowbytes + cb;
    sr.b = (uint32_t)(n0 + load_row<G::B_INS>(0)) * rowbytes + cb;
    sr.touch = (uint32_t)min(m0 + (int)threadIdx.x % BM, rows - 1) * rowbytes;
  };
  const T* bp = static_cast<const T*>(p.b_proj);
  T* y = static_cast<T*>(p.y);
  // Published by the first barrier of run_tiles.
  for (int i = threadIdx.x; i < C; i += G::THREADS) bsm[i] = bp ? (float)bp[i] : 0.f;
  constexpr int kStores = G::TM * (G::TN / 2);  // a full tile's stores per lane
  auto epi = [&](int tile, f32x4 (&acc)[G::TM][G::TN]) -> int {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    const int m0 = rb * BM, n0 = cbk * BN;
    int rbase = m0 + wm * G::WM + i16;
    int c00 = n0 + wn * G::WN;
    // Opaque here: keeps the epilogue's loads and row arithmetic from being
    // scheduled into the main loop, where they would hold registers.
    asm volatile("" : "+v"(rbase), "+s"(c00));
    c00 += 8 * g4;
    // Element offset of each row's un-shifted token (32-bit: tokens * C < 2^30).
    uint32_t dst[G::TM];
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      const int row = rbase + 16 * i;
      dst[i] = row < rows ? (uint32_t)src_token(g, row) * (uint32_t)C : 0xffffffffu;
    }
    float b[G::TN / 2][8];
#pragma unroll
    for (int jh = 0; jh < G::TN / 2; ++jh)
#pragma unroll
      for (int e = 0; e < 8; ++e) b[jh][e] = bsm[c00 + 32 * jh + e];
    // lane: token 16i + i16; channels 32jh + 8 g4 + e.  No loads from global
    // memory here: the stores are the only vector-memory instructions.
    int n = 0;
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      if (dst[i] == 0xffffffffu) continue;
      n += G::TN / 2;
#pragma unroll
      for (int jh = 0; jh < G::TN / 2; ++jh) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][2 * jh][r] + b[jh][r];
          v[4 + r] = acc[i][2 * jh + 1][r] + b[jh][4 + r];
        }
        store8(y + dst[i] + c00 + 32 * jh, v, 1.0f);
      }
    }
    // Per-lane count; EPI_VM needs the wave's count: rows past the end skip
    // stores in some lanes only, so a tile with any such row reports -1.
    return __builtin_amdgcn_readfirstlane(n) == kStores && __all(n == kStores) ? kStores : -1;
  };
  run_tiles<T, BM, BN, WGM, WGN, NK, true, kStores>(static_cast<const char*>(p.buf.o),
                                           (uint32_t)rows * rowbytes,
                                           static_cast<const char*>(p.w_proj), C * rowbytes,
                                           rowbytes, smem, ntiles, src, epi);
}

// ---------------------------------------------------------------------------
// Dense layer of the block's MLP: Y = act(A W^T + bias) (+ R), A [rows, K] and
// R / Y [rows, N] row-major, W [N, K] (nn.Linear layout).
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int WGM, int WGN, int NK, bool GELU, bool RES>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void dense_tiled_kernel(DenseParams d) {
  using G = Cfg<BM, BN, WGM, WGN>;
  using Src = TileSrc<G::A_INS, true>;
  __shared__ __attribute__((aligned(1024))) char smem[G::SMEM];
  const int rows = d.rows, N = d.N;
  const int ncol = N / BN;
  const int ntiles = (rows + BM - 1) / BM * ncol;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
  const int g4 = lane >> 4, i16 = lane & 15;
  const uint32_t cb = load_chunk_bytes();
  const uint32_t rowbytes = (uint32_t)NK * kStageK * 2;

  // Rows past the end of A read zeros (the buffer bound) and are not stored.
  auto src = [&](int tile, Src& sr) {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    const int m0 = rb * BM, n0 = cbk * BN;
    sr.a[0] = (uint32_t)(m0 + load_row<G::A_INS>(0)) * rowbytes + cb;
    sr.b = (uint32_t)(n0 + load_row<G::B_INS>(0)) * rowbytes + cb;
    sr.touch = (uint32_t)min(m0 + (int)threadIdx.x % BM, rows - 1) * rowbytes;
  };
  const T* bias = static_cast<const T*>(d.bias);
  const T* R = static_cast<const T*>(d.res);
  T* Y = static_cast<T*>(d.y);
  auto epi = [&](int tile, f32x4 (&acc)[G::TM][G::TN]) {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    const int m0 = rb * BM, n0 = cbk * BN;
    int rbase = m0 + wm * G::WM + i16;
    int c00 = n0 + wn * G::WN;
    // Opaque here: keeps the epilogue's loads and row arithmetic from being
    // scheduled into the main loop, where they would hold registers.
    asm volatile("" : "+v"(rbase), "+s"(c00));
    c00 += 8 * g4;
    float b[G::TN / 2][8];
#pragma unroll
    for (int jh = 0; jh < G::TN / 2; ++jh) load_bias8(bias, c00 + 32 * jh, b[jh]);
    // lane: row 16i + i16; columns 32jh + 8 g4 + e.
#pragma unroll
    for (int i = 0; i < G::TM; ++i) {
      const int row = rbase + 16 * i;
      if (row >= rows) continue;
#pragma unroll
      for (int jh = 0; jh < G::TN / 2; ++jh) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][2 * jh][r] + b[jh][r];
          v[4 + r] = acc[i][2 * jh + 1][r] + b[jh][4 + r];
        }
        const int64_t o = (int64_t)row * N + c00 + 32 * jh;
        if constexpr (GELU) {
          // GELU(v) = v * Phi(v) = v (1 + erf(v / sqrt 2)) / 2.
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.5f * v[e] * (1.0f + erff(v[e] * 0.70710678118654752f));
        }
        if constexpr (RES) {
          const vec8<T> rr = gload8(R + o);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += (float)rr[e];
        }
        store8(Y + o, v, 1.0f);
      }
    }
  };
  run_tiles<T, BM, BN, WGM, WGN, NK, true>(static_cast<const char*>(d.a), (uint32_t)rows * rowbytes,
                                           static_cast<const char*>(d.w), (uint32_t)N * rowbytes,
                                           rowbytes, smem, ntiles, src, epi);
}

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
  }
  return n;
}

int persistent_grid(int ntiles, int per_cu) {
  return ntiles < per_cu * num_cus() ? ntiles : per_cu * num_cus();
}

// Tiles: 256 x 256 (2 x 2 waves of 128 x 128) when there are at least two per
// CU; else 128 x 128 (2 x 2 waves of 64 x 64) so that small problems still
// spread over the chip.  K = C in 64-wide stages.
template <typename T, typename QT, int NK>
void qkv_tiled_launch(const FwdParams& p, hipStream_t st) {
  const int rows = p.g.B * p.g.H * p.g.W;
  const int big = (rows + 255) / 256 * (3 * p.g.C / 256);
  if (big >= 2 * num_cus()) {
    hipLaunchKernelGGL((qkv_tiled_kernel<T, QT, 256, 256, 2, 2, NK>), dim3(persistent_grid(big, 1)),
                       dim3(256), 0, st, p);
  } else {
    const int small = (rows + 127) / 128 * (3 * p.g.C / 128);
    hipLaunchKernelGGL((qkv_tiled_kernel<T, QT, 128, 128, 2, 2, NK>),
                       dim3(persistent_grid(small, 2)), dim3(256), 0, st, p);
  }
}

template <typename T, typename QT>
hipError_t qkv_tiled_dispatch(const FwdParams& p, hipStream_t st) {
  switch (p.g.C) {
    case 256: qkv_tiled_launch<T, QT, 4>(p, st); break;
    case 512: qkv_tiled_launch<T, QT, 8>(p, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int NK>
void proj_tiled_launch(const FwdParams& p, hipStream_t st) {
  const int rows = p.g.B * p.g.H * p.g.W;
  const int big = (rows + 255) / 256 * (p.g.C / 256);
  if (big >= 2 * num_cus()) {
    hipLaunchKernelGGL((proj_tiled_kernel<T, 256, 256, 2, 2, NK>), dim3(persistent_grid(big, 1)),
                       dim3(256), 0, st, p);
  } else {
    const int small = (rows + 127) / 128 * (p.g.C / 128);
    hipLaunchKernelGGL((proj_tiled_kernel<T, 128, 128, 2, 2, NK>), dim3(persistent_grid(small, 2)),
                       dim3(256), 0, st, p);
  }
}

template <typename T>
hipError_t proj_tiled_dispatch(const FwdParams& p, hipStream_t st) {
  switch (p.g.C) {
    case 256: proj_tiled_launch<T, 4>(p, st); break;
    case 512: proj_tiled_launch<T, 8>(p, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int NK, bool GELU, bool RES>
void dense_tiled_launch(const DenseParams& d, hipStream_t st) {
  const int big = (d.rows + 255) / 256 * (d.N / 256);
  if (d.N % 256 == 0 && big >= 2 * num_cus()) {
    hipLaunchKernelGGL((dense_tiled_kernel<T, 256, 256, 2, 2, NK, GELU, RES>),
                       dim3(persistent_grid(big, 1)), dim3(256), 0, st, d);
  } else {
    const int small = (d.rows + 127) / 128 * (d.N / 128);
    hipLaunchKernelGGL((dense_tiled_kernel<T, 128, 128, 2, 2, NK, GELU, RES>),
                       dim3(persistent_grid(small, 2)), dim3(256), 0, st, d);
  }
}

template <typename T, bool GELU, bool RES>
hipError_t dense_tiled_k(const DenseParams& d, hipStream_t st) {
  switch (d.K) {
    case 256: dense_tiled_launch<T, 4, GELU, RES>(d, st); break;
    case 512: dense_tiled_launch<T, 8, GELU, RES>(d, st); break;
    case 1024: dense_tiled_launch<T, 16, GELU, RES>(d, st); break;
    case 2048: dense_tiled_launch<T, 32, GELU, RES>(d, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dense_tiled_t(const DenseParams& d, bool gelu, hipStream_t st) {
  if (gelu && !d.res) return dense_tiled_k<T, true, false>(d, st);
  if (!gelu && d.res) return dense_tiled_k<T, false, true>(d, st);
  if (!gelu && !d.res) return dense_tiled_k<T, false, false>(d, st);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// FP8 (E4M3) linear layer, y = dec(a) dec(w)^T * sa[:, None] * sw[None, :] +
// bias (the codes and per-row scales of fp8.hip), on the same persistent,
// XCD-contiguous tile walk and direct-to-LDS stages: a 128-byte stage row is
// one 128-deep step of the 16x16x128 8-bit float products (unit block
// scales), whose operand lane holds 32 consecutive bytes (two swizzled 16-byte
// chunks) of one row.  256 x 128 tiles of 4 waves (128 x 64 each), one
// workgroup per CU (the accumulators and two fragment sets need 320
// registers); a stage's fragments are read while the previous stage is
// multiplied.  C^T orientation with the weight rows of each channel-tile pair
// interleaved, as above: a lane ends with 8 consecutive output channels.
// ---------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kFp8MaxN = 4096;  // output channels (column scales and bias in LDS)

template <typename TO, int NK>
__global__ __launch_bounds__(256, 1) void fp8_tiled_kernel(Fp8Linear p) {
  constexpr int BM = 256;
  using G = Cfg<BM, 128, 2, 2>;
  static_assert(NK % 2 == 0 && NK >= kPrefetch, "stage parity and touch distance");
  __shared__ __attribute__((aligned(1024))) char smem[G::SMEM];
  __shared__ float swsm[kFp8MaxN], bsm[kFp8MaxN];  // column scales and bias
  const int rows = (int)p.rows;
  const int ncol = p.N / 128;
  const int ntiles = (rows + BM - 1) / BM * ncol;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int i16 = lane & 15, g4 = lane >> 4;
  const uint32_t cb = load_chunk_bytes();
  const uint32_t rowbytes = (uint32_t)p.K;
  const TileWalk tw = tile_walk(ntiles);
  if (tw.count <= 0) return;

  const i32x4 ra = make_rsrc(p.a, (uint32_t)rows * rowbytes);
  const i32x4 rw = make_rsrc(p.w, (uint32_t)p.N * rowbytes);
  const uint32_t smem_a = lds_addr(smem);
  struct Src {
    uint32_t a, b, touch;
  };
  auto src = [&](int tile, Src& sr) {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    const int m0 = rb * BM, n0 = cbk * 128;
    // Rows past the end read zeros (the buffer resource's bound).
    sr.a = (uint32_t)(m0 + load_row<G::A_INS>(0)) * rowbytes + cb;
    sr.b = (uint32_t)(n0 + load_row<G::B_INS>(0)) * rowbytes + cb;
    sr.touch = (uint32_t)min(m0 + (int)threadIdx.x % BM, rows - 1) * rowbytes;
  };
  auto dma = [&](const Src& sr, int buf, int k) {
    const uint32_t sa = smem_a + buf * G::STAGE, sb = sa + G::A_BYTES;
#pragma unroll
    for (int i = 0; i < G::A_INS; ++i)
      lds_dma16(ra, sa + (wave * G::A_INS + i) * 1024, sr.a, k * 128 + i * 8 * rowbytes);
#pragma unroll
    for (int i = 0; i < G::B_INS; ++i)
      lds_dma16(rw, sb + (wave * G::B_INS + i) * 1024, sr.b, k * 128 + i * 8 * rowbytes);
  };
  auto touch = [&](const Src& sr, int k) {
    lds_dma4(ra, smem_a + 2 * G::STAGE + wave * 256, sr.touch, k * 128);
  };
  // A lane's 32 bytes of a stage row: chunks 2 g4 and 2 g4 + 1, each at its
  // swizzled position (chunk c of row r at c ^ (r % 8)).
  auto frag = [&](const char* base, int row) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row * 128 + (((2 * g4) ^ (row & 7)) << 4));
    const uint4 hi =
        *reinterpret_cast<const uint4*>(base + row * 128 + (((2 * g4 + 1) ^ (row & 7)) << 4));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                 (int)hi.w};
  };
  constexpr int TM = G::TM, TN = G::TN;  // 8 x 4 tiles of 16
  auto read_frags = [&](int buf, i32x8 (&af)[TM], i32x8 (&bf)[TN]) {
    const char* sa = smem + buf * G::STAGE + wm * G::WM * 128;
    const char* sb = smem + buf * G::STAGE + G::A_BYTES + wn * G::WN * 128;
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = frag(sa, 16 * i + i16);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bf[j] = frag(sb, 32 * (j >> 1) + 8 * (i16 >> 2) + 4 * (j & 1) + (i16 & 3));
  };
  f32x4 acc[TM][TN];
  TO* y = static_cast<TO*>(p.y);
  // Published by the prologue's barrier.
  for (int n = threadIdx.x; n < p.N; n += G::THREADS) {
    swsm[n] = p.sw[n];
    bsm[n] = p.bias ? ld_any(p.bias, p.bias_type, n) : 0.f;
  }
  // Row scales of a tile, loaded during its last stage (rows clamped, so that
  // there are always TM loads).
  float sa[TM];
  auto load_sa = [&](int tile) {
    int mbase = (tile / ncol) * BM + wm * G::WM + i16;
    asm volatile("" : "+v"(mbase));
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = p.sa[min(mbase + 16 * i, rows - 1)];
  };
  // Stores per lane of a tile with every row present.
  constexpr int kStores = TM * (TN / 2) * (sizeof(TO) == 4 ? 2 : 1);
  auto epi = [&](int tile) -> int {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    int mbase = rb * BM + wm * G::WM + i16;
    int nbase = cbk * 128 + wn * 64 + 8 * g4;
    asm volatile("" : "+v"(mbase), "+v"(nbase));
    int n_st = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mbase + 16 * i;
      if (m >= rows) continue;
      n_st += kStores / TM;
#pragma unroll
      for (int jp = 0; jp < TN / 2; ++jp) {
        const int n0 = nbase + 32 * jp;
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][2 * jp][r] * sa[i] * swsm[n0 + r] + bsm[n0 + r];
          v[4 + r] = acc[i][2 * jp + 1][r] * sa[i] * swsm[n0 + 4 + r] + bsm[n0 + 4 + r];
        }
        TO* dst = y + (int64_t)m * p.N + nbase + 32 * jp;
        if constexpr (sizeof(TO) == 4) {
          gstore16(dst, uint4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                              __float_as_uint(v[3])});
          gstore16(dst + 4, uint4{__float_as_uint(v[4]), __float_as_uint(v[5]),
                                  __float_as_uint(v[6]), __float_as_uint(v[7])});
        } else {
          vec8<TO> o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = from_f32<TO>(v[e]);
          gstore16(dst, __builtin_bit_cast(uint4, o));
        }
      }
    }
    // The wave's count (EPI in the loop below) only when every lane stored
    // every row; else -1.
    return __builtin_amdgcn_readfirstlane(n_st) == kStores && __all(n_st == kStores) ? kStores
                                                                                     : -1;
  };

  Src cur, nxt;
  int tile = tw.first;
  src(tile, cur);
  src(tw.count > 1 ? tile + tw.stride : tile, nxt);
  // Prologue: stage 0 and the touches of stages 2, 3; then stage 1.  Every
  // stage's loads are followed by exactly one touch, so "stage k+1 landed" is
  // vmcnt(1) whenever no stores came after (and vmcnt(1) waits for them too).
  dma(cur, 0, 0);
  touch(cur, 2);
  wait_vm<1>();
  __syncthreads();
  // Two fragment sets: stage k multiplies set k % 2 while stage k + 1's
  // fragments are read into the other one.
  i32x8 a0[TM], b0[TN], a1[TM], b1[TN];
  read_frags(0, a0, b0);
  dma(cur, 1, 1);
  touch(cur, 3);
  int issued = -1;  // stores of the previous tile's epilogue (see epi)
  for (int it = 0; it < tw.count; ++it) {
    const bool more = it + 1 < tw.count;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto step = [&](int k, const i32x8 (&af)[TM], const i32x8 (&bf)[TN], i32x8 (&an)[TM],
                    i32x8 (&bn)[TN]) {
      if (k + 1 < NK || more) {
        // This wave's loads of the next stage have landed.  At k = 0 they are
        // followed by the touch, the TM row-scale loads and the previous
        // epilogue's stores, which may stay in flight (a full tile's count is
        // exact; otherwise everything is waited for).
        if (k == 0 && issued == kStores)
          wait_vm<1 + TM + kStores>();
        else
          wait_vm<1>();
        __syncthreads();  // ... everyone's; and this stage's buffer is free
        if (k + 2 < NK) dma(cur, k & 1, k + 2);
        else if (more) dma(nxt, k & 1, k + 2 - NK);
        if (k + kPrefetch < NK) touch(cur, k + kPrefetch);
        else touch(more ? nxt : cur, more ? k + kPrefetch - NK : NK - 1);
        read_frags((k + 1) & 1, an, bn);
      }
      if (k == NK - 1) load_sa(tile);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], acc[i][j], 0,
                                                                       0, 0, 127, 0, 127);
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma nounroll
    for (int k = 0; k < NK; k += 2) {
      step(k, a0, b0, a1, b1);
      step(k + 1, a1, b1, a0, b0);
    }
    issued = epi(tile);
    tile += tw.stride;
    cur = nxt;
    if (it + 2 < tw.count) src(tile + tw.stride, nxt);
  }
}

template <typename TO>
hipError_t fp8_tiled_t(const Fp8Linear& p, hipStream_t st) {
  const int tiles = (int)((p.rows + 255) / 256) * (p.N / 128);
  const dim3 grid(persistent_grid(tiles, 1)), block(256);
  switch (p.K) {
    case 512: hipLaunchKernelGGL((fp8_tiled_kernel<TO, 4>), grid, block, 0, st, p); break;
    case 1024: hipLaunchKernelGGL((fp8_tiled_kernel<TO, 8>), grid, block, 0, st, p); break;
    case 1536: hipLaunchKernelGGL((fp8_tiled_kernel<TO, 12>), grid, block, 0, st, p); break;
    case 2048: hipLaunchKernelGGL((fp8_tiled_kernel<TO, 16>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 2:4 structured-sparse linear layer, y = x wp^T + bias (the kept values and
// positions of sparse.hip), on the same tile walk: a 128-byte token stage row
// is one 64-deep step of the 16x16x64 sparse products (twice the dense rate),
// whose token operand lane holds k = 8 g4 .. +7 and 32 + 8 g4 .. +7 (chunks g4
// and 4 + g4).  Per step the weight side is the kept values (64 bytes a
// channel, chunks swizzled) and the positions (16 bytes a channel, 4-byte
// loads), both staged by direct-to-LDS loads with the channels stored
// permuted so that a fragment reads 16 consecutive rows.  256 tokens x 128
// channels per tile, 4 waves of 128 x 64, one workgroup per CU, two fragment
// sets; a lane ends with 8 consecutive output channels of one token.
// ---------------------------------------------------------------------------
constexpr int kSpMaxN = 2048;  // output channels (bias in LDS)

// 16-byte chunk q of row r of a 64-byte-row block sits at q ^ sw64(r): the 16
// consecutive rows of a fragment read then touch distinct bank slots.
__device__ __forceinline__ int sw64(int r) { return ((r >> 1) ^ (r >> 2) ^ (r >> 4)) & 3; }
// LDS row of a 128-channel block -> the channel it holds (pairs of 16-channel
// tiles interleaved: LDS row 16t + 4a + b of a 32-row part holds 8a + 4t + b).
__device__ __forceinline__ int sp_channel_of_row(int l) {
  return (l & ~31) | (((l >> 2) & 3) << 3) | (((l >> 4) & 1) << 2) | (l & 3);
}

template <typename T, int NK>
__global__ __launch_bounds__(256, 1) void sparse24_tiled2_kernel(Sparse24Linear p) {
  typedef T v8 __attribute__((ext_vector_type(8)));
  typedef T v16 __attribute__((ext_vector_type(16)));
  constexpr int BM = 256, BN = 128, WAVES = 4;
  static_assert(NK % 2 == 0 && NK >= kPrefetch, "stage parity and touch distance");
  constexpr int A_BYTES = BM * 128, V_BYTES = BN * 64, C_BYTES = BN * 16;
  constexpr int STAGE = A_BYTES + V_BYTES + C_BYTES;
  constexpr int A_INS = BM / 8 / WAVES;          // 1 KB token-row loads per wave and stage
  constexpr int V_INS = V_BYTES / 1024 / WAVES;  // 1 KB kept-value loads
  constexpr int C_INS = C_BYTES / 256 / WAVES;   // 256 B position loads (4 bytes a lane)
  constexpr int TM = 8, TN = 4;                  // 128 tokens x 64 channels per wave
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + WAVES * 256];
  __shared__ float bsm[kSpMaxN];
  const int rows = (int)p.rows;
  const int ncol = p.N / BN;
  const int ntiles = (rows + BM - 1) / BM * ncol;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int i16 = lane & 15, g4 = lane >> 4;
  const uint32_t cb = load_chunk_bytes();
  const uint32_t rowbytes = (uint32_t)p.K * 2;  // token rows
  const uint32_t vbytes = (uint32_t)p.K;        // kept values of a channel
  const uint32_t cbytes = (uint32_t)p.K / 4;    // positions of a channel
  const TileWalk tw = tile_walk(ntiles);
  if (tw.count <= 0) return;

  const i32x4 rx = make_rsrc(p.x, (uint32_t)rows * rowbytes);
  const i32x4 rv = make_rsrc(p.vals, (uint32_t)p.N * vbytes);
  const i32x4 rc = make_rsrc(p.codes, (uint32_t)p.N * cbytes);
  const uint32_t smem_a = lds_addr(smem);
  // Per-lane source offsets of a tile (stage 0): token rows (linear: the
  // instruction index adds 8 rows), and the kept values / positions of the
  // channel each lane's LDS row holds.
  struct Src {
    uint32_t a, v[V_INS], c[C_INS], touch;
  };
  auto src = [&](int tile, Src& sr) {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    const int m0 = rb * BM, n0 = cbk * BN;
    sr.a = (uint32_t)(m0 + load_row<A_INS>(0)) * rowbytes + cb;  // rows past the end read 0
#pragma unroll
    for (int i = 0; i < V_INS; ++i) {
      const int l = 16 * (wave * V_INS + i) + (lane >> 2), slot = lane & 3;
      sr.v[i] = (uint32_t)(n0 + sp_channel_of_row(l)) * vbytes + ((slot ^ sw64(l)) << 4);
    }
#pragma unroll
    for (int i = 0; i < C_INS; ++i) {
      const int l = 16 * (wave * C_INS + i) + (lane >> 2);
      sr.c[i] = (uint32_t)(n0 + sp_channel_of_row(l)) * cbytes + 4 * (lane & 3);
    }
    sr.touch = (uint32_t)min(m0 + (int)threadIdx.x % BM, rows - 1) * rowbytes;
  };
  auto dma = [&](const Src& sr, int buf, int k) {
    const uint32_t sa = smem_a + buf * STAGE, sv = sa + A_BYTES, sc = sv + V_BYTES;
#pragma unroll
    for (int i = 0; i < A_INS; ++i)
      lds_dma16(rx, sa + (wave * A_INS + i) * 1024, sr.a, k * 128 + i * 8 * rowbytes);
#pragma unroll
    for (int i = 0; i < V_INS; ++i) lds_dma16(rv, sv + (wave * V_INS + i) * 1024, sr.v[i], k * 64);
#pragma unroll
    for (int i = 0; i < C_INS; ++i) lds_dma4(rc, sc + (wave * C_INS + i) * 256, sr.c[i], k * 16);
  };
  auto touch = [&](const Src& sr, int k) {
    lds_dma4(rx, smem_a + 2 * STAGE + wave * 256, sr.touch, k * 128);
  };
  struct Frags {
    v16 x[TM];
    v8 w[TN];
    int wi[TN];
  };
  auto read_frags = [&](int buf, Frags& f) {
    const char* sa = smem + buf * STAGE + wm * 128 * 128;
    const char* sv = smem + buf * STAGE + A_BYTES;
    const char* sc = sv + V_BYTES;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = 16 * i + i16;
      const v8 lo = *reinterpret_cast<const v8*>(sa + r * 128 + ((g4 ^ (r & 7)) << 4));
      const v8 hi = *reinterpret_cast<const v8*>(sa + r * 128 + (((4 + g4) ^ (r & 7)) << 4));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f.x[i][e] = lo[e];
        f.x[i][8 + e] = hi[e];
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int l = wn * 64 + 16 * j + i16;
      f.w[j] = *reinterpret_cast<const v8*>(sv + l * 64 + ((g4 ^ sw64(l)) << 4));
      const uint32_t c4 = *reinterpret_cast<const uint32_t*>(sc + l * 16 + 4 * g4);
      // Four groups' positions (p0 | p1 << 2 a byte) as four nibbles.
      f.wi[j] = (int)((c4 & 0xFu) | ((c4 >> 4) & 0xF0u) | ((c4 >> 8) & 0xF00u) |
                      ((c4 >> 12) & 0xF000u));
    }
  };
  f32x4 acc[TM][TN];
  T* y = static_cast<T*>(p.y);
  const T* bias = static_cast<const T*>(p.bias);
  for (int n = threadIdx.x; n < p.N; n += 256) bsm[n] = bias ? (float)bias[n] : 0.f;
  constexpr int kStores = TM * (TN / 2);
  auto epi = [&](int tile) -> int {
    const int rb = tile / ncol, cbk = tile - (tile / ncol) * ncol;
    int mbase = rb * BM + wm * 128 + i16;
    int nbase = cbk * BN + wn * 64 + 8 * g4;
    asm volatile("" : "+v"(mbase), "+v"(nbase));
    int n_st = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mbase + 16 * i;
      if (m >= rows) continue;
      n_st += TN / 2;
#pragma unroll
      for (int jp = 0; jp < TN / 2; ++jp) {
        const int n0 = nbase + 32 * jp;
        vec8<T> o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o[r] = from_f32<T>(acc[i][2 * jp][r] + bsm[n0 + r]);
          o[4 + r] = from_f32<T>(acc[i][2 * jp + 1][r] + bsm[n0 + 4 + r]);
        }
        gstore16(y + (int64_t)m * p.N + n0, __builtin_bit_cast(uint4, o));
      }
    }
    return __builtin_amdgcn_readfirstlane(n_st) == kStores && __all(n_st == kStores) ? kStores
                                                                                     : -1;
  };

  Src cur, nxt;
  int tile = tw.first;
  src(tile, cur);
  src(tw.count > 1 ? tile + tw.stride : tile, nxt);
  // Prologue (as in run_tiles): stage 0 and the touches of stages 2, 3; then
  // stage 1.  Every stage's loads are followed by exactly one touch.
  dma(cur, 0, 0);
  touch(cur, 2);
  wait_vm<1>();
  __syncthreads();
  Frags f0, f1;
  read_frags(0, f0);
  dma(cur, 1, 1);
  touch(cur, 3);
  bool issued_ok = false;  // the previous tile stored every row (see epi)
  for (int it = 0; it < tw.count; ++it) {
    const bool more = it + 1 < tw.count;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto step = [&](int k, const Frags& fc, Frags& fn) {
      if (k + 1 < NK || more) {
        // The next stage landed (at k = 0 the previous epilogue's stores
        // may stay in flight: they follow it, and their count is exact).
        if (k == 0 && issued_ok)
          wait_vm<1 + kStores>();
        else
          wait_vm<1>();
        __syncthreads();  // everyone's; and this stage's buffer is free
        if (k + 2 < NK) dma(cur, k & 1, k + 2);
        else if (more) dma(nxt, k & 1, k + 2 - NK);
        if (k + kPrefetch < NK) touch(cur, k + kPrefetch);
        else touch(more ? nxt : cur, more ? k + kPrefetch - NK : NK - 1);
        read_frags((k + 1) & 1, fn);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (__is_same(T, h16))
            acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(fc.w[j], fc.x[i], acc[i][j],
                                                                 fc.wi[j], 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(fc.w[j], fc.x[i], acc[i][j],
                                                                  fc.wi[j], 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma nounroll
    for (int k = 0; k < NK; k += 2) {
      step(k, f0, f1);
      step(k + 1, f1, f0);
    }
    issued_ok = epi(tile) == kStores;
    tile += tw.stride;
    cur = nxt;
    if (it + 2 < tw.count) src(tile + tw.stride, nxt);
  }
}

template <typename T>
hipError_t sparse24_tiled2_t(const Sparse24Linear& p, hipStream_t st) {
  const int tiles = (int)((p.rows + 255) / 256) * (p.N / 128);
  const dim3 grid(persistent_grid(tiles, 1)), block(256);
  switch (p.K) {
    case 256: hipLaunchKernelGGL((sparse24_tiled2_kernel<T, 4>), grid, block, 0, st, p); break;
    case 512: hipLaunchKernelGGL((sparse24_tiled2_kernel<T, 8>), grid, block, 0, st, p); break;
    case 1024: hipLaunchKernelGGL((sparse24_tiled2_kernel<T, 16>), grid, block, 0, st, p); break;
    case 1536: hipLaunchKernelGGL((sparse24_tiled2_kernel<T, 24>), grid, block, 0, st, p); break;
    case 2048: hipLaunchKernelGGL((sparse24_tiled2_kernel<T, 32>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// The operand buffer resources take 32-bit byte counts and offsets: A (rows x K,
// 16-bit) must stay below 2 GiB.
bool dense_tiled_supported(int64_t rows, int N, int K, int io) {
  return io != kF32 && N % 128 == 0 && (K == 256 || K == 512 || K == 1024 || K == 2048) &&
         rows * K * 2 < ((int64_t)1 << 31);
}

hipError_t launch_dense_tiled(const DenseParams& d, bool gelu, hipStream_t st) {
  if (!dense_tiled_supported(d.rows, d.N, d.K, d.io)) return hipErrorInvalidValue;
  return d.io == kF16 ? dense_tiled_t<h16>(d, gelu, st) : dense_tiled_t<b16>(d, gelu, st);
}

// K in {512, 1024, 1536, 2048} (4 .. 16 steps of 128), N % 128 == 0 and at
// most kFp8MaxN, both code matrices below 2 GiB, y 16-byte aligned.
bool fp8_tiled_supported(const Fp8Linear& p) {
  return p.rows > 0 && p.N % 128 == 0 && p.N <= kFp8MaxN &&
         (p.K == 512 || p.K == 1024 || p.K == 1536 || p.K == 2048) &&
         p.rows * p.K < ((int64_t)1 << 31) && (int64_t)p.N * p.K < ((int64_t)1 << 31) &&
         (reinterpret_cast<uintptr_t>(p.y) & 15) == 0;
}

hipError_t launch_fp8_tiled(const Fp8Linear& p, int out_io, hipStream_t st) {
  if (!fp8_tiled_supported(p)) return hipErrorInvalidValue;
  if (out_io == kF32) return fp8_tiled_t<float>(p, st);
  if (out_io == kF16) return fp8_tiled_t<h16>(p, st);
  return fp8_tiled_t<b16>(p, st);
}

// K in {256, 512, 1024, 1536, 2048} (4 .. 32 steps of 64), N % 128 == 0 and
// at most kSpMaxN, 16-bit, every operand below 2 GiB, y 16-byte aligned.
bool sparse24_tiled2_supported(const Sparse24Linear& p, int io) {
  return io != kF32 && p.rows > 0 && p.N % 128 == 0 && p.N <= kSpMaxN &&
         (p.K == 256 || p.K == 512 || p.K == 1024 || p.K == 1536 || p.K == 2048) &&
         p.rows * p.K * 2 < ((int64_t)1 << 31) && (int64_t)p.N * p.K < ((int64_t)1 << 31) &&
         (reinterpret_cast<uintptr_t>(p.y) & 15) == 0;
}

hipError_t launch_sparse24_tiled2(const Sparse24Linear& p, int io, hipStream_t st) {
  if (!sparse24_tiled2_supported(p, io)) return hipErrorInvalidValue;
  return io == kF16 ? sparse24_tiled2_t<h16>(p, st) : sparse24_tiled2_t<b16>(p, st);
}

bool tiled_gemm_supported(int C, int io) { return io != kF32 && (C == 256 || C == 512); }

hipError_t launch_qkv_tiled(const FwdParams& p, hipStream_t st) {
  if (!tiled_gemm_supported(p.g.C, p.io)) return hipErrorInvalidValue;
  if (p.io == kF16) return qkv_tiled_dispatch<h16, h16>(p, st);
  if (p.qk == kF16) return qkv_tiled_dispatch<b16, h16>(p, st);
  return qkv_tiled_dispatch<b16, b16>(p, st);
}

hipError_t launch_proj_tiled(const FwdParams& p, hipStream_t st) {
  if (!tiled_gemm_supported(p.g.C, p.io)) return hipErrorInvalidValue;
  if (p.io == kF16) return proj_tiled_dispatch<h16>(p, st);
  return proj_tiled_dispatch<b16>(p, st);
}

}  // namespace swin
