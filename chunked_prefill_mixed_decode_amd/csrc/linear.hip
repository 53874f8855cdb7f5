// Linear layers around the attention step on gfx950: y[M, N] = x[M, K] . w[N, K]^T in bfloat16
// with float32 accumulation -- the QKV projection before the rotary step and the output
// projection after attention.
//
// "Chunked Prefill: Ending the Great Stall" §02: selective batching runs the linear layers over
// all tokens of an iteration (decode and prefill alike) while attention runs per request; its
// piggyback roofline (and "Splitting Prefill From Decode Inside a Step", "Two kernels with
// different limiting resources"): the weights are read once per iteration and serve every token
// in it, so T tokens give about T FLOP per weight byte (bf16) -- weight-bandwidth bound for a
// decode-only step, compute bound once a prefill chunk joins.
//
// One 256-thread workgroup per BM x BN output tile and K split, 64-deep K stages: the x and w
// tiles of a stage are copied HBM -> LDS with the gfx950 16-byte LDS DMA into a ring of stage
// buffers, rows chunk-swizzled (16-byte chunk c of row r at c ^ (r mod 8), so the 32 rows an
// operand read touches at one chunk spread over all 16-byte bank groups); each wave computes a
// BM/2 x BN/2 quarter with v_mfma_f32_32x32x16_bf16.  Three shapes: 128 x 128 with two stage
// buffers (the next stage's copy in flight behind the one being multiplied; 64 KB, two workgroups
// per compute unit -- measured faster than three buffers and one workgroup) and 128 x 192 with
// three (120 KB, one workgroup per unit, for wide layers whose tiles then fill the chip once) for
// the compute-bound mixed step, and 64 x 64 with three (48 KB, two stages of weights in flight)
// for a decode-only step's few rows, where the weight stream is the whole cost and the bytes in
// flight set its rate.  Tiles are ordered so that the workgroups sharing one weight tile
// run on one XCD (workgroup b runs on XCD b mod 8) and read it through that XCD's L2.  A layer
// with few tiles (a decode-only step's rows) splits K so that at least 256 workgroups stream the
// weights: each split writes float32 partials and a second kernel sums them in split order (the
// split depends on the shape alone, so results do not depend on the device).
#include <algorithm>

#include "cb.h"
#include "common.h"

namespace cb {
namespace {

constexpr int kBK = 64;
constexpr int kNAlign = 128;                       // N must be a multiple of this (every tile width)
constexpr int kRowBytes = kBK * 2;                 // bytes of one tile row in one stage
#ifndef CB_LINEAR_SKINNY_M
#define CB_LINEAR_SKINNY_M 64                      // M up to this: 64-row tiles, a deeper ring
#endif
#ifndef CB_LINEAR_SKINNY_STAGES
#define CB_LINEAR_SKINNY_STAGES 3                  // stage buffers of those
#endif
#ifndef CB_LINEAR_SKINNY_BN
#define CB_LINEAR_SKINNY_BN 64                     // and their tile width
#endif
#ifndef CB_LINEAR_MIN_WG
#define CB_LINEAR_MIN_WG 256                       // K is split until the grid has this many
#endif
constexpr int64_t kMinWorkgroups = CB_LINEAR_MIN_WG;
constexpr int kMaxSplit = 16;
constexpr int kMinStagesPerSplit = 4;

// Tile shape of a layer.  Few rows (a decode-only step): 64 x BN_skinny tiles, a deeper ring, K
// split until the weight stream has enough workgroups.  More rows: 128 x 192 tiles (three 40 KB
// stage buffers, one workgroup per compute unit) when N allows and that gives at least
// kMinWorkgroups * 3 / 4 tiles (the budget-512 layer's QKV projection: 256 tiles, 70 against
// 72 us with 128 x 128), else 128 x 128 (two 32 KB buffers, two workgroups per unit) with K split
// as needed (its output projection: 128 x 64 tiles without a split measured 35.8 against 32.7 us).
struct TileShape {
  int32_t bm, bn, ns;
};
TileShape tile_shape(int32_t M, int32_t N) {
  if (M <= CB_LINEAR_SKINNY_M) return {64, CB_LINEAR_SKINNY_BN, CB_LINEAR_SKINNY_STAGES};
  const int64_t mt = (static_cast<int64_t>(M) + 127) / 128;
  if (N % 192 == 0 && mt * (N / 192) >= kMinWorkgroups * 3 / 4) return {128, 192, 3};
  return {128, 128, 2};
}

// K splits for a shape: the smallest power of two giving kMinWorkgroups workgroups, at most
// kMaxSplit, dividing the K stages evenly and keeping kMinStagesPerSplit stages per split.
int32_t k_splits(int64_t tiles, int32_t K) {
  const int32_t stages = K / kBK;
  int32_t s = 1;
  while (s < kMaxSplit && tiles * s < kMinWorkgroups && stages % (2 * s) == 0 &&
         stages / (2 * s) >= kMinStagesPerSplit)
    s *= 2;
  return s;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}
// One 16-byte-per-lane LDS DMA: lane l's 16 bytes from src land at lds_dst + 16 l.  Issued from
// inline asm, so the compiler adds no waits for it; the loop below waits for its copies itself.
// M0 carries the wave-uniform LDS destination (saved and restored; one wait state after writing it).
__device__ __forceinline__ void dma16(const void* src, const char* lds_dst) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(lds_dst));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(dst));
}
__device__ __forceinline__ int swz(int c, int r) { return c ^ (r & 7); }

// Wait until at most `later` stages' copies of this wave are outstanding (copies complete in
// issue order), then the workgroup barrier.
template <int CPS>
__device__ __forceinline__ void wait_stage_copies(int later) {
  if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * CPS) : "memory");
  else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(CPS) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int BM, int BN, int NS>
__global__ __launch_bounds__(256) void linear_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w,
                                                     bf16_t* __restrict__ y, float* __restrict__ part,
                                                     int32_t M, int32_t N, int32_t K, int32_t m_tiles,
                                                     int32_t splits, int32_t items, int32_t per_xcd) {
  static_assert((BM == 64 || BM == 128) && (BN == 64 || BN == 128 || BN == 192) && NS >= 2 && NS <= 4,
                "tile shape and ring depth");
  constexpr int XC = BM / 32;                        // x copies per wave per stage (8 rows each)
  constexpr int WC = BN / 32;                        // w copies per wave per stage
  constexpr int CPS = XC + WC;                       // copies per wave per stage
  constexpr int MI = BM / 64;                        // 32-row fragments of a wave's quarter
  constexpr int NJ = BN / 64;                        // 32-column fragments of it
  constexpr int XBYTES = BM * kRowBytes;
  constexpr int SBYTES = XBYTES + BN * kRowBytes;    // one stage: [x | w]
  __shared__ __attribute__((aligned(1024))) char lds[NS * SBYTES];
  const int32_t b = blockIdx.x;
  const int32_t it = (b & 7) * per_xcd + (b >> 3);   // item = (tile, split), split fastest
  if (it >= items) return;
  const int32_t t = it / splits, split = it - t * splits;
  const int32_t m0 = (t % m_tiles) * BM, n0 = (t / m_tiles) * BN;
  const int32_t nk = K / kBK / splits, kt0 = split * nk;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;

  // Copy j of this wave fills tile bytes [1024 (XC wave + j), + 1024) of x (j < XC) and
  // [1024 (WC wave + j), + 1024) of w: rows 8 (that index) + lane / 8, physical chunk lane % 8
  // (logical chunk lane % 8 ^ row % 8).  Rows of x past M repeat row M - 1 (their results are
  // not stored).
  const char* xs[XC];
  const char* ws[WC];
#pragma unroll
  for (int j = 0; j < XC; ++j) {
    const int r = 8 * (XC * wave + j) + (lane >> 3);
    xs[j] = reinterpret_cast<const char*>(x + static_cast<int64_t>(std::min(m0 + r, M - 1)) * K) + 16 * swz(lane & 7, r);
  }
#pragma unroll
  for (int j = 0; j < WC; ++j) {
    const int r = 8 * (WC * wave + j) + (lane >> 3);
    ws[j] = reinterpret_cast<const char*>(w + static_cast<int64_t>(n0 + r) * K) + 16 * swz(lane & 7, r);
  }
  auto issue = [&](int32_t kt, int buf) {
    const char* xt = lds + buf * SBYTES;
    const char* wt = xt + XBYTES;
    const int64_t koff = static_cast<int64_t>(kt0 + kt) * kRowBytes;
#pragma unroll
    for (int j = 0; j < XC; ++j) dma16(xs[j] + koff, xt + 1024 * (XC * wave + j));
#pragma unroll
    for (int j = 0; j < WC; ++j) dma16(ws[j] + koff, wt + 1024 * (WC * wave + j));
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lr = lane & 31, lh = lane >> 5;
  // Copies run NS - 1 stages ahead of the matrix work.
  for (int p = 0; p < NS - 1; ++p)
    if (p < nk) issue(p, p);
  for (int32_t kt = 0; kt < nk; ++kt) {
    // This wave's copies of stage kt have landed once at most the later stages' copies already
    // issued are outstanding; after the barrier every wave's have, and every wave has finished
    // reading stage kt - 1's buffer, which the next copy overwrites.
    wait_stage_copies<CPS>(min(NS - 2, nk - 1 - kt));
    if (kt + NS - 1 < nk) issue(kt + NS - 1, (kt + NS - 1) % NS);
    const char* xt = lds + (kt % NS) * SBYTES;
    const char* wt = xt + XBYTES;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = 2 * kk + lh;                   // 16-byte chunk: slots 8 (l / 32) .. + 7 of step kk
      Frag<bf16_t> a[MI], bw[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = (BM / 2) * wm + 32 * i + lr;
        a[i].u = *reinterpret_cast<const uint4*>(xt + r * kRowBytes + 16 * swz(c, r));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int r = (BN / 2) * wn + 32 * j + lr;
        bw[j].u = *reinterpret_cast<const uint4*>(wt + r * kRowBytes + 16 * swz(c, r));
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) mma32_k16(acc[i][j], a[i], bw[j]);
    }
  }

  // acc[i][j] register r: row (BM/2) wm + 32 i + acc32_row(lane, r), column (BN/2) wn + 32 j + lane % 32.
  float* pt = splits > 1 ? part + static_cast<int64_t>(split) * M * N : nullptr;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t row = m0 + (BM / 2) * wm + 32 * i + acc32_row(lane, r);
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t o = static_cast<int64_t>(row) * N + n0 + (BN / 2) * wn + 32 * j + lr;
        if (pt) pt[o] = acc[i][j][r];
        else reinterpret_cast<uint16_t*>(y)[o] = f32_to_bf16_bits(acc[i][j][r]);
      }
    }
}

// y = the splits' partials summed in split order, rounded once to bfloat16 (4 outputs a thread).
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float* __restrict__ part, bf16_t* __restrict__ y,
                                                            int64_t n4, int64_t stride, int32_t splits) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4; i += static_cast<int64_t>(gridDim.x) * 256) {
    float4 s = reinterpret_cast<const float4*>(part)[i];
    for (int32_t k = 1; k < splits; ++k) {
      const float4 v = reinterpret_cast<const float4*>(part + k * stride)[i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    reinterpret_cast<uint2*>(y)[i] = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
  }
}

}  // namespace
}  // namespace cb

extern "C" size_t cb_linear_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  using namespace cb;
  if (M < 1 || N < 1 || K < 1 || N % kNAlign || K % kBK) return 0;
  const TileShape ts = tile_shape(M, N);
  const int64_t tiles = ((static_cast<int64_t>(M) + ts.bm - 1) / ts.bm) * (N / ts.bn);
  const int32_t s = k_splits(tiles, K);
  return s > 1 ? static_cast<size_t>(s) * M * N * sizeof(float) : 0;
}

extern "C" int cb_linear(void* stream, int32_t dtype, int32_t M, int32_t N, int32_t K, const void* x,
                         const void* w, void* y, void* workspace, size_t workspace_bytes) {
  using namespace cb;
  if (dtype != CB_BF16) return CB_ERR_INVALID;
  if (M < 0 || N < 1 || K < 1 || N % kNAlign || K % kBK) return CB_ERR_INVALID;
  if (M == 0) return CB_OK;
  if (!x || !w || !y) return CB_ERR_INVALID;
  for (const void* p : {x, w, static_cast<const void*>(y)})
    if (reinterpret_cast<uintptr_t>(p) & 15u) return CB_ERR_INVALID;
  const TileShape ts = tile_shape(M, N);
  const int64_t m_tiles = (static_cast<int64_t>(M) + ts.bm - 1) / ts.bm;
  const int64_t tiles = m_tiles * (N / ts.bn);
  const int32_t splits = k_splits(tiles, K);
  if (splits > 1) {
    if (workspace_bytes < cb_linear_workspace_bytes(M, N, K)) return CB_ERR_CAPACITY;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u)) return CB_ERR_INVALID;
  }
  const int64_t items = tiles * splits;
  const int64_t per_xcd = (items + 7) / 8;
  if (per_xcd * 8 > 0x7fffffff) return CB_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
  auto kernel = ts.bm == 64  ? linear_kernel<64, CB_LINEAR_SKINNY_BN, CB_LINEAR_SKINNY_STAGES>
                : ts.bn == 192 ? linear_kernel<128, 192, 3>
                               : linear_kernel<128, 128, 2>;
  kernel<<<dim3(static_cast<uint32_t>(per_xcd * 8)), dim3(256), 0, st>>>(
      static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w), static_cast<bf16_t*>(y), part, M, N, K,
      static_cast<int32_t>(m_tiles), splits, static_cast<int32_t>(items), static_cast<int32_t>(per_xcd));
  if (hipGetLastError() != hipSuccess) return CB_ERR_HIP;
  if (splits > 1) {
    const int64_t n4 = static_cast<int64_t>(M) * N / 4;
    const int64_t grid = std::min<int64_t>((n4 + 255) / 256, 4096);
    linear_reduce_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st>>>(
        part, static_cast<bf16_t*>(y), n4, static_cast<int64_t>(M) * N, splits);
    if (hipGetLastError() != hipSuccess) return CB_ERR_HIP;
  }
  return CB_OK;
}
