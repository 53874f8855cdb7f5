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
// One workgroup per BM x BN output tile and K split, 64-deep K stages: the x and w tiles of a
// stage are copied HBM -> LDS with the gfx950 16-byte LDS DMA (scalar base plus a loop-invariant
// 32-bit lane offset, so a copy costs a few scalar instructions) into a ring of stage buffers, all
// in flight; rows chunk-swizzled (16-byte chunk c of row r at c ^ ((r / 2) mod 8): the sixteen rows
// an operand read touches at one chunk in one LDS cycle cover all sixteen bank groups); each wave
// computes a block of the tile with v_mfma_f32_32x32x16_bf16, reading the next 16-deep step's
// operands while the current step's products run, and the stage barrier sits before a stage's
// last step, so the next stage's first reads overlap it.  Eight waves (two per SIMD) for the
// compute-bound mixed step's rows, whose waves then hide one another's barrier and read latency;
// four for a decode-only step's few rows, where the weight stream is the whole cost.  Tiles are
// ordered so that the workgroups sharing one weight tile run on one XCD (workgroup b runs on XCD
// b mod 8) and read it through that XCD's L2.  A layer with few tiles (a decode-only step's rows)
// splits K so that at least 256 workgroups stream the weights: each split writes float32
// partials and a second kernel sums them in split order (the split depends on the shape alone,
// so results do not depend on the device).
#include <algorithm>
#include <type_traits>

#include "cb.h"
#include "common.h"

namespace cb {
namespace {

constexpr int kBK = 64;
constexpr int kNAlign = 128;                       // N must be a multiple of this (every tile width)
constexpr int kRowBytes = kBK * 2;                 // bytes of one tile row in one stage
constexpr int kMinWorkgroups = 256;               // K is split until the grid has this many
constexpr int kMaxSplit = 16;
constexpr int kMinStagesPerSplit = 4;
constexpr int32_t kMaxK = 1 << 22;                // keeps a tile's copy offsets within 32 bits

// Tile shape of a layer (rows, columns, ring depth, waves).  Few rows (M <= 64, a decode-only
// step): 64 x 64 tiles, four waves, three stage buffers (48 KB), K split until the weight stream
// has kMinWorkgroups workgroups.  More rows: 128 x 192 tiles (eight waves of 32 x 96, three 40 KB
// buffers, one workgroup per compute unit) when N allows and that gives at least 3/4 of
// kMinWorkgroups tiles (the budget-512 layer's QKV projection: 256 tiles); else 128 x 128 tiles
// when they alone fill the grid, else 64 x 128 (eight waves of 32 x 32; the budget-512 layer's
// output projection: 256 tiles and no K split, 25 against 28.5 us with 128 x 128 tiles split in
// two), K split as needed.
struct TileShape {
  int32_t bm, bn, ns, waves;
};
TileShape tile_shape(int32_t M, int32_t N) {
  if (M <= 64) return {64, 64, 3, 4};
  const int64_t mt = (static_cast<int64_t>(M) + 127) / 128;
  if (N % 192 == 0 && mt * (N / 192) >= kMinWorkgroups * 3 / 4) return {128, 192, 3, 8};
  if (mt * (N / 128) >= kMinWorkgroups) return {128, 128, 3, 8};
  return {64, 128, 3, 8};
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
// One 16-byte-per-lane LDS DMA in the instruction's scalar-base form: lane l's 16 bytes from
// base + voff (base wave-uniform, in SGPRs; voff a 32-bit per-lane offset) land at LDS byte
// address dst + 16 l (dst wave-uniform, in M0).  Issued from inline asm, so the compiler adds no
// waits for it; the loop below waits for its copies itself.  M0 is saved and restored around the
// copy, with one wait state between writing it and the copy that reads it.
__device__ __forceinline__ void dma16_s(const char* base, uint32_t voff, uint32_t dst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(dst));
}
// 16-byte chunk c of tile row r sits at chunk c ^ ((r / 2) mod 8) of its 128-byte LDS row: the
// sixteen rows an operand read touches at one chunk in one LDS cycle cover all sixteen 16-byte
// bank groups of a 256-byte bank line (two rows per line).
__device__ __forceinline__ int swz(int c, int r) { return c ^ ((r >> 1) & 7); }

// Wait until at most L stages' copies of this wave (PER copies each) are outstanding -- copies
// complete in issue order -- and every LDS read of this wave has returned, then the workgroup
// barrier.  L is a run-time value in [0, MAXL].
template <int PER, int MAXL>
__device__ __forceinline__ void wait_copies_barrier(int32_t later) {
  if constexpr (MAXL <= 0) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    if (later >= MAXL) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(MAXL * PER) : "memory");
    else wait_copies_barrier<PER, MAXL - 1>(later);
  }
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// One workgroup of WM x WN waves per BM x BN output tile and K split.  Each wave computes a
// (BM / WM) x (BN / WN) block.  K goes in 64-deep stages through a ring of NS LDS buffers, all NS
// in flight: the copy of stage s + NS goes into the buffer of stage s once every wave has read it.
// The barrier of stage s sits before its last 16-deep step, so the operand reads of stage s + 1's
// first step overlap that step's matrix products.
template <int BM, int BN, int NS, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void linear_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w,
                                                              bf16_t* __restrict__ y, float* __restrict__ part,
                                                              int32_t M, int32_t N, int32_t K, int32_t m_tiles,
                                                              int32_t splits, int32_t items, int32_t per_xcd) {
  constexpr int NW = WM * WN;
  constexpr int XC = BM / 8 / NW;                    // x copies per wave per stage (8 rows, 1 KB each)
  constexpr int WC = BN / 8 / NW;                    // w copies per wave per stage
  static_assert(XC * 8 * NW == BM && WC * 8 * NW == BN && XC >= 1 && WC >= 1, "copies split over the waves");
  constexpr int CPS = XC + WC;
  constexpr int TM = BM / WM, TN = BN / WN;          // a wave's block
  constexpr int MI = TM / 32, NJ = TN / 32;          // its 32 x 32 fragments
  static_assert(MI * 32 == TM && NJ * 32 == TN && NS >= 2, "wave block and ring depth");
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
  const int wm = wave / WN, wn = wave % WN;

  // Copy j of this wave fills tile bytes [1024 (XC wave + j), + 1024) of x (j < XC) and
  // [1024 (WC wave + j), + 1024) of w: rows 8 (that index) + lane / 8, physical chunk lane % 8.
  // Rows of x past M repeat row M - 1 (their results are not stored).  Offsets are from the
  // tile's first row at the split's first column (they fit 32 bits: the launch checks K).
  const uint32_t row_bytes = static_cast<uint32_t>(K) * 2u;
  uint32_t vx[XC], vw[WC];
#pragma unroll
  for (int j = 0; j < XC; ++j) {
    const int r = 8 * (XC * wave + j) + (lane >> 3);
    vx[j] = static_cast<uint32_t>(min(m0 + r, M - 1) - m0) * row_bytes + 16u * swz(lane & 7, r);
  }
#pragma unroll
  for (int j = 0; j < WC; ++j) {
    const int r = 8 * (WC * wave + j) + (lane >> 3);
    vw[j] = static_cast<uint32_t>(r) * row_bytes + 16u * swz(lane & 7, r);
  }
  const char* xb = reinterpret_cast<const char*>(x + static_cast<int64_t>(m0) * K) + static_cast<int64_t>(kt0) * kRowBytes;
  const char* wb = reinterpret_cast<const char*>(w + static_cast<int64_t>(n0) * K) + static_cast<int64_t>(kt0) * kRowBytes;
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  auto issue = [&](int32_t kt, int buf) {
    const char* xs = xb + static_cast<int64_t>(kt) * kRowBytes;
    const char* ws = wb + static_cast<int64_t>(kt) * kRowBytes;
    const uint32_t d = l0 + static_cast<uint32_t>(buf * SBYTES);
#pragma unroll
    for (int j = 0; j < XC; ++j) dma16_s(xs, vx[j], d + 1024u * (XC * wave + j));
#pragma unroll
    for (int j = 0; j < WC; ++j) dma16_s(ws, vw[j], d + XBYTES + 1024u * (WC * wave + j));
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lr = lane & 31, lh = lane >> 5;
  struct Ops {
    Frag<bf16_t> a[MI], b[NJ];
  };
  // Operands of 16-deep step kk of the stage in ring buffer buf.
  auto read = [&](int buf, int kk, Ops& o) {
    const char* xt = lds + buf * SBYTES;
    const char* wt = xt + XBYTES;
    const int c = 2 * kk + lh;                       // 16-byte chunk: slots 8 (l / 32) .. + 7 of the step
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = TM * wm + 32 * i + lr;
      o.a[i].u = *reinterpret_cast<const uint4*>(xt + r * kRowBytes + 16 * swz(c, r));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = TN * wn + 32 * j + lr;
      o.b[j].u = *reinterpret_cast<const uint4*>(wt + r * kRowBytes + 16 * swz(c, r));
    }
  };
  auto mma = [&](const Ops& o) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) mma32_k16(acc[i][j], o.a[i], o.b[j]);
    // The next step's operand reads (issued just before) go ahead of these products.
    __builtin_amdgcn_sched_group_barrier(0x100, MI + NJ, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MI * NJ, 0);
  };

  const int32_t pro = min(NS, nk);
  for (int p = 0; p < pro; ++p) issue(p, p);
  wait_copies_barrier<CPS, NS - 1>(pro - 1);
  Ops r0, r1;
  read(0, 0, r0);
  int32_t s = 0;
  auto stage = [&](auto B) {
    constexpr int buf = decltype(B)::value;
    read(buf, 1, r1);
    mma(r0);
    read(buf, 2, r0);
    mma(r1);
    read(buf, 3, r1);
    mma(r0);
    if (s + 1 < nk) {
      // Stage s + 1 landed everywhere, and every wave has read all of stage s.
      wait_copies_barrier<CPS, NS - 2>(min(NS - 2, nk - 2 - s));
      if (s + NS < nk) issue(s + NS, buf);
      read((buf + 1) % NS, 0, r0);
    }
    mma(r1);
  };
  while (s < nk) {
    bool done = false;
    static_for<0, NS>([&](auto B) {
      if (!done) {
        stage(B);
        done = ++s == nk;
      }
    });
  }

  // acc[i][j] register r: row TM wm + 32 i + acc32_row(lane, r), column TN wn + 32 j + lane % 32.
  float* pt = splits > 1 ? part + static_cast<int64_t>(split) * M * N : nullptr;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t row = m0 + TM * wm + 32 * i + acc32_row(lane, r);
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t o = static_cast<int64_t>(row) * N + n0 + TN * wn + 32 * j + lr;
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
  if (M < 1 || N < 1 || K < 1 || N % kNAlign || K % kBK || K > kMaxK) return 0;
  const TileShape ts = tile_shape(M, N);
  const int64_t tiles = ((static_cast<int64_t>(M) + ts.bm - 1) / ts.bm) * (N / ts.bn);
  const int32_t s = k_splits(tiles, K);
  return s > 1 ? static_cast<size_t>(s) * M * N * sizeof(float) : 0;
}

extern "C" int cb_linear(void* stream, int32_t dtype, int32_t M, int32_t N, int32_t K, const void* x,
                         const void* w, void* y, void* workspace, size_t workspace_bytes) {
  using namespace cb;
  if (dtype != CB_BF16) return CB_ERR_INVALID;
  if (M < 0 || N < 1 || K < 1 || N % kNAlign || K % kBK || K > kMaxK) return CB_ERR_INVALID;
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
  auto kernel = ts.bm == 64 && ts.bn == 64 ? linear_kernel<64, 64, 3, 2, 2>
                : ts.bm == 64              ? linear_kernel<64, 128, 3, 2, 4>
                : ts.bn == 192             ? linear_kernel<128, 192, 3, 4, 2>
                                           : linear_kernel<128, 128, 3, 4, 2>;
  const uint32_t threads = 64u * ts.waves;
  kernel<<<dim3(static_cast<uint32_t>(per_xcd * 8)), dim3(threads), 0, st>>>(
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
