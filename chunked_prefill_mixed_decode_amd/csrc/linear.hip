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
// last two steps, so the next stage's first reads overlap them.  Eight waves (two per SIMD) for the
// compute-bound mixed step's rows, whose waves then hide one another's barrier and read latency;
// four for the 64 x 64 tiles of few rows whose K is split (below).  Tiles are
// ordered so that the workgroups sharing one weight tile run on one XCD (workgroup b runs on XCD
// b mod 8) and read it through that XCD's L2.  Few rows of a wide layer (the decode-only QKV
// projection) take 64 x 32..64 tiles over all of K in 8-wave workgroups that split each stage's
// depth between two wave halves and add the halves in LDS at the end, so 256 workgroups stream
// the weights with no second kernel.  Other layers with few tiles split K so that at least 256
// workgroups stream the weights: each split writes float32 partials and a second kernel sums them
// in split order.  Either way the summation order depends on the shape alone, so results do not
// depend on the device.
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
// The barrier of stage s sits before its last two 16-deep steps, so the operand reads of stage
// s + 1's first step overlap those steps' matrix products.
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
    // With one product per step, the next step's operand reads (issued just before) are put ahead
    // of it (the 64 x 128 tiles: 2% faster); wider wave blocks measured faster without the hint
    // (128 x 192: 3%).
    if constexpr (MI * NJ == 1) {
      __builtin_amdgcn_sched_group_barrier(0x100, MI + NJ, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MI * NJ, 0);
    }
  };

  const int32_t pro = min(NS, nk);
  for (int p = 0; p < pro; ++p) issue(p, p);
  wait_copies_barrier<CPS, NS - 1>(pro - 1);
  Ops r0, r1;
  read(0, 0, r0);
  int32_t s = 0;
  // Steps 2 and 3 are read ahead of the barrier, so two steps of products stay queued behind it
  // (one step measured 1.5-2% slower on the budget-512 layer's QKV projection, 3-4% on its output
  // projection).
  Ops r2, r3;
  auto stage = [&](auto B) {
    constexpr int buf = decltype(B)::value;
    read(buf, 1, r1);
    mma(r0);
    read(buf, 2, r2);
    read(buf, 3, r3);
    mma(r1);
    if (s + 1 < nk) {
      // Stage s + 1 landed everywhere, and every wave has read all of stage s.
      wait_copies_barrier<CPS, NS - 2>(min(NS - 2, nk - 2 - s));
      if (s + NS < nk) issue(s + NS, buf);
      read((buf + 1) % NS, 0, r0);
    }
    mma(r2);
    mma(r3);
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

// Few rows (M <= 64) of a layer wide enough for kMinWorkgroups tiles of 64 x BN: one 8-wave
// workgroup per tile over all of K, so no K split and no second kernel.  A stage's 64 x rows and
// BN weight rows are 8 + BN / 8 one-KB copies: wave v copies x rows 8 v .. 8 v + 7 and, for
// v < BN / 8, weight rows 8 v .. 8 v + 7, into a ring of NS buffers with NS - 1 stages in flight.
// Wave v multiplies row block v % 4 of x against the tile's BN / 16 column blocks over the 32-deep
// half v / 4 of each stage (v_mfma_f32_16x16x32_bf16); at the end the second half's sums meet the
// first's in LDS (first + second), so the result depends on the shape alone.
template <int BN, int NS>
__global__ __launch_bounds__(512) void linear_rows64_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w,
                                                            bf16_t* __restrict__ y, int32_t M, int32_t N, int32_t K) {
  constexpr int NJ = BN / 16;                        // 16-column blocks of the tile
  constexpr int WCP = BN / 8;                        // waves that also copy weight rows
  static_assert(NJ * 16 == BN && WCP >= 1 && WCP <= 8 && NS >= 2, "tile width and ring depth");
  constexpr int XBYTES = 64 * kRowBytes;             // copy c of a stage sits at 1024 c (x: c < 8)
  constexpr int SBYTES = XBYTES + BN * kRowBytes;
  __shared__ __attribute__((aligned(1024))) char lds[NS * SBYTES];
  const int32_t n0 = blockIdx.x * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const bool wcopy = wave < WCP;
  const int32_t nk = K / kBK;
  const uint32_t row_bytes = static_cast<uint32_t>(K) * 2u;
  const int r = 8 * wave + (lane >> 3);              // tile row of this lane's copies
  const uint32_t vx = static_cast<uint32_t>(min(r, M - 1)) * row_bytes + 16u * swz(lane & 7, r);
  const uint32_t vw = static_cast<uint32_t>(r) * row_bytes + 16u * swz(lane & 7, r);
  const char* xb = reinterpret_cast<const char*>(x);
  const char* wb = reinterpret_cast<const char*>(w + static_cast<int64_t>(n0) * K);
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  auto issue = [&](int32_t kt, int buf) {
    const uint32_t d = l0 + static_cast<uint32_t>(buf * SBYTES);
    dma16_s(xb + static_cast<int64_t>(kt) * kRowBytes, vx, d + 1024u * wave);
    if (wcopy) dma16_s(wb + static_cast<int64_t>(kt) * kRowBytes, vw, d + XBYTES + 1024u * wave);
  };
  // Wait for this wave's copies of the current stage (`later` stages issued after it may stay
  // outstanding), then the barrier.
  auto wait = [&](int32_t later) {
    if (wcopy) wait_copies_barrier<2, NS - 2>(later);
    else wait_copies_barrier<1, NS - 2>(later);
  };

  const int q = wave & 3, h = wave >> 2;
  const int lr = lane & 15;
  const int chunk = 4 * h + (lane >> 4);             // 16-byte chunk: K slots 32 h + 8 (l / 16) .. + 7
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < NS - 1; ++p)
    if (p < nk) issue(p, p);
  int32_t s = 0;
  auto stage = [&](auto B) {
    constexpr int buf = decltype(B)::value;
    wait(min(NS - 2, nk - 1 - s));                   // stage s landed everywhere; stage s - 1 read by all
    if (s + NS - 1 < nk) issue(s + NS - 1, (buf + NS - 1) % NS);
    const char* xt = lds + buf * SBYTES;
    const char* wt = xt + XBYTES;
    Frag<bf16_t> a, bw[NJ];
    const int ra = 16 * q + lr;
    a.u = *reinterpret_cast<const uint4*>(xt + ra * kRowBytes + 16 * swz(chunk, ra));
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int rb = 16 * j + lr;
      bw[j].u = *reinterpret_cast<const uint4*>(wt + rb * kRowBytes + 16 * swz(chunk, rb));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) mma16_k32(acc[j], a, bw[j]);
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

  // acc[j] register i: row 16 q + acc16_row(lane, i), column 16 j + lane % 16.  The ring is idle
  // (every copy waited for, every read returned before the last barrier), so its first bytes hold
  // the second half's sums.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  float* red = reinterpret_cast<float*>(lds);
  if (h == 1) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(16 * q + acc16_row(lane, i)) * BN + 16 * j + lr] = acc[j][i];
  }
  __syncthreads();
  if (h == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t row = 16 * q + acc16_row(lane, i);
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float v = acc[j][i] + red[row * BN + 16 * j + lr];
        reinterpret_cast<uint16_t*>(y)[static_cast<int64_t>(row) * N + n0 + 16 * j + lr] = f32_to_bf16_bits(v);
      }
    }
  }
}

// Tile width of the few-rows kernel: the widest of 64, 48, 32 that divides N and gives at least
// kMinWorkgroups tiles; 0 when none does (then 64 x 64 tiles with a K split).  Narrower tiles
// would read x from L2 more than four times per weight byte (the budget-512 layer's output
// projection with 64 x 16 tiles: 14.3 against 12.0 us split).
int rows64_bn(int32_t M, int32_t N) {
  if (M > 64) return 0;
  for (int bn : {64, 48, 32})
    if (N % bn == 0 && N / bn >= kMinWorkgroups) return bn;
  return 0;
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
  if (rows64_bn(M, N)) return 0;
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
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (const int bn = rows64_bn(M, N)) {
    // Four stage buffers (three stages in flight): the budget-512 layer's QKV projection 19.4-20.2
    // us, against 20.3-21.7 with three, five or eight and 34 with two.
    auto k64 = bn == 64 ? linear_rows64_kernel<64, 4> : bn == 48 ? linear_rows64_kernel<48, 4>
                        : linear_rows64_kernel<32, 4>;
    k64<<<dim3(static_cast<uint32_t>(N / bn)), dim3(512), 0, st>>>(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w),
                                                                     static_cast<bf16_t*>(y), M, N, K);
    return hipGetLastError() == hipSuccess ? CB_OK : CB_ERR_HIP;
  }
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
