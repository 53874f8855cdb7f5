// Mixed paged attention for one chunked-prefill step on gfx950.
//
// "Chunked Prefill 的 Token 预算" §02 and §07: a chunk row at position c + i attends keys
// 0..c + i (cached prefix plus its own chunk up to itself).  "Chunked Prefill: Ending the Great
// Stall" §05: each chunk is an ordinary causal attention over the prefix and the chunk, computed
// without materialising the score matrix; §01 and "Splitting Prefill From Decode Inside a Step"
// ("Two kernels with different limiting resources"): decode rows stream the whole cache and are
// bandwidth-bound, chunk rows are dense matrix work and compute-bound.
//
// Kernels on the caller's stream:
//   decode_prep_kernel  one workgroup, only when the caller brings no host-made plan: splits the
//                  decode rows' stage line (32-key stages of every (decode row, KV head, 16-head
//                  block) unit) into one contiguous range per decode wave, each sized by its
//                  workgroup's expected streaming rate.
//   attn_kernel    one launch for both kinds of rows.  The first workgroups hold four independent
//                  decode waves each: a wave streams its stage range, K and V rows of 32 keys
//                  HBM -> LDS by DMA, S^T = K Q^T on 16x16x32 MFMA with up to 16 query heads of
//                  a group as the N dimension, online softmax in the lane that owns the head,
//                  O^T += V^T P^T with V^T read by transposing LDS loads, one float32 partial
//                  (m, l, unnormalised o) per unit its range meets.  The other workgroups are
//                  chunk tiles, one per (chunk, query block, KV head, key split): rows of a tile
//                  are (position, head-in-group) pairs, so all query heads of a GQA group share
//                  one K/V stream; a 4-deep LDS ring of 32-key stages filled by DMA, software-
//                  pipelined so stage j+1's score products (32x32x16 MFMA) run beside stage j's
//                  softmax; causal mask only where a key can exceed a row's position.  One split:
//                  normalised rows written directly; several: float32 partials.
//   combine_kernel log-sum-exp merge of the partials of each (row, head) into out.
// Softmax runs in base 2: weights are 2^(s c - m) with c = scale * log2(e) and m the running
// maximum of s c.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "cb.h"
#include "cb_ext.h"
#include "common.h"

namespace cb {
namespace {

// Tuning constants (compile-time; the defaults are the measured choices on MI355X).
#ifndef CB_DECODE_MIN_STAGES
#define CB_DECODE_MIN_STAGES 8        // shortest decode stage range per wave (32-key stages)
#endif
#ifndef CB_CHUNK_MIN_TILES
#define CB_CHUNK_MIN_TILES 512        // split chunk keys until at least this many tiles (no decodes)
#endif
#ifndef CB_CHUNK_MIN_TILES_MIXED
#define CB_CHUNK_MIN_TILES_MIXED 128  // the same beside decode rows, whose streaming covers long tiles
#endif
#ifndef CB_CHUNK_SPLIT_KEYS
#define CB_CHUNK_SPLIT_KEYS 512       // fewest keys of the longest context per split (no decodes):
#endif                                // each split adds a float32 partial and its merge
#ifndef CB_CHUNK_SPLIT_KEYS_MIXED
#define CB_CHUNK_SPLIT_KEYS_MIXED 64  // the same beside decode rows
#endif
#ifndef CB_DECODE_WG_PER_CU
#define CB_DECODE_WG_PER_CU 2         // four-wave decode workgroups per CU without chunk tiles
#endif
#ifndef CB_DECODE_WG_PER_CU_MIXED
#define CB_DECODE_WG_PER_CU_MIXED 1   // the same beside chunk tiles
#endif
// Relative streaming rates of decode workgroups (percent), from per-wave start/end clocks of
// decode-only and mixed launches on MI355X: workgroups on odd XCDs stream ~8-12% slower than on
// even ones, so each wave's share of the decode work is sized by its workgroup's rate.  The
// workgroup dispatched second onto a compute unit also streams ~11% slower while the first one
// runs, but it speeds up once that one ends: giving it less work measured no faster, so its rate
// is left at 100.
#ifndef CB_DECODE_RATE_SECOND
#define CB_DECODE_RATE_SECOND 100
#endif
#ifndef CB_DECODE_RATE_ODD_XCD
#define CB_DECODE_RATE_ODD_XCD 88
#endif
// A decode workgroup whose compute unit also runs a chunk tile streams ~22% slower while the tile
// runs (per-wave clocks of mixed launches); the tile lasts about CB_DECODE_SHARE_RATIO percent of
// one decode wave stage per key stage of the tile.  Such a workgroup's rate is lowered by
// CB_DECODE_SHARE_SLOW percent times the fraction of the decode launch the tile is estimated to
// last (0 turns the adjustment off; 30 measured the shortest steps of 0, 22 and 30).
#ifndef CB_DECODE_SHARE_SLOW
#define CB_DECODE_SHARE_SLOW 30
#endif
#ifndef CB_DECODE_SHARE_RATIO
#define CB_DECODE_SHARE_RATIO 75
#endif
static_assert(CB_DECODE_RATE_SECOND >= 50 && CB_DECODE_RATE_SECOND <= 100 &&
              CB_DECODE_RATE_ODD_XCD >= 50 && CB_DECODE_RATE_ODD_XCD <= 100, "decode rates in [50, 100]");
static_assert(CB_DECODE_SHARE_SLOW >= 0 && CB_DECODE_SHARE_SLOW <= 40 && CB_DECODE_SHARE_RATIO >= 0 &&
              CB_DECODE_SHARE_RATIO <= 1000, "shared-unit adjustment");
// A split over W <= S / CB_DECODE_MIN_STAGES waves then gives every wave at least one stage: the
// slowest workgroup's rate times CB_DECODE_MIN_STAGES exceeds the fastest one's (10^4).
static_assert(CB_DECODE_MIN_STAGES *
                  (CB_DECODE_RATE_SECOND < 100 - CB_DECODE_SHARE_SLOW ? CB_DECODE_RATE_SECOND : 100 - CB_DECODE_SHARE_SLOW) *
                  CB_DECODE_RATE_ODD_XCD > 10000,
              "non-empty waves");

constexpr int kChunkRows = 128;   // rows per chunk tile: 4 waves x 32
// Chunk tiles let a row's softmax reference lag its running maximum by up to this much (log2
// units): weights 2^(s c - m_ref) stay below 2^8, and the accumulator is rescaled only when a
// maximum jumps further.
constexpr float kRescaleSlack = 8.f;
constexpr int kChunkKeys = 32;    // keys per LDS stage of a chunk tile
#ifndef CB_CHUNK_STAGES
#define CB_CHUNK_STAGES 4             // chunk K/V stages in the LDS ring (copies run NS - 1 ahead)
#endif
constexpr int kChunkStages = CB_CHUNK_STAGES;
static_assert(kChunkStages >= 3 && kChunkStages <= 8, "chunk ring depth");
constexpr int kDecodeKeys = 32;   // keys per decode stage
constexpr int kMaxSplit = 8;
constexpr int kMinBlock = 8;
constexpr int kMaxBlock = 256;
constexpr int kSubKeys = 3840;                       // longest decode sub-range with one block-id load
constexpr int kSubBlocks = 512;                      // >= kSubKeys / kMinBlock + 1
static_assert(kSubKeys % kDecodeKeys == 0 && kSubKeys / kMinBlock + 1 <= kSubBlocks, "sub-range");
constexpr int kMaxDecodeWaves = 8192;                // workspace bound on the decode grid
constexpr int kBlockWindow = 2048;                   // block ids per LDS window (chunk tiles)

struct Plan {
  int32_t G = 1, head_blocks = 1, hw = 1, ups = 1;
  int32_t bmq = 128, q_blocks = 0, n_chunk = 0, nsplit = 1;
  size_t dec_o = 0, dec_ml = 0, chk_o = 0, chk_ml = 0, dec_seq = 0, dec_wave = 0, dec_pos = 0, dec_par = 0,
         dec_unit = 0;
  size_t total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Chunk tiling of a launch for tiles of `rows` query rows: positions per query block, query blocks
// per chunk, tiles before the key split, and the split: keys are split (and merged by the combine)
// until the launch has CB_CHUNK_MIN_TILES 128-row tiles' worth of waves (CB_CHUNK_MIN_TILES_MIXED
// beside decode rows) while each split keeps CB_CHUNK_SPLIT_KEYS keys of the longest context
// (CB_CHUNK_SPLIT_KEYS_MIXED beside decode rows).
struct ChunkSplit {
  int32_t bmq = 1, q_blocks = 0, nsplit = 1;
  int64_t tiles = 0;
};
ChunkSplit chunk_split(int32_t n_chunk, int32_t Hkv, int32_t G, int32_t rows, int32_t nd, int32_t max_q_len,
                       int32_t max_ctx) {
  ChunkSplit c;
  c.bmq = rows / G;
  if (n_chunk <= 0) return c;
  c.q_blocks = (std::max(max_q_len, 1) + c.bmq - 1) / c.bmq;
  c.tiles = static_cast<int64_t>(n_chunk) * c.q_blocks * Hkv;
  const int64_t min_tiles = static_cast<int64_t>(nd > 0 ? CB_CHUNK_MIN_TILES_MIXED : CB_CHUNK_MIN_TILES) * kChunkRows / rows;
  const int32_t min_keys = nd > 0 ? CB_CHUNK_SPLIT_KEYS_MIXED : CB_CHUNK_SPLIT_KEYS;
  while (c.nsplit < kMaxSplit && c.tiles * c.nsplit < min_tiles && max_ctx / (2 * c.nsplit) >= min_keys)
    c.nsplit *= 2;
  return c;
}

// Partitioning decisions, shared by the workspace query and the launch so they always agree.
// Decode partials: one slot per (unit, wave) pair that shares stages, at most units + waves
// slots of hw heads each (a unit is a decode row's KV head and 16-head block).
Plan make_plan(int32_t num_seqs, int32_t nd, int32_t T, int32_t max_q_len, int32_t max_ctx,
               int32_t Hq, int32_t Hkv, int32_t D) {
  Plan p;
  p.G = Hq / Hkv;
  p.head_blocks = (p.G + 15) / 16;
  p.hw = std::min(16, p.G);
  p.ups = Hkv * p.head_blocks;
  p.n_chunk = num_seqs - nd;
  const ChunkSplit cs = chunk_split(p.n_chunk, Hkv, p.G, kChunkRows, nd, max_q_len, max_ctx);
  p.bmq = cs.bmq;
  p.q_blocks = cs.q_blocks;
  p.nsplit = cs.nsplit;
  size_t off = 0;
  const size_t dec_slots = nd > 0 ? static_cast<size_t>(nd) * p.ups + kMaxDecodeWaves : 0;
  p.dec_o = off;  off = align256(off + dec_slots * p.hw * D * sizeof(float));
  p.dec_ml = off; off = align256(off + dec_slots * p.hw * 2 * sizeof(float));
  const size_t chk_rows = p.nsplit > 1 ? static_cast<size_t>(T - nd) * Hq * p.nsplit : 0;
  p.chk_o = off;  off = align256(off + chk_rows * D * sizeof(float));
  p.chk_ml = off; off = align256(off + chk_rows * 2 * sizeof(float));
  p.dec_seq = off;  off = align256(off + (nd > 0 ? static_cast<size_t>(nd + 1) * sizeof(int32_t) : 0));
  p.dec_wave = off; off = align256(off + (nd > 0 ? kMaxDecodeWaves * sizeof(int32_t) : 0));
  p.dec_pos = off;  off = align256(off + (nd > 0 ? (kMaxDecodeWaves + 1) * sizeof(int32_t) : 0));
  p.dec_par = off;  off = align256(off + (nd > 0 ? 4 * sizeof(int32_t) : 0));
  p.dec_unit = off; off = align256(off + (nd > 0 ? static_cast<size_t>(nd) * p.ups * 2 * sizeof(int32_t) : 0));
  p.total = off;
  return p;
}

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_q;
  const int32_t* ctx_lens;
  const int32_t* cu_blocks;
  const int32_t* block_table;
  void* out;
  float* dec_o;          // decode partials, slot-major: [slot][hw][D] and [slot][hw][2]
  float* dec_ml;
  float* chk_o;
  float* chk_ml;
  int32_t* dec_seq;      // [nd + 1] first stage of each decode row on the stage line; [nd] = total
  int32_t* dec_wave;     // [waves] unit holding each wave's first stage
  int32_t* dec_pos;      // [W + 1] first stage of each wave's range; [W] = S
  int32_t* dec_par;      // [0] total stages S, [1] first-round workgroups F, [2] waves with work W
  int32_t* dec_unit;     // [units][2] waves holding each unit's first and last stage (written by them)
  int32_t num_seqs, nd, T, Hq, Hkv, G, bs, bs_shift;
  int32_t head_blocks, hw, ups;
  int32_t bmq, q_blocks, n_chunk, nsplit;
  int32_t max_q_len, max_ctx;
  float scale_log2;
};

// Decode stages (32 keys) of a row with this many cached-plus-current keys.
__device__ __forceinline__ int32_t decode_stages(int32_t ctx) { return ctx > 0 ? (ctx + kDecodeKeys - 1) / kDecodeKeys : 0; }

// ---------------------------------------------------------------------------------------------
// LDS staging.  K and V rows are copied from HBM straight into LDS with the gfx950 16-byte LDS
// DMA (global_load_lds_dwordx4): lane l of one instruction lands at byte 16 l of a 1 KB span.
// Rows are chunk-swizzled: logical 16-byte chunk c of row r sits at chunk c ^ s(r).  Every
// 256-byte row starts at bank 0, so s decides the banks:
//   256+ byte rows: s(r) = 4 (r mod 4) + (r / 4) mod 4.  Sixteen consecutive rows read at one
//     chunk (the K operand reads) get 16 different s; four consecutive rows read at four aligned
//     consecutive chunks (the transposing V reads) differ in bits 2-3 of s, so all 16 (row,
//     chunk) pairs land on different 16-byte bank groups.
//   128-byte rows (two rows per bank line): with q = (r / 2) mod 8, s(r) = 4 (q mod 2) + q / 2,
//     which gives the same two properties.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int lds_chunk(int c, int r, int row_bytes) {
  if (row_bytes >= 256) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  const int q = (r >> 1) & 7;
  return c ^ (((q & 1) << 2) | (q >> 1));
}
// LDS byte address of a pointer into shared memory (the address operand of ds_read).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}
__device__ __forceinline__ void lds_copy16(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src),
                                   (void __attribute__((address_space(3)))*)(lds_dst),
                                   16, 0, 0);
}
// The same copy issued from inline asm.  The compiler does not see it, so it adds no vmcnt waits
// for it anywhere: the code that issues these waits for them itself (wait_vm_barrier).  Copies
// complete in issue order with every other vector-memory operation, so the compiler's own waits
// stay correct (they only become stricter).  M0 carries the wave-uniform LDS destination; it is
// saved and restored around the copy (M0 is reserved, so a clobber would not be honoured), with
// one wait state between the M0 write and the copy that reads it.
__device__ __forceinline__ void lds_copy16_asm(const char* src, const char* lds_dst) {
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
// The same copy from a wave-uniform 64-bit base (SGPRs) plus a 32-bit per-lane offset: the
// instruction's scalar-base form, with no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void lds_copy16_asm_s(const char* base, uint32_t voff, const char* lds_dst) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(lds_dst));
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
// K and V copies of one wave's rows of a stage in one asm block: for each of its NC copy
// instructions j, K then V, from the wave-uniform bases kb[j] / vb[j] plus the lane's 32-bit
// offset voff[j], into the LDS spans dk[j] / dv[j] (wave-uniform).  No immediate offset: the
// LDS DMA adds it to the LDS address as well.  M0 is saved once, set before each copy (one wait
// state before the copy reads it) and restored.
template <int NC>
__device__ __forceinline__ void dma_kv(const char* const (&kb)[NC], const char* const (&vb)[NC], const uint32_t (&voff)[NC],
                                       const uint32_t (&dk)[NC], const uint32_t (&dv)[NC]) {
  static_assert(NC == 1 || NC == 2, "one or two copies per tensor");
  uint32_t saved;
  if constexpr (NC == 1) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff[0]), "s"(kb[0]), "s"(vb[0]), "s"(dk[0]), "s"(dv[0]));
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %7\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "s_mov_b32 m0, %8\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %4\n\t"
        "s_mov_b32 m0, %9\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %5\n\t"
        "s_mov_b32 m0, %10\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %6\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff[0]), "v"(voff[1]), "s"(kb[0]), "s"(vb[0]), "s"(kb[1]), "s"(vb[1]), "s"(dk[0]), "s"(dv[0]),
          "s"(dk[1]), "s"(dv[1]));
  }
}
// Maximum of a lane's 16 scores in eight v_max3_f32 of one asm block (no canonicalising moves
// around each fmaxf, no wait states between the steps; the operands are matrix-core results or
// -inf, never signalling NaNs).
__device__ __forceinline__ float max16_raw(const f32x16& v) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3\n\t"
      "v_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\t"
      "v_max3_f32 %0, %0, %8, %9\n\t"
      "v_max3_f32 %0, %0, %10, %11\n\t"
      "v_max3_f32 %0, %0, %12, %13\n\t"
      "v_max3_f32 %0, %0, %14, %15\n\t"
      "v_max_f32 %0, %0, %16"
      : "=&v"(r)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]),
        "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
  return r;
}
// Scalar (SMEM) load of one int32 from a wave-uniform address, issued without waiting; the
// value may be used only after sload_ready (s_waitcnt lgkmcnt(0), which the value passes
// through, so no use can be scheduled before it).
__device__ __forceinline__ int32_t sload_issue(const int32_t* p) {
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0" : "=s"(v) : "s"(p) : "memory");
  return v;
}
__device__ __forceinline__ void sload_ready(int32_t& v) { asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(v)); }
// Wait for this wave's LDS reads before a DMA overwrites the buffer they read
// (s_waitcnt lgkmcnt(0), vmcnt and expcnt untouched).
__device__ __forceinline__ void lds_reads_done() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// 8 consecutive elements [e0, e0 + 8) of row r.
template <typename T>
__device__ __forceinline__ Frag<T> lds_row_frag(const char* base, int r, int e0, int row_bytes) {
  Frag<T> f;
  const char* row = base + r * row_bytes;
  const int b0 = e0 * static_cast<int>(sizeof(T));
  if constexpr (sizeof(T) == 2) {
    f.u = *reinterpret_cast<const uint4*>(row + 16 * lds_chunk(b0 >> 4, r, row_bytes));
  } else {
    const float4 x = *reinterpret_cast<const float4*>(row + 16 * lds_chunk(b0 >> 4, r, row_bytes));
    const float4 y = *reinterpret_cast<const float4*>(row + 16 * lds_chunk((b0 >> 4) + 1, r, row_bytes));
    f.f[0] = x.x; f.f[1] = x.y; f.f[2] = x.z; f.f[3] = x.w;
    f.f[4] = y.x; f.f[5] = y.y; f.f[6] = y.z; f.f[7] = y.w;
  }
  return f;
}

// The V^T operand of a 16x16x32 step: lane (grp, col) gets dimension 16 dt + col of keys
// 16 h + 4 grp + j (slot 4 h + j), h in {0, 1}, j in 0..3, from a 32-key stage of V rows.
// bf16: two ds_read_b64_tr_b16, whose 16-lane groups return, to lane i, element i % 4 of the
// 8-byte row piece addressed by lane 4 j + i / 4 -- so lane 4 j + q addresses row (key) base + j
// at dimensions 16 dt + 4 q .. + 3.  float: eight 4-byte reads.
template <typename T>
__device__ __forceinline__ Frag<T> lds_vt_frag16(const char* base, int dt, int grp, int col, int row_bytes);
template <>
__device__ __forceinline__ Frag<bf16_t> lds_vt_frag16<bf16_t>(const char* base, int dt, int grp, int col, int row_bytes) {
  typedef __attribute__((ext_vector_type(4))) short s4;
  Frag<bf16_t> f;
  const int j = col >> 2, qd = col & 3;
  const int e = 16 * dt + 4 * qd;                 // first dimension addressed by this lane
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * h + 4 * grp + j;
    const char* addr = base + r * row_bytes + 16 * lds_chunk((2 * e) >> 4, r, row_bytes) + ((2 * e) & 15);
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s4 __attribute__((address_space(3)))*)(const_cast<char*>(addr)));
    w[2 * h] = static_cast<uint16_t>(v[0]) | (static_cast<uint32_t>(static_cast<uint16_t>(v[1])) << 16);
    w[2 * h + 1] = static_cast<uint16_t>(v[2]) | (static_cast<uint32_t>(static_cast<uint16_t>(v[3])) << 16);
  }
  f.u = make_uint4(w[0], w[1], w[2], w[3]);
  return f;
}
template <>
__device__ __forceinline__ Frag<float> lds_vt_frag16<float>(const char* base, int dt, int grp, int col, int row_bytes) {
  Frag<float> f;
  const int dim = 16 * dt + col;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int r = 16 * (jj >> 2) + 4 * grp + (jj & 3);
    f.f[jj] = *reinterpret_cast<const float*>(base + r * row_bytes + 16 * lds_chunk((4 * dim) >> 4, r, row_bytes) + ((4 * dim) & 15));
  }
  return f;
}

// The V^T operand of a 32x32x16 step over keys [16 ps, 16 ps + 16) of a stage: lane l gets
// dimension 32 mt + l % 32 of the keys in slot order 8 (l / 32) + jj <-> key
// 16 ps + 8 (jj / 4) + 4 (l / 32) + jj % 4 (the key order of the S^T accumulator).  bf16: two
// ds_read_b64_tr_b16 (VRegs below), lane 16 grp + 4 j + qd addressing row
// 16 ps + 8 h + 4 (grp / 2) + j at dimensions 32 mt + 16 (grp % 2) + 4 qd .. + 3 for h = 0, 1;
// float: eight 4-byte reads.
template <typename T>
__device__ __forceinline__ Frag<T> lds_vt_frag32(const char* base, int mt, int ps, int lane, int row_bytes);
template <>
__device__ __forceinline__ Frag<float> lds_vt_frag32<float>(const char* base, int mt, int ps, int lane, int row_bytes) {
  Frag<float> f;
  const int dim = 32 * mt + (lane & 31);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int r = 16 * ps + 8 * (jj >> 2) + 4 * (lane >> 5) + (jj & 3);
    f.f[jj] = *reinterpret_cast<const float*>(base + r * row_bytes + 16 * lds_chunk((4 * dim) >> 4, r, row_bytes) + ((4 * dim) & 15));
  }
  return f;
}

// Wait until at most N of this wave's vector-memory operations are outstanding (memory returns
// in issue order, so every older LDS copy has landed), then the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// wait_vm_barrier<later * PER>() for a run-time later in [0, MAXL] (larger values wait as MAXL).
template <int PER, int MAXL>
__device__ __forceinline__ void wait_vm_barrier_later(int32_t later) {
  if constexpr (MAXL <= 0) {
    wait_vm_barrier<0>();
  } else {
    if (later >= MAXL) wait_vm_barrier<MAXL * PER>();
    else wait_vm_barrier_later<PER, MAXL - 1>(later);
  }
}

// f(std::integral_constant<int, I>) for I = 0 .. N - 1, unrolled at compile time.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The operands of one 32-key chunk stage (bf16): K rows (KS ds_read_b128) and V^T (two
// ds_read_b64_tr_b16 per 32x16 piece, the second 16 keys further down).  ka[ks] / va[2 mt + h]
// are the LDS addresses lds_row_frag and the V^T layout above read in ring buffer 0 (piece
// ps = 0); OFF selects the ring buffer (an immediate offset), and ps = 1 is 16 rows further.
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
// Two asm blocks issue them without waiting: K rows (KRegs) and V^T (VRegs), in the ring buffer
// selected by OFF.  The waits below pass every destination register through the wait, so no use
// of them can be scheduled before it.
template <int D> struct KRegs;
template <int D> struct VRegs;
template <> struct KRegs<128> {
  u32x4 k[8];
  template <int OFF>
  __device__ __forceinline__ void read(const uint32_t (&ka)[8]) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%16\n\t"
        "ds_read_b128 %1, %9 offset:%16\n\t"
        "ds_read_b128 %2, %10 offset:%16\n\t"
        "ds_read_b128 %3, %11 offset:%16\n\t"
        "ds_read_b128 %4, %12 offset:%16\n\t"
        "ds_read_b128 %5, %13 offset:%16\n\t"
        "ds_read_b128 %6, %14 offset:%16\n\t"
        "ds_read_b128 %7, %15 offset:%16"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]), "=&v"(k[7])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ka[4]), "v"(ka[5]), "v"(ka[6]), "v"(ka[7]), "n"(OFF));
  }
};
template <> struct KRegs<64> {
  u32x4 k[4];
  template <int OFF>
  __device__ __forceinline__ void read(const uint32_t (&ka)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%8\n\t"
        "ds_read_b128 %1, %5 offset:%8\n\t"
        "ds_read_b128 %2, %6 offset:%8\n\t"
        "ds_read_b128 %3, %7 offset:%8"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "n"(OFF));
  }
};
template <> struct VRegs<128> {
  u32x2 v[2][8];   // [ps][2 mt + h]
  template <int OFF>
  __device__ __forceinline__ void read(const uint32_t (&va)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %2, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %3, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %5, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %6, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %23 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%25\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:%25\n\t"
        "ds_read_b64_tr_b16 %10, %18 offset:%25\n\t"
        "ds_read_b64_tr_b16 %11, %19 offset:%25\n\t"
        "ds_read_b64_tr_b16 %12, %20 offset:%25\n\t"
        "ds_read_b64_tr_b16 %13, %21 offset:%25\n\t"
        "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
        "ds_read_b64_tr_b16 %15, %23 offset:%25"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[0][4]), "=&v"(v[0][5]), "=&v"(v[0][6]), "=&v"(v[0][7]),
          "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3]), "=&v"(v[1][4]), "=&v"(v[1][5]), "=&v"(v[1][6]), "=&v"(v[1][7])
        : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]), "n"(OFF), "n"(OFF + 4096));
  }
};
template <> struct VRegs<64> {
  u32x2 v[2][4];   // [ps][2 mt + h]
  template <int OFF>
  __device__ __forceinline__ void read(const uint32_t (&va)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %10 offset:%13\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%13"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]), "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3])
        : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "n"(OFF), "n"(OFF + 2048));
  }
};
// Wait for the K reads of a stage issued before its V reads (LDS reads of a wave complete in
// order, so at most the V reads may still be outstanding; the counter holds at most 15).
template <int D>
__device__ __forceinline__ void lds_k_ready(KRegs<D>& kr) {
  if constexpr (D == 128)
    asm volatile("s_waitcnt lgkmcnt(15)" : "+v"(kr.k[0]), "+v"(kr.k[1]), "+v"(kr.k[2]), "+v"(kr.k[3]), "+v"(kr.k[4]), "+v"(kr.k[5]), "+v"(kr.k[6]), "+v"(kr.k[7]));
  else
    asm volatile("s_waitcnt lgkmcnt(8)" : "+v"(kr.k[0]), "+v"(kr.k[1]), "+v"(kr.k[2]), "+v"(kr.k[3]));
}
// Wait for every outstanding LDS read of the wave (K rows read with no V reads behind them).
template <int D>
__device__ __forceinline__ void lds_operands_ready(KRegs<D>& kr) {
  if constexpr (D == 128)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kr.k[0]), "+v"(kr.k[1]), "+v"(kr.k[2]), "+v"(kr.k[3]), "+v"(kr.k[4]), "+v"(kr.k[5]), "+v"(kr.k[6]), "+v"(kr.k[7]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kr.k[0]), "+v"(kr.k[1]), "+v"(kr.k[2]), "+v"(kr.k[3]));
}
// The wait for V, ordered after the packed weights P of the stage (they pass through it
// too): the scheduler may otherwise hoist the wait above the score products, so that these
// would also wait for the V reads.
template <int D>
__device__ __forceinline__ void lds_v_ready_after(VRegs<D>& vr, u32x4& p0, u32x4& p1) {
  if constexpr (D == 128)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vr.v[0][0]), "+v"(vr.v[0][1]), "+v"(vr.v[0][2]), "+v"(vr.v[0][3]), "+v"(vr.v[0][4]), "+v"(vr.v[0][5]), "+v"(vr.v[0][6]), "+v"(vr.v[0][7]),
                   "+v"(vr.v[1][0]), "+v"(vr.v[1][1]), "+v"(vr.v[1][2]), "+v"(vr.v[1][3]), "+v"(vr.v[1][4]), "+v"(vr.v[1][5]), "+v"(vr.v[1][6]), "+v"(vr.v[1][7]),
                   "+v"(p0), "+v"(p1));
  else
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vr.v[0][0]), "+v"(vr.v[0][1]), "+v"(vr.v[0][2]), "+v"(vr.v[0][3]), "+v"(vr.v[1][0]), "+v"(vr.v[1][1]), "+v"(vr.v[1][2]), "+v"(vr.v[1][3]),
                   "+v"(p0), "+v"(p1));
}

// ---------------------------------------------------------------------------------------------
// Decode rows.
// ---------------------------------------------------------------------------------------------
// Work layout: a decode row s with context c has units (KV head g, 16-head block hb), each of
// decode_stages(c) 32-key stages.  All units of all rows, in order, form one line of S stages,
// cut into W = min(waves, S / CB_DECODE_MIN_STAGES) contiguous ranges (one at least when S > 0).
// Wave w runs in workgroup w / 4; workgroup b runs on XCD b mod 8, and workgroups [0, F) are the
// first on their compute unit (F = compute units rounded up to a multiple of 8).  Its range is
// [start(w), start(w + 1)) with start(w) = floor(S C(w) / C(W)), C(w) the summed rates of waves
// [0, w): every wave's work is proportional to its rate, so all end together.  A unit is shared by
// the few consecutive waves whose ranges meet it.  Each (unit, wave) pair yields one partial
// (m, l, o) in slot unit + wave: both indices grow along the line, so the slot is unique and a
// unit's partials sit in consecutive slots.
//
// Rates (percent products): 100, or CB_DECODE_RATE_SECOND for workgroups [F, 2F), times 100 or
// CB_DECODE_RATE_ODD_XCD by XCD parity.  Beside chunk tiles, chunk workgroup b (the b-th after
// the decode workgroups) is dispatched onto the compute unit of decode workgroup b < F; when every
// decode wave of the launch has work (W = waves), that workgroup's rate loses CB_DECODE_SHARE_SLOW
// x min(1, rho) percent, rho = the tile's key stages x CB_DECODE_SHARE_RATIO / 100 over the mean
// stages per wave S / W (the share of the decode launch the tile lasts).  Smaller decode loads
// keep the split they have without chunk rows (W = S / CB_DECODE_MIN_STAGES either way), so
// their results do not depend on the chunk rows beside them.
//
// The prep workgroup (or the host, for a plan made there, with the same integer rule) scans the
// rows' stage counts into dec_seq (first stage of each row), picks W, and records each wave's
// start(w) in dec_pos (dec_pos[W] = S) and the unit holding its first stage; dec_par holds
// [S, F, W].
__host__ __device__ __forceinline__ int32_t decode_waves_used(int32_t S, int32_t n_waves) {
  if (S <= 0) return 0;
  const int32_t k = S / CB_DECODE_MIN_STAGES;
  return k < 1 ? 1 : (k > n_waves ? n_waves : k);
}

// Chunk tiles are numbered with the key split fastest, then the query block (last block first:
// under the causal mask later blocks see more keys, so a launch hands out the longest tiles of a
// chunk first and the short ones fill in behind them), the KV head and the chunk.  The tile's
// chunk s, KV head g, query block qb, split sp, the chunk's first row and
// length d, its cached prefix c, and the split's key stages [kt_lo, kt_hi).  False when the query
// block lies past the chunk's end (the tile has no rows).
struct TileSpan {
  int32_t s, g, qb, sp, row0, d, c, kt_lo, kt_hi;
};
struct TileGrid {
  int32_t nd, Hkv, q_blocks, nsplit, bmq;
  int64_t n_tiles, per_xcd;     // tiles; chunk workgroups per XCD (launch order below)
};
// The tile's chunk, KV head, query block and split from its number alone.
__host__ __device__ __forceinline__ void chunk_tile_index(int32_t tile, const TileGrid& tg, TileSpan& t) {
  int32_t x = tile;
  t.sp = x % tg.nsplit; x /= tg.nsplit;
  t.qb = tg.q_blocks - 1 - x % tg.q_blocks; x /= tg.q_blocks;
  t.g = x % tg.Hkv;
  t.s = tg.nd + x / tg.Hkv;
}
// The rest of the span from the chunk's row offsets q0 = cu_q[s], q1 = cu_q[s + 1] and its
// context length ctx = ctx_lens[s].
__host__ __device__ __forceinline__ bool chunk_tile_rows(const TileGrid& tg, int32_t q0, int32_t q1, int32_t ctx,
                                                         TileSpan& t) {
  t.row0 = q0;
  t.d = q1 - q0;
  if (t.qb * tg.bmq >= t.d) return false;
  t.c = ctx - t.d;
  const int32_t rows = (t.qb + 1) * tg.bmq < t.d ? (t.qb + 1) * tg.bmq : t.d;
  const int32_t total = (t.c + rows + kChunkKeys - 1) / kChunkKeys;   // stages up to the block's last key
  const int32_t per = (total + tg.nsplit - 1) / tg.nsplit;
  t.kt_lo = t.sp * per;
  t.kt_hi = total < t.kt_lo + per ? total : t.kt_lo + per;
  return true;
}
__host__ __device__ __forceinline__ bool chunk_tile_span(int32_t tile, const TileGrid& tg, const int32_t* cu_q,
                                                         const int32_t* ctx_lens, TileSpan& t) {
  chunk_tile_index(tile, tg, t);
  return chunk_tile_rows(tg, cu_q[t.s], cu_q[t.s + 1], ctx_lens[t.s], t);
}
// Chunk workgroup cb of a launch runs tile (cb mod 8) per_xcd + cb / 8 (XCD-aware order).
__host__ __device__ __forceinline__ int64_t chunk_wg_tile(int64_t cb, int64_t per_xcd) {
  return (cb & 7) * per_xcd + (cb >> 3);
}
// Key stages of the chunk tile that shares a compute unit with decode workgroup b (0 if none).
__host__ __device__ __forceinline__ int32_t beside_tile_stages(int32_t b, const TileGrid& tg, const int32_t* cu_q,
                                                               const int32_t* ctx_lens) {
  if (tg.n_tiles <= 0 || b >= 8 * tg.per_xcd) return 0;
  const int64_t tile = chunk_wg_tile(b, tg.per_xcd);
  TileSpan t;
  if (tile >= tg.n_tiles || !chunk_tile_span(static_cast<int32_t>(tile), tg, cu_q, ctx_lens, t)) return 0;
  return t.kt_hi > t.kt_lo ? t.kt_hi - t.kt_lo : 0;
}
// Rate of decode workgroup b (see above); ts = beside_tile_stages(b) when W = waves, else 0.
__host__ __device__ __forceinline__ int32_t decode_wg_rate(int32_t b, int32_t F, int32_t ts, int32_t S, int32_t W) {
  int64_t base = b < F ? 100 : CB_DECODE_RATE_SECOND;
  if (b < F && ts > 0) {
    const int64_t slow = static_cast<int64_t>(CB_DECODE_SHARE_SLOW) * CB_DECODE_SHARE_RATIO * ts * W / (100LL * S);
    base -= slow < CB_DECODE_SHARE_SLOW ? slow : CB_DECODE_SHARE_SLOW;
  }
  return static_cast<int32_t>(base * ((b & 1) ? CB_DECODE_RATE_ODD_XCD : 100));
}
// start(w) from the workgroups' rate prefix P (P[b] = summed rates of workgroups [0, b)), four
// waves per workgroup: C(w) = 4 P[w / 4] + (w mod 4) rate(w / 4).  P[b] <= 2048 x 10^4 and S <
// 2^31, so S C(w) fits int64.
__host__ __device__ __forceinline__ int64_t decode_rate_prefix(int32_t w, const int32_t* P) {
  const int32_t b = w >> 2, r = w & 3;
  return 4 * static_cast<int64_t>(P[b]) + (r ? static_cast<int64_t>(r) * (P[b + 1] - P[b]) : 0);
}
__host__ __device__ __forceinline__ int32_t decode_wave_start(int32_t w, int32_t S, int64_t cw, const int32_t* P) {
  return static_cast<int32_t>(static_cast<int64_t>(S) * decode_rate_prefix(w, P) / cw);
}
__device__ __forceinline__ int32_t block_scan_1024(int32_t v, int32_t* scan) {
  const int tid = threadIdx.x;
  scan[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {       // inclusive prefix sum
    const int32_t u = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += u;
    __syncthreads();
  }
  return scan[tid];
}

constexpr int kPrepRows = 8192;   // decode rows whose stage offsets the prep workgroup keeps in LDS

__global__ __launch_bounds__(1024) void decode_prep_kernel(AttnArgs a, int32_t n_waves, int32_t F, TileGrid tg) {
  __shared__ int32_t scan[1024];
  __shared__ int32_t seq_lds[kPrepRows + 1];
  __shared__ int32_t prefix[kMaxDecodeWaves / 4 + 1];   // P[b]: summed rates of workgroups [0, b)
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  // The searches below read the row offsets from LDS when they fit (one LDS round trip per
  // search step instead of a global one).
  const bool in_lds = a.nd <= kPrepRows;
  const int32_t* seq = in_lds ? seq_lds : a.dec_seq;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int32_t base = 0; base < a.nd; base += 1024) {
    const int32_t s = base + tid;
    const int32_t n = s < a.nd ? decode_stages(a.ctx_lens[s]) * a.ups : 0;
    const int32_t incl = block_scan_1024(n, scan);
    if (s < a.nd) {
      a.dec_seq[s] = carry + incl - n;
      if (in_lds) seq_lds[s] = carry + incl - n;
    }
    __syncthreads();                                  // every thread has read carry
    if (tid == 1023) carry += scan[1023];
    __syncthreads();
  }
  const int32_t S = carry;
  const int32_t W = decode_waves_used(S, n_waves);
  const int32_t n_wg = (W + 3) >> 2;
  __syncthreads();                                    // every thread has read carry
  if (tid == 0) {
    a.dec_seq[a.nd] = S;
    if (in_lds) seq_lds[a.nd] = S;
    a.dec_par[0] = S;
    a.dec_par[1] = F;
    a.dec_par[2] = W;
    prefix[0] = 0;
    carry = 0;
  }
  __syncthreads();
  const bool full = W == n_waves;
  for (int32_t base = 0; base < n_wg; base += 1024) {  // workgroup rates, scanned
    const int32_t b = base + tid;
    const int32_t ts = b < n_wg && full ? beside_tile_stages(b, tg, a.cu_q, a.ctx_lens) : 0;
    const int32_t r = b < n_wg ? decode_wg_rate(b, F, ts, S, W) : 0;
    const int32_t incl = block_scan_1024(r, scan);
    if (b < n_wg) prefix[b + 1] = carry + incl;
    __syncthreads();
    if (tid == 1023) carry += scan[1023];
    __syncthreads();
  }
  const int64_t cw = decode_rate_prefix(W, prefix);
  for (int32_t w = tid; w <= W; w += 1024) {
    const int32_t pos = w < W ? decode_wave_start(w, S, cw, prefix) : S;
    a.dec_pos[w] = pos;
    if (w == W) continue;
    int32_t lo = 0, hi = a.nd;                        // seq[lo] <= pos < seq[hi]
    while (hi - lo > 1) {
      const int32_t mid = (lo + hi) >> 1;
      if (seq[mid] <= pos) lo = mid;
      else hi = mid;
    }
    // The row's units each have (seq[lo + 1] - seq[lo]) / ups stages (> 0: pos falls inside it).
    a.dec_wave[w] = lo * a.ups + (pos - seq[lo]) / ((seq[lo + 1] - seq[lo]) / a.ups);
  }
}

// Persistent waves, one per stage range.  A wave walks its range as sub-ranges of at most
// kSubKeys keys inside one unit (block ids of a sub-range are loaded once into LDS); the softmax
// state carries across sub-ranges of the same unit and is written as a partial at the unit's
// last one.  The next sub-range's query and block ids are loaded right after a copy is issued
// (waiting for that copy also covers them) and its first K/V stage is copied during the current
// sub-range's last stage, so the wave keeps one stage in flight from start to end.
// LDS of one decode wave: a K stage, a V stage and the sub-range's block ids.
template <typename T, int D>
struct DecodeLds {
  static constexpr int ROW = D * sizeof(T);
  static constexpr int V = kDecodeKeys * ROW;
  static constexpr int BLK = 2 * kDecodeKeys * ROW;
  static constexpr int BYTES = BLK + kSubBlocks * 4;
  static_assert(BYTES % 1024 == 0, "wave slices keep 1 KB alignment");
};

template <typename T, int D>
__device__ __forceinline__ void decode_wave(const AttnArgs& a, const int32_t* seq_start, const int32_t* wave_unit,
                                            const int32_t* wave_pos, const int32_t* par, const int32_t* ctx_lens,
                                            const int32_t* cu_blocks, int32_t w, int lane, char* lds) {
  constexpr int KS = D / 32;          // 32-slot contraction steps over the head dimension
  constexpr int DT = D / 16;          // 16-dim output tiles
  constexpr int ROW = D * sizeof(T);  // bytes per key row in LDS
  constexpr int RPI = 1024 / ROW;     // key rows per 1 KB copy instruction
  constexpr int NCP = kDecodeKeys / RPI;
  constexpr int NBR = kSubBlocks / 64;   // block ids per lane of one sub-range
  char* sK = lds;
  char* sV = lds + DecodeLds<T, D>::V;
  int32_t* sBlk = reinterpret_cast<int32_t*>(lds + DecodeLds<T, D>::BLK);

  const int32_t W = par[2];             // uniform, read-only here: scalar loads
  if (w >= W) return;
  const int32_t pos_begin = wave_pos[w];
  const int32_t pos_end = wave_pos[w + 1];

  const int32_t col = lane & 15;      // head owned by this lane in S^T / P^T / O^T
  const int32_t grp = lane >> 4;      // slot group
  const int bsh = a.bs_shift;
  const int32_t bmask = (1 << bsh) - 1;
  const T* q = static_cast<const T*>(a.q);
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  const int64_t blk_bytes = static_cast<int64_t>(a.Hkv) * ((int64_t)ROW << bsh);
  const int cp_row = lane / (ROW / 16), cp_pos = lane % (ROW / 16);

  // Cursor on the stage line: position pos inside unit u = (row s, unit r of the row), whose
  // first stage is a_u; n_s stages per unit of row s.
  struct Cursor {
    int32_t pos, u, s, r, a_u, n_s, ctx, cub;
  };
  struct Item {
    int32_t s, cub, k_lo, k_hi, h0, gh, slot;
    int64_t head_bytes;
    bool last;                        // last sub-range of its (unit, wave) partial
  };
  auto load_row = [&](Cursor& c, int32_t s) {        // first unit of row s
    c.s = s;
    c.r = 0;
    c.ctx = ctx_lens[s];
    c.n_s = decode_stages(c.ctx);
    c.cub = cu_blocks[s];
    c.a_u = seq_start[s];
    c.u = s * a.ups;
  };
  Cursor cur_c;
  cur_c.pos = pos_begin;
  {
    const int32_t u0 = wave_unit[w];
    load_row(cur_c, u0 / a.ups);
    cur_c.r = u0 - cur_c.s * a.ups;
    cur_c.u = u0;
    cur_c.a_u += cur_c.r * cur_c.n_s;
  }
  // The sub-range at the cursor; moves the cursor past it (to the next non-empty unit when the
  // unit is finished and the wave's range goes on).
  auto take = [&](Cursor& c) {
    Item it;
    const int32_t unit_end = c.a_u + c.n_s;
    const int32_t seg_end = min(pos_end, unit_end);
    const int32_t sub_end = min(seg_end, c.pos + kSubKeys / kDecodeKeys);
    const int32_t g = c.r / a.head_blocks;
    const int32_t hb = c.r - g * a.head_blocks;
    it.s = c.s;
    it.cub = c.cub;
    it.k_lo = (c.pos - c.a_u) * kDecodeKeys;
    it.k_hi = min((sub_end - c.a_u) * kDecodeKeys, c.ctx);
    it.h0 = g * a.G + 16 * hb;
    it.gh = min(16, a.G - 16 * hb);
    it.slot = c.u + w;
    it.head_bytes = static_cast<int64_t>(g) * ((int64_t)ROW << bsh);
    it.last = sub_end == seg_end;
    // The combine finds a unit's partials (slots u + w0 .. u + w1) from these two records.
    if (lane == 0) {
      if (c.pos == c.a_u) a.dec_unit[2 * c.u] = w;
      if (sub_end == unit_end) a.dec_unit[2 * c.u + 1] = w;
    }
    c.pos = sub_end;
    if (c.pos == unit_end && c.pos < pos_end) {
      if (c.r + 1 < a.ups) {
        ++c.r;
        ++c.u;
        c.a_u = unit_end;
      } else {
        int32_t s = c.s + 1;
        while (decode_stages(ctx_lens[s]) == 0) ++s;   // rows with no keys own no stages
        load_row(c, s);
      }
    }
    return it;
  };

  // Block ids of a sub-range and the query into registers (consumed later: no wait here).
  auto fetch = [&](const Item& it, int32_t (&blk)[NBR], Frag<T> (&qd)[KS]) {
    const int32_t* btab = a.block_table + it.cub + (it.k_lo >> bsh);
    const int32_t nblk = ((it.k_hi - 1) >> bsh) - (it.k_lo >> bsh) + 1;
#pragma unroll
    for (int i = 0; i < NBR; ++i)
      if (64 * i + lane < nblk) blk[i] = btab[64 * i + lane];
    const T* qrow = q + (static_cast<int64_t>(it.s) * a.Hq + it.h0 + col) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (col < it.gh) qd[ks].load(qrow + 32 * ks + 8 * grp);
      else qd[ks].zero();
    }
  };
  auto publish_blocks = [&](const Item& it, const int32_t (&blk)[NBR]) {
    const int32_t nblk = ((it.k_hi - 1) >> bsh) - (it.k_lo >> bsh) + 1;
#pragma unroll
    for (int i = 0; i < NBR; ++i)
      if (64 * i + lane < nblk) sBlk[64 * i + lane] = blk[i];
  };
  // Copy 32 keys' K and V rows straight into LDS (no registers), chunk-swizzled.  Keys past the
  // sub-range repeat its last key; they are masked out of the softmax.
  auto issue = [&](const Item& it, int32_t key0) {
    const int32_t b_lo = it.k_lo >> bsh;
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int r = i * RPI + cp_row;                        // row within the stage
      const int32_t key = min(key0 + r, it.k_hi - 1);
      const int64_t off = static_cast<int64_t>(sBlk[(key >> bsh) - b_lo]) * blk_bytes + it.head_bytes +
                          static_cast<int64_t>(key & bmask) * ROW + 16 * lds_chunk(cp_pos, r, ROW);
      lds_copy16(kc + off, sK + i * 1024);
      lds_copy16(vc + off, sV + i * 1024);
    }
  };

  int32_t blk[NBR];
  Frag<T> qf[KS], qn[KS];
  Item cur = take(cur_c);
  fetch(cur, blk, qf);
  publish_blocks(cur, blk);          // LDS operations of one wave complete in order
  issue(cur, cur.k_lo);

  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  while (true) {
    const bool has_next = cur_c.pos < pos_end;
    const bool one_stage = cur.k_hi - cur.k_lo <= kDecodeKeys;
    Item nxt{};
    if (has_next && one_stage) {
      nxt = take(cur_c);
      fetch(nxt, blk, qn);
    }

    for (int32_t key0 = cur.k_lo; key0 < cur.k_hi; key0 += kDecodeKeys) {
      // Operands of this stage into registers (the copy has landed: the compiler waits for it
      // before the first LDS read), then the next copy, which overlaps the compute below.
      Frag<T> kf[2][KS];
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[kg][ks] = lds_row_frag<T>(sK, 16 * kg + col, 32 * ks + 8 * grp, ROW);
      Frag<T> vt[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vt[dt] = lds_vt_frag16<T>(sV, dt, grp, col, ROW);
      lds_reads_done();
      if (key0 + kDecodeKeys < cur.k_hi) {
        issue(cur, key0 + kDecodeKeys);
        if (key0 == cur.k_lo && has_next) {
          nxt = take(cur_c);
          fetch(nxt, blk, qn);
        }
      } else if (has_next) {
        publish_blocks(nxt, blk);
        issue(nxt, nxt.k_lo);
      }

      // S^T[key, head]: lane holds keys 16 kg + 4 grp + r of head col.
      f32x4 st[2];
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        st[kg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma16_k32(st[kg], kf[kg][ks], qf[ks]);
      }
      float sv[8];
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int32_t key = key0 + 16 * (j >> 2) + 4 * grp + (j & 3);
        const float x = key < cur.k_hi ? st[j >> 2][j & 3] : kNegInf;
        sv[j] = x;
        mx = fmaxf(mx, x);
      }
      mx = wave_xor_max(mx, 16);
      mx = wave_xor_max(mx, 32);
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float pv[8], psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pv[j] = fast_exp2(fmaf(sv[j], a.scale_log2, -m_use));
        psum += pv[j];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      Frag<T> pf;   // P^T slot 8 grp + j <-> key 16 (j / 4) + 4 grp + j % 4 (same order as sv)
      pf.set_all(pv);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt] *= alpha;
        mma16_k32(o[dt], vt[dt], pf);
      }
    }

    if (cur.last) {
      float l_tot = wave_xor_sum(l_run, 16);
      l_tot = wave_xor_sum(l_tot, 32);
      if (col < cur.gh) {
        const int64_t prow = static_cast<int64_t>(cur.slot) * a.hw + col;
        float* po = a.dec_o + prow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<float4*>(po + 16 * dt + 4 * grp) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
        if (grp == 0) *reinterpret_cast<float2*>(a.dec_ml + 2 * prow) = make_float2(m_run, l_tot);
      }
      m_run = kNegInf;
      l_run = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (!has_next) break;
    cur = nxt;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qn[ks];
  }
}

// ---------------------------------------------------------------------------------------------
// Chunk rows.
// ---------------------------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void store4(T* dst, float x0, float x1, float x2, float x3);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* dst, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<float4*>(dst) = make_float4(x0, x1, x2, x3);
}

// LDS of one chunk tile: the K and V stage rings and a block-id window.
template <typename T, int D>
struct ChunkLds {
  static constexpr int ROW = D * sizeof(T);
  static constexpr int NS = sizeof(T) == 2 ? kChunkStages : 2;   // float stages are twice as large
  static constexpr int STAGE = kChunkKeys * ROW;
  static constexpr int V = NS * STAGE;
  static constexpr int BLK = 2 * NS * STAGE;
  static constexpr int BYTES = BLK + kBlockWindow * 4;
};

// NWT waves (32 query rows each) per tile: 4 in every launch with decode rows, 8 (256 rows sharing
// one K/V ring) in some launches without them.
template <typename T, int D, int NWT = 4>
__device__ __forceinline__ void chunk_tile(const AttnArgs& a, int32_t tile, char* lds) {
  constexpr int KS = D / 16;          // 16-slot contraction steps over the head dimension
  constexpr int MT = D / 32;          // 32-dim output tiles
  constexpr int ROW = D * sizeof(T);  // bytes per key row in LDS
  constexpr int RPI = 1024 / ROW;     // key rows per 1 KB copy instruction
  constexpr int RPW = kChunkKeys / NWT;         // key rows each wave copies per stage
  constexpr int NCPW = RPW / RPI;               // copy instructions per wave per tensor
  constexpr int NT = 64 * NWT;                  // threads of the tile
  static_assert(NCPW >= 1 && NCPW * RPI == RPW, "a wave's copies cover whole instructions");
  static_assert(RPI <= kMinBlock && RPW <= kMinBlock, "a copy instruction's rows (and a wave's) share a block");
  constexpr int CPW = 2 * NCPW;                 // copy instructions per wave per stage
  constexpr int NS = ChunkLds<T, D>::NS;
  constexpr int STAGE = ChunkLds<T, D>::STAGE;  // bytes of K (and of V) per stage
  char* sK = lds;
  char* sV = lds + ChunkLds<T, D>::V;
  int32_t* sBlk = reinterpret_cast<int32_t*>(lds + ChunkLds<T, D>::BLK);   // block-table window

  // The chunk's metadata by scalar loads, all four in flight together.
  TileSpan ts;
  const TileGrid tg{a.nd, a.Hkv, a.q_blocks, a.nsplit, a.bmq, 0, 0};
  chunk_tile_index(tile, tg, ts);
  int32_t m_q0 = sload_issue(a.cu_q + ts.s), m_q1 = sload_issue(a.cu_q + ts.s + 1);
  int32_t m_ctx = sload_issue(a.ctx_lens + ts.s), cub = sload_issue(a.cu_blocks + ts.s);
  sload_ready(m_q0);
  sload_ready(m_q1);
  sload_ready(m_ctx);
  sload_ready(cub);
  if (!chunk_tile_rows(tg, m_q0, m_q1, m_ctx, ts)) return;
  const int32_t sp = ts.sp, qb = ts.qb, g = ts.g, row0 = ts.row0, d = ts.d, c = ts.c;
  const int32_t kt_lo = ts.kt_lo, kt_hi = ts.kt_hi;
  const int32_t kv_end = c + min(d, (qb + 1) * a.bmq);        // past the block's last position

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: copy targets stay scalar
  const int col = lane & 31;          // query row of this lane in S^T / P^T / O^T
  const int half = lane >> 5;         // slot group
  const int rr = 32 * wave + col;     // row within the tile
  const int32_t pos_local = qb * a.bmq + rr / a.G;
  const int32_t head = g * a.G + rr % a.G;
  const bool valid = rr < a.bmq * a.G && pos_local < d;
  const int32_t qpos = valid ? c + pos_local : 0x7fffffff;      // padding rows see everything

  const T* q = static_cast<const T*>(a.q);
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  const int32_t* btab = a.block_table + cub;
  const int bsh = a.bs_shift;
  const int32_t bmask = (1 << bsh) - 1;

  Frag<T> qf[KS];
  {
    const T* qrow = q + (static_cast<int64_t>(row0 + pos_local) * a.Hq + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (valid) qf[ks].load(qrow + 16 * ks + 8 * half);
      else qf[ks].zero();
    }
  }

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x16{};

  // K and V rows go HBM -> LDS by DMA (chunk-swizzled rows) into a ring of NS stage buffers; keys
  // at or past kv_end repeat kv_end - 1 and are masked (probability 0).  A copy is issued after
  // the barrier that proves every wave has read the buffer it overwrites.  The float32 path
  // reads block ids from an LDS window [win_lo, win_lo + kBlockWindow) of the block table and
  // issues stage j's copy during stage j - NS + 1; the bf16 path (below) reads them by scalar
  // loads.
  int32_t win_lo = 0;
  const int32_t n_blk = ((kv_end - 1) >> bsh) + 1;
  auto fill_window = [&](int32_t first_block) {   // all loads first, then all LDS writes
    win_lo = first_block;
    const int32_t n = min(kBlockWindow, n_blk - first_block);
    int32_t ids[kBlockWindow / NT];
#pragma unroll
    for (int u = 0; u < kBlockWindow / NT; ++u)
      if (tid + NT * u < n) ids[u] = btab[first_block + tid + NT * u];
#pragma unroll
    for (int u = 0; u < kBlockWindow / NT; ++u)
      if (tid + NT * u < n) sBlk[tid + NT * u] = ids[u];
    __builtin_amdgcn_s_waitcnt(0x0F70);   // no load left pending on any path (see below)
  };
  const int32_t k_last = kv_end - 1;
  const int64_t head_bytes = static_cast<int64_t>(g) * ((int64_t)ROW << bsh);
  const int64_t blk_bytes = static_cast<int64_t>(a.Hkv) * ((int64_t)ROW << bsh);
  const int cp_row = lane / (ROW / 16), cp_pos = lane % (ROW / 16);
  // One copy instruction moves RPI consecutive rows; RPI <= 8 <= bs (both powers of two) and the
  // first row is RPI-aligned, so its rows share one cache block: the block's address is
  // wave-uniform and each lane adds a loop-invariant offset (row in the block, swizzled chunk).
  uint32_t lane_off[NCPW];
#pragma unroll
  for (int j = 0; j < NCPW; ++j)
    lane_off[j] = cp_row * ROW + 16 * lds_chunk(cp_pos, (wave * NCPW + j) * RPI + cp_row, ROW);
  auto issue = [&](int32_t kt, int buf) {
    const int32_t k0 = kt * kChunkKeys;
    if (k0 + kChunkKeys - 1 <= k_last) {             // every key of the stage is real
#pragma unroll
      for (int j = 0; j < NCPW; ++j) {
        const int i = wave * NCPW + j;
        const int32_t key0 = k0 + i * RPI;
        const int32_t blk = __builtin_amdgcn_readfirstlane(sBlk[(key0 >> bsh) - win_lo]);
        const int64_t base = static_cast<int64_t>(blk) * blk_bytes + head_bytes +
                             static_cast<int64_t>(key0 & bmask) * ROW;
        lds_copy16_asm_s(kc + base, lane_off[j], sK + buf * STAGE + i * 1024);
        lds_copy16_asm_s(vc + base, lane_off[j], sV + buf * STAGE + i * 1024);
      }
    } else {                                          // keys past kv_end repeat the last one
#pragma unroll
      for (int j = 0; j < NCPW; ++j) {
        const int i = wave * NCPW + j;
        const int r = i * RPI + cp_row;
        const int32_t key = min(k0 + r, k_last);
        const int64_t off = static_cast<int64_t>(sBlk[(key >> bsh) - win_lo]) * blk_bytes + head_bytes +
                            static_cast<int64_t>(key & bmask) * ROW + 16 * lds_chunk(cp_pos, r, ROW);
        lds_copy16_asm(kc + off, sK + buf * STAGE + i * 1024);
        lds_copy16_asm(vc + off, sV + buf * STAGE + i * 1024);
      }
    }
  };
  // Wait for this wave's copies of the current stage (all but the `later` stages issued after
  // it), then the barrier.
  auto wait_stage = [&](int32_t later) { wait_vm_barrier_later<CPW, NS - 2>(later); };

  // Loop-invariant LDS read addresses of this lane in ring buffer 0 (bf16 operand reads; the
  // buffer is selected by an immediate offset).
  uint32_t ka[KS], va[KS];
  if constexpr (sizeof(T) == 2) {
    const uint32_t k_base = lds_addr(sK), v_base = lds_addr(sV);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int b0 = 2 * (16 * ks + 8 * half);
      ka[ks] = k_base + col * ROW + 16 * lds_chunk(b0 >> 4, col, ROW);
    }
    const int grp = lane >> 4, ii = lane & 15, jj = ii >> 2, qd = ii & 3;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = 32 * mt + 16 * (grp & 1) + 4 * qd;
        const int r = 8 * h + 4 * (grp >> 1) + jj;
        va[2 * mt + h] = v_base + r * ROW + 16 * lds_chunk((2 * e) >> 4, r, ROW) + ((2 * e) & 15);
      }
  }

  // In both paths the ring loop holds no vector-memory operation of the compiler's own, so it adds
  // no waits there.  Float32: an outer loop over block-id windows (a window covers thousands of
  // stages; the copy ring drains at its end), the ring inside.
  const int32_t n_st = kt_hi - kt_lo;
  int32_t j = 0;
  if constexpr (sizeof(T) == 2) {
    // Software-pipelined stages: iteration jj reads V of stage jj and K of stage jj + 1, then
    // issues stage jj + 1's score products (matrix cores) while the softmax of stage jj (vector
    // ALU) runs, then stage jj's P V products.  So each wave keeps the matrix cores fed while
    // its own exponentials run, instead of alternating the two.  Buffer of stage jj - 1 is
    // free once every wave has passed iteration jj's barrier (it read V of jj - 1 and K of jj in
    // iteration jj - 1), so stage jj + NS - 1's copy goes there: NS - 2 stages of work cover it.
    //
    // Each wave copies RPW consecutive key rows of a stage (RPW <= block size, RPW-aligned), so
    // they lie in one cache block: one block id per wave and stage, read by a scalar load one
    // iteration before its copy is issued.  Rows past kv_end repeat kv_end - 1, which lies in the
    // same block as the wave's first real row.
    static_assert(NS >= 3, "pipelined ring needs three buffers");
    if (n_st > 0) {
      const int32_t row_w = RPW * wave;
      const int32_t* bt = btab;
      auto blk_ptr = [&](int32_t jj) { return bt + (min((kt_lo + jj) * kChunkKeys + row_w, k_last) >> bsh); };
      // LDS spans of this wave's copies in ring buffer 0 (wave-uniform integers).
      const uint32_t dk0 = __builtin_amdgcn_readfirstlane(lds_addr(sK)) + wave * NCPW * 1024;
      const uint32_t dv0 = __builtin_amdgcn_readfirstlane(lds_addr(sV)) + wave * NCPW * 1024;
      auto issue_s = [&](int32_t jj, auto B, int32_t blk, auto FULL) {
        constexpr int buf = decltype(B)::value;
        const int32_t k0 = (kt_lo + jj) * kChunkKeys;
        // Block ids are >= 0 and a block's bytes fit 32 bits (the launch checks), so the offset
        // is one 32 x 32 -> 64-bit product.
        const int64_t bb = static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(blk)) *
                                                static_cast<uint32_t>(blk_bytes)) + head_bytes;
        uint32_t dk[NCPW], dv[NCPW];
#pragma unroll
        for (int jc = 0; jc < NCPW; ++jc) {
          dk[jc] = dk0 + buf * STAGE + jc * 1024;
          dv[jc] = dv0 + buf * STAGE + jc * 1024;
        }
        if (decltype(FULL)::value || k0 + row_w + RPW - 1 <= k_last) {   // the wave's rows are all real keys
          // Its RPW rows are RPW-aligned in one block: copy jc starts RPI jc rows further.
          const int64_t roff = static_cast<int64_t>((k0 + row_w) & bmask) * ROW;
          const char* kb[NCPW];
          const char* vb[NCPW];
#pragma unroll
          for (int jc = 0; jc < NCPW; ++jc) {
            kb[jc] = kc + bb + roff + jc * RPI * ROW;
            vb[jc] = vc + bb + roff + jc * RPI * ROW;
          }
          dma_kv<NCPW>(kb, vb, lane_off, dk, dv);
        } else {                                      // keys past kv_end repeat the last one
          uint32_t voff[NCPW];
          const char* kb[NCPW];
          const char* vb[NCPW];
#pragma unroll
          for (int jc = 0; jc < NCPW; ++jc) {
            const int r = (wave * NCPW + jc) * RPI + cp_row;
            const int32_t key = min(k0 + r, k_last);
            voff[jc] = static_cast<uint32_t>((key & bmask) * ROW + 16 * lds_chunk(cp_pos, r, ROW));
            kb[jc] = kc + bb;
            vb[jc] = vc + bb;
          }
          dma_kv<NCPW>(kb, vb, voff, dk, dv);
        }
      };
      // Prologue: block ids and copies of the first NS - 1 stages, the next id, then the first
      // stage's scores.
      int32_t blk0[NS - 1];
#pragma unroll
      for (int p = 0; p < NS - 1; ++p) blk0[p] = sload_issue(blk_ptr(p));
#pragma unroll
      for (int p = 0; p < NS - 1; ++p) sload_ready(blk0[p]);
      constexpr std::false_type kAny{};
      constexpr std::true_type kSteady{};
      static_for<0, NS - 1>([&](auto P) {
        if (decltype(P)::value < n_st) issue_s(decltype(P)::value, P, blk0[decltype(P)::value], kAny);
      });
      int32_t blk_nx = sload_issue(blk_ptr(NS - 1));
      float neg_m = 0.f, raw_limit = kNegInf;     // m_run is -inf until the first rescale
      wait_stage(min(NS - 2, n_st - 1));
      f32x16 s_cur = f32x16{};
      {
        KRegs<D> kr;
        kr.template read<0>(ka);
        lds_operands_ready<D>(kr);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          Frag<T> kf;
          kf.u = make_uint4(kr.k[ks].x, kr.k[ks].y, kr.k[ks].z, kr.k[ks].w);
          mma32_k16(s_cur, kf, qf[ks]);
        }
      }
      // Steady iterations (the bulk of a long tile) know that stages jj .. jj + NS hold only real
      // keys and that stage jj needs no causal mask, so they test nothing at run time.
      auto step = [&](int32_t jj, auto B, auto STEADY) {
        constexpr int buf = decltype(B)::value;
        constexpr int nbuf = (buf + 1) % NS;
        constexpr int pbuf = (buf + NS - 1) % NS;
        constexpr bool steady = decltype(STEADY)::value;
        if (steady || jj + NS - 1 < n_st) sload_ready(blk_nx);   // ahead of the LDS reads, or it waits for them too
        if constexpr (steady) {
          wait_vm_barrier<(NS - 3) * CPW>();    // stage jj + 1 landed everywhere
        } else if (jj + 1 < n_st) {
          wait_stage(min(NS - 3, n_st - jj - 2));
        }
        // K of stage jj + 1 is read even on the last stage (stale ring data, its products
        // unused), so the score products and the softmax share one basic block and can be
        // interleaved.
        VRegs<D> vr;
        KRegs<D> kr;
        kr.template read<nbuf * STAGE>(ka);
        vr.template read<buf * STAGE>(va);
        // The copy of stage jj + NS - 1 (address arithmetic and DMA) goes behind the operand
        // reads, so they start right after the barrier.
        if (steady || jj + NS - 1 < n_st) issue_s(jj + NS - 1, std::integral_constant<int, pbuf>{}, blk_nx, STEADY);

        // Mask and row maximum of stage jj (while the operand reads are in flight).
        const int32_t k0 = (kt_lo + jj) * kChunkKeys;
        f32x16 st = s_cur;
        if (!steady && k0 + kChunkKeys - 1 > c + qb * a.bmq) {   // some key of the stage may pass a row
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (k0 + acc32_row(lane, r) > qpos) st[r] = kNegInf;
        }
        const float mx = max16_raw(st);   // over this lane's half of the row's keys
        // Lazy rescale: the weights are 2^(s c - m_ref) with m_ref a running maximum allowed to
        // lag the true one by up to kRescaleSlack (weights stay below 2^kRescaleSlack), so the
        // accumulator rescale and its exponential run only when some row's maximum jumps past it.
        // The test compares raw scores with (m_ref + slack) / c, kept beside m_ref (its rounding
        // only moves the rare rescale by an ulp).  The wave-wide vote sees both halves of every
        // row, so the halves' maxima are merged only when it fires.
        if (__builtin_amdgcn_ballot_w64(mx > raw_limit)) {
          const float m_new = fmaxf(m_run, half_xor_max(mx) * a.scale_log2);
          const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
          m_run = m_new;
          neg_m = m_run == kNegInf ? 0.f : -m_run;
          raw_limit = (m_run + kRescaleSlack) / a.scale_log2;
        }

        lds_k_ready<D>(kr);                            // K landed; V may still be in flight
        s_cur = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          Frag<T> kf;
          kf.u = make_uint4(kr.k[ks].x, kr.k[ks].y, kr.k[ks].z, kr.k[ks].w);
          mma32_k16(s_cur, kf, qf[ks]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = fast_exp2(fmaf(st[r], a.scale_log2, neg_m));
        Frag<T> pfs[2];
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = st[8 * ps + e];
          pfs[ps].set_all(pv);
        }
        {
          // Row sums of the weights as rounded for the P V products (so numerator and
          // denominator see the same weights): eight bf16 pair dot products into the running sum.
          typedef __attribute__((ext_vector_type(2))) __bf16 b2;
          const b2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
          const uint32_t* u0 = &pfs[0].u.x;
          const uint32_t* u1 = &pfs[1].u.x;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, u0[q]), one2, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, u1[q]), one2, l_run, false);
          }
        }
        {
          u32x4 p0 = __builtin_bit_cast(u32x4, pfs[0].u), p1 = __builtin_bit_cast(u32x4, pfs[1].u);
          lds_v_ready_after<D>(vr, p0, p1);
          pfs[0].u = __builtin_bit_cast(uint4, p0);
          pfs[1].u = __builtin_bit_cast(uint4, p1);
        }
        blk_nx = sload_issue(steady ? bt + (((kt_lo + jj + NS) * kChunkKeys + row_w) >> bsh)
                                    : blk_ptr(jj + NS));   // for the next iteration's copy
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {          // 16-key contraction steps
          const Frag<T>& pf = pfs[ps];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            Frag<T> vt;
            vt.u = make_uint4(vr.v[ps][2 * mt].x, vr.v[ps][2 * mt].y, vr.v[ps][2 * mt + 1].x, vr.v[ps][2 * mt + 1].y);
            mma32_k16(o[mt], vt, pf);
          }
        }
        // Issue order: each score product followed by a share of the softmax arithmetic, then
        // each P V product followed by the rest, so the matrix cores and the vector ALU work side
        // by side within the wave.
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 40 / KS, 0);
        }
#pragma unroll
        for (int i = 0; i < 2 * MT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);
        }
      };
      // Iteration jj is steady when stages up to jj + NS are whole (their keys all lie below
      // kv_end) and stage jj ends at or before the block's first position.
      const int32_t n_whole = min(n_st, max(0, kv_end / kChunkKeys - kt_lo));
      const int32_t n_unmasked = max(0, (c + qb * a.bmq + 1) / kChunkKeys - kt_lo);
      const int32_t n_steady = max(0, min(n_whole - NS, n_unmasked));
      // Unrolled by the ring depth, so each stage's buffer is a compile-time constant.
      for (; j + NS <= n_steady; j += NS)
        static_for<0, NS>([&](auto B) { step(j + decltype(B)::value, B, kSteady); });
      while (j < n_st) {                             // the rest (j is a multiple of NS here)
        bool done = false;
        static_for<0, NS>([&](auto B) {
          if (!done) {
            step(j, B, kAny);
            done = ++j == n_st;
          }
        });
      }
      sload_ready(blk_nx);                             // nothing left in flight
    }
  } else {
    while (j < n_st) {
      fill_window(((kt_lo + j) * kChunkKeys) >> bsh);   // ends with vmcnt(0): nothing left pending
      __syncthreads();                                   // also: every wave is done with the ring
      // Stages whose keys all lie in blocks [win_lo, win_lo + kBlockWindow) (a multiple of 32 keys).
      const int64_t key_end = static_cast<int64_t>(win_lo + kBlockWindow) << bsh;
      const int32_t j_end = kv_end <= key_end ? n_st : static_cast<int32_t>(min<int64_t>(n_st, key_end / kChunkKeys - kt_lo));
      // The ring restarts at buffer 0 in every window; unrolled by NS, each stage's buffer is a
      // compile-time constant (immediate LDS offsets).
      const int32_t j0 = j;
      auto stage = [&](int32_t jj, auto B) {
        constexpr int buf = decltype(B)::value;
        constexpr int next_buf = (buf + NS - 1) % NS;
        const int32_t kt = kt_lo + jj;
        wait_stage(min(NS - 2, j_end - 1 - jj));   // every wave's copy of stage jj has landed
        if (jj + NS - 1 < j_end) issue(kt + NS - 1, next_buf);

        Frag<T> kf[KS];
        Frag<T> vt[2][MT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = lds_row_frag<T>(sK + buf * STAGE, col, 16 * ks + 8 * half, ROW);
#pragma unroll
        for (int ps = 0; ps < 2; ++ps)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) vt[ps][mt] = lds_vt_frag32<T>(sV + buf * STAGE, mt, ps, lane, ROW);

        const int32_t k0 = kt * kChunkKeys;
        f32x16 st = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma32_k16(st, kf[ks], qf[ks]);
        if (k0 + kChunkKeys - 1 > c + qb * a.bmq) {   // some key of the stage may pass a row
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (k0 + acc32_row(lane, r) > qpos) st[r] = kNegInf;
        }
        // Raw scores: the maximum is taken before scaling (scale > 0 keeps the order) and the scale
        // is folded into the exponent, 2^(s c - m).
        float mx = st[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, st[r]);
        mx = half_xor_max(mx);
        const float m_new = fmaxf(m_run, mx * a.scale_log2);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(st[r], a.scale_log2, -m_use));
          st[r] = e;
          psum += e;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {   // some row's maximum moved
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
        }
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {          // 16-key contraction steps
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = st[8 * ps + e];
          Frag<T> pf;
          pf.set_all(pv);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) mma32_k16(o[mt], vt[ps][mt], pf);
        }
      };
#pragma unroll
      for (int p = 0; p < NS - 1; ++p)
        if (j0 + p < j_end) issue(kt_lo + j0 + p, p);
      while (j < j_end) {
        stage(j, std::integral_constant<int, 0>{});
        if (++j == j_end) break;
        stage(j, std::integral_constant<int, 1>{});
        if (++j == j_end) break;
        if constexpr (NS > 2) {
          stage(j, std::integral_constant<int, 2 % NS>{});
          if (++j == j_end) break;
        }
        if constexpr (NS > 3) {
          stage(j, std::integral_constant<int, 3 % NS>{});
          if (++j == j_end) break;
        }
      }
    }
  }

  const float l_tot = wave_xor_sum(l_run, 32);
  if (!valid) return;
  const int32_t row = row0 + pos_local;
  if (a.nsplit == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T* orow = static_cast<T*>(a.out) + (static_cast<int64_t>(row) * a.Hq + head) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4<T>(orow + 32 * mt + 8 * r4 + 4 * half, o[mt][4 * r4] * inv, o[mt][4 * r4 + 1] * inv,
                  o[mt][4 * r4 + 2] * inv, o[mt][4 * r4 + 3] * inv);
  } else {
    const int64_t prow = (static_cast<int64_t>(row - a.nd) * a.Hq + head) * a.nsplit + sp;
    float* po = a.chk_o + prow * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(po + 32 * mt + 8 * r4 + 4 * half) =
            make_float4(o[mt][4 * r4], o[mt][4 * r4 + 1], o[mt][4 * r4 + 2], o[mt][4 * r4 + 3]);
    if (half == 0) *reinterpret_cast<float2*>(a.chk_ml + 2 * prow) = make_float2(m_run, l_tot);
  }
}

// ---------------------------------------------------------------------------------------------
// One launch for both row kinds: workgroups [0, n_dec_wg) hold four independent decode waves
// each (waves 4 b .. 4 b + 3 of the stage split), the rest are chunk tiles.  The decode
// workgroups are dispatched first and stay for the whole decode split, so chunk tiles run on the
// compute units' other workgroup slots while the decode waves stream the cache.
// ---------------------------------------------------------------------------------------------
template <typename T, int D>
constexpr int attn_lds_bytes() {
  return 4 * DecodeLds<T, D>::BYTES > ChunkLds<T, D>::BYTES ? 4 * DecodeLds<T, D>::BYTES : ChunkLds<T, D>::BYTES;
}

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1))) void attn_kernel(
    AttnArgs a, const int32_t* __restrict__ seq_start, const int32_t* __restrict__ wave_unit,
    const int32_t* __restrict__ wave_pos, const int32_t* __restrict__ par, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ cu_blocks, int32_t n_dec_wg, int32_t n_tiles, int32_t per_xcd) {
  __shared__ __attribute__((aligned(1024))) char lds[attn_lds_bytes<T, D>()];
  const int32_t b = blockIdx.x;
  if (b < n_dec_wg) {
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    decode_wave<T, D>(a, seq_start, wave_unit, wave_pos, par, ctx_lens, cu_blocks, 4 * b + wave,
                      static_cast<int>(threadIdx.x & 63), lds + wave * DecodeLds<T, D>::BYTES);
  } else {
    // XCD-aware order: workgroup b runs on XCD b % 8 (n_dec_wg is a multiple of 8); each XCD
    // gets a contiguous run of logical tiles, so the tiles sharing one (chunk, KV head) K/V
    // stream share that XCD's L2.  Chunk workgroup cb shares a compute unit with decode
    // workgroup cb (the decode split accounts for it).
    const int32_t cb = b - n_dec_wg;
    const int32_t tile = static_cast<int32_t>(chunk_wg_tile(cb, per_xcd));
    if (tile < n_tiles) {
      // Chunk waves issue ahead of the decode waves that share their SIMDs (wave priority 1
      // against 0): a decode wave needs few issue slots to keep its copies in flight, and the
      // tiles finish sooner beside it.
      __builtin_amdgcn_s_setprio(1);
      chunk_tile<T, D>(a, tile, lds);
    }
  }
}

// Chunk tiles of NWT waves alone (a launch without decode rows that takes 256-row tiles).
template <typename T, int D, int NWT>
__global__ __launch_bounds__(64 * NWT) __attribute__((amdgpu_waves_per_eu(2))) void chunk_only_kernel(
    AttnArgs a, int32_t n_tiles, int32_t per_xcd) {
  __shared__ __attribute__((aligned(1024))) char lds[ChunkLds<T, D>::BYTES];
  const int32_t tile = static_cast<int32_t>(chunk_wg_tile(blockIdx.x, per_xcd));
  if (tile < n_tiles) chunk_tile<T, D, NWT>(a, tile, lds);
}

// ---------------------------------------------------------------------------------------------
// Merge of split partials: m = max m_p, w_p = 2^(m_p - m), out = sum w_p o_p / sum w_p l_p.
// ---------------------------------------------------------------------------------------------
// One wave per (row, head) item of a launch with decode rows; combine_split_kernel below merges
// the key splits of a launch without them.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, int32_t n_dec_rows, int32_t n_items) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (w >= n_items) return;
  const int32_t ri = static_cast<int32_t>(w / a.Hq);
  const int32_t h = static_cast<int32_t>(w % a.Hq);
  int32_t row, P;
  const float* po;                      // partial i: o at po + i * so, (m, l) at pml + i * sml
  const float* pml;
  int64_t so, sml;
  if (ri < n_dec_rows) {
    // Decode row: the partials of unit u sit in slots u + w for the waves w whose stage ranges
    // meet the unit's stages [a_u, a_u + n).
    row = ri;
    const int32_t g = h / a.G, hh = h - g * a.G;
    const int32_t r = g * a.head_blocks + (hh >> 4);
    const int32_t u = row * a.ups + r;
    // The unit's two records in one load, beside the context length (they are meaningful only
    // when the row has keys).
    const int2 rec = reinterpret_cast<const int2*>(a.dec_unit)[u];
    const int32_t n = decode_stages(a.ctx_lens[row]);
    const int32_t w0 = n > 0 ? rec.x : 0;
    P = n > 0 ? rec.y - w0 + 1 : 0;
    const int64_t base = static_cast<int64_t>(u + w0) * a.hw + (hh & 15);
    po = a.dec_o + base * D;
    pml = a.dec_ml + base * 2;
    so = static_cast<int64_t>(a.hw) * D;
    sml = 2 * a.hw;
  } else {
    row = a.nd + (ri - n_dec_rows);
    P = a.nsplit;
    const int64_t base = (static_cast<int64_t>(row - a.nd) * a.Hq + h) * a.nsplit;
    po = a.chk_o + base * D;
    pml = a.chk_ml + base * 2;
    so = D;
    sml = 2;
  }
  T* orow = static_cast<T*>(a.out) + (static_cast<int64_t>(row) * a.Hq + h) * D;
  if (P <= 8) {
    // Up to eight partials (every chunk split, most decode rows): each lane loads every (m, l)
    // pair (one broadcast load each) and PER adjacent elements of every partial o, all in
    // flight together, then merges serially in partial order -- no cross-lane steps.
    float2 ml[8];
    float xv[8][PER];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      if (v < P) {
        ml[v] = *reinterpret_cast<const float2*>(pml + v * sml);
        if constexpr (PER == 2) {
          const float2 t = *reinterpret_cast<const float2*>(po + v * so + 2 * lane);
          xv[v][0] = t.x;
          xv[v][PER - 1] = t.y;
        } else {
          xv[v][0] = po[v * so + lane];
        }
      }
    }
    float m = kNegInf;
#pragma unroll
    for (int v = 0; v < 8; ++v)
      if (v < P) m = fmaxf(m, ml[v].x);
    const float m_use = m == kNegInf ? 0.f : m;
    float wv[8];
    float Lsum = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      wv[v] = v < P ? exp2f(ml[v].x - m_use) : 0.f;
      if (v < P) Lsum += wv[v] * ml[v].y;
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v)
      if (v < P)
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += (wv[v] * inv) * xv[v][j];
    if constexpr (sizeof(T) == 2) {
      if constexpr (PER == 2) reinterpret_cast<uint32_t*>(orow)[lane] = pack_bf16x2(acc[0], acc[PER - 1]);
      else reinterpret_cast<uint16_t*>(orow)[lane] = f32_to_bf16_bits(acc[0]);
    } else {
      if constexpr (PER == 2) reinterpret_cast<float2*>(orow)[lane] = make_float2(acc[0], acc[PER - 1]);
      else orow[lane] = acc[0];
    }
    return;
  }
  // More partials (long decode rows split over many waves).  The first eight partials' o are
  // loaded up front, beside their (m, l) pairs: the weights need the reductions below, the loads
  // do not.
  float x0[8][PER];
#pragma unroll
  for (int v = 0; v < 8; ++v)
#pragma unroll
    for (int j = 0; j < PER; ++j) x0[v][j] = v < P ? po[v * so + lane + 64 * j] : 0.f;
  // Lanes read the partials' (m, l) pairs side by side; butterfly reductions give every lane the
  // same maximum and total in the same order on every run.
  float m = kNegInf;
  for (int32_t i = lane; i < P; i += 64) m = fmaxf(m, pml[i * sml]);
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) m = wave_xor_max(m, x);
  const float m_use = m == kNegInf ? 0.f : m;
  float Lsum = 0.f;
  for (int32_t i = lane; i < P; i += 64) Lsum += exp2f(pml[i * sml] - m_use) * pml[i * sml + 1];
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) Lsum = wave_xor_sum(Lsum, x);
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  for (int32_t base = 0; base < P; base += 64) {
    const int32_t i = base + lane;
    const float wl = i < P ? exp2f(pml[i * sml] - m_use) * inv : 0.f;
    const int32_t n = min(64, P - base);
    int32_t k = 0;
    if (base == 0) {                          // the prefetched partials, in the same order
      const int32_t n8 = min(n, 8);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        if (v < n8) {
          const float wk = __shfl(wl, v, 64);
#pragma unroll
          for (int j = 0; j < PER; ++j) acc[j] += wk * x0[v][j];
        }
      }
      k = n8;
    }
    for (; k + 8 <= n; k += 8) {              // eight partials' loads in flight together
      float x[8][PER];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < PER; ++j) x[u][j] = po[(base + k + u) * so + lane + 64 * j];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wk = __shfl(wl, k + u, 64);
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += wk * x[u][j];
      }
    }
    for (; k < n; ++k) {
      const float wk = __shfl(wl, k, 64);
      const float* pk = po + (base + k) * so + lane;
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] += wk * pk[64 * j];
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if constexpr (sizeof(T) == 2) {
      reinterpret_cast<uint16_t*>(orow)[lane + 64 * j] = f32_to_bf16_bits(acc[j]);
    } else {
      orow[lane + 64 * j] = acc[j];
    }
  }
}

// Key splits of a launch without decode rows (at most kMaxSplit partials per item, contiguous):
// half a wave per (row, head) item, each lane D / 32 adjacent elements of every partial in one
// load, so a launch has half the waves of one-item waves with twice the bytes each in flight.
// Same merge, in the same order, as combine_kernel's path for up to eight partials.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_split_kernel(AttnArgs a, int32_t n_items) {
  constexpr int E = D / 32;
  static_assert(E == 2 || E == 4, "head dim 64 or 128");
  typedef __attribute__((ext_vector_type(E))) float fxE;
  const int lane = threadIdx.x & 31;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  if (w >= n_items) return;
  const int32_t P = a.nsplit;
  const float* po = a.chk_o + w * P * D + E * lane;     // item w = (row - nd) Hq + head
  const float* pml = a.chk_ml + w * P * 2;
  float2 ml[kMaxSplit];
  fxE xv[kMaxSplit];
#pragma unroll
  for (int v = 0; v < kMaxSplit; ++v) {
    if (v < P) {
      ml[v] = *reinterpret_cast<const float2*>(pml + 2 * v);
      xv[v] = *reinterpret_cast<const fxE*>(po + v * D);
    }
  }
  float m = kNegInf;
#pragma unroll
  for (int v = 0; v < kMaxSplit; ++v)
    if (v < P) m = fmaxf(m, ml[v].x);
  const float m_use = m == kNegInf ? 0.f : m;
  float wv[kMaxSplit];
  float Lsum = 0.f;
#pragma unroll
  for (int v = 0; v < kMaxSplit; ++v) {
    wv[v] = v < P ? exp2f(ml[v].x - m_use) : 0.f;
    if (v < P) Lsum += wv[v] * ml[v].y;
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  float acc[E];
#pragma unroll
  for (int j = 0; j < E; ++j) acc[j] = 0.f;
#pragma unroll
  for (int v = 0; v < kMaxSplit; ++v)
    if (v < P)
#pragma unroll
      for (int j = 0; j < E; ++j) acc[j] += (wv[v] * inv) * xv[v][j];
  T* orow = static_cast<T*>(a.out) + (static_cast<int64_t>(a.nd) * a.Hq + w) * D + E * lane;
  if constexpr (sizeof(T) == 2) {
    if constexpr (E == 4)
      *reinterpret_cast<uint2*>(orow) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    else
      *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(acc[0], acc[1]);
  } else {
    if constexpr (E == 4)
      *reinterpret_cast<float4*>(orow) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    else
      *reinterpret_cast<float2*>(orow) = make_float2(acc[0], acc[1]);
  }
}

// Compute units of the device that owns the stream (cached per device).
int compute_units(hipStream_t st) {
  static std::atomic<int> cached[64] = {};      // 0 = not looked up yet; any thread may fill it
  int dev = 0;
  if (hipStreamGetDevice(st, &dev) != hipSuccess && hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Decode waves of an attention launch on the stream's device: four per decode workgroup, one
// workgroup per compute unit beside chunk tiles, two when there are none.
// Decode workgroups dispatched first onto their compute units: the compute units rounded up to a
// multiple of 8 (whole rounds over the XCDs).
int32_t first_round_wgs(hipStream_t st) { return (compute_units(st) + 7) / 8 * 8; }

// The chunk tile grid of a launch: n_tiles tiles (numbered as chunk_tile_span reads them) on
// 8 per_xcd chunk workgroups.
TileGrid tile_grid(int32_t nd, int32_t Hkv, int32_t n_chunk, int32_t q_blocks, int32_t nsplit, int32_t bmq) {
  TileGrid tg{nd, Hkv, q_blocks, nsplit, bmq, 0, 0};
  tg.n_tiles = n_chunk > 0 ? static_cast<int64_t>(n_chunk) * q_blocks * Hkv * nsplit : 0;
  tg.per_xcd = (tg.n_tiles + 7) / 8;
  return tg;
}

int32_t decode_waves(hipStream_t st, bool has_chunks) {
  const int cus8 = first_round_wgs(st);
  return 4 * std::min(kMaxDecodeWaves / 4, (has_chunks ? CB_DECODE_WG_PER_CU_MIXED : CB_DECODE_WG_PER_CU) * cus8);
}

// The launches of one call, in order on the caller's stream: the decode stage split (skipped with
// a host-made plan, which a.dec_seq / dec_wave / dec_par then point into), the attention kernel
// (decode waves and chunk tiles together) and the combine.
template <typename T, int D>
int launch_all(hipStream_t st, const AttnArgs& a0, const Plan& p, void* const* events, bool planned) {
  auto rec = [&](int i) {
    if (events && events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), st);
  };
  AttnArgs a = a0;
  // A launch without decode rows (bf16, head dim 128) takes 8-wave tiles of 256 rows when its
  // longest chunk fills one and the tiles give every compute unit a workgroup without a key
  // split: one K/V ring then serves twice the rows (long-context chunk-only launch 15.2 -> 14.8
  // ms).  Where keys must be split (the budget-512 layer's chunks) they measured no faster, so
  // those keep 4-wave tiles.  No split needs no chunk partials, so the workspace sized by the
  // 4-wave plan suffices.
  bool wide = false;
  if constexpr (sizeof(T) == 2 && D == 128) {
    if (a.nd == 0 && a.n_chunk > 0) {
      const ChunkSplit w8 = chunk_split(a.n_chunk, a.Hkv, a.G, 2 * kChunkRows, 0, a.max_q_len, a.max_ctx);
      if (a.max_q_len >= w8.bmq && w8.nsplit == 1 && w8.tiles >= compute_units(st)) {
        wide = true;
        a.bmq = w8.bmq;
        a.q_blocks = w8.q_blocks;
        a.nsplit = w8.nsplit;
      }
    }
  }
  const TileGrid tg = tile_grid(a.nd, a.Hkv, a.n_chunk, a.q_blocks, a.nsplit, a.bmq);
  const int64_t n_tiles = tg.n_tiles, per_xcd = tg.per_xcd;
  int32_t n_dec_wg = 0;
  if (a.nd > 0) {
    n_dec_wg = decode_waves(st, a.n_chunk > 0) / 4;
    if (!planned) {
      decode_prep_kernel<<<dim3(1), dim3(1024), 0, st>>>(a, 4 * n_dec_wg, first_round_wgs(st), tg);
      if (hipGetLastError() != hipSuccess) return CB_ERR_HIP;
    }
  }
  const int64_t grid = n_dec_wg + per_xcd * 8;
  if (grid > 0x7fffffff) return CB_ERR_INVALID;
  if (grid > 0) {
    rec(0);
    rec(2);
    if constexpr (sizeof(T) == 2 && D == 128) {
      if (wide)
        chunk_only_kernel<T, D, 8><<<dim3(static_cast<uint32_t>(grid)), dim3(512), 0, st>>>(
            a, static_cast<int32_t>(n_tiles), static_cast<int32_t>(per_xcd));
    }
    if (!wide) {
      attn_kernel<T, D><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st>>>(
          a, a.dec_seq, a.dec_wave, a.dec_pos, a.dec_par, a.ctx_lens, a.cu_blocks, n_dec_wg,
          static_cast<int32_t>(n_tiles), static_cast<int32_t>(per_xcd));
    }
    if (hipGetLastError() != hipSuccess) return CB_ERR_HIP;
    rec(1);
    rec(3);
  }
  const int32_t n_chunk_rows = a.nsplit > 1 ? a.T - a.nd : 0;
  const int64_t items = static_cast<int64_t>(a.nd + n_chunk_rows) * a.Hq;
  if (items > 0) {
    const int64_t grid = a.nd == 0 ? (items + 7) / 8 : (items + 3) / 4;
    if (grid > 0x7fffffff) return CB_ERR_INVALID;
    rec(4);
    if (a.nd == 0)
      combine_split_kernel<T, D><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st>>>(a, static_cast<int32_t>(items));
    else
      combine_kernel<T, D><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st>>>(a, a.nd, static_cast<int32_t>(items));
    if (hipGetLastError() != hipSuccess) return CB_ERR_HIP;
    rec(5);
  }
  return CB_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t decode_plan_ints(int32_t nd, int32_t n_waves) {
  return 4 + static_cast<size_t>(nd) + 1 + 2 * static_cast<size_t>(n_waves) + 1;
}

// Host version of decode_prep_kernel's split, with the same rule, so that a launch with the plan
// computes bit for bit what it computes after the split kernel.  ctx: context lengths of all
// rows (decode rows first); cu_q: query row offsets (read only for chunk tiles).  Layout of out:
// [0] S, [1] F, [2] W, [3] n_waves; the row stage offsets seq[0..nd] (seq[nd] = S); n_waves slots
// whose first W hold each wave's first unit; n_waves + 1 slots whose first W + 1 hold start(0..W).
int decode_plan_host(const int32_t* cu_q, const int32_t* ctx, int32_t nd, int32_t ups, int32_t n_waves,
                     int32_t F, const TileGrid& tg, int32_t* out, size_t cap) {
  if (n_waves < 1 || n_waves > kMaxDecodeWaves) return CB_ERR_INVALID;
  if (cap < decode_plan_ints(nd, n_waves)) return CB_ERR_CAPACITY;
  int32_t* seq = out + 4;
  int64_t S = 0;
  for (int32_t s = 0; s < nd; ++s) {
    if (ctx[s] < 0) return CB_ERR_INVALID;
    seq[s] = static_cast<int32_t>(S);
    S += static_cast<int64_t>(ctx[s] > 0 ? (ctx[s] + kDecodeKeys - 1) / kDecodeKeys : 0) * ups;
    if (S > 0x7fff0000 - static_cast<int64_t>(kMaxDecodeWaves) * 2) return CB_ERR_INVALID;
  }
  seq[nd] = static_cast<int32_t>(S);
  const int32_t W = decode_waves_used(static_cast<int32_t>(S), n_waves);
  const int32_t n_wg = (W + 3) >> 2;
  int32_t P[kMaxDecodeWaves / 4 + 1];
  P[0] = 0;
  const bool full = W == n_waves;
  for (int32_t b = 0; b < n_wg; ++b) {
    const int32_t ts = full ? beside_tile_stages(b, tg, cu_q, ctx) : 0;
    P[b + 1] = P[b] + decode_wg_rate(b, F, ts, static_cast<int32_t>(S), W);
  }
  const int64_t cw = decode_rate_prefix(W, P);
  out[0] = static_cast<int32_t>(S);
  out[1] = F;
  out[2] = W;
  out[3] = n_waves;
  int32_t* wave = seq + nd + 1;
  int32_t* pos = wave + n_waves;
  int32_t lo = 0;
  for (int32_t w = 0; w < W; ++w) {                 // wave starts grow: walk the rows once
    const int32_t p = decode_wave_start(w, static_cast<int32_t>(S), cw, P);
    pos[w] = p;
    while (seq[lo + 1] <= p) ++lo;                  // seq[lo] <= p < seq[lo + 1]
    const int32_t n_s = (seq[lo + 1] - seq[lo]) / ups;
    wave[w] = lo * ups + (p - seq[lo]) / n_s;
  }
  pos[W] = static_cast<int32_t>(S);
  return CB_OK;
}

bool valid_shape(int32_t num_seqs, int32_t nd, int32_t T, int32_t max_q_len, int32_t max_dctx,
                 int32_t max_ctx, int32_t Hq, int32_t Hkv, int32_t D) {
  if (num_seqs < 0 || nd < 0 || nd > num_seqs || T < num_seqs || T - nd < num_seqs - nd) return false;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv || Hq / Hkv > kChunkRows) return false;
  if (D != 64 && D != 128) return false;
  if (max_q_len < 0 || max_dctx < 0 || max_ctx < 0) return false;
  if (num_seqs > nd && (max_q_len < 1 || max_ctx < 1)) return false;
  if (nd > 0 && max_dctx < 1) return false;
  // Decode stage positions (and one wave's range past them) must stay in int32.
  const int64_t units = static_cast<int64_t>(nd) * Hkv * ((Hq / Hkv + 15) / 16);
  if (units * ((static_cast<int64_t>(max_dctx) + kDecodeKeys - 1) / kDecodeKeys) > 0x7fff0000 - (int64_t)kMaxDecodeWaves * 2)
    return false;
  return true;
}

}  // namespace
}  // namespace cb

extern "C" size_t cb_attn_workspace_bytes(int32_t num_seqs, int32_t num_decodes, int32_t T,
                                          int32_t max_q_len, int32_t max_decode_ctx,
                                          int32_t max_ctx, int32_t Hq, int32_t Hkv, int32_t D) {
  if (!cb::valid_shape(num_seqs, num_decodes, T, max_q_len, max_decode_ctx, max_ctx, Hq, Hkv, D))
    return 0;
  return cb::make_plan(num_seqs, num_decodes, T, max_q_len, max_ctx, Hq, Hkv, D).total;
}

extern "C" int32_t cb_attn_decode_waves(void* stream, int32_t has_chunks) {
  return cb::decode_waves(static_cast<hipStream_t>(stream), has_chunks != 0);
}

extern "C" size_t cb_decode_plan_ints(int32_t num_decodes, int32_t n_waves) {
  if (num_decodes < 0 || n_waves < 1) return 0;
  return cb::decode_plan_ints(num_decodes, n_waves);
}

extern "C" int cb_decode_plan(void* stream, int32_t num_seqs, int32_t num_decodes, int32_t max_q_len,
                              int32_t max_ctx, int32_t Hq, int32_t Hkv, const int32_t* cu_seqlens_q,
                              const int32_t* context_lens, int32_t* out, size_t cap_ints) {
  using namespace cb;
  if (num_decodes < 1 || num_seqs < num_decodes || !context_lens || !out) return CB_ERR_INVALID;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv || Hq / Hkv > kChunkRows) return CB_ERR_INVALID;
  const bool chunks = num_seqs > num_decodes;
  if (chunks && (!cu_seqlens_q || max_q_len < 1 || max_ctx < 1)) return CB_ERR_INVALID;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // The same chunk tiling as the attention call with these shape arguments (the token count and
  // head size only size its workspace).
  const Plan p = make_plan(num_seqs, num_decodes, num_seqs, max_q_len, max_ctx, Hq, Hkv, 64);
  const TileGrid tg = tile_grid(num_decodes, Hkv, p.n_chunk, p.q_blocks, p.nsplit, p.bmq);
  return decode_plan_host(cu_seqlens_q, context_lens, num_decodes, p.ups, decode_waves(st, chunks),
                          first_round_wgs(st), tg, out, cap_ints);
}

extern "C" int cb_mixed_paged_attention_timed(
    void* stream, int32_t dtype, int32_t num_seqs, int32_t num_decodes, int32_t T,
    int32_t max_q_len, int32_t max_decode_ctx, int32_t max_ctx, int32_t Hq, int32_t Hkv,
    int32_t D, int32_t block_size, float scale, const void* q, const void* k_cache,
    const void* v_cache, const int32_t* cu_seqlens_q, const int32_t* context_lens,
    const int32_t* cu_blocks, const int32_t* block_table, void* out, void* workspace,
    size_t workspace_bytes, const int32_t* decode_plan, int32_t plan_waves, void* const* events) {
  using namespace cb;
  if (dtype != CB_F32 && dtype != CB_BF16) return CB_ERR_INVALID;
  if (!valid_shape(num_seqs, num_decodes, T, max_q_len, max_decode_ctx, max_ctx, Hq, Hkv, D))
    return CB_ERR_INVALID;
  if (block_size < kMinBlock || block_size > kMaxBlock || (block_size & (block_size - 1)) ||
      !(scale > 0.f))
    return CB_ERR_INVALID;
  if (num_seqs == 0) return CB_OK;
  if (!q || !k_cache || !v_cache || !cu_seqlens_q || !context_lens || !cu_blocks || !block_table || !out)
    return CB_ERR_INVALID;
  const void* ptrs[] = {q, k_cache, v_cache, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return CB_ERR_INVALID;
  const Plan p = make_plan(num_seqs, num_decodes, T, max_q_len, max_ctx, Hq, Hkv, D);
  if (p.total > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))) return CB_ERR_INVALID;
  if (workspace_bytes < p.total) return CB_ERR_CAPACITY;

  AttnArgs a{};
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.cu_q = cu_seqlens_q; a.ctx_lens = context_lens; a.cu_blocks = cu_blocks; a.block_table = block_table;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.dec_o = reinterpret_cast<float*>(ws + p.dec_o);
  a.dec_ml = reinterpret_cast<float*>(ws + p.dec_ml);
  a.chk_o = reinterpret_cast<float*>(ws + p.chk_o);
  a.chk_ml = reinterpret_cast<float*>(ws + p.chk_ml);
  a.dec_seq = reinterpret_cast<int32_t*>(ws + p.dec_seq);
  a.dec_wave = reinterpret_cast<int32_t*>(ws + p.dec_wave);
  a.dec_pos = reinterpret_cast<int32_t*>(ws + p.dec_pos);
  a.dec_par = reinterpret_cast<int32_t*>(ws + p.dec_par);
  a.dec_unit = reinterpret_cast<int32_t*>(ws + p.dec_unit);
  a.num_seqs = num_seqs; a.nd = num_decodes; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.G = p.G;
  a.bs = block_size;
  a.bs_shift = __builtin_ctz(static_cast<unsigned>(block_size));
  a.head_blocks = p.head_blocks; a.hw = p.hw; a.ups = p.ups;
  a.bmq = p.bmq; a.q_blocks = p.q_blocks; a.n_chunk = p.n_chunk; a.nsplit = p.nsplit;
  a.max_q_len = max_q_len; a.max_ctx = max_ctx;
  a.scale_log2 = scale * 1.4426950408889634f;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool planned = decode_plan != nullptr && num_decodes > 0;
  if (planned) {
    if (plan_waves != decode_waves(st, p.n_chunk > 0) || !aligned16(decode_plan)) return CB_ERR_INVALID;
    int32_t* plan = const_cast<int32_t*>(decode_plan);
    a.dec_par = plan;
    a.dec_seq = plan + 4;
    a.dec_wave = plan + 4 + num_decodes + 1;
    a.dec_pos = a.dec_wave + plan_waves;
  }
  if (dtype == CB_BF16) {
    return D == 128 ? launch_all<bf16_t, 128>(st, a, p, events, planned)
                    : launch_all<bf16_t, 64>(st, a, p, events, planned);
  }
  return D == 128 ? launch_all<float, 128>(st, a, p, events, planned) : launch_all<float, 64>(st, a, p, events, planned);
}

extern "C" int cb_mixed_paged_attention(
    void* stream, int32_t dtype, int32_t num_seqs, int32_t num_decodes, int32_t T,
    int32_t max_q_len, int32_t max_decode_ctx, int32_t max_ctx, int32_t Hq, int32_t Hkv,
    int32_t D, int32_t block_size, float scale, const void* q, const void* k_cache,
    const void* v_cache, const int32_t* cu_seqlens_q, const int32_t* context_lens,
    const int32_t* cu_blocks, const int32_t* block_table, void* out, void* workspace,
    size_t workspace_bytes) {
  return cb_mixed_paged_attention_timed(stream, dtype, num_seqs, num_decodes, T, max_q_len,
                                        max_decode_ctx, max_ctx, Hq, Hkv, D, block_size, scale, q,
                                        k_cache, v_cache, cu_seqlens_q, context_lens, cu_blocks,
                                        block_table, out, workspace, workspace_bytes, nullptr, 0,
                                        nullptr);
}

// ---------------------------------------------------------------------------------------------
// The same call for callers that cannot allocate (graph capture, tight serving loops): its
// workspace is a file-scope device array of kScratchBytes.  Each GPU holds its own copy at its own
// address, found once per device with hipGetSymbolAddress (with that device current) and kept;
// host code passes only that address, never the array's name.  Nothing in it must start at zero:
// every word the kernels read is written earlier in the same call.  Calls that overlap in time on
// one GPU share the array and race.
// ---------------------------------------------------------------------------------------------
namespace cb {
namespace {
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

int scratch_address(hipStream_t st, void** addr) {
  int dev = -1;
  if (hipStreamGetDevice(st, &dev) != hipSuccess && hipGetDevice(&dev) != hipSuccess) return CB_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CB_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return CB_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return CB_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return CB_ERR_HIP;
    if (e != hipSuccess || ptr == nullptr) return CB_ERR_HIP;
    g_scratch_addr[dev] = ptr;
  }
  *addr = g_scratch_addr[dev];
  return CB_OK;
}
}  // namespace
}  // namespace cb

extern "C" int cb_mixed_paged_attention_noalloc(
    void* stream, int32_t dtype, int32_t num_seqs, int32_t num_decodes, int32_t T,
    int32_t max_q_len, int32_t max_decode_ctx, int32_t max_ctx, int32_t Hq, int32_t Hkv,
    int32_t D, int32_t block_size, float scale, const void* q, const void* k_cache,
    const void* v_cache, const int32_t* cu_seqlens_q, const int32_t* context_lens,
    const int32_t* cu_blocks, const int32_t* block_table, void* out) {
  using namespace cb;
  if (!valid_shape(num_seqs, num_decodes, T, max_q_len, max_decode_ctx, max_ctx, Hq, Hkv, D))
    return CB_ERR_INVALID;
  if (make_plan(num_seqs, num_decodes, T, max_q_len, max_ctx, Hq, Hkv, D).total > kScratchBytes)
    return CB_ERR_CAPACITY;
  void* ws = nullptr;
  const int rc = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (rc != CB_OK) return rc;
  return cb_mixed_paged_attention(stream, dtype, num_seqs, num_decodes, T, max_q_len, max_decode_ctx,
                                  max_ctx, Hq, Hkv, D, block_size, scale, q, k_cache, v_cache,
                                  cu_seqlens_q, context_lens, cu_blocks, block_table, out, ws,
                                  kScratchBytes);
}
