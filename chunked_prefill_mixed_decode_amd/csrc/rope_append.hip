// Rotary embedding at absolute positions fused with the paged KV append.
//
// "Chunked Prefill 的 Token 预算" §06: every new key/value goes to the physical slot named by
// slot_mapping; §07: rows carry absolute positions, so a chunk's rotary phases continue where
// the previous chunk stopped.  "Chunked Prefill: Ending the Great Stall" §05: the paged cache is
// filled token by token, blind to chunk boundaries.
//
// Rotary variant (the pages fix none): rotate-half over the full head dimension, float32 table
// built on the host (cb_rope_cos_sin: fp64 angle, extended-precision cos/sin), each product and sum rounded to
// float32 on its own (contraction is disabled here), then round-to-nearest-even into the element
// type.  Memory-bound: every thread moves 2 x 8 elements of one head of one row.
#include <cmath>
#include <limits>

#include "cb.h"
#include "common.h"

#pragma clang fp contract(off)

namespace cb {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_kv_append_kernel(
    int32_t T_rows, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, const T* __restrict__ q,
    const T* __restrict__ k, const T* __restrict__ v, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ slot_mapping, const float* __restrict__ cos_sin, int32_t max_pos,
    T* q_out, T* __restrict__ k_cache, T* __restrict__ v_cache, int64_t num_slots) {
  const int32_t half = D / 2;
  const int32_t per_head = half / 8;           // threads per head: each takes 8 pairs
  const int32_t heads = (q ? Hq : 0) + 2 * Hkv;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(T_rows) * heads * per_head;
  if (item >= total) return;
  const int32_t c = static_cast<int32_t>(item % per_head);
  const int32_t hs = static_cast<int32_t>((item / per_head) % heads);
  const int32_t t = static_cast<int32_t>(item / (static_cast<int64_t>(per_head) * heads));
  const int32_t p = positions[t];
  if (p < 0 || p >= max_pos) return;
  const int32_t i0 = 8 * c;

  int32_t kind, h;                              // 0 = q, 1 = k, 2 = v
  if (q && hs < Hq) {
    kind = 0;
    h = hs;
  } else {
    const int32_t r = hs - (q ? Hq : 0);
    kind = r < Hkv ? 1 : 2;
    h = r < Hkv ? r : r - Hkv;
  }

  T* dst;
  if (kind == 0) {
    dst = q_out + (static_cast<int64_t>(t) * Hq + h) * D;
  } else {
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t blk = slot / bs, off = slot % bs;
    dst = (kind == 1 ? k_cache : v_cache) + ((blk * Hkv + h) * bs + off) * D;
  }
  const T* src = kind == 0 ? q + (static_cast<int64_t>(t) * Hq + h) * D
                           : (kind == 1 ? k : v) + (static_cast<int64_t>(t) * Hkv + h) * D;

  Frag<T> a, b;
  a.load(src + i0);
  b.load(src + half + i0);
  if (kind == 2) {                              // V is stored unrotated
    a.store(dst + i0);
    b.store(dst + half + i0);
    return;
  }
  const float* cs = cos_sin + static_cast<int64_t>(p) * D;
  float lo[8], hi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x1 = a.get(j), x2 = b.get(j);
    const float cj = cs[i0 + j], sj = cs[half + i0 + j];
    // Plain operators inside this file's contract(off) region: each product and each sum is
    // its own rounded float32 operation (library rounding helpers defined in headers outside the
    // region would still be fused after inlining).
    const float a1 = x1 * cj, b1 = x2 * sj, a2 = x2 * cj, b2 = x1 * sj;
    lo[j] = a1 - b1;
    hi[j] = a2 + b2;
  }
  a.set_all(lo);
  b.set_all(hi);
  a.store(dst + i0);
  b.store(dst + half + i0);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace cb

extern "C" int cb_rope_cos_sin(float* out, int32_t max_pos, int32_t D, double base) {
  if (!out || max_pos < 0 || D < 2 || (D & 1) || !(base > 0.0)) return CB_ERR_INVALID;
  // The table is defined with x87 extended precision (64-bit significand) for the cosine and sine;
  // a host whose long double differs would produce other bits, so it is refused.
  if (std::numeric_limits<long double>::digits != 64) return CB_ERR_INVALID;
  const int32_t half = D / 2;
  for (int32_t i = 0; i < half; ++i) {
    const double theta = std::pow(base, (-2.0 * i) / D);
    for (int32_t p = 0; p < max_pos; ++p) {
      // fp64 angle; cosine and sine in extended precision, rounded once to float32 (a double
      // result would double-round and lose relative accuracy near the functions' zeros)
      const long double ang = static_cast<long double>(static_cast<double>(p) * theta);
      out[static_cast<int64_t>(p) * D + i] = static_cast<float>(cosl(ang));
      out[static_cast<int64_t>(p) * D + half + i] = static_cast<float>(sinl(ang));
    }
  }
  return CB_OK;
}

extern "C" int cb_rope_kv_append(void* stream, int32_t dtype, int32_t T, int32_t Hq, int32_t Hkv,
                                 int32_t D, int32_t block_size, const void* q, const void* k,
                                 const void* v, const int32_t* positions,
                                 const int32_t* slot_mapping, const float* cos_sin,
                                 int32_t max_pos, void* q_out, void* k_cache, void* v_cache,
                                 int64_t num_blocks) {
  using namespace cb;
  if (dtype != CB_F32 && dtype != CB_BF16) return CB_ERR_INVALID;
  if (T < 0 || Hq < 1 || Hkv < 1 || block_size < 1 || max_pos < 1 || num_blocks < 0)
    return CB_ERR_INVALID;
  if (D != 64 && D != 128) return CB_ERR_INVALID;
  if (T == 0) return CB_OK;
  if (!k || !v || !positions || !slot_mapping || !cos_sin || !k_cache || !v_cache)
    return CB_ERR_INVALID;
  if (q && !q_out) return CB_ERR_INVALID;
  const void* ptrs[] = {q, k, v, q_out, k_cache, v_cache};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return CB_ERR_INVALID;
  const int32_t heads = (q ? Hq : 0) + 2 * Hkv;
  const int64_t total = static_cast<int64_t>(T) * heads * (D / 16);
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffff) return CB_ERR_INVALID;
  const int64_t num_slots = num_blocks * block_size;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == CB_BF16) {
    rope_kv_append_kernel<bf16_t><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st>>>(
        T, Hq, Hkv, D, block_size, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
        static_cast<const bf16_t*>(v), positions, slot_mapping, cos_sin, max_pos,
        static_cast<bf16_t*>(q_out), static_cast<bf16_t*>(k_cache), static_cast<bf16_t*>(v_cache),
        num_slots);
  } else {
    rope_kv_append_kernel<float><<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st>>>(
        T, Hq, Hkv, D, block_size, static_cast<const float*>(q), static_cast<const float*>(k),
        static_cast<const float*>(v), positions, slot_mapping, cos_sin, max_pos,
        static_cast<float*>(q_out), static_cast<float*>(k_cache), static_cast<float*>(v_cache),
        num_slots);
  }
  return hipGetLastError() == hipSuccess ? CB_OK : CB_ERR_HIP;
}
