/* Optional extensions of the mixed-step library (libcb.so): a host-made decode work split and a
 * timed variant of the attention call.  Nothing here is needed to run a step --
 * cb_mixed_paged_attention in cb.h is complete on its own -- but a serving loop that already has
 * the step's metadata on the host saves the split kernel and one kernel boundary per step with
 * cb_decode_plan, and a benchmark can time the attention kernels with the timed variant.  Both
 * expose the launch's decode grid (the plan must match the call's wave count), so they are kept
 * apart from the core interface.
 *
 * Sources: "Chunked Prefill: Ending the Great Stall" §01 (decode rows stream the whole cache, so
 * their work is split by bytes streamed) and "Chunked Prefill 的 Token 预算" §04 (per-step timing
 * records). */
#ifndef CB_EXT_H
#define CB_EXT_H

#include "cb.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The decode rows' work split, made on the host (so that the attention call needs no split
 * kernel).  Decode rows stream their keys as 32-key stages of (row, KV head, 16-head group)
 * units; all units' stages, in order, form one line of S stages, cut into W contiguous ranges,
 * one per decode wave with work.  Each wave's share is proportional to the measured streaming rate
 * of its workgroup (the first or second workgroup on its compute unit, even or odd XCD, and, beside
 * chunk rows, how long the chunk tile on the same compute unit runs), so the waves end together.
 * cb_attn_decode_waves is the number of decode waves an attention call on this stream's device
 * launches (has_chunks: whether the step has chunk rows); cb_decode_plan_ints the int32 capacity a
 * plan needs; cb_decode_plan writes the plan for a call on the same stream's device with the same
 * num_seqs, num_decodes >= 1, max_q_len, max_ctx, Hq and Hkv, from the step's host metadata (the
 * values cb_build_step emitted): context_lens of all num_seqs rows, decode rows first, and
 * cu_seqlens_q (num_seqs + 1 offsets; read only when num_seqs > num_decodes, may be NULL
 * otherwise).  out (host memory) receives [S, F (workgroups dispatched first onto their compute
 * units), W, n_waves], the stage offset of each decode row (num_decodes + 1), n_waves slots whose
 * first W hold the first unit of each wave with work, and n_waves + 1 slots whose first W + 1 hold
 * each wave's first stage and then S.  It makes no device call beyond reading the device's compute
 * unit count once.  The device copy (16-byte aligned) is passed to the call below with its n_waves
 * (out[3]), which must equal the call's own decode wave count (else CB_ERR_INVALID).  The result is
 * bit for bit the same as with the split kernel.  CB_ERR_CAPACITY if cap_ints is too small,
 * CB_ERR_INVALID on bad arguments. */
int32_t cb_attn_decode_waves(void* stream, int32_t has_chunks);
size_t cb_decode_plan_ints(int32_t num_decodes, int32_t n_waves);
int cb_decode_plan(void* stream, int32_t num_seqs, int32_t num_decodes, int32_t max_q_len, int32_t max_ctx,
                   int32_t Hq, int32_t Hkv, const int32_t* cu_seqlens_q, const int32_t* context_lens,
                   int32_t* out, size_t cap_ints);

/* The same operation, optionally with a host-made decode plan (decode_plan: device copy of
 * cb_decode_plan's output, plan_waves its n_waves; NULL = split on the device), recording
 * caller-created HIP events (hipEvent_t, passed as void*) on the stream around its kernels for
 * timing: events[0] / events[1] and events[2] / events[3] before / after the attention kernel
 * (decode and chunk rows share it), events[4] / events[5] before / after the combine kernel.
 * events may be NULL and any entry may be NULL. */
int cb_mixed_paged_attention_timed(void* stream, int32_t dtype, int32_t num_seqs,
                                   int32_t num_decodes, int32_t T, int32_t max_q_len,
                                   int32_t max_decode_ctx, int32_t max_ctx, int32_t Hq,
                                   int32_t Hkv, int32_t D, int32_t block_size, float scale,
                                   const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                   const int32_t* cu_blocks, const int32_t* block_table,
                                   void* out, void* workspace, size_t workspace_bytes,
                                   const int32_t* decode_plan, int32_t plan_waves,
                                   void* const* events);

#ifdef __cplusplus
}
#endif
#endif /* CB_EXT_H */
