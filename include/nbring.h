/*
 * nbring -- the global-layer ring attention of one context-parallel rank on
 * MI355X (gfx950): per-chunk attention returning (out, lse), the online-softmax
 * merges, and the per-chunk backward with the global out and lse.
 *
 * Sources (NeMo AutoModel gemma4_moe.cp_attention page):
 *   - _run_gemma4_cp_ffpa_varlen_ring_forward: rank r's queries (its chunk of
 *     the global sequence) visit the K/V chunks of owners r, r-1, ..., 0; each
 *     chunk's attention gives (out, lse), merged into fp32 accumulators; pad
 *     query rows stay 0;
 *   - _ffpa_varlen_forward_chunk / _chunk_dense_eligible: the own chunk runs
 *     causally, an earlier owner's chunk non-causally; a query meets only keys
 *     of its own document (_build_packed_ring_segments);
 *   - _merge_ffpa_packed_chunk: the -inf-safe online-softmax merge (a row
 *     neither side covered keeps out 0, lse -inf);
 *   - _merge_live_chunk_: the same merge in place at the live rows only;
 *   - _ffpa_varlen_backward_chunk: each chunk's backward with the *global*
 *     merged out and lse; the chunks' dQ add up (_grad_add_live_), each chunk's
 *     dK/dV is its owner's contribution (_route_kv_grads_to_owners).
 * Readings where the page is silent: positions are global (query row i at
 * q_start + i, key j at k_start + j); a query attends key j iff both lie in the
 * same document and k_start + j <= q_start + i, so a chunk that ends before the
 * shard is non-causal by construction and the shard's own chunk causal; no
 * left window (global layers); lse is the natural log of the softmax
 * denominator, -inf (with out 0) for a row without keys in the chunk.
 *
 * Documents: the segment buffer comes from nb_segment_build over the prefix
 * [0, q_start + L) of the global doc map with window_left = -1 and the shard's
 * L: its row_klo then holds each query row's document start in global
 * positions, which serves every chunk.
 *
 * Conventions are those of nbattn.h (device pointers owned by the caller, work
 * enqueued on `stream`, checks before any launch, NB_* status codes, NB_BF16 /
 * NB_F32 for `dtype`, head dim 64 / 128 / 256, and 512 -- the global layers'
 * head dim, which the cp_attention page's FFPA path runs -- on the chunk
 * attention calls).  At D = 512 each 32-row query group of the forward is
 * split over two waves, one per half of the head dim, and the backward always
 * takes the stored-dS form (see nb_ring_chunk_bwd_workspace_bytes).
 */
#ifndef NBRING_H
#define NBRING_H

#include <stddef.h>
#include <stdint.h>

#include "nbattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One chunk's forward: q [B, Hq, L, D] (the shard, global positions q_start ..),
 * k, v [B, Hkv, Lk, D] (the chunk, global positions k_start ..; 0 <= k_start <=
 * q_start, L <= Lk), seg_buf as above.  out [B, Hq, L, D] (dtype) and lse
 * [B, Hq, L] (fp32) receive the chunk's attention alone.  Errors as
 * nb_attn_fwd, plus NB_ERR_INVALID_ARG when k_start > q_start. */
int nb_ring_chunk_fwd(const void* q, const void* k, const void* v, void* out, float* lse, const int32_t* seg_buf,
                      int B, int Hq, int Hkv, int L, int Lk, int D, int q_start, int k_start, float scale, int dtype,
                      void* stream);

/* In-place -inf-safe merge over R = B * Hq * L rows of D values:
 * lse = log(e^lse_acc + e^lse_step), out_acc = the two outs weighted by
 * exp(lse_x - lse).  A row whose lse_step is -inf is left untouched (nothing to
 * merge), so the rows neither side covers keep out 0, lse -inf.  out_acc,
 * lse_acc fp32; out_step dtype, lse_step fp32; out_acc and out_step 16-byte
 * aligned; D a power of two in [4, 1024].  init != 0: nothing is merged yet --
 * the accumulators are set to the step on every row (their contents ignored). */
int nb_ring_merge(float* out_acc, float* lse_acc, const void* out_step, const float* lse_step, int64_t R, int D,
                  int dtype, int init, void* stream);

/* The rows of the shard that have keys in the chunk (k_start, Lk): live_index
 * [B * L] receives their flat indices b * L + i in ascending order and *n_live
 * (device int32) their count.  A row is live iff it is not padding and its
 * document starts at or before the chunk's last key it may attend. */
int nb_ring_live_rows(const int32_t* seg_buf, int B, int L, int Lk, int q_start, int k_start, int32_t* live_index,
                      int32_t* n_live, void* stream);

/* The merge at the live rows only (_merge_live_chunk_): for every head h and
 * every entry x < *n_live of live_index (flat b * L + i), row (b, h, i) of the
 * [B, H, L, D] / [B, H, L] arrays is merged as by nb_ring_merge; every other row
 * is left alone.  n_live_max bounds *n_live (it sizes the launch). */
int nb_ring_merge_live(float* out_acc, float* lse_acc, const void* out_step, const float* lse_step,
                       const int32_t* live_index, const int32_t* n_live, int n_live_max, int B, int H, int L, int D,
                       int dtype, void* stream);

/* The merged fp32 output as the attention output: out = out_acc rounded to
 * dtype; for bf16, out_resid (optional, may be NULL; int8, R * D bytes) = the
 * rounding residual codes of out (as nb_attn_fwd's o_resid, nbattn.h), which
 * the backward adds back for an fp32-accurate Delta; for float32 out_resid is
 * ignored.  R rows of D values. */
int nb_ring_finalize(const float* out_acc, void* out, void* out_resid, int64_t R, int D, int dtype, void* stream);

/* Flags of nb_ring_chunk_bwd. */
#define NB_RING_DELTA_READY 1  /* ws already holds Delta = rowsum(dout * o): written by an earlier call on the
                                  same ws with the same dout, o, o_resid, seg_buf and B, Hq, L (Delta does not
                                  depend on the chunk) */
#define NB_RING_DQ_F32_SET 2   /* dq is an fp32 [B, Hq, L, D] buffer and receives the contribution */
#define NB_RING_DQ_F32_ADD 4   /* dq is fp32 and the contribution is added to it (the chunks' dQ summed) */

/* One chunk's backward with the global out (o, o_resid from nb_ring_finalize)
 * and the global lse (the merged lse_acc): dq [B, Hq, L, D] receives the chunk's
 * dQ contribution (dtype; fp32 set or accumulated per flags), dk, dv
 * [B, Hkv, Lk, D] the chunk's dK/dV (its owner's share from this shard; 0 at
 * keys no query reaches).  Workspace: at least nb_attn_bwd_workspace_bytes(B,
 * Hq, Hkv, L, Lk, D, dtype); given nb_ring_chunk_bwd_workspace_bytes, the dK/dV
 * pass stores dS and dQ is formed from it (dK, dV bit-identical to the
 * recompute form, dQ within the usual tolerance).  At D = 512 that workspace
 * is required (NB_ERR_WORKSPACE below it; NB_ERR_UNSUPPORTED when the dS band
 * would exceed 2 GiB).  Arguments as nb_ring_chunk_fwd otherwise; unknown
 * flags, or both dQ flags, are NB_ERR_INVALID_ARG. */
int nb_ring_chunk_bwd(const void* dout, const void* q, const void* k, const void* v, const void* o,
                      const void* o_resid, const float* lse, const int32_t* seg_buf, int B, int Hq, int Hkv, int L,
                      int Lk, int D, int q_start, int k_start, float scale, int dtype, void* dq, void* dk, void* dv,
                      int flags, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace for nb_ring_chunk_bwd's stored-dS form: those of
 * nb_attn_bwd_workspace_bytes plus, at D = 256 and 512, a banded dS buffer with room
 * for bands as wide as the chunk (B * Hq * round_up(L, 32) rows of
 * round_up(Lk + 96, 32) elements of dtype; at most 2 GiB, else none).  Equal to
 * nb_attn_bwd_workspace_bytes at other head dims.  Without a window every row's
 * band may span the chunk, so the dS round trip grows with the rows that reach
 * it: on a 4096-token chunk at B = 1, Hq = 16 the shard's own (causal) chunk
 * takes longer this way than with the recompute, a chunk few rows reach less. */
size_t nb_ring_chunk_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int Lk, int D, int dtype);

/* acc[x] += src[x] for n elements (fp32 acc, dtype src; 16-byte aligned, n a
 * multiple of 4): the chunks' dQ contributions summed in fp32.  init != 0:
 * acc[x] = src[x] (the first contribution). */
int nb_ring_grad_add(float* acc, const void* src, int64_t n, int dtype, int init, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NBRING_H */
