/*
 * nbattn -- neighbourhood attention for one context-parallel rank (MI355X / gfx950).
 *
 * A local query shard Q attends over its collected K/V neighbourhood: the
 * causally valid ring chunks (owners <= cp_rank) concatenated in ascending
 * order, or a left halo plus the local chunk.  The query shard is the suffix of
 * the neighbourhood, so local query row i sits at neighbourhood position
 * p = S - L + i (bottom-right alignment).  Sources, all NeMo AutoModel API pages:
 *   - cp_local_ring page, module docstring: one bottom-right causal call with a
 *     left window over the concatenated neighbourhood; per-document varlen
 *     segments; a forward that saves what its backward needs (no recompute);
 *   - cp_local_ring page, sliding_ring_compute_fa_fwd / _bwd: out[B,Hq,L,D] and
 *     (dQ, dK by owner, dV by owner);
 *   - cp_local_ring page, _fold_pad and _owner_grad_dict;
 *   - blockdiag_cp.kernels page, _cp_blockdiag_mask and _cp_blockdiag_varlen:
 *     a query attends a key iff same document, neither is padding (id 0), key
 *     not after the query; the varlen form equals that mask + attention on the
 *     real rows, padding rows are zeros;
 *   - blockdiag_cp.kernels page, _varlen_backend_unavailable_reason and
 *     _varlen_metadata_unavailable_reason: failures are found before any
 *     kernel is launched.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises (except nb_segment_header, a debug
 *     helper that does synchronise).  Work is enqueued on `stream` (a
 *     hipStream_t, NULL = the default stream) and the call returns at once.
 *   - Layouts are contiguous row-major: Q/O/dO/dQ [B,Hq,L,D]; K/V/dK/dV
 *     [B,Hkv,S,D]; LSE [B,Hq,L] float32; doc ids / pad mask [B,S].
 *   - GQA: q head h reads kv head h / (Hq / Hkv).
 *   - window_left W >= 0: key j is visible from position p iff p - j <= W
 *     (FlashAttention's window_size[0]: W+1 keys including the query's own);
 *     W < 0: no window.
 *   - Errors are detected before anything is enqueued: a non-OK return leaves
 *     the stream untouched.  NB_ERR_LAUNCH reports a HIP launch failure.
 *   - Thread-safe and stateless (except nb_attn_bwd_noalloc, whose static
 *     workspace calls on one GPU share); calls on one stream are ordered by the
 *     stream.
 */
#ifndef NBATTN_H
#define NBATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum nb_status {
  NB_OK = 0,
  NB_ERR_INVALID_ARG = 1,  /* null pointer, bad size, Hq % Hkv != 0, L > S, ... */
  NB_ERR_UNSUPPORTED = 2,  /* D not in {64,128,256}, unknown dtype, dropout != 0 */
  NB_ERR_WORKSPACE = 3,    /* workspace or segment buffer smaller than required */
  NB_ERR_LAUNCH = 4,       /* a HIP launch failed (hipGetLastError) */
  NB_ERR_DEVICE = 5        /* no usable gfx950 device / HIP runtime error */
};

enum nb_dtype {
  NB_BF16 = 0, /* bfloat16 inputs/outputs, fp32 accumulation (main path) */
  NB_F32 = 1   /* float32 inputs/outputs (debug path, same kernels) */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char* nb_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int nb_version(void);

/* ------------------------------------------------------------------------ *
 * Segment buffer (int32), produced by nb_segment_build, read by the kernels.
 * Offsets are in int32 elements, with N = B * L:
 *   [0, 16)            header: n_seg, max_q, max_k, status, lo, B, L, S,
 *                      window_left, n_real, then 6 reserved words
 *   cu_q   [N + 1]     cumulative query-segment lengths (cu_seqlens_q)
 *   cu_k   [N + 1]     cumulative key-segment lengths (cu_seqlens_k); cu_q[i]
 *                      pairs with cu_k[i]
 *   q_row0 [N]         b * L + first local query row of segment i
 *   k_row0 [N]         b * S + first key of segment i
 *   row_seg[N]         segment of local query row (b, i), -1 for padding rows
 *   row_klo[N]         first key of that row's segment (neighbourhood position);
 *                      p + 1 for padding rows (an empty key range)
 *   kcov_lo[B]         first covered key of batch row b (S if none)
 *   fwd_order[B * ceil(L / 128)]
 *                      per batch row, the indices of its 128-row query tiles
 *                      by decreasing band work (ties: higher index first); the
 *                      identity when a row has more than 2048 tiles.  The
 *                      forward launches its tiles in this order; it changes
 *                      no result
 *   scratch            builder-private (per-tile records, completion counters,
 *                      duplicate-id set)
 * Entries past n_seg (past n_seg + 1 for cu_q / cu_k) are unspecified.
 * ------------------------------------------------------------------------ */
#define NB_SEG_HEADER 16
enum {
  NB_HDR_NSEG = 0, NB_HDR_MAXQ = 1, NB_HDR_MAXK = 2, NB_HDR_STATUS = 3, NB_HDR_LO = 4,
  NB_HDR_B = 5, NB_HDR_L = 6, NB_HDR_S = 7, NB_HDR_WINDOW = 8, NB_HDR_NREAL = 9
};
/* status bit 0: some id > 0 occurs in two separate runs of one row (the
 * per-document contract is violated; segments then follow runs). */
#define NB_SEG_STATUS_SPLIT_DOC 1

/* Element offsets of each array inside the segment buffer. */
size_t nb_segment_offset_cu_q(int B, int L);
size_t nb_segment_offset_cu_k(int B, int L);
size_t nb_segment_offset_q_row0(int B, int L);
size_t nb_segment_offset_k_row0(int B, int L);
size_t nb_segment_offset_row_seg(int B, int L);
size_t nb_segment_offset_row_klo(int B, int L);
size_t nb_segment_offset_kcov_lo(int B, int L);
size_t nb_segment_offset_fwd_order(int B, int L);

/* int32 elements the caller must provide for seg_buf (0 on invalid sizes). */
size_t nb_segment_buffer_elems(int B, int L, int S);

/*
 * Fold padding into the doc map and build the per-document varlen segments of
 * the shard, on the device, without any device-to-host transfer.
 *   cp_local_ring page, _fold_pad (pad -> id 0) and _cached_sliding_segments
 *   (the key start of the straddling document is clipped at
 *   lo = max(0, S - L - W) when W >= 0, else 0); blockdiag_cp.kernels page,
 *   _cp_blockdiag_varlen (one segment per document the local rows touch: query
 *   part = its local rows, key part = document start .. last local row) and
 *   precompute_blockdiag_varlen_meta (built once per step, reused by every
 *   layer and both passes).
 * A document is a maximal run of one id > 0; ids <= 0 are padding.
 *   doc_ids    [B,S] int32 device, neighbourhood doc map
 *   pad_mask   [B,S] uint8 device, nonzero = padding, or NULL
 *   folded_ids [B,S] int32 device, out: doc_ids with padding set to 0
 *   seg_buf    device, out, 16-byte aligned,
 *              seg_buf_elems >= nb_segment_buffer_elems(B, L, S)
 * Requires 1 <= L <= S, B >= 1.  Segments are valid by construction.
 */
int nb_segment_build(const int32_t* doc_ids, const uint8_t* pad_mask, int B, int S, int L,
                     int window_left, int32_t* folded_ids, int32_t* seg_buf,
                     size_t seg_buf_elems, void* stream);

/* Debug: copy the 16-word header to host memory (synchronises the stream). */
int nb_segment_header(const int32_t* seg_buf, int32_t* host_header, void* stream);

/* Bytes of workspace nb_attn_fwd needs (currently 0). */
size_t nb_attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int L, int S, int D, int dtype);

/*
 * Forward: for every real query row and q head, softmax attention over the
 * keys of its document band [max(row_klo, p - W), p]; saves LSE.
 *   cp_local_ring page, sliding_ring_compute_fa_fwd; blockdiag_cp.kernels page,
 *   _cp_blockdiag_varlen.
 *   q   [B,Hq,L,D], k/v [B,Hkv,S,D]   (dtype), device
 *   o   [B,Hq,L,D] out (dtype); padding rows written 0
 *   o_resid [B,Hq,L,D] int8 out, or NULL: the rounding residual of o, one
 *       signed byte per element.  With a the fp32 result, v = bf16(a) the
 *       stored value and u = 2^(max(e, 1) - 134) its ulp (e = v's biased
 *       exponent field), the code is a - v in units of u / 254, rounded to
 *       nearest even and clamped to [-127, 127]; v + code * u / 254 is within
 *       u / 508 of a (about 17 significant bits).  Saved for the backward,
 *       whose Delta = dO . O then uses an fp32-accurate O; for bf16 the
 *       backward is only within tolerance with it.  float32: ignored (pass
 *       NULL; O is the fp32 result itself).
 *   lse [B,Hq,L] float32 out: natural-log sum of exp(scale * q.k) over the
 *       band; -inf for padding rows
 *   seg_buf from nb_segment_build with the same B, L, S and window_left
 *   scale > 0 (callers pass D^-0.5 for the default), dropout_p must be 0.
 */
int nb_attn_fwd(const void* q, const void* k, const void* v, void* o, void* o_resid, float* lse,
                const int32_t* seg_buf, int B, int Hq, int Hkv, int L, int S, int D, float scale,
                int window_left, float dropout_p, int dtype, void* ws, size_t ws_bytes,
                void* stream);

/* Bytes of workspace nb_attn_bwd needs: the Delta rows (B * Hq * L floats),
 * then the work orders of the two passes, the backward kernel's counters and
 * the list of deferred dQ items (B * ceil(S / 32) + 10 + B * ceil(L / 32) +
 * B * Hq * ceil(L / 32) ints), each part 256-byte aligned. */
size_t nb_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int S, int D, int dtype);

/* The same plus, with a left window 0 <= window_left <= 4096 and D = 256, a
 * banded dS buffer (B * Hq * round_up(L, 32) rows of round_up(window_left + 96,
 * 32) elements of dtype; at most 2 GiB, else none).  Given a workspace of this
 * size, nb_attn_bwd, nb_attn_bwd_main and nb_attn_bwd_chunks on a windowed
 * neighbourhood have the dK/dV pass store dS and form dQ = dS K from it instead
 * of recomputing S and dP (dK, dV unchanged bit for bit; dQ within the usual
 * tolerance).  Equal to nb_attn_bwd_workspace_bytes without a window or at
 * another D. */
size_t nb_attn_bwd_workspace_bytes_window(int B, int Hq, int Hkv, int L, int S, int D, int dtype, int window_left);

/*
 * Backward with no forward recompute: dQ and dK/dV from the saved O and LSE.
 *   cp_local_ring page, sliding_ring_compute_fa_bwd (returns dQ and per-owner
 *   dK/dV) and _owner_grad_dict (owners this shard did not attend get zeros).
 *   dout, q, o [B,Hq,L,D]; k, v [B,Hkv,S,D]; lse [B,Hq,L] (from nb_attn_fwd);
 *   o_resid    the int8 residual codes nb_attn_fwd saved, or NULL (Delta from o
 *              alone); ignored for float32
 *   dq [B,Hq,L,D] out (0 on padding rows)
 *   dk, dv [B,Hkv,S,D] out; every row is written, keys no query attended are 0
 *   owner_off  HOST int32 [n_owner + 1], ascending neighbourhood offsets of the
 *              owner chunks, owner_off[0] = 0, owner_off[n_owner] = S;
 *              dK of owner o is dk[:, :, owner_off[o]:owner_off[o+1]]
 *   owner_attended DEVICE uint8 [n_owner] out: 1 iff some real query attended
 *              a key of chunk o (may be NULL when n_owner == 0)
 *   1 <= n_owner <= 64, or n_owner == 0 with owner_off / owner_attended NULL.
 *   ws: workspace of at least nb_attn_bwd_workspace_bytes bytes.
 */
int nb_attn_bwd(const void* dout, const void* q, const void* k, const void* v, const void* o,
                const void* o_resid, const float* lse, const int32_t* seg_buf, const int32_t* folded_ids, int B,
                int Hq, int Hkv, int L, int S, int D, float scale, int window_left, int dtype,
                void* dq, void* dk, void* dv, const int32_t* owner_off, int n_owner,
                uint8_t* owner_attended, void* ws, size_t ws_bytes, void* stream);

/*
 * The steps nb_attn_bwd runs, for callers that schedule them separately (for
 * instance to hand dK/dV to the owner exchange while other work runs) and for
 * per-kernel timing.  Same arguments and conventions as nb_attn_bwd.
 *   nb_attn_bwd_prep: Delta = dO . (o + o_resid) into ws, and the work orders
 *                     (longest items first) of the two passes.
 *   nb_attn_bwd_main: dq, dk, dv: both passes in one persistent grid (the
 *                     short dQ items fill the tail of the dK/dV items); needs
 *                     an nb_attn_bwd_prep call on the same stream and ws before
 *                     each call.  nb_attn_bwd = prep + main + owner flags.
 *   nb_attn_bwd_dq:   Delta into ws, then dq alone.
 *   nb_attn_bwd_dkdv: dk, dv alone; needs the Delta an earlier nb_attn_bwd_dq
 *                     or nb_attn_bwd_prep call on the same stream left in ws.
 *   nb_owner_attended: owner_attended[o] = 1 iff some real query attended a key
 *                     of chunk o (cp_local_ring page, _owner_grad_dict).
 * The workspace is written by every one of them (Delta, work orders, queue
 * counters); calls sharing a workspace must be ordered on one stream.
 */
int nb_attn_bwd_prep(const void* dout, const void* o, const void* o_resid, const int32_t* seg_buf, int B,
                     int Hq, int Hkv, int L, int S, int D, int window_left, int dtype, void* ws,
                     size_t ws_bytes, void* stream);
int nb_attn_bwd_main(const void* dout, const void* q, const void* k, const void* v, const float* lse,
                     const int32_t* seg_buf, int B, int Hq, int Hkv, int L, int S, int D, float scale,
                     int window_left, int dtype, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                     void* stream);
int nb_attn_bwd_dq(const void* dout, const void* q, const void* k, const void* v, const void* o,
                   const void* o_resid, const float* lse, const int32_t* seg_buf, int B, int Hq,
                   int Hkv, int L, int S, int D, float scale, int window_left, int dtype, void* dq,
                   void* ws, size_t ws_bytes, void* stream);
int nb_attn_bwd_dkdv(const void* dout, const void* q, const void* k, const void* v,
                     const float* lse, const int32_t* seg_buf, int B, int Hq, int Hkv, int L, int S,
                     int D, float scale, int window_left, int dtype, void* dk, void* dv,
                     void* ws, size_t ws_bytes, void* stream);
int nb_owner_attended(const int32_t* seg_buf, const int32_t* folded_ids, int B, int L, int S,
                      const int32_t* owner_off, int n_owner, uint8_t* owner_attended, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): nb_attn_bwd
 * with no workspace argument.  Its workspace (Delta, work orders, queue
 * counters, deferred dQ list) lives in a static device array of the library,
 * one per GPU, of nb_attn_bwd_noalloc_max_workspace_bytes() bytes (8 MiB),
 * held until the process ends.  Nothing is allocated or freed by the call.
 *   Arguments, layouts and results as nb_attn_bwd (the recompute form of the
 *   dQ pass: no stored-dS buffer); dq, dk, dv are bit-identical to nb_attn_bwd
 *   with a workspace of nb_attn_bwd_workspace_bytes.
 *   NB_ERR_WORKSPACE when nb_attn_bwd_workspace_bytes(...) for these sizes
 *   exceeds the static array (checked before anything is enqueued).
 *   Every call on one GPU uses that GPU's one array: calls that overlap on one
 *   GPU (on different streams, or from different threads) race and must be
 *   ordered by the caller.  The array keeps the last call's contents; the call
 *   rewrites everything it reads (the prep kernel sets the queue counters to 0).
 */
size_t nb_attn_bwd_noalloc_max_workspace_bytes(void);
int nb_attn_bwd_noalloc(const void* dout, const void* q, const void* k, const void* v, const void* o,
                        const void* o_resid, const float* lse, const int32_t* seg_buf, const int32_t* folded_ids,
                        int B, int Hq, int Hkv, int L, int S, int D, float scale, int window_left, int dtype,
                        void* dq, void* dk, void* dv, const int32_t* owner_off, int n_owner,
                        uint8_t* owner_attended, void* stream);

/* ------------------------------------------------------------------------ *
 * Zero-copy neighbourhood: K/V straight from the owners' chunk buffers.
 *
 * cp_local_ring page, module docstring and _concat_neighborhood: the
 * neighbourhood is the causally valid chunks concatenated in ascending owner
 * order, and with a left window only the keys the window reaches matter.
 * These entry points take the chunks as a table instead of a concatenated copy:
 * neighbourhood keys [off_c, off_c + chunk_len[c]) (off_c = sum of the earlier
 * lengths, S = the total) are rows chunk_start[c] .. of chunk c's buffers
 * K, V [B, Hkv, chunk_rows[c], D] (HOST arrays of n_chunk device pointers and
 * sizes, 1 <= n_chunk <= 16, chunk_len >= 1, chunk_start + chunk_len <=
 * chunk_rows).  So a windowed ring rank passes the last W' rows of the previous
 * chunk(s) and its own chunk, and nothing is copied.  seg_buf comes from
 * nb_segment_build over the same neighbourhood's doc ids [B, S].  Chunk
 * buffers are 16-byte aligned.  Results are bit-identical to nb_attn_fwd /
 * nb_attn_bwd on the concatenated neighbourhood (the same key tiles in the same
 * order).  Errors: NB_ERR_INVALID_ARG for a table outside the bounds above,
 * lengths not summing to S, or a null or misaligned chunk pointer; otherwise as
 * nb_attn_fwd / nb_attn_bwd.
 */
int nb_attn_fwd_chunks(const void* q, const void* const* k_chunk, const void* const* v_chunk,
                       const int32_t* chunk_len, const int32_t* chunk_start, const int32_t* chunk_rows,
                       int n_chunk, void* o, void* o_resid, float* lse, const int32_t* seg_buf, int B, int Hq,
                       int Hkv, int L, int S, int D, float scale, int window_left, float dropout_p, int dtype,
                       void* ws, size_t ws_bytes, void* stream);

/* The backward with the chunk table: dk_chunk[c], dv_chunk[c] (host arrays of
 * device pointers) are whole chunk-gradient buffers [B, Hkv, chunk_rows[c], D],
 * fully written -- the gradients of the chunk's neighbourhood keys (0 where no
 * query attends) and 0 on its rows outside [chunk_start, chunk_start +
 * chunk_len).  chunk_attended (device [n_chunk], or NULL) receives the
 * nb_owner_attended flags with the chunks as owners (folded_ids then required).
 * Workspace as for nb_attn_bwd (nb_attn_bwd_workspace_bytes_window's size
 * selects the stored-dS form here too). */
int nb_attn_bwd_chunks(const void* dout, const void* q, const void* const* k_chunk, const void* const* v_chunk,
                       const int32_t* chunk_len, const int32_t* chunk_start, const int32_t* chunk_rows,
                       int n_chunk, const void* o, const void* o_resid, const float* lse, const int32_t* seg_buf,
                       const int32_t* folded_ids, int B, int Hq, int Hkv, int L, int S, int D, float scale,
                       int window_left, int dtype, void* dq, void* const* dk_chunk, void* const* dv_chunk,
                       uint8_t* chunk_attended, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NBATTN_H */
