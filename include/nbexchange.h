/*
 * nbexchange -- block-diagonal context-parallel K/V exchange plans, and the
 * needed-range exchange emulated for every rank on one device (MI355X / gfx950).
 *
 * Sources (NeMo AutoModel blockdiag_cp.exchange page):
 *   - the global left-halo plan (its description): with cp_size ranks and the
 *     global sequence split into equal chunks of L = N / cp_size tokens (rank r
 *     owns [r L, (r+1) L)), rank r needs the contiguous K/V range
 *     [s_first_r, real_end_r): its boundary document's straddle (owned by
 *     earlier ranks) plus its own chunk.  back_r = r L - s_first_r; one
 *     neighbour exchange suffices (use_halo) iff back_r <= L for every rank.
 *     Every rank derives the plan from the same replicated document ids;
 *   - _LeftHaloExchange: one uniform-size step; each rank receives the last
 *     halo_size tokens of the previous rank's chunk and keeps the last back_r;
 *   - the per-(source, destination) split sizes and local gather index, and
 *     _NeededKVExchange: source s sends destination r the intersection of its
 *     chunk with r's range (a token once per rank that needs it; the send
 *     buffer is the chunk gathered through send_index); r concatenates the
 *     pieces in source order into its range.  The backward adds each
 *     destination's gradient back onto the source token (index_add).
 * Readings where the page is silent: padding (nonzero pad mask) is folded to
 * id 0 and id 0 is never a document; s_first_r is the start of the run of equal
 * nonzero ids holding position r L (r L itself when that position is padding);
 * real_end_r is one past chunk r's last non-padding position, and a chunk with
 * none needs nothing (s_first_r = real_end_r = r L); with several batch rows the
 * range is the union over the rows; halo_size = max_r back_r.
 *
 * Conventions are those of nbattn.h (device pointers owned by the caller, work
 * enqueued on `stream`, checks before any launch, NB_* status codes, NB_BF16 /
 * NB_F32).  On one device "rank r's chunk" is the slice [r L, (r+1) L) of one
 * global tensor; the emulated exchange moves exactly the tokens the real one
 * would, rank by rank.
 */
#ifndef NBEXCHANGE_H
#define NBEXCHANGE_H

#include <stddef.h>
#include <stdint.h>

#include "nbattn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define NB_XCH_MAX_RANKS 64

/* Plan buffer (int32), with P = cp_size, offsets in elements:
 *   [0, 8)              use_halo (1/0), halo_size, L, P, total received tokens
 *                       (sum over r of R_r = real_end_r - s_first_r), 3 reserved
 *   s_first  [P]        at 8
 *   real_end [P]        at 8 + P
 *   back     [P]        at 8 + 2P
 *   splits   [P * P]    at 8 + 3P; splits[s * P + r] = tokens source s sends
 *                       destination r (row s: s's in_splits; column r: r's
 *                       out_splits)
 *   send_off [P * (P+1)] at 8 + 3P + P*P; send_off[s * (P+1) + r] = start of
 *                       the piece for destination r in s's send buffer
 *                       (send_off[s * (P+1) + P] = s's send count)
 *   recv_off [P * (P+1)] after send_off; recv_off[r * (P+1) + s] = start of
 *                       source s's piece in r's received range
 */
size_t nb_exchange_plan_elems(int cp_size);

/* Plan from doc_ids [B, N] (int32; N a multiple of cp_size) and pad_mask
 * [B, N] (uint8, nonzero = padding) or NULL.  plan: device int32 buffer of at
 * least nb_exchange_plan_elems(cp_size) elements, fully written.  Errors:
 * NB_ERR_INVALID_ARG (null pointer, B < 1, N < 1, cp_size outside
 * [1, NB_XCH_MAX_RANKS], N % cp_size != 0), NB_ERR_WORKSPACE (plan too small). */
int nb_exchange_plan(const int32_t* doc_ids, const uint8_t* pad_mask, int B, int N, int cp_size,
                     int32_t* plan, size_t plan_elems, void* stream);

/* send_index of every source: send_index[s * N + k] for k < send count of s is
 * the local position (0 .. L-1) of the k-th token of s's send buffer (the
 * pieces for destinations 0, 1, ... one after another); entries past the send
 * count are not written.  send_index: device int32 buffer of at least
 * nb_exchange_send_index_elems(cp_size, N) elements (each source sends at most
 * P L = N tokens). */
size_t nb_exchange_send_index_elems(int cp_size, int N);
int nb_exchange_send_index(const int32_t* plan, int cp_size, int N, int32_t* send_index, size_t elems,
                           void* stream);

/* Forward of the needed-range exchange for every rank: x is the global
 * [B, C, N, D] tensor (rank s owns x[:, :, s L : (s+1) L]); recv is a HOST array
 * of cp_size device pointers, recv[r] -> [B, C, R_r, D] (R_r from the plan;
 * the caller reads the plan to size them).  recv[r] may be NULL only when
 * R_r = 0.  The received range is the pieces of every source in source order,
 * i.e. x[:, :, s_first_r : real_end_r].  x and every non-null recv[r] 16-byte
 * aligned, D * element size a multiple of 16 bytes, B * C <= 65535. */
int nb_exchange_gather(const void* x, const int32_t* plan, int B, int C, int N, int D, int cp_size, int dtype,
                       void* const* recv, void* stream);

/* Backward: grad_recv[r] -> [B, C, R_r, D] (host array of device pointers;
 * NULL = a zero gradient); grad_x [B, C, N, D] receives, for every token, the
 * sum over the ranks that needed it (ascending rank order, fp32 accumulation,
 * one rounding to the output type) and 0 where no rank needed it. */
int nb_exchange_scatter_add(void* const* grad_recv, const int32_t* plan, int B, int C, int N, int D, int cp_size,
                            int dtype, void* grad_x, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NBEXCHANGE_H */
