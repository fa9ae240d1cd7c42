// Device-side pad fold + per-document varlen segment builder (no host sync).
//
// NeMo AutoModel cp_local_ring page: _fold_pad folds padding into the doc map
// as id 0; _cached_sliding_segments builds the segments once per step (the
// reference pays a device-to-host copy and Python pairing for it), with the
// straddling document's key start clipped at lo = max(0, S - L - W).
// blockdiag_cp.kernels page, _cp_blockdiag_varlen: one segment per document
// the local query rows touch; query part = its local rows, key part = document
// start .. last local row (bottom-right alignment), cu_seqlens_q[i] paired
// with cu_seqlens_k[i].
//
// One workgroup of 1024 threads walks the batch rows in order and each row in
// tiles of 8192 positions, carrying the running counts across tiles and rows,
// so segment indices are global and ordered by (row, position) without any
// host round trip.  Per position it needs the start of its run (a prefix max of
// run starts) and, at the last position of a run reaching the query shard, the
// running segment count, query-row count and key-length sum (prefix sums).
// Duplicate document ids across separate runs of a row are detected with an
// open-addressing set in the buffer's scratch area (status bit 0).
#include "nb_device.h"
#include "nb_kernels.h"

namespace nb {

namespace {
constexpr int SB_NT = 1024;
constexpr int SB_ITEMS = 8;
constexpr int SB_TILE = SB_NT * SB_ITEMS;
constexpr int SB_WAVES = SB_NT / 64;

// Exclusive block-wide scan (sum, or max when MX); `total` gets the block aggregate.
template <bool MX>
__device__ int block_excl_scan(int x, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int ident = MX ? INT_MIN : 0;
  int v = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d);
    if (lane >= d) v = MX ? max(v, y) : v + y;
  }
  if (lane == 63) sh[wid] = v;
  __syncthreads();
  if (wid == 0) {
    int t = lane < SB_WAVES ? sh[lane] : ident;
#pragma unroll
    for (int d = 1; d < SB_WAVES; d <<= 1) {
      const int y = __shfl_up(t, d);
      if (lane >= d) t = MX ? max(t, y) : t + y;
    }
    if (lane < SB_WAVES) sh[SB_WAVES + lane] = t;
  }
  __syncthreads();
  const int before_wave = wid ? sh[SB_WAVES + wid - 1] : ident;
  int before_lane = __shfl_up(v, 1);
  if (lane == 0) before_lane = ident;
  total = sh[2 * SB_WAVES - 1];
  __syncthreads();
  return MX ? max(before_wave, before_lane) : before_wave + before_lane;
}

__device__ __forceinline__ int folded_at(const SegParams& p, int b, int j) {
  const size_t x = (size_t)b * p.S + j;
  int v = p.doc_ids[x];
  if (p.pad_mask != nullptr && p.pad_mask[x] != 0) v = 0;
  return v;
}

// Insert a document id into the row's id set; returns true if it was present.
__device__ bool id_seen_before(int* table, int mask, int id) {
  uint32_t h = ((uint32_t)id * 2654435761u) & (uint32_t)mask;
  while (true) {
    const int old = atomicCAS(&table[h], 0, id);
    if (old == 0) return false;
    if (old == id) return true;
    h = (h + 1) & (uint32_t)mask;
  }
}
}  // namespace

__global__ __launch_bounds__(SB_NT) void segment_build_kernel(SegParams p) {
  __shared__ int sh[2 * SB_WAVES];
  const int S = p.S, L = p.L, off = S - L;
  const int lo = p.window >= 0 ? max(0, off - p.window) : 0;
  int32_t* __restrict__ seg = p.seg;
  int32_t* cu_q = seg + p.lay.cu_q;
  int32_t* cu_k = seg + p.lay.cu_k;
  int32_t* q_row0 = seg + p.lay.q_row0;
  int32_t* k_row0 = seg + p.lay.k_row0;
  int32_t* row_seg = seg + p.lay.row_seg;
  int32_t* row_klo = seg + p.lay.row_klo;
  int32_t* kcov_lo = seg + p.lay.kcov_lo;
  int* table = seg + p.lay.hash;
  const int hmask = p.lay.hash_size - 1;

  int n_seg = 0, cuq = 0, cuk = 0, maxq = 0, maxk = 0, dup = 0;
  if (threadIdx.x == 0) { cu_q[0] = 0; cu_k[0] = 0; }

  for (int b = 0; b < p.B; ++b) {
    for (int x = threadIdx.x; x < p.lay.hash_size; x += SB_NT) table[x] = 0;
    if (threadIdx.x == 0) kcov_lo[b] = S;
    __threadfence();
    __syncthreads();
    int carry_start = -1, row_nseg = 0, row_realq = 0, row_klen = 0;

    for (int t0 = 0; t0 < S; t0 += SB_TILE) {
      const int jb = t0 + threadIdx.x * SB_ITEMS;
      int f[SB_ITEMS];
#pragma unroll
      for (int u = 0; u < SB_ITEMS; ++u) f[u] = (jb + u < S) ? folded_at(p, b, jb + u) : 0;
      const int fprev = (jb > 0 && jb - 1 < S) ? folded_at(p, b, jb - 1) : 0;
      const int fnext = (jb + SB_ITEMS < S) ? folded_at(p, b, jb + SB_ITEMS) : 0;
#pragma unroll
      for (int u = 0; u < SB_ITEMS; ++u)
        if (jb + u < S) p.folded[(size_t)b * S + jb + u] = f[u];

      // pass 1: last run start among this thread's positions
      int my_last_start = -1;
#pragma unroll
      for (int u = 0; u < SB_ITEMS; ++u) {
        const int pv = u ? f[u - 1] : fprev;
        if (f[u] > 0 && pv != f[u]) my_last_start = jb + u;
      }
      int tile_last_start;
      const int start_before = max(carry_start, block_excl_scan<true>(my_last_start, sh, tile_last_start));

      // pass 2: per-thread counts of segment ends, real query rows, key lengths
      int n_end = 0, n_realq = 0, klen = 0, mq = 0, mk = 0;
      {
        int cur = start_before;
#pragma unroll
        for (int u = 0; u < SB_ITEMS; ++u) {
          const int j = jb + u;
          const int pv = u ? f[u - 1] : fprev;
          const int nx = (u + 1 < SB_ITEMS) ? f[u + 1] : fnext;
          if (f[u] > 0 && pv != f[u]) cur = j;
          if (f[u] > 0 && j >= off) ++n_realq;
          if (f[u] > 0 && nx != f[u] && j >= off) {
            ++n_end;
            const int ql = j + 1 - max(cur, off), kl = j + 1 - max(cur, lo);
            klen += kl;
            mq = max(mq, ql);
            mk = max(mk, kl);
          }
        }
      }
      int tot_end, tot_realq, tot_klen, tile_mq, tile_mk;
      const int end_before = block_excl_scan<false>(n_end, sh, tot_end);
      const int realq_before = block_excl_scan<false>(n_realq, sh, tot_realq);
      const int klen_before = block_excl_scan<false>(klen, sh, tot_klen);
      block_excl_scan<true>(mq, sh, tile_mq);
      block_excl_scan<true>(mk, sh, tile_mk);

      // pass 3: emit
      {
        int cur = start_before;
        int e_run = row_nseg + end_before;            // segments of this row ended before j
        int q_run = cuq + row_realq + realq_before;   // real query rows before j (all rows)
        int k_run = cuk + row_klen + klen_before;     // key lengths of segments before j
#pragma unroll
        for (int u = 0; u < SB_ITEMS; ++u) {
          const int j = jb + u;
          if (j >= S) break;
          const int pv = u ? f[u - 1] : fprev;
          const int nx = (u + 1 < SB_ITEMS) ? f[u + 1] : fnext;
          const bool doc = f[u] > 0;
          if (doc && pv != f[u]) {
            cur = j;
            if (id_seen_before(table, hmask, f[u])) dup = 1;
          }
          if (j >= off) {
            const int qi = (size_t)b * L + (j - off);
            row_seg[qi] = doc ? n_seg + e_run : -1;
            row_klo[qi] = doc ? max(cur, lo) : j + 1;
            if (doc) ++q_run;
          }
          if (doc && nx != f[u] && j >= off) {
            const int sid = n_seg + e_run;
            const int k0 = max(cur, lo);
            k_run += j + 1 - k0;
            cu_q[sid + 1] = q_run;
            cu_k[sid + 1] = k_run;
            q_row0[sid] = b * L + (max(cur, off) - off);
            k_row0[sid] = b * S + k0;
            if (e_run == 0) kcov_lo[b] = k0;
            ++e_run;
          }
        }
      }
      carry_start = max(carry_start, tile_last_start);
      row_nseg += tot_end;
      row_realq += tot_realq;
      row_klen += tot_klen;
      maxq = max(maxq, tile_mq);
      maxk = max(maxk, tile_mk);
    }
    n_seg += row_nseg;
    cuq += row_realq;
    cuk += row_klen;
    __syncthreads();
  }
  dup = __syncthreads_or(dup);
  if (threadIdx.x == 0) {
    seg[0] = n_seg;
    seg[1] = maxq;
    seg[2] = maxk;
    seg[3] = dup ? 1 : 0;
    seg[4] = lo;
    seg[5] = p.B;
    seg[6] = L;
    seg[7] = S;
    seg[8] = p.window;
    seg[9] = cuq;
    for (int x = 10; x < 16; ++x) seg[x] = 0;
  }
}

SegLayout seg_layout(int B, int L, int S) {
  SegLayout l;
  const size_t N = (size_t)B * L;
  l.cu_q = 16;
  l.cu_k = l.cu_q + N + 1;
  l.q_row0 = l.cu_k + N + 1;
  l.k_row0 = l.q_row0 + N;
  l.row_seg = l.k_row0 + N;
  l.row_klo = l.row_seg + N;
  l.kcov_lo = l.row_klo + N;
  size_t h = l.kcov_lo + B;
  h = (h + 63) & ~(size_t)63;
  l.hash = h;
  int hs = 64;
  while (hs < 2 * S) hs <<= 1;
  l.hash_size = hs;
  return l;
}

size_t seg_buffer_elems(int B, int L, int S) {
  const SegLayout l = seg_layout(B, L, S);
  return l.hash + (size_t)l.hash_size;
}

hipError_t launch_segment_build(const SegParams& p, hipStream_t s) {
  hipLaunchKernelGGL(segment_build_kernel, dim3(1), dim3(SB_NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace nb
