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
// Two launches over tiles of 2048 positions of one batch row each:
//   1. stats (one workgroup per tile): fold the padding, write the folded ids,
//      clear the duplicate-id set, and reduce the tile to a few numbers -- its
//      last run start, its segment ends (ends at or after the shard start),
//      real query rows, and the key lengths / maxima of the segments whose run
//      starts inside the tile; a segment end whose run began in an earlier
//      tile (at most one per tile) is recorded by position;
//   2. emit (one workgroup per tile): first a scan of the tile records in
//      (row, tile) order -- the run start carried into the tile (a segmented
//      prefix max), the completed key lengths of the carried-in segments, and
//      exclusive prefix sums of segment ends, query rows and key lengths (the
//      owner of tile 0 writes the header) -- then per-position outputs and
//      per-segment cu_seqlens / row offsets from those prefixes plus in-tile
//      scans.
//      Run starts are inserted into an open-addressing set keyed by (row, id)
//      to detect an id that occurs in two separate runs (status bit 0);
//      The last emit workgroup of a batch row to finish then orders the row's
//      query tiles for the forward's launch, longest band first (scheduling
//      only: any order gives the same results).
// Segment indices are global and ordered by (row, position).
#include "../../include/nbattn.h"
#include "nb_device.h"
#include "nb_kernels.h"

namespace nb {

namespace {
constexpr int SB_NT = 256;
constexpr int SB_ITEMS = 8;
constexpr int SB_TILE = SB_NT * SB_ITEMS;
constexpr int SB_WAVES = SB_NT / 64;

// Exclusive block-wide scan (sum, or max when MX) over NT threads; `total`
// gets the block aggregate.  `sh` holds 2 * NT / 64 elements.
template <bool MX, int NT, typename V>
__device__ V block_excl_scan(V x, V* sh, V& total) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const V ident = MX ? (V)(sizeof(V) == 8 ? LLONG_MIN : INT_MIN) : (V)0;
  V v = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const V y = __shfl_up(v, d);
    if (lane >= d) v = MX ? max(v, y) : v + y;
  }
  if (lane == 63) sh[wid] = v;
  __syncthreads();
  if (wid == 0) {
    V t = lane < NWV ? sh[lane] : ident;
#pragma unroll
    for (int d = 1; d < NWV; d <<= 1) {
      const V y = __shfl_up(t, d);
      if (lane >= d) t = MX ? max(t, y) : t + y;
    }
    if (lane < NWV) sh[NWV + lane] = t;
  }
  __syncthreads();
  const V before_wave = wid ? sh[NWV + wid - 1] : ident;
  V before_lane = __shfl_up(v, 1);
  if (lane == 0) before_lane = ident;
  total = sh[2 * NWV - 1];
  __syncthreads();
  return MX ? max(before_wave, before_lane) : before_wave + before_lane;
}

__device__ __forceinline__ int folded_at(const SegParams& p, int b, int j) {
  const size_t x = (size_t)b * p.S + j;
  int v = p.doc_ids[x];
  if (p.pad_mask != nullptr && p.pad_mask[x] != 0) v = 0;
  return v;
}

// Insert (row, id) into the set; returns true if it was present.  Entries are
// (row + 1, id) pairs packed in 64 bits; 0 marks an empty slot.
__device__ bool id_seen_before(unsigned long long* table, uint32_t mask, int row, int id) {
  const unsigned long long key = ((unsigned long long)(unsigned)(row + 1) << 32) | (unsigned)id;
  uint32_t h = ((uint32_t)id * 2654435761u + (uint32_t)row * 40503u) & mask;
  while (true) {
    const unsigned long long old = atomicCAS(&table[h], 0ull, key);
    if (old == 0ull || old == key) return old == key;
    h = (h + 1) & (uint32_t)mask;
  }
}

// per-tile records in the scratch area (int32 each)
enum { T_LAST_START, T_N_END, T_N_REALQ, T_KLEN_INT, T_MQ_INT, T_MK_INT, T_EXT_END, T_STAT };
constexpr int kTileRec = 8;

// Per-thread view of its SB_ITEMS positions: folded ids plus both neighbours.
struct Span {
  int f[SB_ITEMS];
  int fprev, fnext, jb;
};

__device__ __forceinline__ void load_span(const SegParams& p, const int32_t* src, int b, int t0, Span& sp) {
  sp.jb = t0 + threadIdx.x * SB_ITEMS;
  const int32_t* row = src + (size_t)b * p.S;
#pragma unroll
  for (int u = 0; u < SB_ITEMS; ++u) sp.f[u] = (sp.jb + u < p.S) ? row[sp.jb + u] : 0;
  sp.fprev = (sp.jb > 0 && sp.jb - 1 < p.S) ? row[sp.jb - 1] : 0;
  sp.fnext = (sp.jb + SB_ITEMS < p.S) ? row[sp.jb + SB_ITEMS] : 0;
}
}  // namespace

__global__ __launch_bounds__(SB_NT) void seg_stats_kernel(SegParams p) {
  __shared__ int sh[2 * SB_WAVES];
  const int S = p.S, L = p.L, off = S - L;
  const int lo = p.window >= 0 ? max(0, off - p.window) : 0;
  const int T = (S + SB_TILE - 1) / SB_TILE;
  const int b = blockIdx.x / T, k = blockIdx.x % T;
  const int t0 = k * SB_TILE;
  int32_t* rec = p.seg + p.lay.tiles + (size_t)blockIdx.x * kTileRec;

  // fold the padding (doc ids -> folded ids), then work on the folded ids
  Span sp;
  sp.jb = t0 + threadIdx.x * SB_ITEMS;
#pragma unroll
  for (int u = 0; u < SB_ITEMS; ++u) sp.f[u] = (sp.jb + u < S) ? folded_at(p, b, sp.jb + u) : 0;
  sp.fprev = (sp.jb > 0 && sp.jb - 1 < S) ? folded_at(p, b, sp.jb - 1) : 0;
  sp.fnext = (sp.jb + SB_ITEMS < S) ? folded_at(p, b, sp.jb + SB_ITEMS) : 0;
#pragma unroll
  for (int u = 0; u < SB_ITEMS; ++u)
    if (sp.jb + u < S) p.folded[(size_t)b * S + sp.jb + u] = sp.f[u];

  // this workgroup's slice of the duplicate-id set
  unsigned long long* table = reinterpret_cast<unsigned long long*>(p.seg + p.lay.hash);
  for (size_t x = (size_t)blockIdx.x * SB_NT + threadIdx.x; x < p.lay.hash_size; x += (size_t)gridDim.x * SB_NT)
    table[x] = 0ull;
  if (k == 0 && threadIdx.x == 0) {
    p.seg[p.lay.kcov_lo + b] = S;
    p.seg[p.lay.done + b] = 0;   // emit workgroups of row b that have finished
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) p.seg[NB_HDR_STATUS] = 0;

  // run starts: the tile's last, and per thread the last one before it (in-tile)
  int my_last = -1;
#pragma unroll
  for (int u = 0; u < SB_ITEMS; ++u) {
    const int pv = u ? sp.f[u - 1] : sp.fprev;
    if (sp.f[u] > 0 && pv != sp.f[u]) my_last = sp.jb + u;
  }
  int tile_last;
  const int before = block_excl_scan<true, SB_NT>(my_last, sh, tile_last);

  // segment ends: those whose run starts in the tile are complete here; the
  // one (if any) whose run began in an earlier tile is left to the scan
  int n_end = 0, n_realq = 0, klen = 0, mq = 0, mk = 0, ext = -1;
  int cur = before;
#pragma unroll
  for (int u = 0; u < SB_ITEMS; ++u) {
    const int j = sp.jb + u;
    const int pv = u ? sp.f[u - 1] : sp.fprev;
    const int nx = (u + 1 < SB_ITEMS) ? sp.f[u + 1] : sp.fnext;
    if (j >= S) break;
    if (sp.f[u] > 0 && pv != sp.f[u]) cur = j;
    if (sp.f[u] > 0 && j >= off) ++n_realq;
    if (sp.f[u] > 0 && nx != sp.f[u] && j >= off) {
      ++n_end;
      if (cur >= 0) {
        const int ql = j + 1 - max(cur, off), kl = j + 1 - max(cur, lo);
        klen += kl;
        mq = max(mq, ql);
        mk = max(mk, kl);
      } else {
        ext = j;
      }
    }
  }
  int tot;
  block_excl_scan<false, SB_NT>(n_end, sh, tot);
  if (threadIdx.x == 0) rec[T_N_END] = tot;
  block_excl_scan<false, SB_NT>(n_realq, sh, tot);
  if (threadIdx.x == 0) rec[T_N_REALQ] = tot;
  block_excl_scan<false, SB_NT>(klen, sh, tot);
  if (threadIdx.x == 0) rec[T_KLEN_INT] = tot;
  block_excl_scan<true, SB_NT>(mq, sh, tot);
  if (threadIdx.x == 0) rec[T_MQ_INT] = tot;
  block_excl_scan<true, SB_NT>(mk, sh, tot);
  if (threadIdx.x == 0) rec[T_MK_INT] = tot;
  block_excl_scan<true, SB_NT>(ext, sh, tot);
  if (threadIdx.x == 0) {
    rec[T_EXT_END] = tot;
    rec[T_LAST_START] = tile_last;
  }
}

// Prefixes of tile `mine` from the records of all tiles, in (row, tile) order:
// the run start carried into it (segmented prefix max over its row), and the
// segment ends, real query rows and key lengths of all earlier tiles (the
// carried-in segment of each tile completed with its carried start).  Every
// emit workgroup runs this over the (few) tile records; the one that owns
// tile 0 also writes the header totals.
struct TilePrefix {
  int start_before, seg_before, q_before, k_before, row_seg0;
};

__device__ TilePrefix tile_prefix(const SegParams& p, int mine, bool write_header) {
  __shared__ long long shl[2 * SB_WAVES];
  __shared__ int shi[2 * SB_WAVES];
  __shared__ TilePrefix out;
  const int S = p.S, L = p.L, off = S - L;
  const int lo = p.window >= 0 ? max(0, off - p.window) : 0;
  const int T = (S + SB_TILE - 1) / SB_TILE;
  const int n = p.B * T;
  const int32_t* tiles = p.seg + p.lay.tiles;
  long long carry_key = LLONG_MIN, carry_rkey = LLONG_MIN;
  int carry_seg = 0, carry_q = 0, carry_k = 0, maxq = 0, maxk = 0;
  for (int c0 = 0; c0 < n; c0 += SB_NT) {
    const int i = c0 + threadIdx.x;
    const bool in = i < n;
    const int32_t* rec = tiles + (size_t)(in ? i : 0) * kTileRec;
    const int b = in ? i / T : 0;
    // segmented prefix max of run starts within the row: key (row, start + 1)
    const long long key = in ? (long long)b * ((long long)S + 1) + (rec[T_LAST_START] + 1) : LLONG_MIN;
    long long agg;
    const long long kb = max(carry_key, block_excl_scan<true, SB_NT>(key, shl, agg));
    const int sb = (in && kb >= (long long)b * ((long long)S + 1)) ? (int)(kb - (long long)b * ((long long)S + 1)) - 1 : -1;
    // complete the carried-in segment of the tile
    int klen = 0, mq = 0, mk = 0, n_end = 0, n_realq = 0;
    if (in) {
      n_end = rec[T_N_END];
      n_realq = rec[T_N_REALQ];
      klen = rec[T_KLEN_INT];
      mq = rec[T_MQ_INT];
      mk = rec[T_MK_INT];
      const int ext = rec[T_EXT_END];
      if (ext >= 0) {
        klen += ext + 1 - max(sb, lo);
        mq = max(mq, ext + 1 - max(sb, off));
        mk = max(mk, ext + 1 - max(sb, lo));
      }
    }
    int tot_seg, tot_q, tot_k, cmq, cmk;
    const int seg_before = carry_seg + block_excl_scan<false, SB_NT>(n_end, shi, tot_seg);
    const int q_before = carry_q + block_excl_scan<false, SB_NT>(n_realq, shi, tot_q);
    const int k_before = carry_k + block_excl_scan<false, SB_NT>(klen, shi, tot_k);
    block_excl_scan<true, SB_NT>(mq, shi, cmq);
    block_excl_scan<true, SB_NT>(mk, shi, cmk);
    // segments before the row's first tile: segmented max of (row, seg_before)
    // over the rows' first tiles
    const long long rkey = (in && i % T == 0) ? (long long)b * (1ll << 32) + seg_before : LLONG_MIN;
    long long ragg;
    const long long rk = max(carry_rkey, block_excl_scan<true, SB_NT>(rkey, shl, ragg));
    if (i == mine) {
      out.start_before = sb;
      out.seg_before = seg_before;
      out.q_before = q_before;
      out.k_before = k_before;
      out.row_seg0 = (i % T == 0) ? seg_before : (int)(rk & 0xFFFFFFFFll);
    }
    carry_key = max(carry_key, agg);
    carry_rkey = max(carry_rkey, ragg);
    carry_seg += tot_seg;
    carry_q += tot_q;
    carry_k += tot_k;
    maxq = max(maxq, cmq);
    maxk = max(maxk, cmk);
  }
  if (write_header && threadIdx.x == 0) {
    int32_t* seg = p.seg;
    seg[NB_HDR_NSEG] = carry_seg;
    seg[NB_HDR_MAXQ] = maxq;
    seg[NB_HDR_MAXK] = maxk;
    // NB_HDR_STATUS: cleared by the stats pass, set by the emit pass
    seg[NB_HDR_LO] = lo;
    seg[NB_HDR_B] = p.B;
    seg[NB_HDR_L] = L;
    seg[NB_HDR_S] = S;
    seg[NB_HDR_WINDOW] = p.window;
    seg[NB_HDR_NREAL] = carry_q;
    for (int x = 10; x < NB_SEG_HEADER; ++x) seg[x] = 0;
    seg[p.lay.cu_q] = 0;
    seg[p.lay.cu_k] = 0;
  }
  __syncthreads();
  return out;
}

// The forward's query tiles of batch row b by decreasing work (run by the
// last emit workgroup of the row, once all its row_klo are written).  A
// tile's work: the keys of each 32-row group's band union (the key tiles that
// group computes) plus those of the tile's union (the tiles its workgroup
// steps through).  Bands as the forward forms them for the neighbourhood
// call: row i at key position S - L + i, [max(row_klo, p - W), p].  The
// hardware starts workgroups in grid order as slots free up, so launching the
// long tiles first keeps short ones for the end (list scheduling, longest
// first).
__device__ void fwd_order_row(const SegParams& p, int b) {
  static_assert(kFwdOrderRows % 64 == 0 && SB_NT % 64 == 0, "a wave's 64 rows lie in one tile");
  __shared__ unsigned long long keys[kFwdOrderMax];
  __shared__ int t_lo[kFwdOrderMax], t_hi[kFwdOrderMax];   // the tile's union
  __shared__ unsigned t_work[kFwdOrderMax];                 // sum of its groups' spans
  const int tid = threadIdx.x;
  const int nq = (p.L + kFwdOrderRows - 1) / kFwdOrderRows;
  int32_t* out = p.seg + p.lay.fwd_order + (size_t)b * nq;
  const int32_t* klo = p.seg + p.lay.row_klo + (size_t)b * p.L;
  if (nq > kFwdOrderMax) {
    for (int t = tid; t < nq; t += SB_NT) out[t] = t;
    return;
  }
  for (int t = tid; t < nq; t += SB_NT) {
    t_lo[t] = INT_MAX;
    t_hi[t] = INT_MIN;
    t_work[t] = 0u;
  }
  __syncthreads();
  // One 32-row group per thread and pass: its 32 band starts are loaded
  // together (one load latency), then the group's union [lo, hi) over its
  // real rows goes into its tile's sums.
  const int ng = (p.L + 31) / 32;
  for (int gi = tid; gi < ng; gi += SB_NT) {
    const int i0 = 32 * gi;
    int kl[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) kl[r] = i0 + r < p.L ? klo[i0 + r] : 0;
    int lo = INT_MAX, hi = INT_MIN;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int pq = p.S - p.L + i0 + r;
      int bs = max(0, kl[r]);
      if (p.window >= 0) bs = max(bs, pq - p.window);
      if (i0 + r < p.L && bs <= pq) {
        lo = min(lo, bs);
        hi = max(hi, pq + 1);
      }
    }
    if (lo < hi) {
      const int t = i0 / kFwdOrderRows;
      atomicAdd(&t_work[t], (unsigned)(hi - lo));
      atomicMin(&t_lo[t], lo);
      atomicMax(&t_hi[t], hi);
    }
  }
  __syncthreads();
  int N = 1;
  while (N < nq) N <<= 1;
  for (int t = tid; t < N; t += SB_NT) {
    unsigned long long key = ~0ull;   // padding sorts last
    if (t < nq) {
      unsigned work = t_work[t];
      if (t_lo[t] < t_hi[t]) work += (unsigned)(t_hi[t] - t_lo[t]);
      key = work_key(work, t, nq);
    }
    keys[t] = key;
  }
  if (nq <= SB_NT) {
    // one tile per thread: its rank is the number of smaller keys (the keys
    // are distinct), the same order the sort below gives
    __syncthreads();
    if (tid < nq) {
      const unsigned long long k = keys[tid];
      int rank = 0;
      for (int u = 0; u < nq; ++u) rank += keys[u] < k ? 1 : 0;
      out[rank] = tid;
    }
    return;
  }
  order_by_work<SB_NT>(keys, nq, N, out);
}

__global__ __launch_bounds__(SB_NT) void seg_emit_kernel(SegParams p) {
  __shared__ int sh[2 * SB_WAVES];
  const int S = p.S, L = p.L, off = S - L;
  const int lo = p.window >= 0 ? max(0, off - p.window) : 0;
  const int T = (S + SB_TILE - 1) / SB_TILE;
  const int b = blockIdx.x / T, k = blockIdx.x % T;
  const TilePrefix tp = tile_prefix(p, blockIdx.x, blockIdx.x == 0);
  const int start_before = tp.start_before, seg_before = tp.seg_before;
  const int q_before = tp.q_before, k_before = tp.k_before, row_seg0 = tp.row_seg0;
  int32_t* seg = p.seg;
  int32_t* cu_q = seg + p.lay.cu_q;
  int32_t* cu_k = seg + p.lay.cu_k;
  int32_t* q_row0 = seg + p.lay.q_row0;
  int32_t* k_row0 = seg + p.lay.k_row0;
  int32_t* row_seg = seg + p.lay.row_seg;
  int32_t* row_klo = seg + p.lay.row_klo;
  int32_t* kcov_lo = seg + p.lay.kcov_lo;
  unsigned long long* table = reinterpret_cast<unsigned long long*>(seg + p.lay.hash);
  const uint32_t hmask = (uint32_t)(p.lay.hash_size - 1);

  Span sp;
  load_span(p, p.folded, b, k * SB_TILE, sp);

  int my_last = -1;
#pragma unroll
  for (int u = 0; u < SB_ITEMS; ++u) {
    const int pv = u ? sp.f[u - 1] : sp.fprev;
    if (sp.f[u] > 0 && pv != sp.f[u]) my_last = sp.jb + u;
  }
  int tmp;
  const int before = max(start_before, block_excl_scan<true, SB_NT>(my_last, sh, tmp));
  int n_end = 0, n_realq = 0, klen = 0;
  {
    int cur = before;
#pragma unroll
    for (int u = 0; u < SB_ITEMS; ++u) {
      const int j = sp.jb + u;
      if (j >= S) break;
      const int pv = u ? sp.f[u - 1] : sp.fprev;
      const int nx = (u + 1 < SB_ITEMS) ? sp.f[u + 1] : sp.fnext;
      if (sp.f[u] > 0 && pv != sp.f[u]) cur = j;
      if (sp.f[u] > 0 && j >= off) ++n_realq;
      if (sp.f[u] > 0 && nx != sp.f[u] && j >= off) {
        ++n_end;
        klen += j + 1 - max(cur, lo);
      }
    }
  }
  int e_run = seg_before + block_excl_scan<false, SB_NT>(n_end, sh, tmp);
  int q_run = q_before + block_excl_scan<false, SB_NT>(n_realq, sh, tmp);
  int k_run = k_before + block_excl_scan<false, SB_NT>(klen, sh, tmp);
  int dup = 0;
  int cur = before;
#pragma unroll
  for (int u = 0; u < SB_ITEMS; ++u) {
    const int j = sp.jb + u;
    if (j >= S) break;
    const int pv = u ? sp.f[u - 1] : sp.fprev;
    const int nx = (u + 1 < SB_ITEMS) ? sp.f[u + 1] : sp.fnext;
    const bool doc = sp.f[u] > 0;
    if (doc && pv != sp.f[u]) {
      cur = j;
      if (id_seen_before(table, hmask, b, sp.f[u])) dup = 1;
    }
    if (j >= off) {
      const int qi = b * L + (j - off);   // < B * L since off <= j < S
      row_seg[qi] = doc ? e_run : -1;
      row_klo[qi] = doc ? max(cur, lo) : j + 1;
      if (doc) ++q_run;
    }
    if (doc && nx != sp.f[u] && j >= off && e_run < p.B * L) {   // (every segment owns >= 1 query row)
      const int k0 = max(cur, lo);
      k_run += j + 1 - k0;
      cu_q[e_run + 1] = q_run;
      cu_k[e_run + 1] = k_run;
      q_row0[e_run] = b * L + (max(cur, off) - off);
      k_row0[e_run] = b * S + k0;
      if (e_run == row_seg0) kcov_lo[b] = k0;
      ++e_run;
    }
  }
  if (__syncthreads_or(dup) && threadIdx.x == 0) atomicOr(seg + NB_HDR_STATUS, NB_SEG_STATUS_SPLIT_DOC);

  // The last of the row's T workgroups to finish orders its forward tiles:
  // each publishes its writes (fence) before its count; the last one fences
  // again before it reads the others' row_klo.
  __shared__ int last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(seg + p.lay.done + b, 1) == T - 1;
  __syncthreads();
  if (last) {
    __threadfence();
    fwd_order_row(p, b);
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
  l.fwd_order = (l.kcov_lo + B + 15) & ~(size_t)15;
  size_t t = l.fwd_order + (size_t)B * ((L + kFwdOrderRows - 1) / kFwdOrderRows);
  t = (t + 63) & ~(size_t)63;
  l.tiles = t;
  const size_t n_tiles = (size_t)B * ((S + SB_TILE - 1) / SB_TILE);
  l.done = l.tiles + n_tiles * kTileRec;
  size_t h = l.done + (size_t)B;
  h = (h + 63) & ~(size_t)63;   // 8-byte set entries, 256-byte aligned
  l.hash = h;
  size_t hs = 64;
  while (hs < 2 * (size_t)B * (size_t)S) hs <<= 1;
  l.hash_size = hs;
  return l;
}

size_t seg_buffer_elems(int B, int L, int S) {
  const SegLayout l = seg_layout(B, L, S);
  return l.hash + 2 * (size_t)l.hash_size;
}

hipError_t launch_segment_build(const SegParams& p, hipStream_t s) {
  const unsigned n_tiles = (unsigned)(p.B * ((p.S + SB_TILE - 1) / SB_TILE));
  hipLaunchKernelGGL(seg_stats_kernel, dim3(n_tiles), dim3(SB_NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seg_emit_kernel, dim3(n_tiles), dim3(SB_NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace nb
