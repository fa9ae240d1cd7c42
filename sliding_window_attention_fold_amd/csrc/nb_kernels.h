// Internal launch interface between the C-ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nb {

// The forward's query tiles: kFwdOrderRows rows of one (batch row, q head).
// The segment builder orders each batch row's tiles by decreasing band work
// (fwd_order, B * ceil(L / kFwdOrderRows) entries) when there are at most
// kFwdOrderMax of them, else writes the identity.
constexpr int kFwdOrderRows = 128;
constexpr int kFwdOrderMax = 2048;

struct SegLayout {
  size_t cu_q, cu_k, q_row0, k_row0, row_seg, row_klo, kcov_lo;
  size_t fwd_order;
  size_t tiles;   // builder scratch: per-tile records
  size_t done;    // builder scratch: per batch row, emit workgroups finished
  size_t hash;    // builder scratch: (row, id) set, hash_size 8-byte entries
  size_t hash_size;  // power of two >= 2 * B * S
};

SegLayout seg_layout(int B, int L, int S);
size_t seg_buffer_elems(int B, int L, int S);

struct SegParams {
  const int32_t* doc_ids;
  const uint8_t* pad_mask;
  int32_t* folded;
  int32_t* seg;
  SegLayout lay;
  int B, S, L, window;
};

// K/V of the neighbourhood as a table of per-chunk buffers (no concatenated
// copy): neighbourhood keys [off[c], off[c+1]) are rows start[c] .. of chunk c's
// buffers K, V (and dK, dV) [B, Hkv, rows[c], D].  One chunk with start 0 and
// rows S is the concatenated neighbourhood.
constexpr int kMaxKvChunks = 16;
// How a kernel variant finds K/V rows (template argument): one concatenated
// buffer; the chunk table for work whose key range touches at most two chunks
// (scalar bases, see KvPair); the chunk table for any key range (a lookup per
// tile, for the rare ranges over three or more chunks).
constexpr int kKvConcat = 0, kKvPair = 1, kKvAny = 2;
struct KvChunks {
  int n;
  int off[kMaxKvChunks + 1];
  int start[kMaxKvChunks];
  int rows[kMaxKvChunks];
  const void* k[kMaxKvChunks];
  const void* v[kMaxKvChunks];
  void* dk[kMaxKvChunks];
  void* dv[kMaxKvChunks];
};

// Chunk of neighbourhood key j (0 <= j < S) and the index of its row (batch b,
// kv head: bh = b * Hkv + h) in that chunk's buffers, counted in rows.  One pass over
// the chunks with uniform indices, so per-lane keys need no indexed loads.
__device__ __forceinline__ int kv_locate(const KvChunks& c, int bh, int j, size_t* row) {
  int x = 0;
  size_t r = (size_t)bh * c.rows[0] + c.start[0] + j;
  for (int y = 1; y < c.n; ++y) {
    if (j >= c.off[y]) {
      x = y;
      r = (size_t)bh * c.rows[y] + c.start[y] + (j - c.off[y]);
    }
  }
  *row = r;
  return x;
}

struct FwdParams {
  const void* q;
  KvChunks kv;
  void* o;
  void* o_lo;        // optional (bf16): rounding residual codes of o, one byte per element (nb_device.h: resid_code)
  float* lse;
  const int32_t* row_klo;
  // Optional (null: grid order): per batch row, its query tiles in the order
  // to launch them (longest first; the segment builder's fwd_order).
  const int32_t* qt_order;
  int B, Hq, Hkv, L, S, window;
  // Query row i sits at key position q_off + i; row_klo values count keys from
  // k_origin.  Neighbourhood attention: q_off = S - L, k_origin = 0.  A ring
  // chunk: row_klo in global positions, k_origin = the chunk's first global
  // position, q_off = the shard's first global position - k_origin (>= S for
  // an earlier owner's chunk, whose keys then all precede the queries).
  int q_off, k_origin;
  float scale_log2;  // softmax scale * log2(e)
};

constexpr int kMaxOwners = 64;
struct OwnerParams {
  const int32_t* folded;
  const int32_t* kcov_lo;
  uint8_t* attended;
  int B, S, n_owner;
  int off[kMaxOwners + 1];
};

struct BwdParams {
  const void* q;
  KvChunks kv;       // K, V read and dK, dV written through the chunk table
  const void* o;
  const void* o_lo;  // optional residual codes saved by the forward (bf16; ignored for float32)
  const void* dout;
  const float* lse;
  float* delta;
  int* order;        // workspace: dK/dV key tiles (b * n_tiles + tile) by decreasing work
  int* counters;     // workspace: kNumCounters counters (work queues, deferred dQ items)
  int* qorder;       // workspace: dQ query tiles (b * n_tiles + tile) by decreasing work
  int* cross;        // workspace: dQ items deferred by the chunk-table backward
  const int32_t* row_klo;
  void* dq;
  int B, Hq, Hkv, L, S, window;
  int q_off, k_origin;   // as in FwdParams
  int dq_mode;       // kDqStore: dq is T, written; kDqSetF32 / kDqAddF32: dq is fp32, set / added to
  // Optional banded dS (windowed neighbourhoods): per (batch row, q head,
  // 32-row query tile) ds_w / 32 blocks of 32 rows x 32 keys (row-major T), the
  // tile's keys from its first row's band start rounded down to 32.  Within a
  // row, key k of the block sits at k with bits 2 and 3 swapped (ds_slot), so
  // the eight keys one lane feeds to a 32x32x16 product are contiguous.  Non-null:
  // the dK/dV items store dS there and dQ = dS K runs as a separate pass
  // instead of the dQ items.
  void* dsbuf;
  int ds_w;
  int ds_bytes;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  // Optional (n_owner > 0): the owners' attended flags, computed by extra
  // workgroups of the prep kernel (they depend on the segments alone).
  OwnerParams own;
};


hipError_t launch_segment_build(const SegParams& p, hipStream_t s);

// Compute units of the current device (sizes persistent grids; decides
// whether a grid runs in one round).
inline int device_cu_count() {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
    n_cu = 256;
  return n_cu;
}
hipError_t launch_attn_fwd(const FwdParams& p, int D, bool f32, hipStream_t s);
// Backward launches: kBwdPrep = Delta + work orders; kBwdMain = both passes in
// one persistent grid (after kBwdPrep); kBwdDq = Delta + dQ pass; kBwdDkdv =
// dK/dV pass (after kBwdPrep or kBwdDq on the same workspace); kBwdOrders =
// the work orders alone (Delta left in the workspace by an earlier kBwdPrep).
enum { kBwdPrep = 0, kBwdMain = 1, kBwdDq = 2, kBwdDkdv = 3, kBwdOrders = 4 };
enum { kDqStore = 0, kDqSetF32 = 1, kDqAddF32 = 2 };
hipError_t launch_bwd(const BwdParams& p, int D, bool f32, int what, hipStream_t s);
// Zeros the dK/dV rows of the chunk buffers that lie outside the neighbourhood.
hipError_t launch_kv_zero_outside(const KvChunks& c, int BH, int row_bytes, hipStream_t s);
// Elements of the dK/dV and dQ work-order arrays and of the deferred dQ item
// list (enough for tiles of >= 32); the workspace also holds kNumCounters
// counters: the kNumQueues work queues of the backward kernel, then the length
// of the deferred list and the follow-up kernel's position in it.
size_t dkdv_order_elems(int B, int S);
size_t dq_order_elems(int B, int L);
size_t dq_cross_elems(int B, int Hq, int L);
constexpr int kNumQueues = 8;
constexpr int kCrossCount = kNumQueues, kCrossNext = kNumQueues + 1, kNumCounters = kNumQueues + 2;
hipError_t launch_owner_flags(const OwnerParams& p, hipStream_t s);

}  // namespace nb
