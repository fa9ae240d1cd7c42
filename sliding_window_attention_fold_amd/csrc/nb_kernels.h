// Internal launch interface between the C-ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nb {

struct SegLayout {
  size_t cu_q, cu_k, q_row0, k_row0, row_seg, row_klo, kcov_lo;
  size_t tiles;   // builder scratch: per-tile records
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

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  void* o_lo;        // optional: rounding residual of o (fp32 value minus stored value)
  float* lse;
  const int32_t* row_klo;
  int B, Hq, Hkv, L, S, window;
  float scale_log2;  // softmax scale * log2(e)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* o_lo;  // optional residual saved by the forward
  const void* dout;
  const float* lse;
  float* delta;
  int* order;        // workspace: dK/dV key tiles (b * n_tiles + tile) by decreasing work
  int* counters;     // workspace: kNumQueues work-queue counters of the backward kernel
  int* qorder;       // workspace: dQ query tiles (b * n_tiles + tile) by decreasing work
  const int32_t* row_klo;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, L, S, window;
  float scale;       // softmax scale
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

hipError_t launch_segment_build(const SegParams& p, hipStream_t s);
hipError_t launch_attn_fwd(const FwdParams& p, int D, bool f32, hipStream_t s);
// Backward launches: kBwdPrep = Delta + work orders; kBwdMain = both passes in
// one persistent grid (after kBwdPrep); kBwdDq = Delta + dQ pass; kBwdDkdv =
// dK/dV pass (after kBwdPrep or kBwdDq on the same workspace).
enum { kBwdPrep = 0, kBwdMain = 1, kBwdDq = 2, kBwdDkdv = 3 };
hipError_t launch_bwd(const BwdParams& p, int D, bool f32, int what, hipStream_t s);
// Elements of the dK/dV and dQ work-order arrays (enough for tiles of >= 32);
// the workspace also holds kNumQueues queue counters.
size_t dkdv_order_elems(int B, int S);
size_t dq_order_elems(int B, int L);
constexpr int kNumQueues = 8;
hipError_t launch_owner_flags(const OwnerParams& p, hipStream_t s);

}  // namespace nb
