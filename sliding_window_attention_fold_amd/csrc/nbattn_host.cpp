// C-ABI of nbattn: argument checks before any launch, then dispatch to the HIP
// kernels on the caller's stream.  Nothing here allocates or synchronises
// (except the debug header read).
//
// The checks mirror blockdiag_cp.kernels page, _varlen_backend_unavailable_reason
// and _varlen_metadata_unavailable_reason (NeMo AutoModel): every reason a
// kernel cannot run is found on the host without launching anything, and the
// varlen metadata the kernels index with is produced on the device by the
// segment builder, valid by construction, instead of being validated with a
// device-to-host copy.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/nbattn.h"
#include "../../include/nbring.h"
#include "nb_kernels.h"

namespace {

constexpr int64_t kMaxIndex = (int64_t)1 << 30;  // positions and row counts stay in int32 math

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dims_ok(int B, int L, int S) {
  if (B < 1 || L < 1 || S < 1 || L > S) return false;
  if (B > 65535) return false;
  if ((int64_t)B * S >= kMaxIndex || (int64_t)S >= kMaxIndex) return false;
  return true;
}

int map_hip(hipError_t e) {
  if (e == hipSuccess) return NB_OK;
  if (e == hipErrorNoDevice || e == hipErrorInvalidDevice || e == hipErrorNoBinaryForGpu) return NB_ERR_DEVICE;
  return NB_ERR_LAUNCH;
}

// allow512: head dim 512 (the global layers) is accepted -- by the ring chunk
// entry points only, whose backward takes the stored-dS form it requires.
int attn_common_checks(const void* const* ptrs, int nptrs, int B, int Hq, int Hkv, int L, int S, int D,
                       float scale, int dtype, bool allow512 = false) {
  for (int x = 0; x < nptrs; ++x)
    if (ptrs[x] == nullptr || !aligned16(ptrs[x])) return NB_ERR_INVALID_ARG;
  if (!dims_ok(B, L, S)) return NB_ERR_INVALID_ARG;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hq > 65535) return NB_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !std::isfinite(scale)) return NB_ERR_INVALID_ARG;
  if (dtype != NB_BF16 && dtype != NB_F32) return NB_ERR_UNSUPPORTED;
  if (D != 64 && D != 128 && D != 256 && !(allow512 && D == 512)) return NB_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq * L >= kMaxIndex * 2 || (int64_t)B * Hkv * S >= kMaxIndex * 2) return NB_ERR_INVALID_ARG;
  return NB_OK;
}

// The concatenated neighbourhood as a one-chunk table.
nb::KvChunks one_chunk(int S, const void* k, const void* v, void* dk, void* dv) {
  nb::KvChunks c;
  std::memset(&c, 0, sizeof(c));
  c.n = 1;
  c.off[0] = 0;
  c.off[1] = S;
  c.start[0] = 0;
  c.rows[0] = S;
  c.k[0] = k;
  c.v[0] = v;
  c.dk[0] = dk;
  c.dv[0] = dv;
  return c;
}

// A caller's chunk table: n chunks of len[c] keys starting at row start[c] of
// buffers with rows[c] rows per (batch, kv head); S = sum of len.
int chunk_table(const void* const* k, const void* const* v, void* const* dk, void* const* dv, const int32_t* len,
                const int32_t* start, const int32_t* rows, int n, int B, int Hkv, int S, nb::KvChunks* out) {
  if (n < 1 || n > nb::kMaxKvChunks || len == nullptr || start == nullptr || rows == nullptr) return NB_ERR_INVALID_ARG;
  if (k == nullptr || v == nullptr) return NB_ERR_INVALID_ARG;
  nb::KvChunks c;
  std::memset(&c, 0, sizeof(c));
  c.n = n;
  int64_t acc = 0;
  for (int x = 0; x < n; ++x) {
    if (len[x] < 1 || start[x] < 0 || rows[x] < 1 || (int64_t)start[x] + len[x] > rows[x]) return NB_ERR_INVALID_ARG;
    if ((int64_t)B * Hkv * rows[x] >= kMaxIndex * 2) return NB_ERR_INVALID_ARG;
    if (k[x] == nullptr || v[x] == nullptr || !aligned16(k[x]) || !aligned16(v[x])) return NB_ERR_INVALID_ARG;
    if (dk != nullptr && (dk[x] == nullptr || !aligned16(dk[x]))) return NB_ERR_INVALID_ARG;
    if (dv != nullptr && (dv[x] == nullptr || !aligned16(dv[x]))) return NB_ERR_INVALID_ARG;
    c.off[x] = (int)acc;
    c.start[x] = start[x];
    c.rows[x] = rows[x];
    c.k[x] = k[x];
    c.v[x] = v[x];
    c.dk[x] = dk ? dk[x] : nullptr;
    c.dv[x] = dv ? dv[x] : nullptr;
    acc += len[x];
  }
  if (acc != S) return NB_ERR_INVALID_ARG;
  c.off[n] = S;
  *out = c;
  return NB_OK;
}

}  // namespace

extern "C" {

const char* nb_status_string(int status) {
  switch (status) {
    case NB_OK: return "ok";
    case NB_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or shape)";
    case NB_ERR_UNSUPPORTED:
      return "unsupported (head dim not in {64,128,256} -- 512 on the ring chunk calls --, unknown dtype, or dropout)";
    case NB_ERR_WORKSPACE: return "workspace or segment buffer too small";
    case NB_ERR_LAUNCH: return "HIP kernel launch failed";
    case NB_ERR_DEVICE: return "no usable gfx950 device";
    default: return "unknown status";
  }
}

int nb_version(void) { return 100; }

size_t nb_segment_offset_cu_q(int B, int L) { return nb::seg_layout(B, L, 1).cu_q; }
size_t nb_segment_offset_cu_k(int B, int L) { return nb::seg_layout(B, L, 1).cu_k; }
size_t nb_segment_offset_q_row0(int B, int L) { return nb::seg_layout(B, L, 1).q_row0; }
size_t nb_segment_offset_k_row0(int B, int L) { return nb::seg_layout(B, L, 1).k_row0; }
size_t nb_segment_offset_row_seg(int B, int L) { return nb::seg_layout(B, L, 1).row_seg; }
size_t nb_segment_offset_row_klo(int B, int L) { return nb::seg_layout(B, L, 1).row_klo; }
size_t nb_segment_offset_kcov_lo(int B, int L) { return nb::seg_layout(B, L, 1).kcov_lo; }
size_t nb_segment_offset_fwd_order(int B, int L) { return nb::seg_layout(B, L, 1).fwd_order; }

size_t nb_segment_buffer_elems(int B, int L, int S) {
  if (!dims_ok(B, L, S)) return 0;
  return nb::seg_buffer_elems(B, L, S);
}

int nb_segment_build(const int32_t* doc_ids, const uint8_t* pad_mask, int B, int S, int L, int window_left,
                     int32_t* folded_ids, int32_t* seg_buf, size_t seg_buf_elems, void* stream) {
  if (doc_ids == nullptr || folded_ids == nullptr || seg_buf == nullptr) return NB_ERR_INVALID_ARG;
  if (!aligned16(seg_buf)) return NB_ERR_INVALID_ARG;
  if (!dims_ok(B, L, S)) return NB_ERR_INVALID_ARG;
  if (seg_buf_elems < nb::seg_buffer_elems(B, L, S)) return NB_ERR_WORKSPACE;
  nb::SegParams p;
  p.doc_ids = doc_ids;
  p.pad_mask = pad_mask;
  p.folded = folded_ids;
  p.seg = seg_buf;
  p.lay = nb::seg_layout(B, L, S);
  p.B = B;
  p.S = S;
  p.L = L;
  p.window = window_left < 0 ? -1 : window_left;
  return map_hip(nb::launch_segment_build(p, (hipStream_t)stream));
}

int nb_segment_header(const int32_t* seg_buf, int32_t* host_header, void* stream) {
  if (seg_buf == nullptr || host_header == nullptr) return NB_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(host_header, seg_buf, NB_SEG_HEADER * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return map_hip(e);
}

size_t nb_attn_fwd_workspace_bytes(int, int, int, int, int, int, int) { return 0; }

}  // extern "C"

namespace {

// q_off / k_origin: see FwdParams (the neighbourhood call: S - L and 0).
int attn_fwd_kv(const void* q, const nb::KvChunks& kv, void* o, void* o_resid, float* lse, const int32_t* seg_buf,
                int B, int Hq, int Hkv, int L, int S, int D, float scale, int window_left, float dropout_p, int dtype,
                void* stream, int q_off = -1, int k_origin = 0) {
  if (o_resid != nullptr && !aligned16(o_resid)) return NB_ERR_INVALID_ARG;
  if (dropout_p != 0.f) return NB_ERR_UNSUPPORTED;
  nb::FwdParams p;
  p.q = q;
  p.kv = kv;
  p.o = o;
  p.o_lo = o_resid;
  p.lse = lse;
  const nb::SegLayout lay = nb::seg_layout(B, L, S);
  p.row_klo = seg_buf + lay.row_klo;
  // the builder's launch order is for the neighbourhood geometry (q_off < 0)
  p.qt_order = q_off < 0 ? seg_buf + lay.fwd_order : nullptr;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.L = L;
  p.S = S;
  p.window = window_left < 0 ? -1 : window_left;
  p.q_off = q_off < 0 ? S - L : q_off;
  p.k_origin = k_origin;
  p.scale_log2 = scale * 1.4426950408889634f;
  return map_hip(nb::launch_attn_fwd(p, D, dtype == NB_F32, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int nb_attn_fwd(const void* q, const void* k, const void* v, void* o, void* o_resid, float* lse, const int32_t* seg_buf, int B,
                int Hq, int Hkv, int L, int S, int D, float scale, int window_left, float dropout_p, int dtype,
                void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  const void* ptrs[] = {q, k, v, o, lse, seg_buf};
  int st = attn_common_checks(ptrs, 6, B, Hq, Hkv, L, S, D, scale, dtype);
  if (st != NB_OK) return st;
  return attn_fwd_kv(q, one_chunk(S, k, v, nullptr, nullptr), o, o_resid, lse, seg_buf, B, Hq, Hkv, L, S, D, scale,
                     window_left, dropout_p, dtype, stream);
}

int nb_attn_fwd_chunks(const void* q, const void* const* k_chunk, const void* const* v_chunk,
                       const int32_t* chunk_len, const int32_t* chunk_start, const int32_t* chunk_rows, int n_chunk,
                       void* o, void* o_resid, float* lse, const int32_t* seg_buf, int B, int Hq, int Hkv, int L,
                       int S, int D, float scale, int window_left, float dropout_p, int dtype, void* ws,
                       size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  const void* ptrs[] = {q, o, lse, seg_buf};
  int st = attn_common_checks(ptrs, 4, B, Hq, Hkv, L, S, D, scale, dtype);
  if (st != NB_OK) return st;
  nb::KvChunks kv;
  st = chunk_table(k_chunk, v_chunk, nullptr, nullptr, chunk_len, chunk_start, chunk_rows, n_chunk, B, Hkv, S, &kv);
  if (st != NB_OK) return st;
  return attn_fwd_kv(q, kv, o, o_resid, lse, seg_buf, B, Hq, Hkv, L, S, D, scale, window_left, dropout_p, dtype,
                     stream);
}

namespace {
size_t delta_bytes(int B, int Hq, int L) { return (((size_t)B * Hq * L * sizeof(float)) + 255) & ~(size_t)255; }
// dK/dV work order, the backward kernel's counters, dQ work order, deferred dQ items
size_t order_bytes(int B, int Hq, int L, int S) {
  return ((nb::dkdv_order_elems(B, S) + nb::kNumCounters + nb::dq_order_elems(B, L) +
           nb::dq_cross_elems(B, Hq, L)) * sizeof(int) + 255) & ~(size_t)255;
}
}  // namespace

size_t nb_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int S, int D, int dtype) {
  (void)Hkv;
  (void)D;
  (void)dtype;
  if (B < 1 || Hq < 1 || L < 1 || S < 1) return 0;
  return delta_bytes(B, Hq, L) + order_bytes(B, Hq, L, S);
}

}  // extern "C"

namespace {
// The banded dS of the windowed backward: row width (keys) and bytes; 0 when
// the window is absent or too wide for the buffer to pay, or at head dims
// below 256, where the dQ items that recompute S and dP measured faster (their
// dK/dV steps have no spare registers for the stores' bookkeeping there either).
constexpr int kMaxDsWindow = 4096;
// Keys per 32-row tile of the banded dS buffer when no row's band is wider
// than `span` keys: the first row's band start rounded down to 32, then up to
// the last row's position, 31 rows further.
int ds_width(int span) { return (span + 96 + 31) / 32 * 32; }
size_t ds_bytes_span(int B, int Hq, int L, int D, int span, int dtype) {
  if ((D != 256 && D != 512) || span < 0 || B < 1 || Hq < 1 || L < 1) return 0;
  const size_t n = ((size_t)B * Hq * ((L + 31) / 32 * 32) * ds_width(span) * (dtype == NB_F32 ? 4 : 2) + 255) &
                   ~(size_t)255;
  return n < ((size_t)1 << 31) ? n : 0;   // buffer offsets stay in 31 bits
}
size_t ds_bytes(int B, int Hq, int L, int D, int window, int dtype) {
  return (window > kMaxDsWindow || D != 256) ? 0 : ds_bytes_span(B, Hq, L, D, window, dtype);
}
// Turns the stored-dS backward on when the workspace holds the buffer.
void enable_ds(nb::BwdParams& p, void* ws, size_t ws_bytes, int B, int Hq, int Hkv, int L, int S, int D,
               int window_left, int dtype) {
  const size_t base = nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dtype);
  const size_t db = ds_bytes(B, Hq, L, D, window_left, dtype);
  if (db == 0 || ws_bytes < base + db) return;
  p.dsbuf = reinterpret_cast<char*>(ws) + base;
  p.ds_w = ds_width(window_left);
  p.ds_bytes = (int)db;
}
}  // namespace

extern "C" {

size_t nb_attn_bwd_workspace_bytes_window(int B, int Hq, int Hkv, int L, int S, int D, int dtype, int window_left) {
  const size_t base = nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dtype);
  return base == 0 ? 0 : base + ds_bytes(B, Hq, L, D, window_left, dtype);
}

size_t nb_ring_chunk_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int Lk, int D, int dtype) {
  const size_t base = nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, Lk, D, dtype);
  return base == 0 ? 0 : base + ds_bytes_span(B, Hq, L, D, Lk, dtype);
}

}  // extern "C"

namespace {

nb::BwdParams bwd_params(const void* dout, const void* q, const nb::KvChunks& kv, const void* o,
                         const void* o_resid, const float* lse, const int32_t* seg_buf, int B, int Hq, int Hkv,
                         int L, int S, float scale, int window_left, void* dq, void* ws, int q_off = -1,
                         int k_origin = 0) {
  nb::BwdParams p;
  p.q = q;
  p.kv = kv;
  p.o = o;
  p.o_lo = o_resid;
  p.dout = dout;
  p.lse = lse;
  p.delta = reinterpret_cast<float*>(ws);
  p.order = reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + delta_bytes(B, Hq, L));
  p.counters = p.order + nb::dkdv_order_elems(B, S);
  p.qorder = p.counters + nb::kNumCounters;
  p.cross = p.qorder + nb::dq_order_elems(B, L);
  p.row_klo = seg_buf + nb::seg_layout(B, L, S).row_klo;
  p.dq = dq;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.L = L;
  p.S = S;
  p.window = window_left < 0 ? -1 : window_left;
  p.q_off = q_off < 0 ? S - L : q_off;
  p.k_origin = k_origin;
  p.dq_mode = nb::kDqStore;
  p.dsbuf = nullptr;
  p.ds_w = 0;
  p.ds_bytes = 0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  std::memset(&p.own, 0, sizeof(p.own));   // no owner flags unless an entry point asks
  return p;
}

int owner_checks(const int32_t* folded_ids, int S, const int32_t* owner_off, int n_owner,
                 const uint8_t* owner_attended) {
  if (n_owner < 0 || n_owner > nb::kMaxOwners) return NB_ERR_INVALID_ARG;
  if (n_owner == 0) return NB_OK;
  if (owner_off == nullptr || owner_attended == nullptr || folded_ids == nullptr) return NB_ERR_INVALID_ARG;
  if (owner_off[0] != 0 || owner_off[n_owner] != S) return NB_ERR_INVALID_ARG;
  for (int x = 0; x < n_owner; ++x)
    if (owner_off[x + 1] < owner_off[x]) return NB_ERR_INVALID_ARG;
  return NB_OK;
}

// The owner-flag arguments (checked by owner_checks; n_owner 0: none).
nb::OwnerParams owner_params(const int32_t* seg_buf, const int32_t* folded_ids, int B, int L, int S,
                             const int32_t* owner_off, int n_owner, uint8_t* owner_attended) {
  nb::OwnerParams op;
  std::memset(&op, 0, sizeof(op));
  if (n_owner == 0) return op;
  op.folded = folded_ids;
  op.kcov_lo = seg_buf + nb::seg_layout(B, L, S).kcov_lo;
  op.attended = owner_attended;
  op.B = B;
  op.S = S;
  op.n_owner = n_owner;
  for (int x = 0; x <= n_owner; ++x) op.off[x] = owner_off[x];
  return op;
}

int launch_owner(const int32_t* seg_buf, const int32_t* folded_ids, int B, int L, int S, const int32_t* owner_off,
                 int n_owner, uint8_t* owner_attended, hipStream_t s) {
  if (n_owner == 0) return NB_OK;
  return map_hip(nb::launch_owner_flags(owner_params(seg_buf, folded_ids, B, L, S, owner_off, n_owner,
                                                     owner_attended), s));
}

}  // namespace

extern "C" {

int nb_attn_bwd_dq(const void* dout, const void* q, const void* k, const void* v, const void* o,
                   const void* o_resid, const float* lse, const int32_t* seg_buf, int B, int Hq, int Hkv, int L,
                   int S, int D, float scale, int window_left, int dtype, void* dq, void* ws, size_t ws_bytes,
                   void* stream) {
  const void* ptrs[] = {dout, q, k, v, o, lse, seg_buf, dq, ws};
  int st = attn_common_checks(ptrs, 9, B, Hq, Hkv, L, S, D, scale, dtype);
  if (st != NB_OK) return st;
  if (o_resid != nullptr && !aligned16(o_resid)) return NB_ERR_INVALID_ARG;
  if (ws_bytes < nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dtype)) return NB_ERR_WORKSPACE;
  const nb::BwdParams p = bwd_params(dout, q, one_chunk(S, k, v, nullptr, nullptr), o, o_resid, lse, seg_buf, B,
                                     Hq, Hkv, L, S, scale, window_left, dq, ws);
  return map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdDq, (hipStream_t)stream));
}

int nb_attn_bwd_dkdv(const void* dout, const void* q, const void* k, const void* v, const float* lse,
                     const int32_t* seg_buf, int B, int Hq, int Hkv, int L, int S, int D, float scale,
                     int window_left, int dtype, void* dk, void* dv, void* ws, size_t ws_bytes,
                     void* stream) {
  const void* ptrs[] = {dout, q, k, v, lse, seg_buf, dk, dv, ws};
  int st = attn_common_checks(ptrs, 9, B, Hq, Hkv, L, S, D, scale, dtype);
  if (st != NB_OK) return st;
  if (ws_bytes < nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dtype)) return NB_ERR_WORKSPACE;
  const nb::BwdParams p = bwd_params(dout, q, one_chunk(S, k, v, dk, dv), nullptr, nullptr, lse, seg_buf, B, Hq,
                                     Hkv, L, S, scale, window_left, nullptr, ws);
  return map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdDkdv, (hipStream_t)stream));
}

int nb_attn_bwd_prep(const void* dout, const void* o, const void* o_resid, const int32_t* seg_buf, int B, int Hq,
                     int Hkv, int L, int S, int D, int window_left, int dtype, void* ws, size_t ws_bytes,
                     void* stream) {
  const void* ptrs[] = {dout, o, seg_buf, ws};
  int st = attn_common_checks(ptrs, 4, B, Hq, Hkv, L, S, D, 1.0f, dtype);
  if (st != NB_OK) return st;
  if (o_resid != nullptr && !aligned16(o_resid)) return NB_ERR_INVALID_ARG;
  if (ws_bytes < nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dtype)) return NB_ERR_WORKSPACE;
  const nb::BwdParams p = bwd_params(dout, nullptr, one_chunk(S, nullptr, nullptr, nullptr, nullptr), o, o_resid,
                                     nullptr, seg_buf, B, Hq, Hkv, L, S, 1.0f, window_left, nullptr, ws);
  return map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdPrep, (hipStream_t)stream));
}

int nb_attn_bwd_main(const void* dout, const void* q, const void* k, const void* v, const float* lse,
                     const int32_t* seg_buf, int B, int Hq, int Hkv, int L, int S, int D, float scale,
                     int window_left, int dtype, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                     void* stream) {
  const void* ptrs[] = {dout, q, k, v, lse, seg_buf, dq, dk, dv, ws};
  int st = attn_common_checks(ptrs, 10, B, Hq, Hkv, L, S, D, scale, dtype);
  if (st != NB_OK) return st;
  if (ws_bytes < nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dtype)) return NB_ERR_WORKSPACE;
  nb::BwdParams p = bwd_params(dout, q, one_chunk(S, k, v, dk, dv), nullptr, nullptr, lse, seg_buf, B, Hq, Hkv, L,
                               S, scale, window_left, dq, ws);
  enable_ds(p, ws, ws_bytes, B, Hq, Hkv, L, S, D, window_left, dtype);
  return map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdMain, (hipStream_t)stream));
}

int nb_owner_attended(const int32_t* seg_buf, const int32_t* folded_ids, int B, int L, int S,
                      const int32_t* owner_off, int n_owner, uint8_t* owner_attended, void* stream) {
  if (seg_buf == nullptr || !dims_ok(B, L, S)) return NB_ERR_INVALID_ARG;
  int st = owner_checks(folded_ids, S, owner_off, n_owner, owner_attended);
  if (st != NB_OK) return st;
  return launch_owner(seg_buf, folded_ids, B, L, S, owner_off, n_owner, owner_attended, (hipStream_t)stream);
}

int nb_attn_bwd_chunks(const void* dout, const void* q, const void* const* k_chunk, const void* const* v_chunk,
                       const int32_t* chunk_len, const int32_t* chunk_start, const int32_t* chunk_rows, int n_chunk,
                       const void* o, const void* o_resid, const float* lse, const int32_t* seg_buf,
                       const int32_t* folded_ids, int B, int Hq, int Hkv, int L, int S, int D, float scale,
                       int window_left, int dtype, void* dq, void* const* dk_chunk, void* const* dv_chunk,
                       uint8_t* chunk_attended, void* ws, size_t ws_bytes, void* stream) {
  const void* ptrs[] = {dout, q, o, lse, seg_buf, dq, ws};
  int st = attn_common_checks(ptrs, 7, B, Hq, Hkv, L, S, D, scale, dtype);
  if (st != NB_OK) return st;
  if (o_resid != nullptr && !aligned16(o_resid)) return NB_ERR_INVALID_ARG;
  if (ws_bytes < nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dtype)) return NB_ERR_WORKSPACE;
  if (dk_chunk == nullptr || dv_chunk == nullptr) return NB_ERR_INVALID_ARG;
  nb::KvChunks kv;
  st = chunk_table(k_chunk, v_chunk, dk_chunk, dv_chunk, chunk_len, chunk_start, chunk_rows, n_chunk, B, Hkv, S, &kv);
  if (st != NB_OK) return st;
  int32_t off[nb::kMaxKvChunks + 1];
  for (int x = 0; x <= n_chunk; ++x) off[x] = kv.off[x];
  if (chunk_attended != nullptr) {
    st = owner_checks(folded_ids, S, off, n_chunk, chunk_attended);
    if (st != NB_OK) return st;
  }
  hipStream_t s = (hipStream_t)stream;
  nb::BwdParams p = bwd_params(dout, q, kv, o, o_resid, lse, seg_buf, B, Hq, Hkv, L, S, scale, window_left, dq, ws);
  enable_ds(p, ws, ws_bytes, B, Hq, Hkv, L, S, D, window_left, dtype);
  if (chunk_attended != nullptr)   // the flags come from the prep kernel
    p.own = owner_params(seg_buf, folded_ids, B, L, S, off, n_chunk, chunk_attended);
  st = map_hip(nb::launch_kv_zero_outside(kv, B * Hkv, D * (dtype == NB_F32 ? 4 : 2), s));
  if (st != NB_OK) return st;
  st = map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdPrep, s));
  if (st != NB_OK) return st;
  return map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdMain, s));
}

int nb_attn_bwd(const void* dout, const void* q, const void* k, const void* v, const void* o, const void* o_resid,
                const float* lse, const int32_t* seg_buf, const int32_t* folded_ids, int B, int Hq, int Hkv, int L,
                int S, int D, float scale, int window_left, int dtype, void* dq, void* dk, void* dv,
                const int32_t* owner_off, int n_owner, uint8_t* owner_attended, void* ws, size_t ws_bytes,
                void* stream) {
  const void* ptrs[] = {dout, q, k, v, o, lse, seg_buf, dq, dk, dv, ws};
  int st = attn_common_checks(ptrs, 11, B, Hq, Hkv, L, S, D, scale, dtype);
  if (st != NB_OK) return st;
  if (o_resid != nullptr && !aligned16(o_resid)) return NB_ERR_INVALID_ARG;
  if (ws_bytes < nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dtype)) return NB_ERR_WORKSPACE;
  st = owner_checks(folded_ids, S, owner_off, n_owner, owner_attended);
  if (st != NB_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  nb::BwdParams p = bwd_params(dout, q, one_chunk(S, k, v, dk, dv), o, o_resid, lse, seg_buf, B, Hq, Hkv, L, S,
                               scale, window_left, dq, ws);
  enable_ds(p, ws, ws_bytes, B, Hq, Hkv, L, S, D, window_left, dtype);
  p.own = owner_params(seg_buf, folded_ids, B, L, S, owner_off, n_owner, owner_attended);   // computed in prep
  st = map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdPrep, s));
  if (st != NB_OK) return st;
  return map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdMain, s));
}

int nb_ring_chunk_fwd(const void* q, const void* k, const void* v, void* out, float* lse, const int32_t* seg_buf,
                      int B, int Hq, int Hkv, int L, int Lk, int D, int q_start, int k_start, float scale, int dtype,
                      void* stream) {
  const void* ptrs[] = {q, k, v, out, lse, seg_buf};
  int st = attn_common_checks(ptrs, 6, B, Hq, Hkv, L, Lk, D, scale, dtype, true);
  if (st != NB_OK) return st;
  if (k_start < 0 || k_start > q_start || (int64_t)q_start + L >= kMaxIndex) return NB_ERR_INVALID_ARG;
  return attn_fwd_kv(q, one_chunk(Lk, k, v, nullptr, nullptr), out, nullptr, lse, seg_buf, B, Hq, Hkv, L, Lk, D,
                     scale, -1, 0.f, dtype, stream, q_start - k_start, k_start);
}

int nb_ring_chunk_bwd(const void* dout, const void* q, const void* k, const void* v, const void* o,
                      const void* o_resid, const float* lse, const int32_t* seg_buf, int B, int Hq, int Hkv, int L,
                      int Lk, int D, int q_start, int k_start, float scale, int dtype, void* dq, void* dk, void* dv,
                      int flags, void* ws, size_t ws_bytes, void* stream) {
  const void* ptrs[] = {dout, q, k, v, o, lse, seg_buf, dq, dk, dv, ws};
  int st = attn_common_checks(ptrs, 11, B, Hq, Hkv, L, Lk, D, scale, dtype, true);
  if (st != NB_OK) return st;
  if (o_resid != nullptr && !aligned16(o_resid)) return NB_ERR_INVALID_ARG;
  if (k_start < 0 || k_start > q_start || (int64_t)q_start + L >= kMaxIndex) return NB_ERR_INVALID_ARG;
  if (flags & ~(NB_RING_DELTA_READY | NB_RING_DQ_F32_SET | NB_RING_DQ_F32_ADD)) return NB_ERR_INVALID_ARG;
  if ((flags & NB_RING_DQ_F32_SET) && (flags & NB_RING_DQ_F32_ADD)) return NB_ERR_INVALID_ARG;
  if (ws_bytes < nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, Lk, D, dtype)) return NB_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  nb::BwdParams p = bwd_params(dout, q, one_chunk(Lk, k, v, dk, dv), o, o_resid, lse, seg_buf, B, Hq, Hkv, L, Lk,
                               scale, -1, dq, ws, q_start - k_start, k_start);
  p.dq_mode = (flags & NB_RING_DQ_F32_SET) ? nb::kDqSetF32 : (flags & NB_RING_DQ_F32_ADD) ? nb::kDqAddF32
                                                                                            : nb::kDqStore;
  // with room for a dS band as wide as the chunk: the stored-dS form (the
  // only form at D = 512, where a dQ pass recomputing S and dP does not fit)
  const size_t base = nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, Lk, D, dtype);
  const size_t db = ds_bytes_span(B, Hq, L, D, Lk, dtype);
  if (D == 512 && db == 0) return NB_ERR_UNSUPPORTED;          // dS band over 2 GiB
  if (D == 512 && ws_bytes < base + db) return NB_ERR_WORKSPACE;
  if (db != 0 && ws_bytes >= base + db) {
    p.dsbuf = reinterpret_cast<char*>(ws) + base;
    p.ds_w = ds_width(Lk);
    p.ds_bytes = (int)db;
  }
  st = map_hip(nb::launch_bwd(p, D, dtype == NB_F32, (flags & NB_RING_DELTA_READY) ? nb::kBwdOrders : nb::kBwdPrep,
                              s));
  if (st != NB_OK) return st;
  return map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdMain, s));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The backward without a caller workspace (nb_attn_bwd_noalloc).  Its
// workspace -- Delta, the work orders, the queue counters and the deferred dQ
// list, laid out exactly as nb_attn_bwd's -- lives in this file-scope device
// array, one copy per GPU, held until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in): each
// device's address comes from hipGetSymbolAddress, taken once per device with
// that device current, and is what the kernels receive.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (resolved on the first call on that device).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NB_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return e == hipSuccess ? NB_ERR_DEVICE : map_hip(e);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return NB_OK;
}
}  // namespace

extern "C" {

size_t nb_attn_bwd_noalloc_max_workspace_bytes(void) { return kNoAllocScratchBytes; }

int nb_attn_bwd_noalloc(const void* dout, const void* q, const void* k, const void* v, const void* o,
                        const void* o_resid, const float* lse, const int32_t* seg_buf, const int32_t* folded_ids,
                        int B, int Hq, int Hkv, int L, int S, int D, float scale, int window_left, int dtype,
                        void* dq, void* dk, void* dv, const int32_t* owner_off, int n_owner,
                        uint8_t* owner_attended, void* stream) {
  // the same checks as nb_attn_bwd, with the size limit of the static workspace
  const void* ptrs[] = {dout, q, k, v, o, lse, seg_buf, dq, dk, dv};
  int st = attn_common_checks(ptrs, 10, B, Hq, Hkv, L, S, D, scale, dtype);
  if (st != NB_OK) return st;
  if (o_resid != nullptr && !aligned16(o_resid)) return NB_ERR_INVALID_ARG;
  const size_t need = nb_attn_bwd_workspace_bytes(B, Hq, Hkv, L, S, D, dtype);
  if (need == 0 || need > kNoAllocScratchBytes) return NB_ERR_WORKSPACE;
  st = owner_checks(folded_ids, S, owner_off, n_owner, owner_attended);
  if (st != NB_OK) return st;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != NB_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // recompute form (no dS buffer); the prep kernel writes Delta and the work
  // orders and sets the queue counters to zero, so nothing carried over from
  // an earlier call is read
  nb::BwdParams p = bwd_params(dout, q, one_chunk(S, k, v, dk, dv), o, o_resid, lse, seg_buf, B, Hq, Hkv, L, S,
                               scale, window_left, dq, ws);
  p.own = owner_params(seg_buf, folded_ids, B, L, S, owner_off, n_owner, owner_attended);
  st = map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdPrep, s));
  if (st != NB_OK) return st;
  return map_hip(nb::launch_bwd(p, D, dtype == NB_F32, nb::kBwdMain, s));
}

}  // extern "C"
