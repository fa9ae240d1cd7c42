// Global-layer ring attention pieces that are not attention proper: the
// online-softmax merges, the live-row list, the final rounding of the merged
// output and the fp32 sum of the chunks' dQ.
//
// NeMo AutoModel gemma4_moe.cp_attention page: _merge_ffpa_packed_chunk (the
// -inf-safe merge: lse = log(e^lse_acc + e^lse_step), outs weighted by
// exp(lse_x - lse), a row neither side covered stays 0), _merge_live_chunk_
// (the same merge in place at the live rows only) and _grad_add_live_ (the
// chunks' gradients added up).  The per-chunk attention itself runs on the
// neighbourhood kernels (attn_fwd.hip, attn_bwd.hip) with global positions.
//
// All of it is HBM-bound streaming: a row's D values are spread over D / 4
// lanes with 16-byte fp32 accesses (8-byte bf16), consecutive rows in
// consecutive lanes, so a wave reads whole contiguous rows.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/nbring.h"
#include "nb_device.h"

namespace nb {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// One row's merge, by the D / 4 lanes that hold it (lane part c: values 4c..4c+3).
// A row may span several waves (D > 256), so every lane reads the row's two
// LSEs, then the whole workgroup meets at a barrier, and only then does the
// row's lane 0 overwrite lse_acc: no lane can read the new value.  Lanes
// without a row (`row` < 0) take part in the barrier only.
template <typename T>
__device__ __forceinline__ void merge_row(float* out_acc, float* lse_acc, const T* out_step, const float* lse_step,
                                          int64_t row, int D, int c) {
  float a = -INFINITY, b = -INFINITY;
  if (row >= 0) {
    b = lse_step[row];
    a = lse_acc[row];
  }
  __syncthreads();
  if (row < 0 || b == -INFINITY) return;   // no row, or the chunk gave this row nothing
  const float m = fmaxf(a, b);             // finite: b is
  const float lse = m + logf(expf(a - m) + expf(b - m));
  const float wa = expf(a - lse), wb = expf(b - lse);
  float* o = out_acc + (size_t)row * D + 4 * c;
  const f32x4 x = *reinterpret_cast<const f32x4*>(o);
  const f32x4 y = load4<T>(out_step + (size_t)row * D + 4 * c);
  *reinterpret_cast<f32x4*>(o) = f32x4{wa * x[0] + wb * y[0], wa * x[1] + wb * y[1], wa * x[2] + wb * y[2],
                                       wa * x[3] + wb * y[3]};
  if (c == 0) lse_acc[row] = lse;
}

// init: nothing merged yet -- the accumulators become the step (every row).
template <typename T>
__global__ __launch_bounds__(kThreads) void merge_kernel(float* out_acc, float* lse_acc, const T* out_step,
                                                         const float* lse_step, int64_t R, int D, int init) {
  const int tpr = D / 4, rpb = kThreads / tpr;
  const int64_t row = (int64_t)blockIdx.x * rpb + threadIdx.x / tpr;
  const int c = threadIdx.x % tpr;
  if (init) {
    if (row >= R) return;
    *reinterpret_cast<f32x4*>(out_acc + (size_t)row * D + 4 * c) = load4<T>(out_step + (size_t)row * D + 4 * c);
    if (c == 0) lse_acc[row] = lse_step[row];
    return;
  }
  merge_row<T>(out_acc, lse_acc, out_step, lse_step, row < R ? row : -1, D, c);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void merge_live_kernel(float* out_acc, float* lse_acc, const T* out_step,
                                                              const float* lse_step, const int32_t* live_index,
                                                              const int32_t* n_live, int64_t tasks, int H, int L,
                                                              int D) {
  const int tpr = D / 4, rpb = kThreads / tpr;
  const int64_t t = (int64_t)blockIdx.x * rpb + threadIdx.x / tpr;   // (live row, head), head fastest
  int64_t row = -1;
  if (t < tasks) {
    const int64_t x = t / H;
    if (x < *n_live) {
      const int h = (int)(t % H);
      const int flat = live_index[x];
      const int b = flat / L, i = flat % L;
      row = ((int64_t)b * H + h) * L + i;
    }
  }
  merge_row<T>(out_acc, lse_acc, out_step, lse_step, row, D, threadIdx.x % tpr);
}

// One workgroup: the live rows in ascending order (a block-wide running scan).
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void live_rows_kernel(const int32_t* row_klo, int N, int L, int Lk,
                                                                 int q_off, int k_origin, int32_t* live_index,
                                                                 int32_t* n_live) {
  __shared__ int wsum[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int total = 0;
  for (int base = 0; base < N; base += kScanThreads) {
    const int idx = base + tid;
    bool live = false;
    if (idx < N) {
      const int i = idx % L;
      const int bs = max(0, row_klo[idx] - k_origin);
      live = bs <= min(q_off + i, Lk - 1);
    }
    const unsigned long long m = __ballot(live);
    const int below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __popcll(m);
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int x = 0; x < kScanThreads / 64; ++x) {
      before += x < w ? wsum[x] : 0;
      all += wsum[x];
    }
    if (live) live_index[total + before + below] = idx;
    total += all;
    __syncthreads();   // wsum is rewritten by the next round
  }
  if (tid == 0) *n_live = total;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void finalize_kernel(const float* acc, T* out, uint8_t* resid, int64_t n4) {
  const int64_t x = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (x >= n4) return;
  const f32x4 a = reinterpret_cast<const f32x4*>(acc)[x];
  store_quad<T>(out + 4 * x, a[0], a[1], a[2], a[3]);
  if constexpr (sizeof(T) == 2) {   // bf16: the residual codes (nb_device.h: resid_code)
    if (resid != nullptr) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) word |= resid_code(a[e], (bf16)a[e]) << (8 * e);
      reinterpret_cast<uint32_t*>(resid)[x] = word;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void grad_add_kernel(float* acc, const T* src, int64_t n4, int init) {
  const int64_t x = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (x >= n4) return;
  const f32x4 b = load4<T>(src + 4 * x);
  if (init) {
    reinterpret_cast<f32x4*>(acc)[x] = b;
    return;
  }
  const f32x4 a = reinterpret_cast<f32x4*>(acc)[x];
  reinterpret_cast<f32x4*>(acc)[x] = f32x4{a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// a row's D / 4 lanes sit in one workgroup (the merge's barrier orders the
// reads of lse_acc before its rewrite)
bool row_width_ok(int D) { return D >= 4 && D <= 4 * kThreads && (D & (D - 1)) == 0; }
constexpr int64_t kMaxGrid = (int64_t)1 << 31;

int status(hipError_t e) { return e == hipSuccess ? NB_OK : NB_ERR_LAUNCH; }

}  // namespace
}  // namespace nb

extern "C" {

int nb_ring_merge(float* out_acc, float* lse_acc, const void* out_step, const float* lse_step, int64_t R, int D,
                  int dtype, int init, void* stream) {
  using namespace nb;
  if (!out_acc || !lse_acc || !out_step || !lse_step) return NB_ERR_INVALID_ARG;
  if (!aligned16(out_acc) || !aligned16(out_step) || R < 0 || !row_width_ok(D)) return NB_ERR_INVALID_ARG;
  if (dtype != NB_BF16 && dtype != NB_F32) return NB_ERR_UNSUPPORTED;
  if (R == 0) return NB_OK;
  const int rpb = kThreads / (D / 4);
  const int64_t grid = (R + rpb - 1) / rpb;
  if (grid >= kMaxGrid) return NB_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == NB_F32)
    hipLaunchKernelGGL(merge_kernel<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, out_acc, lse_acc,
                       (const float*)out_step, lse_step, R, D, init);
  else
    hipLaunchKernelGGL(merge_kernel<bf16>, dim3((unsigned)grid), dim3(kThreads), 0, s, out_acc, lse_acc,
                       (const bf16*)out_step, lse_step, R, D, init);
  return status(hipGetLastError());
}

int nb_ring_live_rows(const int32_t* seg_buf, int B, int L, int Lk, int q_start, int k_start, int32_t* live_index,
                      int32_t* n_live, void* stream) {
  using namespace nb;
  if (!seg_buf || !live_index || !n_live) return NB_ERR_INVALID_ARG;
  if (B < 1 || L < 1 || Lk < 1 || k_start < 0 || k_start > q_start || (int64_t)B * L >= ((int64_t)1 << 30))
    return NB_ERR_INVALID_ARG;
  const int32_t* row_klo = seg_buf + nb_segment_offset_row_klo(B, L);
  hipLaunchKernelGGL(live_rows_kernel, dim3(1), dim3(kScanThreads), 0, (hipStream_t)stream, row_klo, B * L, L, Lk,
                     q_start - k_start, k_start, live_index, n_live);
  return status(hipGetLastError());
}

int nb_ring_merge_live(float* out_acc, float* lse_acc, const void* out_step, const float* lse_step,
                       const int32_t* live_index, const int32_t* n_live, int n_live_max, int B, int H, int L, int D,
                       int dtype, void* stream) {
  using namespace nb;
  if (!out_acc || !lse_acc || !out_step || !lse_step || !live_index || !n_live) return NB_ERR_INVALID_ARG;
  if (!aligned16(out_acc) || !aligned16(out_step) || !row_width_ok(D)) return NB_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || L < 1 || n_live_max < 0 || (int64_t)n_live_max > (int64_t)B * L) return NB_ERR_INVALID_ARG;
  if (dtype != NB_BF16 && dtype != NB_F32) return NB_ERR_UNSUPPORTED;
  if (n_live_max == 0) return NB_OK;
  const int rpb = kThreads / (D / 4);
  const int64_t tasks = (int64_t)n_live_max * H;
  const int64_t grid = (tasks + rpb - 1) / rpb;
  if (grid >= kMaxGrid) return NB_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == NB_F32)
    hipLaunchKernelGGL(merge_live_kernel<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, out_acc, lse_acc,
                       (const float*)out_step, lse_step, live_index, n_live, tasks, H, L, D);
  else
    hipLaunchKernelGGL(merge_live_kernel<bf16>, dim3((unsigned)grid), dim3(kThreads), 0, s, out_acc, lse_acc,
                       (const bf16*)out_step, lse_step, live_index, n_live, tasks, H, L, D);
  return status(hipGetLastError());
}

int nb_ring_finalize(const float* out_acc, void* out, void* out_resid, int64_t R, int D, int dtype, void* stream) {
  using namespace nb;
  if (!out_acc || !out || !aligned16(out_acc) || !aligned16(out)) return NB_ERR_INVALID_ARG;
  if (out_resid && !aligned16(out_resid)) return NB_ERR_INVALID_ARG;
  if (R < 0 || D < 4 || D % 4 != 0) return NB_ERR_INVALID_ARG;
  if (dtype != NB_BF16 && dtype != NB_F32) return NB_ERR_UNSUPPORTED;
  const int64_t n4 = R * D / 4;
  if (n4 == 0) return NB_OK;
  const int64_t grid = (n4 + kThreads - 1) / kThreads;
  if (grid >= kMaxGrid) return NB_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == NB_F32)
    hipLaunchKernelGGL(finalize_kernel<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, out_acc, (float*)out,
                       nullptr, n4);
  else
    hipLaunchKernelGGL(finalize_kernel<bf16>, dim3((unsigned)grid), dim3(kThreads), 0, s, out_acc, (bf16*)out,
                       (uint8_t*)out_resid, n4);
  return status(hipGetLastError());
}

int nb_ring_grad_add(float* acc, const void* src, int64_t n, int dtype, int init, void* stream) {
  using namespace nb;
  if (!acc || !src || !aligned16(acc) || !aligned16(src) || n < 0 || n % 4 != 0) return NB_ERR_INVALID_ARG;
  if (dtype != NB_BF16 && dtype != NB_F32) return NB_ERR_UNSUPPORTED;
  const int64_t n4 = n / 4;
  if (n4 == 0) return NB_OK;
  const int64_t grid = (n4 + kThreads - 1) / kThreads;
  if (grid >= kMaxGrid) return NB_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == NB_F32)
    hipLaunchKernelGGL(grad_add_kernel<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, acc, (const float*)src, n4,
                       init);
  else
    hipLaunchKernelGGL(grad_add_kernel<bf16>, dim3((unsigned)grid), dim3(kThreads), 0, s, acc, (const bf16*)src, n4,
                       init);
  return status(hipGetLastError());
}

}  // extern "C"
