// Block-diagonal context-parallel K/V exchange: the plans, and the needed-range
// exchange emulated for every rank on one device.
//
// NeMo AutoModel blockdiag_cp.exchange page: the global left-halo plan (needed
// range [s_first_r, real_end_r) of every rank, straddle back_r, use_halo), the
// per-(source, destination) split sizes and local gather index, and
// _NeededKVExchange (forward: each destination receives the pieces of its
// range in source order; backward: index_add of every destination's gradient
// onto the source tokens).  Readings where the page is silent are stated in
// nbexchange.h.
//
// The plan is integer work over the replicated document ids (one workgroup
// per rank: block-wide reductions per row; then one workgroup for the splits
// and offsets).  On one device the exchange's
// forward is, per rank, one contiguous copy of x[:, :, s_first_r:real_end_r]
// (the pieces of all sources in source order are exactly that slice); the
// backward sums, per token, the gradients of the ranks that needed it, in
// ascending rank order in fp32.  Both are HBM-bound 16-byte streams.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "../../include/nbexchange.h"

namespace nb {
namespace {

constexpr int kHdr = 8;
constexpr int kPlanThreads = 1024;
constexpr int kStreamThreads = 256;

struct PlanLayout {
  int s_first, real_end, back, splits, send_off, recv_off, total;
  __host__ __device__ explicit PlanLayout(int P) {
    s_first = kHdr;
    real_end = s_first + P;
    back = real_end + P;
    splits = back + P;
    send_off = splits + P * P;
    recv_off = send_off + P * (P + 1);
    total = recv_off + P * (P + 1);
  }
};

struct XchPtrs {
  void* p[NB_XCH_MAX_RANKS];
};

__device__ int block_max(int v, int* red) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();   // red may still be read by the previous call
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int r = red[0];
  for (int x = 1; x < nw; ++x) r = max(r, red[x]);
  return r;
}

// Folded id at (b, j): padding and ids <= 0 are not documents (0).
__device__ __forceinline__ int folded(const int32_t* ids, const uint8_t* pad, int N, int b, int j) {
  const size_t o = (size_t)b * N + j;
  const int v = ids[o];
  return (v > 0 && (pad == nullptr || pad[o] == 0)) ? v : 0;
}

// Needed range of rank blockIdx.x: union over the rows of [start of the run
// holding r L, one past the chunk's last non-padding position).
__global__ __launch_bounds__(kPlanThreads) void xch_range_kernel(const int32_t* ids, const uint8_t* pad, int B,
                                                                 int N, int P, int32_t* plan) {
  __shared__ int red[kPlanThreads / 64];
  const int tid = threadIdx.x, r = blockIdx.x;
  const int L = N / P;
  const int lo = r * L, hi = lo + L;
  int first = INT_MAX, end = -1;
  for (int b = 0; b < B; ++b) {
    // last non-padding position of the row's chunk
    int m = -1;
    for (int j = lo + tid; j < hi; j += kPlanThreads)
      if (folded(ids, pad, N, b, j) != 0) m = j;
    m = block_max(m, red);
    if (m < 0) continue;   // the row has no real token in this chunk
    end = max(end, m + 1);
    // start of the run of equal ids holding position lo: the last j <= lo
    // whose left neighbour carries another id (0 if none)
    const int id = folded(ids, pad, N, b, lo);
    int s = lo;
    if (id != 0) {
      int t = 0;
      for (int j = 1 + tid; j <= lo; j += kPlanThreads)
        if (folded(ids, pad, N, b, j - 1) != id) t = j;
      s = block_max(t, red);
    }
    first = min(first, s);
  }
  if (tid == 0) {
    const PlanLayout lay(P);
    plan[lay.s_first + r] = end < 0 ? lo : first;
    plan[lay.real_end + r] = end < 0 ? lo : end;
  }
}

// The rest of the plan from the ranges: straddles, splits, offsets, header.
__global__ __launch_bounds__(kPlanThreads) void xch_offsets_kernel(int N, int P, int32_t* plan) {
  __shared__ int sf[NB_XCH_MAX_RANKS], re[NB_XCH_MAX_RANKS];
  __shared__ int spl[NB_XCH_MAX_RANKS * NB_XCH_MAX_RANKS];
  const int tid = threadIdx.x;
  const int L = N / P;
  const PlanLayout lay(P);
  if (tid < P) {
    sf[tid] = plan[lay.s_first + tid];
    re[tid] = plan[lay.real_end + tid];
  }
  __syncthreads();
  for (int x = tid; x < P * P; x += kPlanThreads) {
    const int s = x / P, r = x % P;
    const int a = max(s * L, sf[r]), e = min((s + 1) * L, re[r]);
    spl[x] = max(0, e - a);
    plan[lay.splits + x] = spl[x];
  }
  if (tid < P) plan[lay.back + tid] = tid * L - sf[tid];
  __syncthreads();
  if (tid < P) {
    // sender tid: where each destination's piece starts in its send buffer
    int acc = 0;
    for (int r = 0; r < P; ++r) {
      plan[lay.send_off + tid * (P + 1) + r] = acc;
      acc += spl[tid * P + r];
    }
    plan[lay.send_off + tid * (P + 1) + P] = acc;
    // destination tid: where each source's piece starts in its range
    acc = 0;
    for (int s = 0; s < P; ++s) {
      plan[lay.recv_off + tid * (P + 1) + s] = acc;
      acc += spl[s * P + tid];
    }
    plan[lay.recv_off + tid * (P + 1) + P] = acc;
  }
  if (tid == 0) {
    int use_halo = 1, halo = 0, total = 0;
    for (int r = 0; r < P; ++r) {
      const int back = r * L - sf[r];
      use_halo &= back <= L ? 1 : 0;
      halo = max(halo, back);
      total += re[r] - sf[r];
    }
    plan[0] = use_halo;
    plan[1] = halo;
    plan[2] = L;
    plan[3] = P;
    plan[4] = total;
    plan[5] = plan[6] = plan[7] = 0;
  }
}

__global__ __launch_bounds__(kStreamThreads) void xch_send_index_kernel(const int32_t* plan, int N, int P,
                                                                        int32_t* send_index) {
  const PlanLayout lay(P);
  const int s = blockIdx.x, L = N / P;
  int32_t* out = send_index + (size_t)s * N;
  for (int r = 0; r < P; ++r) {
    const int a = max(s * L, plan[lay.s_first + r]);
    const int n = plan[lay.splits + s * P + r];
    const int base = plan[lay.send_off + s * (P + 1) + r];
    for (int t = threadIdx.x; t < n; t += kStreamThreads) out[base + t] = a - s * L + t;
  }
}

// recv[r][bc] = x[bc][s_first_r : real_end_r], 16 bytes per thread.
__global__ __launch_bounds__(kStreamThreads) void xch_gather_kernel(const uint4* __restrict__ x,
                                                                    const int32_t* plan, int N, int VPR, int P,
                                                                    XchPtrs recv) {
  const PlanLayout lay(P);
  const int r = blockIdx.z, bc = blockIdx.y;
  const int sf = plan[lay.s_first + r];
  const int R = plan[lay.real_end + r] - sf;
  uint4* dst0 = reinterpret_cast<uint4*>(recv.p[r]);
  if (R <= 0 || dst0 == nullptr) return;
  const uint4* src = x + ((size_t)bc * N + sf) * VPR;
  uint4* dst = dst0 + (size_t)bc * R * VPR;
  const size_t n = (size_t)R * VPR;
  for (size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kStreamThreads)
    dst[i] = src[i];
}

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int E = 4;
  typedef float V __attribute__((ext_vector_type(4)));
};
template <>
struct Vec16<__bf16> {
  static constexpr int E = 8;
  typedef __bf16 V __attribute__((ext_vector_type(8)));
};

// gx[bc][j] = sum over ranks r (ascending) whose range holds j of
// grad_r[bc][j - s_first_r]; 0 if none.  fp32 sums, one rounding at the store.
template <typename T>
__global__ __launch_bounds__(kStreamThreads) void xch_scatter_add_kernel(XchPtrs grads, const int32_t* plan,
                                                                         int N, int VPR, int P, T* gx) {
  typedef typename Vec16<T>::V V;
  constexpr int E = Vec16<T>::E;
  __shared__ int sf[NB_XCH_MAX_RANKS], re[NB_XCH_MAX_RANKS];
  const PlanLayout lay(P);
  for (int r = threadIdx.x; r < P; r += kStreamThreads) {
    sf[r] = plan[lay.s_first + r];
    re[r] = plan[lay.real_end + r];
  }
  __syncthreads();
  const int bc = blockIdx.y;
  const size_t n = (size_t)N * VPR;
  V* out = reinterpret_cast<V*>(gx) + (size_t)bc * n;
  for (size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kStreamThreads) {
    const int j = (int)(i / VPR), c = (int)(i % VPR);
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    // loads of up to four ranks in flight before their sums (the sums keep rank order)
    for (int r0 = 0; r0 < P; r0 += 4) {
      V v[4];
      bool h[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u;
        h[u] = r < P && j >= sf[r] && j < re[r] && grads.p[r] != nullptr;
        if (h[u]) {
          const int R = re[r] - sf[r];
          v[u] = reinterpret_cast<const V*>(grads.p[r])[((size_t)bc * R + (j - sf[r])) * VPR + c];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (h[u]) {
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] += (float)v[u][e];
        }
    }
    V o;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = (T)acc[e];
    out[i] = o;
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int map_hip(hipError_t e) {
  if (e == hipSuccess) return NB_OK;
  if (e == hipErrorNoDevice || e == hipErrorInvalidDevice || e == hipErrorNoBinaryForGpu) return NB_ERR_DEVICE;
  return NB_ERR_LAUNCH;
}

bool ranks_ok(int N, int P) { return P >= 1 && P <= NB_XCH_MAX_RANKS && N >= 1 && N % P == 0; }

// Shared checks of the two streaming calls; VPR = 16-byte vectors per token row.
int stream_checks(const void* dense, const int32_t* plan, int B, int C, int N, int D, int P, int dtype,
                  void* const* ptrs, int* VPR) {
  if (dense == nullptr || plan == nullptr || ptrs == nullptr || !aligned16(dense)) return NB_ERR_INVALID_ARG;
  if (!ranks_ok(N, P) || B < 1 || C < 1 || D < 1 || (int64_t)B * C > 65535) return NB_ERR_INVALID_ARG;
  if (dtype != NB_BF16 && dtype != NB_F32) return NB_ERR_UNSUPPORTED;
  const int es = dtype == NB_BF16 ? 2 : 4;
  if ((D * es) % 16 != 0) return NB_ERR_INVALID_ARG;
  if ((int64_t)N * D * es / 16 >= ((int64_t)1 << 31)) return NB_ERR_INVALID_ARG;
  for (int r = 0; r < P; ++r)
    if (ptrs[r] != nullptr && !aligned16(ptrs[r])) return NB_ERR_INVALID_ARG;
  *VPR = D * es / 16;
  return NB_OK;
}

unsigned stream_blocks(int N, int VPR) {
  const int64_t need = ((int64_t)N * VPR + kStreamThreads - 1) / kStreamThreads;
  return (unsigned)(need < 1024 ? (need < 1 ? 1 : need) : 1024);
}

}  // namespace
}  // namespace nb

extern "C" {

size_t nb_exchange_plan_elems(int cp_size) {
  if (cp_size < 1 || cp_size > NB_XCH_MAX_RANKS) return 0;
  return (size_t)nb::PlanLayout(cp_size).total;
}

int nb_exchange_plan(const int32_t* doc_ids, const uint8_t* pad_mask, int B, int N, int cp_size, int32_t* plan,
                     size_t plan_elems, void* stream) {
  if (doc_ids == nullptr || plan == nullptr) return NB_ERR_INVALID_ARG;
  if (B < 1 || B > 65535 || !nb::ranks_ok(N, cp_size) || (int64_t)B * N >= ((int64_t)1 << 31))
    return NB_ERR_INVALID_ARG;
  if (plan_elems < nb_exchange_plan_elems(cp_size)) return NB_ERR_WORKSPACE;
  hipLaunchKernelGGL(nb::xch_range_kernel, dim3(cp_size), dim3(nb::kPlanThreads), 0, (hipStream_t)stream, doc_ids,
                     pad_mask, B, N, cp_size, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return nb::map_hip(e);
  hipLaunchKernelGGL(nb::xch_offsets_kernel, dim3(1), dim3(nb::kPlanThreads), 0, (hipStream_t)stream, N, cp_size,
                     plan);
  return nb::map_hip(hipGetLastError());
}

size_t nb_exchange_send_index_elems(int cp_size, int N) {
  if (!nb::ranks_ok(N, cp_size)) return 0;
  return (size_t)cp_size * N;
}

int nb_exchange_send_index(const int32_t* plan, int cp_size, int N, int32_t* send_index, size_t elems,
                           void* stream) {
  if (plan == nullptr || send_index == nullptr || !nb::ranks_ok(N, cp_size)) return NB_ERR_INVALID_ARG;
  if ((int64_t)cp_size * N >= ((int64_t)1 << 31)) return NB_ERR_INVALID_ARG;
  if (elems < nb_exchange_send_index_elems(cp_size, N)) return NB_ERR_WORKSPACE;
  hipLaunchKernelGGL(nb::xch_send_index_kernel, dim3(cp_size), dim3(nb::kStreamThreads), 0, (hipStream_t)stream,
                     plan, N, cp_size, send_index);
  return nb::map_hip(hipGetLastError());
}

int nb_exchange_gather(const void* x, const int32_t* plan, int B, int C, int N, int D, int cp_size, int dtype,
                       void* const* recv, void* stream) {
  int vpr = 0;
  const int e = nb::stream_checks(x, plan, B, C, N, D, cp_size, dtype, recv, &vpr);
  if (e != NB_OK) return e;
  nb::XchPtrs ptrs{};
  for (int r = 0; r < cp_size; ++r) ptrs.p[r] = recv[r];
  const dim3 grid(nb::stream_blocks(N, vpr), (unsigned)(B * C), (unsigned)cp_size);
  hipLaunchKernelGGL(nb::xch_gather_kernel, grid, dim3(nb::kStreamThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(x), plan, N, vpr, cp_size, ptrs);
  return nb::map_hip(hipGetLastError());
}

int nb_exchange_scatter_add(void* const* grad_recv, const int32_t* plan, int B, int C, int N, int D, int cp_size,
                            int dtype, void* grad_x, void* stream) {
  int vpr = 0;
  const int e = nb::stream_checks(grad_x, plan, B, C, N, D, cp_size, dtype, grad_recv, &vpr);
  if (e != NB_OK) return e;
  nb::XchPtrs ptrs{};
  for (int r = 0; r < cp_size; ++r) ptrs.p[r] = grad_recv[r];
  const dim3 grid(nb::stream_blocks(N, vpr), (unsigned)(B * C));
  if (dtype == NB_BF16)
    hipLaunchKernelGGL(nb::xch_scatter_add_kernel<__bf16>, grid, dim3(nb::kStreamThreads), 0, (hipStream_t)stream,
                       ptrs, plan, N, vpr, cp_size, reinterpret_cast<__bf16*>(grad_x));
  else
    hipLaunchKernelGGL(nb::xch_scatter_add_kernel<float>, grid, dim3(nb::kStreamThreads), 0, (hipStream_t)stream,
                       ptrs, plan, N, vpr, cp_size, reinterpret_cast<float*>(grad_x));
  return nb::map_hip(hipGetLastError());
}

}  // extern "C"
