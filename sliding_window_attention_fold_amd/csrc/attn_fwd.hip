// Forward of neighbourhood attention: per document, bottom-right causal, left
// window, GQA; saves the log-sum-exp for the backward.
//
// NeMo AutoModel cp_local_ring page (sliding_ring_compute_fa_fwd and the module
// docstring) and blockdiag_cp.kernels page (_cp_blockdiag_varlen): a real query
// row at neighbourhood position p attends the keys of its own document that are
// not after p and, with a window W, not more than W before it.  The segment
// builder hands every row its document's first key (row_klo), so the band of
// row p is [max(row_klo, p - W), p]; padding rows have an empty band and get
// O = 0, LSE = -inf.  Optionally the rounding residual of O is saved too, so
// the backward's Delta = dO . O is formed from an fp32-accurate O.
//
// Work decomposition: one workgroup per (128 query rows, q head, batch row);
// four waves of 32 rows each.  Q stays in registers as the B operand of
// S^T = K Q^T, so every lane owns one query row: its softmax statistics are
// lane-local up to one exchange with the lane 32 away.  K tiles are staged in
// LDS row-major (A operand of S^T), V tiles transposed with the accumulator row
// permutation (A operand of O^T = V^T P^T), P^T is fed from the S^T
// accumulators directly.  Key tiles outside the union of the rows' bands are
// never visited; tiles inside every band of a wave skip the element mask.
#include <math.h>

#include "nb_device.h"
#include "nb_kernels.h"

namespace nb {

template <typename T, int D>
struct FwdCfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  static constexpr int BN = 64;
  static constexpr int KP = D + Pad<T>::elems;    // K tile pitch (elements)
  static constexpr int VP = BN + Pad<T>::elems;   // V^T tile pitch (elements)
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(FwdParams p) {
  typedef FwdCfg<T, D> C;
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) T Ks[C::BN * C::KP];
  __shared__ __attribute__((aligned(16))) T Vt[D * C::VP];
  __shared__ int red[4][2];

  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, ln = lane & 31;
  const int off = p.S - p.L;
  const int i = qt * C::BM + 32 * w + ln;
  const bool in_range = i < p.L;
  const int pos = off + i;
  int bs = pos + 1;
  if (in_range) {
    bs = max(0, p.row_klo[(size_t)b * p.L + i]);  // clamp: never index before the neighbourhood
    if (p.window >= 0) bs = max(bs, pos - p.window);
  }
  const bool real = in_range && bs <= pos;

  // Key range of the wave and of the workgroup (union of the rows' bands).
  const int w_lo = wave_min_i(real ? bs : INT_MAX);
  const int w_hi = wave_max_i(real ? pos + 1 : INT_MIN);
  const int w_bs_max = wave_max_i(real ? bs : INT_MIN);
  const int w_p_min = wave_min_i(real ? pos : INT_MAX);
  const bool w_all_real = wave_min_i(real ? 1 : 0) != 0;
  if (lane == 0) { red[w][0] = w_lo; red[w][1] = w_hi; }
  __syncthreads();
  int kstart = INT_MAX, kend = INT_MIN;
#pragma unroll
  for (int x = 0; x < C::NW; ++x) { kstart = min(kstart, red[x][0]); kend = max(kend, red[x][1]); }

  const size_t qrow = ((size_t)b * p.Hq + h) * p.L + i;
  const T* __restrict__ kbase = reinterpret_cast<const T*>(p.k) + ((size_t)b * p.Hkv + kvh) * p.S * D;
  const T* __restrict__ vbase = reinterpret_cast<const T*>(p.v) + ((size_t)b * p.Hkv + kvh) * p.S * D;

  F qf[D / 16];
  {
    const T* qp = reinterpret_cast<const T*>(p.q) + qrow * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = in_range ? load_frag<T>(qp + 16 * kk + 8 * g) : zero_frag<T>();
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) oacc[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int j0 = kstart; j0 < kend; j0 += C::BN) {
    const int nvalid = min(C::BN, p.S - j0);
    __syncthreads();
    stage_rows<T, C::BN, D, C::KP, C::NT>(Ks, kbase + (size_t)j0 * D, nvalid);
    stage_rows_transposed<T, C::BN, D, C::VP, C::NT>(Vt, vbase + (size_t)j0 * D, nvalid);
    __syncthreads();
    if (j0 >= w_hi || j0 + C::BN <= w_lo) continue;
    const bool full = w_all_real && j0 >= w_bs_max && j0 + C::BN - 1 <= w_p_min;

    f32x16 sacc[C::BN / 32];
#pragma unroll
    for (int sb = 0; sb < C::BN / 32; ++sb) {
      sacc[sb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const F a = load_frag<T>(Ks + (32 * sb + ln) * C::KP + 16 * kk + 8 * g);
        sacc[sb] = mma(a, qf[kk], sacc[sb]);
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < C::BN / 32; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[sb][r] * p.scale_log2;
        if (!full) {
          const int j = j0 + 32 * sb + acc_row(r, g);
          if (j < bs || j > pos) x = -INFINITY;
        }
        sacc[sb][r] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_ref);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) oacc[d] *= alpha;
#pragma unroll
    for (int sb = 0; sb < C::BN / 32; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(sacc[sb][r] - m_ref);
        sacc[sb][r] = e;
        l_run += e;
      }
    }
    m_run = m_new;
#pragma unroll
    for (int m = 0; m < C::BN / 16; ++m) {
      const F pf = acc_to_frag<T>(sacc[m >> 1], m & 1);
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const F a = load_frag<T>(Vt + (32 * d + ln) * C::VP + 16 * m + 8 * g);
        oacc[d] = mma(a, pf, oacc[d]);
      }
    }
  }

  const float l = l_run + __shfl_xor(l_run, 32);
  if (!in_range) return;
  const float inv = real ? 1.f / l : 0.f;
  T* op = reinterpret_cast<T*>(p.o) + qrow * D;
  T* olp = p.o_lo ? reinterpret_cast<T*>(p.o_lo) + qrow * D : nullptr;
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int dd = 32 * d + 8 * rq + 4 * g;
      store_quad_split<T>(op + dd, olp ? olp + dd : nullptr, oacc[d][4 * rq] * inv, oacc[d][4 * rq + 1] * inv,
                          oacc[d][4 * rq + 2] * inv, oacc[d][4 * rq + 3] * inv);
    }
  }
  if (g == 0) p.lse[qrow] = real ? (m_run + log2f(l)) * kLn2 : -INFINITY;
}

template <typename T, int D>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  typedef FwdCfg<T, D> C;
  dim3 grid((p.L + C::BM - 1) / C::BM, p.Hq, p.B);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), grid, dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const FwdParams& p, int D, bool f32, hipStream_t s) {
  if (f32) {
    if (D == 64) return launch_fwd_t<float, 64>(p, s);
    if (D == 128) return launch_fwd_t<float, 128>(p, s);
    if (D == 256) return launch_fwd_t<float, 256>(p, s);
  } else {
    if (D == 64) return launch_fwd_t<bf16, 64>(p, s);
    if (D == 128) return launch_fwd_t<bf16, 128>(p, s);
    if (D == 256) return launch_fwd_t<bf16, 256>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nb
