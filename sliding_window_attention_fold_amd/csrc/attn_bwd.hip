// Backward of neighbourhood attention with no forward recompute.
//
// NeMo AutoModel cp_local_ring page, sliding_ring_compute_fa_bwd: the backward
// runs from the saved output and log-sum-exp and returns dQ and the per-owner
// dK/dV.  With P = exp(scale * q.k - LSE) on the band and 0 elsewhere:
//   Delta_i = sum_d dO_id O_id        (equals sum_j P_ij dP_ij)
//   dP = dO V^T,  dS = P * (dP - Delta)
//   dV = sum_{h in group} P^T dO_h,   dK = scale * sum_{h in group} dS^T Q_h,
//   dQ = scale * dS K.
// Two passes keep every output owned by exactly one workgroup (no atomics, the
// result is bitwise reproducible):
//   1. dQ:     one workgroup per (128 query rows, q head, batch row); Q and dO in
//      registers, K/V staged row-major and K transposed per key tile.  Its
//      prologue forms Delta = dO . O (O = stored value + saved rounding residual)
//      and publishes it for pass 2;
//   2. dK/dV:  one workgroup per (128 keys, kv head, batch row), four waves of
//      32 keys; K and V stay in registers, the loop runs over the group's q
//      heads and the 32-row query tiles whose bands reach the keys, with Q and dO
//      staged in LDS both row-major (A operands of S and dP) and transposed (A
//      operands of dV^T and dK^T).  Keys no query attends come out as exact 0.
#include <math.h>

#include "nb_device.h"
#include "nb_kernels.h"

namespace nb {

// ---------------------------------------------------------------- dK / dV

template <typename T, int D>
struct DkvCfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BK = 32 * NW;               // keys per workgroup
  static constexpr int BQ = 32;                    // query rows per step
  static constexpr int RP = D + Pad<T>::elems;      // row-major pitch
  static constexpr int TP = BQ + Pad<T>::elems;     // transposed pitch
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BwdParams p) {
  typedef DkvCfg<T, D> C;
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) T Qs[C::BQ * C::RP];
  __shared__ __attribute__((aligned(16))) T dOs[C::BQ * C::RP];
  __shared__ __attribute__((aligned(16))) T Qt[D * C::TP];
  __shared__ __attribute__((aligned(16))) T dOt[D * C::TP];
  __shared__ float lse_s[C::BQ], delta_s[C::BQ];
  __shared__ int bs_s[C::BQ];
  __shared__ int n_tiles_s;

  const int kt = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int grp = p.Hq / p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, ln = lane & 31;
  const int off = p.S - p.L;
  const int j0 = kt * C::BK;                      // first key of the workgroup
  const int jw = j0 + 32 * w;                     // first key of the wave
  const int j = jw + ln;                          // this lane's key (C column / B operand)
  const int jmax = min(j0 + C::BK, p.S) - 1;      // last key of the workgroup

  // Query tiles whose bands can reach [j0, jmax]: rows from max(0, j0 - off);
  // the band start bs_i = max(row_klo_i, p_i - W) is nondecreasing in i, so the
  // tiles whose first row starts its band at or before jmax form a prefix.
  const int i_first = max(0, j0 - off);
  const int t_first = i_first / C::BQ;
  const int n_q_tiles = (p.L + C::BQ - 1) / C::BQ;
  if (tid == 0) n_tiles_s = 0;
  __syncthreads();
  for (int base = t_first; base < n_q_tiles; base += C::NT) {
    const int t = base + tid;
    int pred = 0;
    if (t < n_q_tiles) {
      const int i = t * C::BQ;
      int bsi = p.row_klo[(size_t)b * p.L + i];
      if (p.window >= 0) bsi = max(bsi, off + i - p.window);
      pred = bsi <= jmax;
    }
    const int cnt = __syncthreads_count(pred);
    if (tid == 0) n_tiles_s += cnt;
    if (cnt < C::NT) break;
    __syncthreads();
  }
  __syncthreads();
  const int t_end = t_first + n_tiles_s;

  const T* __restrict__ kp = reinterpret_cast<const T*>(p.k) + (((size_t)b * p.Hkv + kvh) * p.S + j) * D;
  const T* __restrict__ vp = reinterpret_cast<const T*>(p.v) + (((size_t)b * p.Hkv + kvh) * p.S + j) * D;
  const bool key_ok = j < p.S;
  F kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    kf[kk] = key_ok ? load_frag<T>(kp + 16 * kk + 8 * g) : zero_frag<T>();
    vf[kk] = key_ok ? load_frag<T>(vp + 16 * kk + 8 * g) : zero_frag<T>();
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) { dkacc[d] = f32x16{}; dvacc[d] = f32x16{}; }

  for (int hh = 0; hh < grp; ++hh) {
    const int h = kvh * grp + hh;
    const size_t rowbase = ((size_t)b * p.Hq + h) * p.L;
    for (int t = t_first; t < t_end; ++t) {
      const int i0 = t * C::BQ;
      const int nrows = min(C::BQ, p.L - i0);
      __syncthreads();
      const T* qsrc = reinterpret_cast<const T*>(p.q) + (rowbase + i0) * D;
      const T* dsrc = reinterpret_cast<const T*>(p.dout) + (rowbase + i0) * D;
      stage_rows<T, C::BQ, D, C::RP, C::NT>(Qs, qsrc, nrows);
      stage_rows<T, C::BQ, D, C::RP, C::NT>(dOs, dsrc, nrows);
      stage_rows_transposed<T, C::BQ, D, C::TP, C::NT>(Qt, qsrc, nrows);
      stage_rows_transposed<T, C::BQ, D, C::TP, C::NT>(dOt, dsrc, nrows);
      if (tid < C::BQ) {
        const int i = i0 + tid;
        int bsi = off + i + 1;  // empty band
        float lse2 = 0.f, dl = 0.f;
        if (i < p.L) {
          const int pos = off + i;
          bsi = max(0, p.row_klo[(size_t)b * p.L + i]);
          if (p.window >= 0) bsi = max(bsi, pos - p.window);
          if (bsi <= pos) {
            lse2 = p.lse[rowbase + i] * kLog2e;
            dl = p.delta[rowbase + i];
          }
        }
        bs_s[tid] = bsi;
        lse_s[tid] = lse2;
        delta_s[tid] = dl;
      }
      __syncthreads();

      // rows of this tile: positions off+i0 .. off+i0+nrows-1
      const int p_min = off + i0, p_max = off + i0 + nrows - 1;
      const int bs_min = bs_s[0], bs_max = bs_s[nrows - 1];
      if (jw > p_max || jw + 31 < bs_min) continue;
      // every (row, key) pair of the wave inside the band: no element mask
      const bool full = (nrows == C::BQ) && jw >= bs_max && jw + 31 <= p_min;

      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const F a = load_frag<T>(Qs + ln * C::RP + 16 * kk + 8 * g);
        sacc = mma(a, kf[kk], sacc);
        const F c = load_frag<T>(dOs + ln * C::RP + 16 * kk + 8 * g);
        dpacc = mma(c, vf[kk], dpacc);
      }
      // accumulator r: query row acc_row(r, g) of the tile, key j
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = acc_row(r, g);
        const int pos = off + i0 + qi;
        float pr = exp2f(sacc[r] * p.scale_log2 - lse_s[qi]);
        if (!full) {
          if (qi >= nrows || j < bs_s[qi] || j > pos) pr = 0.f;
        }
        sacc[r] = pr;
        dpacc[r] = pr * (dpacc[r] - delta_s[qi]);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const F pf = acc_to_frag<T>(sacc, m);
        const F sf = acc_to_frag<T>(dpacc, m);
#pragma unroll
        for (int d = 0; d < D / 32; ++d) {
          const F a = load_frag<T>(dOt + (32 * d + ln) * C::TP + 16 * m + 8 * g);
          dvacc[d] = mma(a, pf, dvacc[d]);
          const F c = load_frag<T>(Qt + (32 * d + ln) * C::TP + 16 * m + 8 * g);
          dkacc[d] = mma(c, sf, dkacc[d]);
        }
      }
    }
  }

  if (!key_ok) return;
  T* dkp = reinterpret_cast<T*>(p.dk) + (((size_t)b * p.Hkv + kvh) * p.S + j) * D;
  T* dvp = reinterpret_cast<T*>(p.dv) + (((size_t)b * p.Hkv + kvh) * p.S + j) * D;
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int dd = 32 * d + 8 * rq + 4 * g;
      store_quad<T>(dkp + dd, dkacc[d][4 * rq] * p.scale, dkacc[d][4 * rq + 1] * p.scale,
                    dkacc[d][4 * rq + 2] * p.scale, dkacc[d][4 * rq + 3] * p.scale);
      store_quad<T>(dvp + dd, dvacc[d][4 * rq], dvacc[d][4 * rq + 1], dvacc[d][4 * rq + 2],
                    dvacc[d][4 * rq + 3]);
    }
  }
}

// ---------------------------------------------------------------- dQ

template <typename T, int D>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  static constexpr int BN = (sizeof(T) == 4 && D == 256) ? 32 : 64;
  static constexpr int RP = D + Pad<T>::elems;
  static constexpr int TP = BN + Pad<T>::elems;
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdParams p) {
  typedef DqCfg<T, D> C;
  typedef typename Frag<T>::type F;
  __shared__ __attribute__((aligned(16))) T Ks[C::BN * C::RP];
  __shared__ __attribute__((aligned(16))) T Vs[C::BN * C::RP];
  __shared__ __attribute__((aligned(16))) T Kt[D * C::TP];
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
  F qf[D / 16], df[D / 16];
  {
    const T* qp = reinterpret_cast<const T*>(p.q) + qrow * D;
    const T* dp = reinterpret_cast<const T*>(p.dout) + qrow * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      qf[kk] = in_range ? load_frag<T>(qp + 16 * kk + 8 * g) : zero_frag<T>();
      df[kk] = in_range ? load_frag<T>(dp + 16 * kk + 8 * g) : zero_frag<T>();
    }
  }
  const float lse2 = real ? p.lse[qrow] * kLog2e : 0.f;
  // Delta_i = dO_i . O_i with O taken as the stored value plus its saved
  // rounding residual; published for the dK/dV pass, which runs after this one.
  float dl = 0.f;
  {
    float part = 0.f;
    if (in_range) {
      const T* op = reinterpret_cast<const T*>(p.o) + qrow * D;
      const T* olp = p.o_lo ? reinterpret_cast<const T*>(p.o_lo) + qrow * D : nullptr;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const F ov = load_frag<T>(op + 16 * kk + 8 * g);
        const F ol = olp ? load_frag<T>(olp + 16 * kk + 8 * g) : zero_frag<T>();
#pragma unroll
        for (int t = 0; t < 8; ++t) part += to_f32(df[kk][t]) * (to_f32(ov[t]) + to_f32(ol[t]));
      }
    }
    dl = part + __shfl_xor(part, 32);
    if (!real) dl = 0.f;
    if (in_range && g == 0) p.delta[qrow] = dl;
  }
  const T* __restrict__ kbase = reinterpret_cast<const T*>(p.k) + ((size_t)b * p.Hkv + kvh) * p.S * D;
  const T* __restrict__ vbase = reinterpret_cast<const T*>(p.v) + ((size_t)b * p.Hkv + kvh) * p.S * D;

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) dqacc[d] = f32x16{};

  for (int j0 = kstart; j0 < kend; j0 += C::BN) {
    const int nvalid = min(C::BN, p.S - j0);
    __syncthreads();
    stage_rows<T, C::BN, D, C::RP, C::NT>(Ks, kbase + (size_t)j0 * D, nvalid);
    stage_rows<T, C::BN, D, C::RP, C::NT>(Vs, vbase + (size_t)j0 * D, nvalid);
    stage_rows_transposed<T, C::BN, D, C::TP, C::NT>(Kt, kbase + (size_t)j0 * D, nvalid);
    __syncthreads();
    if (j0 >= w_hi || j0 + C::BN <= w_lo) continue;
    const bool full = w_all_real && j0 >= w_bs_max && j0 + C::BN - 1 <= w_p_min;

    f32x16 sacc[C::BN / 32], dpacc[C::BN / 32];
#pragma unroll
    for (int sb = 0; sb < C::BN / 32; ++sb) {
      sacc[sb] = f32x16{};
      dpacc[sb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const F a = load_frag<T>(Ks + (32 * sb + ln) * C::RP + 16 * kk + 8 * g);
        sacc[sb] = mma(a, qf[kk], sacc[sb]);
        const F c = load_frag<T>(Vs + (32 * sb + ln) * C::RP + 16 * kk + 8 * g);
        dpacc[sb] = mma(c, df[kk], dpacc[sb]);
      }
    }
#pragma unroll
    for (int sb = 0; sb < C::BN / 32; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = exp2f(sacc[sb][r] * p.scale_log2 - lse2);
        if (!full) {
          const int jj = j0 + 32 * sb + acc_row(r, g);
          if (!real || jj < bs || jj > pos) pr = 0.f;
        }
        dpacc[sb][r] = pr * (dpacc[sb][r] - dl);
      }
    }
#pragma unroll
    for (int m = 0; m < C::BN / 16; ++m) {
      const F sf = acc_to_frag<T>(dpacc[m >> 1], m & 1);
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const F a = load_frag<T>(Kt + (32 * d + ln) * C::TP + 16 * m + 8 * g);
        dqacc[d] = mma(a, sf, dqacc[d]);
      }
    }
  }

  if (!in_range) return;
  T* dqp = reinterpret_cast<T*>(p.dq) + qrow * D;
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      store_quad<T>(dqp + 32 * d + 8 * rq + 4 * g, dqacc[d][4 * rq] * p.scale,
                    dqacc[d][4 * rq + 1] * p.scale, dqacc[d][4 * rq + 2] * p.scale,
                    dqacc[d][4 * rq + 3] * p.scale);
    }
  }
}

// ---------------------------------------------------------------- launch

template <typename T, int D>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
  {  // dQ first: it also publishes Delta for the dK/dV pass
    typedef DqCfg<T, D> C;
    dim3 grid((p.L + C::BM - 1) / C::BM, p.Hq, p.B);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D>), grid, dim3(C::NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    typedef DkvCfg<T, D> C;
    dim3 grid((p.S + C::BK - 1) / C::BK, p.Hkv, p.B);
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D>), grid, dim3(C::NT), 0, s, p);
    return hipGetLastError();
  }
}

hipError_t launch_attn_bwd(const BwdParams& p, int D, bool f32, hipStream_t s) {
  if (f32) {
    if (D == 64) return launch_bwd_t<float, 64>(p, s);
    if (D == 128) return launch_bwd_t<float, 128>(p, s);
    if (D == 256) return launch_bwd_t<float, 256>(p, s);
  } else {
    if (D == 64) return launch_bwd_t<bf16, 64>(p, s);
    if (D == 128) return launch_bwd_t<bf16, 128>(p, s);
    if (D == 256) return launch_bwd_t<bf16, 256>(p, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- owner flags

// attended[o] = 1 iff some batch row has a covered key in chunk o: a key j is
// covered iff j >= kcov_lo[b] and folded[b, j] > 0 (every covered key is
// attended by at least one real query row, see the segment builder).
__global__ __launch_bounds__(256) void owner_flags_kernel(OwnerParams p) {
  const int o = blockIdx.x;
  const int a = p.off[o], e = p.off[o + 1];
  int found = 0;
  for (int b = 0; b < p.B && !found; ++b) {
    const int lo = max(a, p.kcov_lo[b]);
    for (int jj = lo + threadIdx.x; jj < e; jj += 256) {
      if (p.folded[(size_t)b * p.S + jj] > 0) { found = 1; break; }
    }
    found = __syncthreads_or(found);
  }
  if (threadIdx.x == 0) p.attended[o] = found ? 1 : 0;
}

hipError_t launch_owner_flags(const OwnerParams& p, hipStream_t s) {
  hipLaunchKernelGGL(owner_flags_kernel, dim3(p.n_owner), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace nb
