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
// lane-local up to one exchange with the lane 32 away.  K and V tiles are
// copied global -> LDS asynchronously (double-buffered) and stay row-major: K
// rows are the A operand of S^T, V is read transposed (ds_read_b64_tr_b16) as
// the A operand of O^T = V^T P^T, and P^T is fed from the S^T accumulators
// directly.  Key tiles outside the union of the rows' bands are never visited;
// tiles inside every band of a wave skip the element mask.
#include <math.h>

#include "nb_device.h"
#include "nb_kernels.h"
#include "nb_kv.h"

namespace nb {

// Two workgroups share a CU (bf16, D <= 256): while one runs its softmax on the
// vector units, the other keeps the matrix cores busy, which a single wave per
// SIMD cannot do on its own.  That needs <= 256 registers per wave and <= 80 KB
// of LDS per workgroup, hence 32-key tiles at D = 256.  The float32 debug path
// keeps one workgroup per CU.
//
// Head-dim split (D = 512, the global layers): a wave holding a 32-row group's
// Q fragments and O accumulator over all 512 dims would need ~400 registers,
// so two waves share each 32-row group, one per half of D.  Each forms the
// partial scores of its half, the two halves meet in LDS (every wave adds the
// two partials in the same order, so both hold bit-identical scores and run
// the same softmax), and each accumulates O over its own half.  bf16: eight
// waves (four row groups x two halves) with double-buffered K/V tiles, exactly
// 160 KB of LDS with the exchange; float32: four waves (two row groups) and one
// K/V tile pair (a float32 tile pair is 128 KB).
// SH (bf16, D = 128, short bands: a left window of at most kFwdShortWindow
// keys): 32-key tiles and less read-ahead, so that the K/V buffers and
// registers let three workgroups share a CU -- with bands of a few hundred
// keys a workgroup's loop is short and its load latency dominates; measured on
// the batched short-document workload: the forward 8 % faster, and 7.5 %
// slower on long bands, which keep 64-key tiles.
constexpr int kFwdShortWindow = 512;
template <typename T, int D, bool SH = false>
struct FwdCfg {
  static constexpr int DS = D >= 512 ? 2 : 1;        // waves per 32-row group (halves of D)
  static constexpr int DW = D / DS;                  // head dims of one wave's Q fragments and O
  static constexpr int NRG = (DS == 1 || sizeof(T) == 2) ? 4 : 2;   // 32-row groups per workgroup
  static constexpr int NW = NRG * DS;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NRG;
  static constexpr int BN = (D <= 128 && !SH) ? 64 : 32;  // keys per tile
  static constexpr int OCC = SH ? 3 : (sizeof(T) == 2 && D <= 256) ? 2 : 1;  // workgroups per CU
  static constexpr int NBUF = (sizeof(T) * D > 1024) ? 1 : 2;      // K/V tile pairs in LDS
  // operand fragments read ahead of their MFMA (fewer at 256 dims per wave,
  // where the Q fragments and O accumulators leave little room)
  static constexpr int AHEAD_S = (DW <= 128 && !SH) ? 4 : 2;
  static constexpr int AHEAD_PV = (DW <= 128 && !SH) ? 3 : 2;
  static_assert(!SH || (sizeof(T) == 2 && D == 128), "the short-band shape is for bf16 at 128 dims");
};

// LDS of the forward: the K/V tile pairs and the key-range reduction; with the
// head-dim split also the partial scores, [wave][32-key block][value quad][lane]
// (the reduction, done before the first tile, shares their space).
// After the key loop (bf16), each wave's 32 rows of O leave through LDS
// (nb_device.h: RowStage).  Measured on the 256-dim sliding layer: the forward
// 4 % faster, where every workgroup reaches its stores at about the same time.
template <typename T, int D, bool SH = false>
using FwdStage = RowStage<T, FwdCfg<T, D, SH>::NW, FwdCfg<T, D, SH>::DW>;
template <typename T, int D, bool SH = false, bool SPLIT = (FwdCfg<T, D, SH>::DS > 1)>
struct FwdSmem;
template <typename T, int D, bool SH>
struct FwdSmem<T, D, SH, false> {
  typedef FwdCfg<T, D, SH> C;
  union {
    struct {
      __attribute__((aligned(1024))) T K[C::NBUF][Tile<T, C::BN, D>::ELEMS];
      __attribute__((aligned(1024))) T V[C::NBUF][Tile<T, C::BN, D>::ELEMS];
      int red[C::NW][2];
    };
    FwdStage<T, D, SH> ost;
  };
};
template <typename T, int D, bool SH>
struct FwdSmem<T, D, SH, true> {
  typedef FwdCfg<T, D, SH> C;
  union {
    struct {
      __attribute__((aligned(1024))) T K[C::NBUF][Tile<T, C::BN, D>::ELEMS];
      __attribute__((aligned(1024))) T V[C::NBUF][Tile<T, C::BN, D>::ELEMS];
      union {
        f32x4 xs[C::NW][C::BN / 32][4][64];
        int red[C::NW][2];
      };
    };
    FwdStage<T, D, SH> ost;
  };
};

// KV selects how K/V rows are found: kKvConcat, one concatenated buffer
// (p.kv.k[0] / p.kv.v[0], S rows per (batch, kv head)); kKvPair, the chunk
// table for workgroups whose key range touches at most two chunks (the rest
// return at once); kKvAny, the chunk table for the workgroups whose range
// touches three or more (the rest return).  A chunk-table forward launches
// kKvPair, then kKvAny over the same grid when the chunk lengths allow such
// ranges, so the common loop carries none of the general lookup's registers.
template <typename T, int D, int KV, bool SH = false>
__global__ __launch_bounds__((FwdCfg<T, D, SH>::NT), (FwdCfg<T, D, SH>::OCC)) void attn_fwd_kernel(FwdParams p) {
  typedef FwdCfg<T, D, SH> C;
  typedef Tile<T, C::BN, D> TL;
  typedef typename Frag<T>::type F;
  // two K/V tile pairs (one is being filled by DMA while the other is read),
  // or one where a float32 pair fills most of the LDS
  __shared__ FwdSmem<T, D, SH> sm;
  T* const K0 = sm.K[0];
  T* const V0 = sm.V[0];
  T* const K1 = sm.K[C::NBUF - 1];
  T* const V1 = sm.V[C::NBUF - 1];
  int (*red)[2] = sm.red;

  // Work order: the kv group (batch row, kv head) varies fastest, so with the
  // round-robin dispatch over 8 XCDs every group stays on one XCD and the K/V
  // window its query tiles share stays in that XCD's L2; the group's q heads
  // come next, then the query tiles, in grid order or, when the grid takes
  // more than one round of workgroups, longest band first (qt_order).
  const int grp = p.Hq / p.Hkv;
  const int ngroups = p.B * p.Hkv;
  const int gid = blockIdx.x % ngroups, rest = blockIdx.x / ngroups;
  const int b = gid / p.Hkv, kvh = gid % p.Hkv;
  const int h = kvh * grp + rest % grp, rank = rest / grp;
  const int qt = p.qt_order ? p.qt_order[(size_t)b * ((p.L + C::BM - 1) / C::BM) + rank] : rank;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, ln = lane & 31;
  const int rg = C::DS > 1 ? w % C::NRG : w;   // 32-row group
  const int hf = C::DS > 1 ? w / C::NRG : 0;   // half of D (head-dim split)
  const int i = qt * C::BM + 32 * rg + ln;
  const bool in_range = i < p.L;
  const int pq = p.q_off + i;               // the row's key position
  const int pos = min(pq, p.S - 1);         // its band's last key
  int bs = pq + 1;
  if (in_range) {
    bs = max(0, p.row_klo[(size_t)b * p.L + i] - p.k_origin);  // clamp: never index before the keys
    if (p.window >= 0) bs = max(bs, pq - p.window);
  }
  const bool real = in_range && bs <= pos;

  // Key range of the wave and of the workgroup (union of the rows' bands).
  // (wave reductions are uniform; readfirstlane lets the compiler see it, so
  // the tile decisions below are scalar branches)
  const int w_lo = __builtin_amdgcn_readfirstlane(wave_min_i(real ? bs : INT_MAX));
  const int w_hi = __builtin_amdgcn_readfirstlane(wave_max_i(real ? pos + 1 : INT_MIN));
  const int w_bs_max = __builtin_amdgcn_readfirstlane(wave_max_i(real ? bs : INT_MIN));
  const int w_p_min = __builtin_amdgcn_readfirstlane(wave_min_i(real ? pos : INT_MAX));
  const bool w_all_real = __builtin_amdgcn_readfirstlane(wave_min_i(real ? 1 : 0)) != 0;
  if (lane == 0) { red[w][0] = w_lo; red[w][1] = w_hi; }
  __syncthreads();
  int kstart = INT_MAX, kend = INT_MIN;
#pragma unroll
  for (int x = 0; x < C::NW; ++x) { kstart = min(kstart, red[x][0]); kend = max(kend, red[x][1]); }
  kstart = __builtin_amdgcn_readfirstlane(kstart);   // uniform: scalar tile bounds and addresses
  kend = __builtin_amdgcn_readfirstlane(kend);

  const size_t qrow = ((size_t)b * p.Hq + h) * p.L + i;
  const int bh = b * p.Hkv + kvh;
  // kbase + j * D is key j's row (the concatenated buffer)
  const T* __restrict__ kbase = reinterpret_cast<const T*>(p.kv.k[0]) + (size_t)bh * p.S * D;
  const T* __restrict__ vbase = reinterpret_cast<const T*>(p.kv.v[0]) + (size_t)bh * p.S * D;
  const KvPair<T, C::BN> pair = KV == kKvConcat ? KvPair<T, C::BN>() : KvPair<T, C::BN>(p.kv, bh, kstart, kend, D);
  if constexpr (KV != kKvConcat) {
    if (pair.ok != (KV == kKvPair)) return;   // uniform: the other launch owns it
  }
  const TileDma<T, C::BN, D, C::NW> dma;   // K and V tiles share one layout
  auto load = [&](T* Ks, T* Vs, int j0) __attribute__((always_inline)) {
    if constexpr (KV == kKvAny) {
      kv_tile_load<T, C::BN, D, C::NW>(dma, p.kv, bh, j0, min(C::BN, p.S - j0), Ks, Vs);
    } else if constexpr (KV == kKvPair) {
      pair.load(dma, j0, Ks, Vs);
    } else {
      const int nv = min(C::BN, p.S - j0);
      if constexpr (C::DS > 1) {
        // Unseen copies (nb_device.h): the loop's own wait before each tile's
        // barrier orders the reads; the compiler would otherwise wait for the
        // next tile's copies before this tile's V reads.  Measured: 25 %
        // faster at D = 512; at D <= 256 the builtin copies are as fast or
        // faster (config 4 -3 %), so they stay there.
        dma.issue_unseen(Ks, kbase + (size_t)j0 * D, nv);
        dma.issue_unseen(Vs, vbase + (size_t)j0 * D, nv);
      } else {
        dma.issue(Ks, kbase + (size_t)j0 * D, nv);
        dma.issue(Vs, vbase + (size_t)j0 * D, nv);
      }
    }
  };
  if (kstart < kend) load(K0, V0, kstart);

  F qf[C::DW / 16];
  {
    // rows past L read row L-1 (in bounds) and are zeroed
    const T* qp = reinterpret_cast<const T*>(p.q) + (((size_t)b * p.Hq + h) * p.L + min(i, p.L - 1)) * D + hf * C::DW;
#pragma unroll
    for (int kk = 0; kk < C::DW / 16; ++kk) {
      qf[kk] = load_frag<T>(qp + 16 * kk + 8 * g);
      if (!in_range) qf[kk] = zero_frag<T>();
    }
  }

  const TileAccess<T, TL> acc(ln, lane);  // K rows: this lane reads key row 32*sb + ln

  f32x16 oacc[C::DW / 32];
#pragma unroll
  for (int d = 0; d < C::DW / 32; ++d) oacc[d] = f32x16{};
  // m_ref: exponent reference of the row (log2 units, scaled scores); l_run: the
  // row's sum of 2^(s - m_ref) over this lane's keys (the other half is in lane^32).
  float m_ref = -INFINITY, l_run = 0.f;

  auto compute = [&](const T* Ks, const T* Vs, int j0) __attribute__((always_inline)) {
    constexpr int NSB = C::BN / 32;
    const bool active = !(j0 >= w_hi || j0 + C::BN <= w_lo);
    if constexpr (C::DS == 1) {
      if (!active) return;
    }
    const bool full = w_all_real && j0 >= w_bs_max && j0 + C::BN - 1 <= w_p_min;
    f32x16 sacc[NSB];
    constexpr int NK = C::DW / 16;   // contraction steps of this wave's dims
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) sacc[sb] = f32x16{};
    if (active) {
      lds_mfma_pipeline<NSB * NK, C::AHEAD_S, F>(
          [&](int x) { return acc.row(Ks, x / NK, x % NK + hf * NK); },
          [&](int x, const F& a) { sacc[x / NK] = mma(a, qf[x % NK], sacc[x / NK]); });
    }
    if constexpr (C::DS > 1) {
      // the two halves' partial scores meet in LDS; every wave of the workgroup
      // reaches the barrier, active or not
      if (active) {
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            sm.xs[w][sb][qd][lane] = f32x4{sacc[sb][4 * qd], sacc[sb][4 * qd + 1], sacc[sb][4 * qd + 2],
                                           sacc[sb][4 * qd + 3]};
      }
      __syncthreads();
      if (!active) return;
      const int partner = hf ? w - C::NRG : w + C::NRG;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 o = sm.xs[partner][sb][qd][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e)   // half 0's partial first, in both waves
            sacc[sb][4 * qd + e] = hf ? o[e] + sacc[sb][4 * qd + e] : sacc[sb][4 * qd + e] + o[e];
        }
      }
    }
    // The element mask, only on tiles that a band edge crosses (one uniform
    // branch around the whole block: per element the compiler would turn it
    // into selects executed on every tile).
    if (!full) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * sb + acc_row(r, g);
          if ((j < bs) | (j > pos)) sacc[sb][r] = -INFINITY;
        }
      }
    }
    // Row maximum of the raw scores; scaling by the positive scale_log2
    // commutes with the maximum (rounding is monotonic), so the scale folds
    // into the exponent's fma below.
    float tmax = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[sb][r]);
    }
    tmax = fmaxf(tmax, other_half(tmax)) * p.scale_log2;
    // Move the reference (and rescale O) when some row's maximum passed it by
    // more than kRefLag (0: any growth); the wave decides together so the
    // branch is uniform, and rows whose maximum did not grow scale by 1.
    if (__any(tmax > m_ref + kRefLag)) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < C::DW / 32; ++d) oacc[d] *= alpha;
      m_ref = m_new;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(sacc[sb][r], p.scale_log2, -m_use));
        sacc[sb][r] = e;
        l_run += e;
      }
    }
    F pf[C::BN / 16];
#pragma unroll
    for (int m = 0; m < C::BN / 16; ++m) pf[m] = acc_to_frag<T>(sacc[m >> 1], m & 1);
    constexpr int ND = C::DW / 32;
    lds_mfma_pipeline<C::BN / 16 * ND, C::AHEAD_PV, F>(
        [&](int x) { return acc.col(Vs, x % ND + hf * ND, x / ND); },
        [&](int x, const F& a) { oacc[x % ND] = mma(a, pf[x / ND], oacc[x % ND]); });
  };

  if constexpr (C::NBUF == 2) {
    // Double-buffered key loop: the DMA of the next tile is issued right after
    // the barrier that frees its buffer, then the current tile is computed.
    for (int j0 = kstart; j0 < kend; j0 += 2 * C::BN) {
      wait_global();
      __syncthreads();
      if (j0 + C::BN < kend) load(K1, V1, j0 + C::BN);
      __builtin_amdgcn_sched_barrier(0);
      compute(K0, V0, j0);
      if (j0 + C::BN >= kend) break;
      wait_global();
      __syncthreads();
      if (j0 + 2 * C::BN < kend) load(K0, V0, j0 + 2 * C::BN);
      __builtin_amdgcn_sched_barrier(0);
      compute(K1, V1, j0 + C::BN);
    }
  } else {
    // One tile pair: the next tile's copy waits until every wave is done
    // with the current one.
    for (int j0 = kstart; j0 < kend; j0 += C::BN) {
      wait_global();
      __syncthreads();
      compute(K0, V0, j0);
      __syncthreads();
      if (j0 + C::BN < kend) load(K0, V0, j0 + C::BN);
    }
  }

  const float l = l_run + other_half(l_run);
  const float inv = real ? 1.f / l : 0.f;
  if constexpr (FwdStage<T, D, SH>::ON) {
    T* const st = &sm.ost.r[w][0][0];
    const int i_grp = qt * C::BM + 32 * rg;   // the wave's first row (uniform: a scalar store base)
    const size_t grp0 = (((size_t)b * p.Hq + h) * p.L + i_grp) * D + hf * C::DW;
    const int nrows = min(32, p.L - i_grp);
    __syncthreads();   // every wave is done with the K/V tiles the staging overwrites
    stage_rows_in<T, C::DW>(st, oacc, inv);
    stage_rows_store<T, C::DW>(st, reinterpret_cast<T*>(p.o) + grp0, D, nrows);
    if (p.o_lo != nullptr) {
      // what the rounding to bf16 left over, as one byte per element (the
      // same products rounded again; the staged O rows were read back first:
      // a wave's LDS operations complete in order)
      uint8_t* const sc = reinterpret_cast<uint8_t*>(st);
      stage_codes_in<C::DW>(sc, oacc, inv);
      stage_codes_store<C::DW>(sc, reinterpret_cast<uint8_t*>(p.o_lo) + grp0, D, nrows);
    }
    if (g == 0 && hf == 0 && in_range) p.lse[qrow] = real ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
    return;
  }
  // float32: O is the fp32 result itself (no residual)
  if (!in_range) return;
  T* op = reinterpret_cast<T*>(p.o) + qrow * D + hf * C::DW;
#pragma unroll
  for (int d = 0; d < C::DW / 32; ++d) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int dd = 32 * d + 8 * rq + 4 * g;
      store_quad<T>(op + dd, oacc[d][4 * rq] * inv, oacc[d][4 * rq + 1] * inv, oacc[d][4 * rq + 2] * inv,
                    oacc[d][4 * rq + 3] * inv);
    }
  }
  if (g == 0 && hf == 0) p.lse[qrow] = real ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
}

// The concatenated neighbourhood: one chunk of S rows starting at row 0.
static bool kv_concatenated(const KvChunks& c, int S) { return c.n == 1 && c.start[0] == 0 && c.rows[0] == S; }

template <typename T, int D, bool SH = false>
static hipError_t launch_fwd_t(const FwdParams& p_in, hipStream_t s) {
  typedef FwdCfg<T, D, SH> C;
  dim3 grid((unsigned)((p_in.L + C::BM - 1) / C::BM) * p_in.Hq * p_in.B);
  // The launch order only pays when workgroups wait for slots (and it is
  // built for kFwdOrderRows-row tiles).
  FwdParams p = p_in;
  if (C::BM != kFwdOrderRows || (long long)grid.x <= (long long)device_cu_count() * C::OCC) p.qt_order = nullptr;
  if constexpr (D >= 512) {   // the global layers' head dim: one concatenated K/V buffer only
    if (!kv_concatenated(p.kv, p.S)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, kKvConcat>), grid, dim3(C::NT), 0, s, p);
    return hipGetLastError();
  } else {
    if (kv_concatenated(p.kv, p.S)) {
      hipLaunchKernelGGL((attn_fwd_kernel<T, D, kKvConcat, SH>), grid, dim3(C::NT), 0, s, p);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, kKvPair, SH>), grid, dim3(C::NT), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !kv_may_need_general(p.kv, p.window, C::BM, C::BN)) return e;
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, kKvAny, SH>), grid, dim3(C::NT), 0, s, p);
    return hipGetLastError();
  }
}

hipError_t launch_attn_fwd(const FwdParams& p, int D, bool f32, hipStream_t s) {
  if (f32) {
    if (D == 64) return launch_fwd_t<float, 64>(p, s);
    if (D == 128) return launch_fwd_t<float, 128>(p, s);
    if (D == 256) return launch_fwd_t<float, 256>(p, s);
    if (D == 512) return launch_fwd_t<float, 512>(p, s);
  } else {
    if (D == 64) return launch_fwd_t<bf16, 64>(p, s);
    if (D == 128)   // short bands (a small left window): the three-per-CU shape
      return p.window >= 0 && p.window <= kFwdShortWindow ? launch_fwd_t<bf16, 128, true>(p, s)
                                                          : launch_fwd_t<bf16, 128>(p, s);
    if (D == 256) return launch_fwd_t<bf16, 256>(p, s);
    if (D == 512) return launch_fwd_t<bf16, 512>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nb
