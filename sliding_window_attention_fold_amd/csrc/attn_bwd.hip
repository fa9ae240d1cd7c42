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
//   1. dQ:     one workgroup per (query rows, q head, batch row).  bf16 at
//      D <= 128: eight query groups of 32 rows (256 rows), one wave each,
//      forming S, P, dP, dS and all of dQ; otherwise four query groups, each
//      served by a pair of waves (Q side: S, P; dO side: dP; they swap P and dP
//      through LDS and each accumulates half of dQ).  K/V tiles are copied into LDS asynchronously (double-buffered); K^T
//      is read transposed from the same row-major tile.  Its prologue forms
//      Delta = dO . O (O = stored value + saved rounding residual) and
//      publishes it for pass 2;
//   2. dK/dV:  one workgroup per (128 keys, kv head, batch row): four key groups
//      of 32 keys, each served by a pair of waves (K side: S, P, dV; V side:
//      dP, dS, dK; P crosses through LDS).  A one-workgroup pre-pass orders
//      the key tiles by decreasing work so the longest start first.  The loop runs over the group's q
//      heads and the 32-row query tiles whose bands reach the keys.  Q and dO
//      tiles (plus their rows' LSE, Delta, band start) are copied into LDS
//      asynchronously and read row-wise (A operands of S and dP) and transposed
//      (A operands of dV^T and dK^T).  Keys no query attends come out as exact 0.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "nb_device.h"
#include "nb_kernels.h"
#include "nb_kv.h"

namespace nb {

// ---------------------------------------------------------------- dK / dV

// NKG key groups of 32 keys, two waves (roles) per group.  Role A holds the
// group's K rows, forms S = Q K^T and P, hands P to its partner through LDS and
// accumulates dV^T = dO^T P; role B holds the V rows, forms dP = dO V^T, takes
// P, forms dS = P (dP - Delta) and accumulates dK^T = Q^T dS.  Splitting the
// roles keeps each wave under 256 registers at D = 256 (K or V rows plus one
// accumulator), so two waves share each SIMD and hide each other's latency
// (measured: one wave per SIMD with 512 registers and deep operand read-ahead,
// four waves per workgroup, ran the backward 1.5x slower).
// Workgroup shape: eight waves (four groups of 32 keys or 32 query rows, two
// roles each); the LDS of one workgroup is 160 KB / OCC at most.
// At D = 512 (the global layers) a wave holding 32 keys' K or V rows over all
// 512 dims plus half of their gradient's columns needs ~300 registers: four
// waves per workgroup (one per SIMD, 512 registers each).
template <typename T, int D>
struct BwdShape {
  static constexpr int OCC = 1;
  static constexpr int NT = D >= 512 ? 256 : 512;
  static constexpr int LDS_BUDGET = 160 * 1024 / OCC;
};

template <typename T, int D>
struct DkvCfg {
  static constexpr int NT = BwdShape<T, D>::NT;
  static constexpr int NW = NT / 64;
  // Column halves of the gradient accumulators: at D = 512 each role runs on
  // two waves, which form the same S (or dP, dS) and keep one half of dV^T
  // (dK^T) each -- the S / dP products are done twice (1.5x the dK/dV pass's
  // matrix work) but no partial sums cross between waves.
  static constexpr int HS = D >= 512 ? 2 : 1;
  static constexpr int DA = D / HS;      // columns of one wave's accumulator
  static constexpr int NKG = NW / (2 * HS);   // key groups of 32 keys
  static constexpr int BK = 32 * NKG;  // keys per workgroup
  static constexpr int BQ = 32;        // query rows per step
  // operand fragments read ahead of their MFMA; 0 = plain loop (the float path
  // and D = 512 have no registers to spare).  At D = 256 the room comes from
  // the XOR-addressed readers (XREAD: one and two address registers per lane
  // instead of sixteen), in the dK/dV-only kernel (AHEAD_DS); the kernel that
  // also runs dQ items carries their registers and reads none ahead.
  static constexpr bool XREAD = sizeof(T) == 2 && D == 256;
  static constexpr int AHEAD = (D <= 128 && sizeof(T) == 2) ? 4 : 0;
  static constexpr int AHEAD_DS = XREAD ? 3 : AHEAD;
  static constexpr int TILE_BYTES = BQ * D * (int)sizeof(T);
  static constexpr int PEX_BYTES = NKG * 4 * 64 * 16;   // one P hand-over buffer
  static constexpr int META_BYTES = 3 * 64 * 4;         // LSE, Delta, band starts of one step
  static constexpr bool fits(int ns, int npex) {
    return ns * (2 * TILE_BYTES + META_BYTES) + npex * PEX_BYTES + 1024 <= BwdShape<T, D>::LDS_BUDGET;
  }
  // Schedules (measured per head size):
  //  - skewed (D > 128): role B one step behind role A; ring slots for the
  //    previous step, the current one and one step of copies in flight, two
  //    hand-over buffers;
  //  - in step, three slots (copies two steps ahead), two hand-over buffers,
  //    one barrier per step;
  //  - in step, two slots, one hand-over buffer, two barriers per step.
  //  - one slot (float32 at D = 512, whose Q + dO tiles take 128 KB): the
  //    next step's copies wait for the end of the current step.
  static constexpr bool SKEW = D > 128 && HS == 1 && fits(3, 2);
  static constexpr int STAGES = SKEW ? (fits(4, 2) ? 4 : 3) : fits(3, 2) ? 3 : fits(2, 1) ? 2 : 1;
  static constexpr int NPEX = STAGES >= 3 ? 2 : 1;
};

// LDS of one dK/dV item: a ring of (Q, dO, row metadata) buffers -- filled by
// DMA ahead of the step that reads them -- and the P hand-over from role A to
// role B.
template <typename T, int D>
struct DkvTiles {
  typedef Tile<T, DkvCfg<T, D>::BQ, D> TL;
  static constexpr int NS = DkvCfg<T, D>::STAGES;
  __attribute__((aligned(1024))) T Q[NS][TL::ELEMS];
  __attribute__((aligned(1024))) T G[NS][TL::ELEMS];
};
template <typename T, int D>
struct DkvMeta {
  static constexpr int NS = DkvCfg<T, D>::STAGES;
  __attribute__((aligned(256))) float lse[NS][64], dl[NS][64];
  __attribute__((aligned(256))) int klo[NS][64];
  // P hand-over, double-buffered with three slots (no barrier separates one
  // step's read from the next step's write)
  __attribute__((aligned(256))) f32x4 pex[DkvCfg<T, D>::NPEX][DkvCfg<T, D>::NKG][4][64];  // [buf][key group][value quad][lane][4]
  int n_tiles_s;
};
// Where the row metadata goes decides the register cost of its addresses (an
// LDS read reaches 64 KB past its address register): the skewed schedule reads
// two slots' metadata per step and keeps it below the tiles; the in-step
// schedules keep the tiles at the bottom (measured: fewer scalar spills).
template <typename T, int D>
struct DkvSmemMetaFirst : DkvMeta<T, D>, DkvTiles<T, D> {};
template <typename T, int D>
struct DkvSmemTilesFirst : DkvTiles<T, D>, DkvMeta<T, D> {};
template <typename T, int D>
using DkvSmem = typename std::conditional<DkvCfg<T, D>::SKEW, DkvSmemMetaFirst<T, D>, DkvSmemTilesFirst<T, D>>::type;

// The dK/dV item's rows on their way out (nb_device.h: RowStage).
template <typename T, int D>
using DkvStage = RowStage<T, DkvCfg<T, D>::NW, DkvCfg<T, D>::DA>;

// Slot of key k (0..31) in a row of a stored 32 x 32 dS block: k with bits 2
// and 3 swapped.  A lane's B fragment of a 32x32x16 product covers keys
// 4g + {0..3} and 8 + 4g + {0..3} of a 16-key half (g = lane / 32), the
// accumulator order of S; in this order they are one contiguous run of eight.
__device__ __forceinline__ constexpr int ds_slot(int k) { return (k & 0x13) | ((k & 4) << 1) | ((k & 8) >> 1); }

// One dK/dV item f: (kv head, batch row, key tile) with the kv head fastest
// and the (batch row, key tile) pairs in the order of decreasing work
// (work_order_kernel), so the long tiles start first.
// DS: the item may store dS (p.dsbuf non-null); compiled into the dK/dV-only
// kernel alone, so the combined kernel carries none of its registers.
// AC (in-step schedules, D <= 128): role A issues every tile copy, so role B
// waves never stall issuing copies; chosen for neighbourhoods without a left
// window (long bands), where it measured 2-3 % faster -- on short windowed
// bands (batched short documents) it measured 4 % slower.
template <typename T, int D, bool CH, bool DS, bool AC = false>
__device__ __forceinline__ void dkdv_item(const BwdParams& p, DkvSmem<T, D>& sm, DkvStage<T, D>& stage, int f) {
  typedef DkvCfg<T, D> C;
  typedef Tile<T, C::BQ, D> TL;
  typedef typename Frag<T>::type F;
  auto& pex = sm.pex;
  int& n_tiles_s = sm.n_tiles_s;
  const int grp = p.Hq / p.Hkv;
  const int n_kt = (p.S + C::BK - 1) / C::BK;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, ln = lane & 31;
  const int kg = w % C::NKG;                      // key group
  const int wr = w / C::NKG;                      // role and accumulator half
  const bool role_a = wr < C::HS;                 // A: S, P, dV   B: dP, dS, dK
  const int hf = wr % C::HS;                      // the half of dV^T / dK^T this wave keeps
  constexpr int NDA = C::DA / 32;                 // 32-wide column blocks of the accumulator
  const int off = p.q_off;                        // row i sits at key position off + i
  const int kor = p.k_origin;                     // row_klo values count keys from here
  // (at D = 256 the one- and two-register readers leave room to read ahead)
  typedef typename std::conditional<C::XREAD, TileAccessX<TL>, TileAccess<T, TL>>::type Access;
  const Access acc(ln, lane);
  // Q and dO tiles share one layout.  In the skewed schedule role A (waves 0 ..
  // NKG - 1) issues every copy: role B's dS stores count in the same vector
  // memory counter as copies, so a role-B wait for a step's copies would also
  // wait for the stores issued after them -- and role A has the slack.
  const TileDma<T, C::BQ, D, (C::SKEW || AC) ? C::NKG : C::NW> dma;
  const int kvh = f % p.Hkv;
  const int code = p.order[f / p.Hkv];
  const int b = code / n_kt, kt = code % n_kt;
  const int j0 = kt * C::BK;                      // first key of the workgroup
  const int jw = j0 + 32 * kg;                    // first key of the group
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
      int bsi = p.row_klo[(size_t)b * p.L + i] - kor;
      if (p.window >= 0) bsi = max(bsi, off + i - p.window);
      pred = bsi <= jmax;
    }
    // count through the waves' ballots (no extra LDS beyond n_tiles_s)
    const int wc = __popcll(__ballot(pred));
    if (lane == 0 && wc) atomicAdd(&n_tiles_s, wc);
    __syncthreads();
    if (n_tiles_s < base - t_first + C::NT) break;   // the prefix ended in this chunk
    __syncthreads();
  }
  __syncthreads();
  const int n_t = n_tiles_s;
  const int n_iter = grp * n_t;      // (q head of the group, query tile) steps
  if (n_iter == 0) {
    // no query reaches these keys: dK = dV = 0 over the whole tile (16-byte stores)
    constexpr int V16 = 16 / (int)sizeof(T);
    constexpr int RV = D / V16;   // 16-byte vectors per row
    const int bh = b * p.Hkv + kvh;
    const int n16 = min(C::BK, p.S - j0) * RV;
    if constexpr (CH) {
      const KvSpan<T> sk(p.kv, kDK, bh, j0, jmax, D), sv(p.kv, kDV, bh, j0, jmax, D);
      for (int x = tid; x < n16; x += C::NT) {
        const int j = j0 + x / RV, c = x % RV;
        T* rk = sk.ok ? sk.row(j, D) : kv_row<T>(p.kv, kDK, bh, j, D);
        T* rv = sv.ok ? sv.row(j, D) : kv_row<T>(p.kv, kDV, bh, j, D);
        reinterpret_cast<uint4*>(rk)[c] = uint4{0u, 0u, 0u, 0u};
        reinterpret_cast<uint4*>(rv)[c] = uint4{0u, 0u, 0u, 0u};
      }
    } else {
      const size_t base = ((size_t)bh * p.S + j0) * D;
      uint4* dkp = reinterpret_cast<uint4*>(reinterpret_cast<T*>(p.kv.dk[0]) + base);
      uint4* dvp = reinterpret_cast<uint4*>(reinterpret_cast<T*>(p.kv.dv[0]) + base);
      for (int x = tid; x < n16; x += C::NT) {
        dkp[x] = uint4{0u, 0u, 0u, 0u};
        dvp[x] = uint4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }

  // Step order (skewed schedule): step it visits (q head, tile) number
  // (it - t_first) mod n_iter, so step s reads query tile s (absolute) for
  // every item whose range holds it.  The items of one kv head run side by
  // side on one XCD, so the up to (W + BK) / BK items that read a tile read it
  // at about the same time and all but the first copy it from the L2 (sliding
  // layer: 135 instead of 307 MB fetched past the L2, same time).  Only the
  // order of the sum over the steps changes.  The in-step schedules (D <= 128)
  // keep the plain order: rotated, they ran about 1 % slower.
  const int rot = C::SKEW ? (n_iter - t_first % n_iter) % n_iter : 0;
  auto step_of = [&](int it) {
    const int x = it + rot;
    return x >= n_iter ? x - n_iter : x;
  };
  // the item's sources (rows of the group's first q head; a few base pointers
  // instead of the whole parameter block live across the loop)
  const size_t hb = ((size_t)b * p.Hq + (size_t)kvh * grp) * p.L;
  const T* const q_it = reinterpret_cast<const T*>(p.q) + hb * D;
  const T* const do_it = reinterpret_cast<const T*>(p.dout) + hb * D;
  const float* const lse_it = p.lse + hb;
  const float* const dl_it = p.delta + hb;
  const int* const klo_it = p.row_klo + (size_t)b * p.L;
  const int Lr = p.L;
  // Unseen copies (nb_device.h): the compiler cannot tell a copy's LDS
  // destination from the slot a later LDS read uses and would wait for the
  // copies of later steps before the step's reads; every schedule below orders
  // each slot's reads after that slot's copies with its own waits.
  auto load = [&](T* Qs, T* Gs, float* ls, float* ds, int* ks, int it) {
    const int sx = step_of(it), hh = sx / n_t, t = t_first + sx % n_t;
    const int i0 = t * C::BQ;
    const int nr = min(C::BQ, Lr - i0);
    const size_t rb = (size_t)hh * Lr + i0;
    if ((!C::SKEW && !AC) || role_a) {
      dma.issue_unseen(Qs, q_it + rb * D, nr);
      dma.issue_unseen(Gs, do_it + rb * D, nr);
    }
    if (w == 0) dma_words<true>(ls, lse_it + rb, nr);
    if (w == 1) dma_words<true>(ds, dl_it + rb, nr);
    if (w == 2) dma_words<true>(ks, klo_it + i0, nr);
  };
  constexpr int NS = C::STAGES;
  auto load_slot = [&](int slot, int it) {
    load(sm.Q[slot], sm.G[slot], sm.lse[slot], sm.dl[slot], sm.klo[slot], it);
  };
  // prologue: the copies of the first steps (all that run ahead of step 0)
#pragma unroll
  for (int x = 0; x < (NS == 1 ? 1 : C::SKEW ? NS - 2 : NS - 1); ++x)
    if (x < n_iter) load_slot(x, x);

  // this lane's key row of K (role A) or V (role B): the B operand of S = Q K^T
  // or dP = dO V^T
  F kv[D / 16];
  {
    const T* src;
    if constexpr (CH) {
      const KvSpan<const T> sp(p.kv, role_a ? kK : kV, b * p.Hkv + kvh, j0, jmax, D);
      src = sp.ok ? sp.row(min(j, p.S - 1), D) : kv_row<T>(p.kv, role_a ? kK : kV, b * p.Hkv + kvh,
                                                                  min(j, p.S - 1), D);
    } else {
      const size_t kr = ((size_t)b * p.Hkv + kvh) * p.S + min(j, p.S - 1);
      src = reinterpret_cast<const T*>(role_a ? p.kv.k[0] : p.kv.v[0]) + kr * D;
    }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kv[kk] = load_frag<T>(src + 16 * kk + 8 * g);
  }
  f32x16 gacc[NDA];   // dV^T (role A) or dK^T (role B) of the group's keys, columns of half hf
#pragma unroll
  for (int d = 0; d < NDA; ++d) gacc[d] = f32x16{};

  // One step's facts from its slot's band starts (uniform over the workgroup):
  // the tile's rows, whether the group's keys meet their bands at all, and
  // whether every (row, key) pair is inside them (no element mask).
  struct StepInfo {
    int i0, nrows;
    bool active, full;
  };
  auto info = [&](const int* ks, int it) {
    StepInfo si;
    si.i0 = (t_first + step_of(it) % n_t) * C::BQ;
    si.nrows = min(C::BQ, p.L - si.i0);
    // rows of this tile: positions off+i0 .. off+i0+nrows-1; band starts are nondecreasing
    const int p_min = off + si.i0, p_max = off + si.i0 + si.nrows - 1;
    auto band = [&](int qi) {
      const int bq = max(0, ks[qi] - kor);
      return p.window >= 0 ? max(bq, off + si.i0 + qi - p.window) : bq;
    };
    // (readfirstlane lets the compiler branch on the scalar unit)
    const int bs_min = __builtin_amdgcn_readfirstlane(band(0));
    const int bs_max = __builtin_amdgcn_readfirstlane(band(si.nrows - 1));
    si.active = !(jw > p_max || jw + 31 < bs_min);
    si.full = (si.nrows == C::BQ) && jw >= bs_max && jw + 31 <= p_min;
    return si;
  };
  // acc += rows of src (Q or dO) x this lane's K or V row: S^T or dP^T blocks
  constexpr int AH = DS ? C::AHEAD_DS : C::AHEAD;   // (see DkvCfg)
  auto rows_x_kv = [&](const T* src, f32x16& sacc) {
    if constexpr (AH > 0) {
      lds_mfma_pipeline<D / 16, AH, F>([&](int kk) { return acc.row(src, 0, kk); },
                                             [&](int kk, const F& a) { sacc = mma(a, kv[kk], sacc); });
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) sacc = mma(acc.row(src, 0, kk), kv[kk], sacc);
    }
  };
  // role A: S -> P in place (exp2 against the rows' LSE, 0 outside the band),
  // then published for role B; accumulator r is query row acc_row(r, g), key j
  auto to_p = [&](f32x16& sacc, const float* ls, const int* ks, const StepInfo& si, auto& px) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      // rows 8*rq + 4*g + e: their LSE as one 16-byte read
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + 8 * rq + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[4 * rq + e] = fast_exp2(fmaf(sacc[4 * rq + e], p.scale_log2, -l4[e] * kLog2e));
    }
    // the element mask, only on steps a band edge crosses: one uniform branch
    // around the whole block (per element the compiler turns it into selects
    // executed on every step)
    if (!si.full) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int4 k4 = *reinterpret_cast<const int4*>(ks + 8 * rq + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qi = 8 * rq + 4 * g + e;
          int bq = max(0, k4[e] - kor);
          if (p.window >= 0) bq = max(bq, off + si.i0 + qi - p.window);
          const bool in = (qi < si.nrows) & (j >= bq) & (j <= off + si.i0 + qi);
          sacc[4 * rq + e] = in ? sacc[4 * rq + e] : 0.f;
        }
      }
    }
    if (hf == 0) {   // (at D = 512 the other role-A wave holds the same P)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        px[kg][qd][lane] = f32x4{sacc[4 * qd], sacc[4 * qd + 1], sacc[4 * qd + 2], sacc[4 * qd + 3]};
    }
  };
  // role B: dP -> dS = P (dP - Delta) in place, P from role A
  auto to_ds = [&](f32x16& sacc, const auto& px, const float* ds) {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const f32x4 pq = px[kg][qd][lane];
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(ds + 8 * qd + 4 * g);  // rows acc_row(4*qd + e, g)
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[4 * qd + e] = pq[e] * (sacc[4 * qd + e] - d4[e]);
    }
  };
  // role B: step it's dS (this lane's key j, rows acc_row(r, g)) into the
  // banded buffer, when there is one (the dQ pass then reads it).  The buffer
  // is 32-row x 32-key blocks (row-major, 32 * 32 elements each): a lane's 16
  // values go through one buffer resource, a scalar block offset, one lane
  // offset for the whole item and a constant offset per row.
  const int ds_nb = p.ds_w >> 5;                      // blocks per 32-row tile
  const int ds_ntq = (p.L + 31) >> 5;                 // 32-row tiles per head
  auto store_ds = [&](const f32x16& ds, int it, const int* ks) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int ds_lane = (ds_slot(ln) + 4 * g * 32) * (int)sizeof(T);   // (formed here: nothing extra held in the loop)
    const int sx = step_of(it), hh = sx / n_t, tq = t_first + sx % n_t, i0 = tq * C::BQ;
    int bs0 = max(0, ks[0] - kor);
    if (p.window >= 0) bs0 = max(bs0, off + i0 - p.window);
    bs0 = __builtin_amdgcn_readfirstlane(bs0);
    const int blk = ((b * p.Hq + kvh * grp + hh) * ds_ntq + tq) * ds_nb + ((jw - (bs0 & ~31)) >> 5);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(p.dsbuf, (short)0, p.ds_bytes, kBufferWord3);
    const int nrows = p.L - i0;
    if (j < p.S && hf == 0) {   // (at D = 512 the other role-B wave holds the same dS)
      auto put = [&](int r) __attribute__((always_inline)) {
        const int voff = ds_lane + (8 * (r >> 2) + (r & 3)) * 32 * (int)sizeof(T);
        if constexpr (sizeof(T) == 2) {
          const bf16 v = to_elem<bf16>(ds[r]);
          // non-temporal (aux 2): the band streams through once, and cached it
          // evicted the Q / dO tiles other items re-read (the pass fetched 417
          // instead of 307 MB past the L2 on the sliding layer)
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), rs, voff,
                                                    blk * 32 * 32 * 2, 2);
        } else {
          const float v = ds[r];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, voff, blk * 32 * 32 * 4, 0);
        }
      };
      if (nrows >= C::BQ) {   // uniform: a whole tile of rows, no per-row test (no exec mask per store)
#pragma unroll
        for (int r = 0; r < 16; ++r) put(r);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_row(r, g) < nrows) put(r);
      }
    }
#endif
  };
  // gacc += src^T (P or dS): dV^T = dO^T P (role A) or dK^T = Q^T dS (role B)
  auto accumulate = [&](const T* src, const f32x16& sacc) {
    const int d0 = hf * NDA;   // first column block of this wave's half
    if constexpr (AH > 0) {
      const F sf[2] = {acc_to_frag<T>(sacc, 0), acc_to_frag<T>(sacc, 1)};
      constexpr int ND = NDA;
      lds_mfma_pipeline<2 * ND, AH, F>(
          [&](int x) { return acc.col(src, d0 + x % ND, x / ND); },
          [&](int x, const F& a) { gacc[x % ND] = mma(a, sf[x / ND], gacc[x % ND]); });
    } else {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const F sf = acc_to_frag<T>(sacc, m);
#pragma unroll
        for (int d = 0; d < NDA; ++d) gacc[d] = mma(acc.col(src, d0 + d, m), sf, gacc[d]);
      }
    }
  };

  if constexpr (C::SKEW) {
    // Role B runs one step behind role A: in step t role A forms S, P and dV
    // of step t while role B finishes step t - 1 (dS from the P role A
    // published then, dK) and forms dP of step t.  Neither waits for the other
    // inside a step; the one barrier per step (at its end) publishes P, retires
    // a ring slot and makes the next step's copies visible.  The ring holds the
    // previous step (role B's Q and Delta), the current one and LA steps of
    // copies in flight.  The loop is not unrolled over the slots: a copy of
    // the step per slot and role outgrows the instruction cache.
    constexpr int LA = NS - 2;
    static_assert(C::NKG >= 3, "the row metadata copies come from role-A waves 0, 1, 2");
    const int n_vm = 2 * dma.count() + (w < 3 ? 1 : 0);   // a role-A wave's copies per step
    wait_global();   // the prologue's copies (steps 0 .. LA - 1)
    __syncthreads();
    // Each role runs a loop of its own (same copies and barriers, one branch
    // per item rather than per step: the register allocator then sees one
    // role's live values at a time).
    auto run = [&](auto is_a) {
      constexpr bool A = decltype(is_a)::value;
      f32x16 dp = f32x16{};   // role B: dP of the previous step
      bool act_prev = false;  // role B: the previous step met the group's keys
      // The vector memory traffic of a step -- role A's copies of step t + LA
      // (into step t - 2's slot) and role B's dS stores -- is spread out: the
      // copies go out after role A's S products, the stores after role B's dK
      // products.  Issued together at the top of the step they queued behind
      // each other (measured: the backward 3 % slower; either move alone did
      // not pay).
      auto stage = [&](int t, int x) {
        const int slot_next = x + LA < NS ? x + LA : x + LA - NS;
        if constexpr (A) {
          bool copied = false;
          if (t < n_iter) {
            const StepInfo si = info(sm.klo[x], t);
            if (si.active) {
              f32x16 sacc = f32x16{};
              rows_x_kv(sm.Q[x], sacc);
              if (t + LA < n_iter) load_slot(slot_next, t + LA);
              copied = true;
              to_p(sacc, sm.lse[x], sm.klo[x], si, pex[t & 1]);
              __builtin_amdgcn_sched_barrier(0);   // keep the phases' operands apart
              accumulate(sm.G[x], sacc);
            }
          }
          if (!copied && t + LA < n_iter) load_slot(slot_next, t + LA);
        } else {
          const int xp = x == 0 ? NS - 1 : x - 1;
          if (act_prev) {
            to_ds(dp, pex[(t - 1) & 1], sm.dl[xp]);
            accumulate(sm.Q[xp], dp);
            if (DS && p.dsbuf) store_ds(dp, t - 1, sm.klo[xp]);
          }
          __builtin_amdgcn_sched_barrier(0);
          act_prev = false;
          if (t < n_iter) {
            act_prev = info(sm.klo[x], t).active;
            if (act_prev) {
              dp = f32x16{};
              rows_x_kv(sm.G[x], dp);
            }
          }
        }
        // step t + 1's copies complete (those of later steps may stay in flight);
        // role B issued none and leaves its dS stores in flight
        if constexpr (A) {
          const int later = min(t + LA, n_iter - 1) - (t + 1);
          if (t + 1 < n_iter) wait_global_le(later > 0 ? n_vm * later : 0);
        }
        __syncthreads();
      };
      for (int t = 0, x = 0; t <= n_iter; ++t, x = (x + 1 == NS) ? 0 : x + 1) stage(t, x);
    };
    if (role_a) run(std::true_type{});
    else run(std::false_type{});
  } else if constexpr (NS >= 3) {
    // Role B in step with role A, one barrier per step, at the hand-over: by
    // then every wave has finished the previous step, so the copies of step
    // it + 2 go into its slot right after the barrier, and the copies of step
    // it + 1 (issued two steps earlier) are complete and visible for its first
    // half.  The ring is unrolled NS times so every slot's LDS address is a
    // constant.
    auto stage = [&](int it, int x) {
      auto& px = pex[it & 1];
      const StepInfo si = info(sm.klo[x], it);
      f32x16 sacc = f32x16{};
      if (si.active) {
        rows_x_kv(role_a ? sm.Q[x] : sm.G[x], sacc);
        if (role_a) to_p(sacc, sm.lse[x], sm.klo[x], si, px);
      }
      if (it + 1 < n_iter) wait_global();
      __syncthreads();   // the hand-over
      if (it + 2 < n_iter) load_slot((x + 2) % NS, it + 2);
      if (si.active) {
        if (!role_a) {
          to_ds(sacc, px, sm.dl[x]);
          if (DS && p.dsbuf) store_ds(sacc, it, sm.klo[x]);
        }
        accumulate(role_a ? sm.G[x] : sm.Q[x], sacc);
      }
    };
    wait_global();   // the prologue's copies
    __syncthreads();
    for (int it = 0; it < n_iter; it += NS) {
#pragma unroll
      for (int x = 0; x < NS; ++x)
        if (it + x < n_iter) stage(it + x, x);
    }
  } else if constexpr (NS == 1) {
    // One slot: step it's copies go out once every wave is done with step
    // it - 1; P crosses at a barrier inside the step.
    auto stage = [&](int it) {
      if (it > 0) {
        __syncthreads();   // step it - 1 is done with the slot
        load_slot(0, it);
      }
      wait_global();
      __syncthreads();
      const StepInfo si = info(sm.klo[0], it);
      f32x16 sacc = f32x16{};
      if (si.active) {
        rows_x_kv(role_a ? sm.Q[0] : sm.G[0], sacc);
        if (role_a) to_p(sacc, sm.lse[0], sm.klo[0], si, pex[0]);
      }
      __syncthreads();   // the hand-over
      if (si.active) {
        if (!role_a) {
          to_ds(sacc, pex[0], sm.dl[0]);
          if (DS && p.dsbuf) store_ds(sacc, it, sm.klo[0]);
        }
        accumulate(role_a ? sm.G[0] : sm.Q[0], sacc);
      }
    };
    for (int it = 0; it < n_iter; ++it) stage(it);
  } else {
    // Two slots, role B in step with role A: copies for step it + 1 go out
    // after the barrier at the top of step it (which also makes step it's
    // copies visible); P crosses at a second barrier inside the step.
    auto stage = [&](int it, int x) {
      wait_global();
      __syncthreads();
      if (it + 1 < n_iter) load_slot((x + 1) % NS, it + 1);
      __builtin_amdgcn_sched_barrier(0);
      const StepInfo si = info(sm.klo[x], it);
      f32x16 sacc = f32x16{};
      if (si.active) {
        rows_x_kv(role_a ? sm.Q[x] : sm.G[x], sacc);
        if (role_a) to_p(sacc, sm.lse[x], sm.klo[x], si, pex[0]);
      }
      __syncthreads();   // the hand-over
      if (si.active) {
        if (!role_a) {
          to_ds(sacc, pex[0], sm.dl[x]);
          if (DS && p.dsbuf) store_ds(sacc, it, sm.klo[x]);
        }
        accumulate(role_a ? sm.G[x] : sm.Q[x], sacc);
      }
    };
    for (int it = 0; it < n_iter; it += NS) {
#pragma unroll
      for (int x = 0; x < NS; ++x)
        if (it + x < n_iter) stage(it + x, x);
    }
  }

  if constexpr (DkvStage<T, D>::ON) {
    const float sc = role_a ? 1.f : p.scale;
    const int bh = b * p.Hkv + kvh;
    const int nrows = min(32, p.S - jw);
    __syncthreads();   // every wave is done with the ring and the hand-over the staging overwrites
    if constexpr (CH) {
      const KvSpan<T> sp(p.kv, role_a ? kDV : kDK, bh, j0, jmax, D);
      stage_rows_in<T, C::DA>(&stage.r[w][0][0], gacc, sc);
      stage_rows_store_at<T, C::DA>(&stage.r[w][0][0], nrows, [&](int r) {
        return (sp.ok ? sp.row(jw + r, D) : kv_row<T>(p.kv, role_a ? kDV : kDK, bh, jw + r, D)) + hf * C::DA;
      });
    } else {
      T* const base = reinterpret_cast<T*>(role_a ? p.kv.dv[0] : p.kv.dk[0]) + ((size_t)bh * p.S + jw) * D + hf * C::DA;
      stage_rows_in<T, C::DA>(&stage.r[w][0][0], gacc, sc);
      stage_rows_store<T, C::DA>(&stage.r[w][0][0], base, D, nrows);
    }
    return;
  }
  if (j < p.S) {
    T* dst;
    if constexpr (CH) {
      const KvSpan<T> sp(p.kv, role_a ? kDV : kDK, b * p.Hkv + kvh, j0, jmax, D);
      dst = sp.ok ? sp.row(j, D) : kv_row<T>(p.kv, role_a ? kDV : kDK, b * p.Hkv + kvh, j, D);
    }
    else
      dst = reinterpret_cast<T*>(role_a ? p.kv.dv[0] : p.kv.dk[0]) + (((size_t)b * p.Hkv + kvh) * p.S + j) * D;
    const float sc = role_a ? 1.f : p.scale;
    dst += hf * C::DA;
#pragma unroll
    for (int d = 0; d < NDA; ++d) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        store_quad<T>(dst + 32 * d + 8 * rq + 4 * g, gacc[d][4 * rq] * sc, gacc[d][4 * rq + 1] * sc,
                      gacc[d][4 * rq + 2] * sc, gacc[d][4 * rq + 3] * sc);
      }
    }
  }
}


// ---------------------------------------------------------------- dQ

// Eight waves: four query groups of 32 rows, two roles per group.  Role A holds
// the rows' Q and forms S^T = K Q^T and P; role B holds dO and forms
// dP^T = V dO^T.  They swap P and dP through LDS, both form dS, and each
// accumulates half of dQ's columns (A the first D/2, B the rest).  Each wave
// then needs one operand block plus half an accumulator, so two waves share
// each SIMD at D = 256; the matrix-core work is the same as one wave doing all.
template <typename T, int D>
struct DqCfg {
  // FUSED (bf16, D <= 128): every wave is a query group of its own and forms S,
  // P, dP and dS for its 32 rows and all of dQ -- Q and dO rows plus the whole
  // accumulator fit 256 registers at these head dims -- so no P / dP crosses
  // between waves and the step keeps one barrier, for the K/V ring.
  static constexpr bool FUSED = sizeof(T) == 2 && D <= 128;
  static constexpr int NQG = FUSED ? BwdShape<T, D>::NT / 64 : BwdShape<T, D>::NT / 128;   // query groups of 32 rows
  static constexpr int NW = FUSED ? NQG : 2 * NQG;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NQG;               // query rows per workgroup
  static constexpr int BN = (D * sizeof(T) <= 256) ? 64 : 32;   // keys per tile
  // operand fragments read ahead of their MFMA; 0 = plain loop (float path)
  static constexpr int AHEAD = (sizeof(T) != 2) ? 0 : (D <= 128) ? 3 : 2;   // (4 at D <= 128: ~1 % slower)
  static constexpr int DQW = FUSED ? D : D / 2;   // columns of one wave's dQ part
};
// The dQ item's rows on their way out (nb_device.h: RowStage).
template <typename T, int D>
using DqStage = RowStage<T, DqCfg<T, D>::NW, DqCfg<T, D>::DQW>;

// LDS of one dQ item: two K/V tile pairs (one filled by DMA while the other is
// read) and the P / dP exchange of each query group.
template <typename T, int D>
struct DqSmem {
  typedef Tile<T, DqCfg<T, D>::BN, D> TL;
  static constexpr int NSB = DqCfg<T, D>::BN / 32;
  static constexpr int TILE_BYTES = TL::ELEMS * (int)sizeof(T);
  static constexpr int NQG = DqCfg<T, D>::FUSED ? 1 : DqCfg<T, D>::NQG;   // (fused: the exchange only hosts the wave bounds)
  static constexpr int XCH_BYTES = 2 * NQG * NSB * 4 * 64 * 16;
  // three K/V slots and a double-buffered exchange (one barrier per step) when
  // they fit, else two slots and one exchange buffer (two barriers per step)
  static constexpr bool RING3 = 6 * TILE_BYTES + 2 * XCH_BYTES <= BwdShape<T, D>::LDS_BUDGET;
  static constexpr int NS = RING3 ? 3 : 2;
  static constexpr int NX = RING3 ? 2 : 1;
  __attribute__((aligned(1024))) T K[NS][TL::ELEMS];
  __attribute__((aligned(1024))) T V[NS][TL::ELEMS];
  __attribute__((aligned(256))) f32x4 xch[NX][2][NQG][NSB][4][64];  // [buf][P | dP][group][block][value quad][lane][4]
};

// One dQ item f: (kv head, q head of its group, batch row, query tile) with
// the kv head fastest and the (batch row, query tile) pairs longest band first.
// KV as in the forward (kKvConcat / kKvPair / kKvAny); under kKvPair an item
// whose key range touches three or more chunks is appended to p.cross and left
// to the follow-up kernel, which runs it as kKvAny.
template <typename T, int D, int KV>
__device__ __forceinline__ void dq_item(const BwdParams& p, DqSmem<T, D>& sm, DqStage<T, D>& stage, int f) {
  typedef DqCfg<T, D> C;
  typedef Tile<T, C::BN, D> TL;
  typedef typename Frag<T>::type F;
  constexpr int NSB = C::BN / 32;
  constexpr int NM = C::BN / 16;
  constexpr int DH = C::FUSED ? D / 32 : D / 64;   // 32-wide d blocks of dQ per wave
  constexpr int NS = DqSmem<T, D>::NS;
  // wave bounds: scratch at the start of the exchange, dead before the first
  // exchange write (barriers separate them)
  int (*red)[2] = reinterpret_cast<int (*)[2]>(&sm.xch[0][0][0][0][0][0]);
  const int grp = p.Hq / p.Hkv;
  const int n_qt = (p.L + C::BM - 1) / C::BM;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, ln = lane & 31;
  const int qg = w % C::NQG;            // query group
  const bool role_a = C::FUSED || w < C::NQG;   // A: Q, S, P   B: dO, dP   (fused: both)
  typedef TileAccess<T, TL> Access;
  const Access acc(ln, lane);
  const TileDma<T, C::BN, D, C::NW> dma;   // K and V tiles share one layout
  const int kvh = f % p.Hkv;
  const int h = kvh * grp + (f / p.Hkv) % grp;
  const int code = p.qorder[f / p.Hq];
  const int b = code / n_qt, qt = code % n_qt;
  const int i = qt * C::BM + 32 * qg + ln;
  const bool in_range = i < p.L;
  const int pq = p.q_off + i;               // the row's key position
  const int pos = min(pq, p.S - 1);         // its band's last key
  int bs = pq + 1;
  if (in_range) {
    bs = max(0, p.row_klo[(size_t)b * p.L + i] - p.k_origin);  // clamp: never index before the keys
    if (p.window >= 0) bs = max(bs, pq - p.window);
  }
  const bool real = in_range && bs <= pos;
  // (uniform; readfirstlane makes the tile decisions scalar branches)
  const int w_lo = __builtin_amdgcn_readfirstlane(wave_min_i(real ? bs : INT_MAX));
  const int w_hi = __builtin_amdgcn_readfirstlane(wave_max_i(real ? pos + 1 : INT_MIN));
  const int w_bs_max = __builtin_amdgcn_readfirstlane(wave_max_i(real ? bs : INT_MIN));
  const int w_p_min = __builtin_amdgcn_readfirstlane(wave_min_i(real ? pos : INT_MAX));
  const bool w_all_real = __builtin_amdgcn_readfirstlane(wave_min_i(real ? 1 : 0)) != 0;
  if (lane == 0) { red[w][0] = w_lo; red[w][1] = w_hi; }

  const size_t qrow = ((size_t)b * p.Hq + h) * p.L + i;
  const size_t qrow_c = ((size_t)b * p.Hq + h) * p.L + min(i, p.L - 1);  // rows past L read row L-1
  // this lane's row of Q (role A) or dO (role B): the B operand of S^T or dP^T
  // (fused: Q in rf, dO in rg)
  F rf[D / 16];
  F rg[C::FUSED ? D / 16 : 1];
  {
    const T* src = reinterpret_cast<const T*>(role_a ? p.q : p.dout) + qrow_c * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      rf[kk] = load_frag<T>(src + 16 * kk + 8 * g);
      if (!in_range) rf[kk] = zero_frag<T>();
    }
    if constexpr (C::FUSED) {
      const T* so = reinterpret_cast<const T*>(p.dout) + qrow_c * D;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        rg[kk] = load_frag<T>(so + 16 * kk + 8 * g);
        if (!in_range) rg[kk] = zero_frag<T>();
      }
    }
  }
  // Delta of the row (bwd_delta_kernel), 0 for padding rows
  const float dl = real ? p.delta[qrow_c] : 0.f;
  const float lse2 = real ? p.lse[qrow_c] * kLog2e : 0.f;
  __syncthreads();
  int kstart = INT_MAX, kend = INT_MIN;
#pragma unroll
  for (int x = 0; x < C::NW; ++x) { kstart = min(kstart, red[x][0]); kend = max(kend, red[x][1]); }
  kstart = __builtin_amdgcn_readfirstlane(kstart);   // uniform: scalar tile bounds and addresses
  kend = __builtin_amdgcn_readfirstlane(kend);

  const int bh = b * p.Hkv + kvh;
  // kbase + j * D is key j's row (the concatenated buffer; chunks: see the forward)
  const T* __restrict__ kbase = reinterpret_cast<const T*>(p.kv.k[0]) + (size_t)bh * p.S * D;
  const T* __restrict__ vbase = reinterpret_cast<const T*>(p.kv.v[0]) + (size_t)bh * p.S * D;
  const KvPair<T, C::BN> pair = KV == kKvConcat ? KvPair<T, C::BN>() : KvPair<T, C::BN>(p.kv, bh, kstart, kend, D);
  if constexpr (KV == kKvPair) {
    if (!pair.ok) {   // uniform
      if (threadIdx.x == 0) p.cross[atomicAdd(&p.counters[kCrossCount], 1)] = f;
      return;
    }
  }
  const int nt = kstart < kend ? (kend - kstart + C::BN - 1) / C::BN : 0;   // key tiles of the item
  if (nt == 0 && p.dq_mode == kDqAddF32) return;   // uniform: no key, nothing to add
  auto load = [&](int slot, int n) {
    const int j0 = kstart + n * C::BN;
    if constexpr (KV == kKvAny) {
      kv_tile_load<T, C::BN, D, C::NW>(dma, p.kv, bh, j0, min(C::BN, p.S - j0), sm.K[slot], sm.V[slot]);
    } else if constexpr (KV == kKvPair) {
      pair.load(dma, j0, sm.K[slot], sm.V[slot]);
    } else {   // unseen copies: the schedules below wait for each slot themselves
      const int nv = min(C::BN, p.S - j0);
      dma.issue_unseen(sm.K[slot], kbase + (size_t)j0 * D, nv);
      dma.issue_unseen(sm.V[slot], vbase + (size_t)j0 * D, nv);
    }
  };
#pragma unroll
  for (int x = 0; x < NS - 1; ++x)
    if (x < nt) load(x, x);

  const int dh0 = (C::FUSED || role_a) ? 0 : DH;      // first 32-wide d block of this wave's dQ part
  f32x16 dqacc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) dqacc[d] = f32x16{};

  // fused: S and dP of the wave's rows, P and dS in place, then (after the
  // ring's barrier) dQ^T += K^T dS^T over all of D
  auto step_fused = [&](const T* Ks, const T* Vs, int n, auto&& mid) {
    const int j0 = kstart + n * C::BN;
    const bool active = !(j0 >= w_hi || j0 + C::BN <= w_lo);
    const bool full = w_all_real && j0 >= w_bs_max && j0 + C::BN - 1 <= w_p_min;
    constexpr int NK = D / 16;
    f32x16 sacc[NSB], dpa[NSB];
    if (active) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) sacc[sb] = dpa[sb] = f32x16{};
      lds_mfma_pipeline<NSB * NK, C::AHEAD, F>(
          [&](int x) { return acc.row(Ks, x / NK, x % NK); },
          [&](int x, const F& a) { sacc[x / NK] = mma(a, rf[x % NK], sacc[x / NK]); });
      lds_mfma_pipeline<NSB * NK, C::AHEAD, F>(
          [&](int x) { return acc.row(Vs, x / NK, x % NK); },
          [&](int x, const F& a) { dpa[x / NK] = mma(a, rg[x % NK], dpa[x / NK]); });
      // accumulator r of block sb: key j0 + 32*sb + acc_row(r, g), query row i (this lane)
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] = fast_exp2(fmaf(sacc[sb][r], p.scale_log2, -lse2));
      }
      if (!full) {   // one uniform branch around the element mask (see the dK/dV item)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jj = j0 + 32 * sb + acc_row(r, g);
            if ((!real) | (jj < bs) | (jj > pos)) sacc[sb][r] = 0.f;
          }
        }
      }
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] = sacc[sb][r] * (dpa[sb][r] - dl);
      }
    }
    mid();   // the ring's barrier (and maintenance)
    if (!active) return;
    F sf[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) sf[m] = acc_to_frag<T>(sacc[m >> 1], m & 1);
    lds_mfma_pipeline<NM * DH, C::AHEAD, F>(
        [&](int x) { return acc.col(Ks, x % DH, x / DH); },
        [&](int x, const F& a) { dqacc[x % DH] = mma(a, sf[x / DH], dqacc[x % DH]); });
  };
  auto step = [&](const T* Ks, const T* Vs, int n, auto&& mid) {
    if constexpr (C::FUSED) {
      step_fused(Ks, Vs, n, mid);
      return;
    }
    const int j0 = kstart + n * C::BN;
    auto& xb = sm.xch[DqSmem<T, D>::NX > 1 ? (n & 1) : 0];
    f32x4 (*xp)[NSB][4][64] = xb[0];
    f32x4 (*xdp)[NSB][4][64] = xb[1];
    const bool active = !(j0 >= w_hi || j0 + C::BN <= w_lo);   // same for both roles of the group
    const bool full = w_all_real && j0 >= w_bs_max && j0 + C::BN - 1 <= w_p_min;
    f32x16 sacc[NSB];
    if (active) {
      const T* src = role_a ? Ks : Vs;
      constexpr int NK = D / 16;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) sacc[sb] = f32x16{};
      if constexpr (C::AHEAD > 0) {
        lds_mfma_pipeline<NSB * NK, C::AHEAD, F>(
            [&](int x) { return acc.row(src, x / NK, x % NK); },
            [&](int x, const F& a) { sacc[x / NK] = mma(a, rf[x % NK], sacc[x / NK]); });
      } else {
#pragma unroll
        for (int x = 0; x < NSB * NK; ++x) sacc[x / NK] = mma(acc.row(src, x / NK, x % NK), rf[x % NK], sacc[x / NK]);
      }
      if (role_a) {
        // accumulator r of block sb: key j0 + 32*sb + acc_row(r, g), query row i (this lane)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[sb][r] = fast_exp2(fmaf(sacc[sb][r], p.scale_log2, -lse2));
        }
        if (!full) {   // one uniform branch around the element mask (see the dK/dV item)
#pragma unroll
          for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int jj = j0 + 32 * sb + acc_row(r, g);
              if ((!real) | (jj < bs) | (jj > pos)) sacc[sb][r] = 0.f;
            }
          }
        }
      }
      f32x4 (*mine)[4][64] = role_a ? xp[qg] : xdp[qg];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          mine[sb][qd][lane] = f32x4{sacc[sb][4 * qd], sacc[sb][4 * qd + 1], sacc[sb][4 * qd + 2], sacc[sb][4 * qd + 3]};
    }
    mid();   // the exchange barrier (and ring maintenance)
    if (!active) return;
    // dS = P (dP - Delta), with the partner's half taken from LDS
    f32x4 (*theirs)[4][64] = role_a ? xdp[qg] : xp[qg];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const f32x4 o = theirs[sb][qd][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * qd + e;
          const float pr = role_a ? sacc[sb][r] : o[e];
          const float dp = role_a ? o[e] : sacc[sb][r];
          sacc[sb][r] = pr * (dp - dl);
        }
      }
    }
    F sf[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) sf[m] = acc_to_frag<T>(sacc[m >> 1], m & 1);
    // This role's d blocks as compile-time indices (one branch per role): a
    // block index known only at run time would index the column reader's
    // per-lane address arrays at run time, and the compiler then keeps those
    // arrays in LDS and loads every read's address from there (bank-conflicted).
    auto dq_product_rt = [&](int d0) __attribute__((always_inline)) {
      if constexpr (C::AHEAD > 0) {
        lds_mfma_pipeline<NM * DH, C::AHEAD, F>(
            [&](int x) { return acc.col(Ks, d0 + x % DH, x / DH); },
            [&](int x, const F& a) { dqacc[x % DH] = mma(a, sf[x / DH], dqacc[x % DH]); });
      } else {
#pragma unroll
        for (int x = 0; x < NM * DH; ++x) dqacc[x % DH] = mma(acc.col(Ks, d0 + x % DH, x / DH), sf[x / DH], dqacc[x % DH]);
      }
    };
    auto dq_product = [&](auto half) __attribute__((always_inline)) {
      constexpr int d0 = decltype(half)::value * DH;
      if constexpr (C::AHEAD > 0) {
        lds_mfma_pipeline<NM * DH, C::AHEAD, F>(
            [&](int x) { return acc.col(Ks, d0 + x % DH, x / DH); },
            [&](int x, const F& a) { dqacc[x % DH] = mma(a, sf[x / DH], dqacc[x % DH]); });
      } else {
#pragma unroll
        for (int x = 0; x < NM * DH; ++x) dqacc[x % DH] = mma(acc.col(Ks, d0 + x % DH, x / DH), sf[x / DH], dqacc[x % DH]);
      }
    };
    if constexpr (sizeof(T) == 2 && D <= 128) {
      if (role_a) dq_product(std::integral_constant<int, 0>{});
      else dq_product(std::integral_constant<int, 1>{});
    } else {
      // (at D >= 256 a role's first block is a multiple of the reader's block
      // count, so the array index is a compile-time constant already)
      dq_product_rt(dh0);
    }
  };

  if constexpr (DqSmem<T, D>::RING3) {
    // one barrier per step, at the exchange: copies of tile n + 2 go into the
    // slot tile n - 1 used, and tile n + 1's copies (issued two steps earlier)
    // are complete and visible before its first half
    auto stage = [&](int n, int slot) {
      step(sm.K[slot], sm.V[slot], n, [&]() {
        if (n + 1 < nt) wait_global();
        __syncthreads();
        if (n + 2 < nt) load((slot + 2) % NS, n + 2);
      });
    };
    wait_global();
    __syncthreads();
    for (int n = 0; n < nt; n += NS) {
#pragma unroll
      for (int x = 0; x < NS; ++x)
        if (n + x < nt) stage(n + x, x);
    }
  } else {
    auto stage = [&](int n, int slot) {
      wait_global();
      __syncthreads();
      if (n + 1 < nt) load((slot + 1) % NS, n + 1);
      __builtin_amdgcn_sched_barrier(0);
      step(sm.K[slot], sm.V[slot], n, [&]() { __syncthreads(); });
    };
    for (int n = 0; n < nt; n += NS) {
#pragma unroll
      for (int x = 0; x < NS; ++x)
        if (n + x < nt) stage(n + x, x);
    }
  }

  if constexpr (DqStage<T, D>::ON) {
    static_assert(DH * 32 == C::DQW, "a wave's dQ part");
    if (p.dq_mode == kDqStore) {
      const int i_grp = qt * C::BM + 32 * qg;   // the wave's first row (uniform: a scalar store base)
      T* const st = &stage.r[w][0][0];
      __syncthreads();   // every wave is done with the K/V ring and the exchange the staging overwrites
      stage_rows_in<T, C::DQW>(st, dqacc, p.scale);
      stage_rows_store<T, C::DQW>(st, reinterpret_cast<T*>(p.dq) + (((size_t)b * p.Hq + h) * p.L + i_grp) * D + 32 * dh0,
                                  D, min(32, p.L - i_grp));
      return;
    }
  }
  if (in_range && p.dq_mode == kDqStore) {
    T* dqp = reinterpret_cast<T*>(p.dq) + qrow * D;
#pragma unroll
    for (int d = 0; d < DH; ++d) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        store_quad<T>(dqp + 32 * (dh0 + d) + 8 * rq + 4 * g, dqacc[d][4 * rq] * p.scale,
                      dqacc[d][4 * rq + 1] * p.scale, dqacc[d][4 * rq + 2] * p.scale,
                      dqacc[d][4 * rq + 3] * p.scale);
      }
    }
  } else if (in_range) {   // fp32 dQ accumulator: set, or add this call's contribution
    float* dqp = reinterpret_cast<float*>(p.dq) + qrow * D;
#pragma unroll
    for (int d = 0; d < DH; ++d) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4* dst = reinterpret_cast<f32x4*>(dqp + 32 * (dh0 + d) + 8 * rq + 4 * g);
        f32x4 x = f32x4{dqacc[d][4 * rq] * p.scale, dqacc[d][4 * rq + 1] * p.scale, dqacc[d][4 * rq + 2] * p.scale,
                        dqacc[d][4 * rq + 3] * p.scale};
        if (p.dq_mode == kDqAddF32) {
          const f32x4 a = *dst;
          x = f32x4{a[0] + x[0], a[1] + x[1], a[2] + x[2], a[3] + x[3]};
        }
        *dst = x;
      }
    }
  }
}


// ---------------------------------------------------------------- dQ from stored dS

// dQ = scale * dS K from the banded dS the dK/dV items stored (windowed
// neighbourhoods), with no recompute of S or dP.  One workgroup per (128 query
// rows, q head, batch row), four waves of 32 rows; the work is the forward's
// P V half: K tiles copied into LDS asynchronously and read transposed as the A
// operand of dQ^T = K^T dS^T, the B operand (dS^T, this lane's query row) read
// from the buffer in the accumulator order the forward feeds P^T in.  A wave
// reads the same 32-key blocks the dK/dV items wrote for its 32-row tile: from
// the first row's band start rounded down to 32 up to the last row's position.
// KV: kKvConcat (one neighbourhood buffer) or kKvPair (the chunk table: K tiles
// through KvPair, and through the general lookup when the workgroup's key range
// touches three or more chunks).
template <typename T, int D>
struct DqsCfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;
  // keys per tile (no Q fragments to hold: room for 64 at D = 256; 32 for a
  // float32 tile at D = 512, so two of them fit the LDS)
  static constexpr int BN = (sizeof(T) * D > 1024) ? 32 : 64;
  static constexpr int AHEAD = (D <= 128) ? 3 : 2;   // as the forward's P V half
  static constexpr int OCC = (sizeof(T) == 2 && D <= 256) ? 2 : 1;
};

// Its LDS: two K tiles and the key-range reduction; after the loop, the dQ rows
// on their way out.
template <typename T, int D>
struct DqsSmem {
  typedef DqsCfg<T, D> C;
  union {
    struct {
      __attribute__((aligned(1024))) T K0[Tile<T, C::BN, D>::ELEMS];
      __attribute__((aligned(1024))) T K1[Tile<T, C::BN, D>::ELEMS];
      int red[C::NW][2];
    };
    RowStage<T, C::NW, D> st;
  };
};

template <typename T, int D, int KV>
__global__ __launch_bounds__(256, (DqsCfg<T, D>::OCC)) void dq_ds_kernel(BwdParams p) {
  typedef DqsCfg<T, D> C;
  typedef Tile<T, C::BN, D> TL;
  typedef typename Frag<T>::type F;
  __shared__ DqsSmem<T, D> sm;
  T* const K0 = sm.K0;
  T* const K1 = sm.K1;
  int (*red)[2] = sm.red;
  const int grp = p.Hq / p.Hkv;
  const int ngroups = p.B * p.Hkv;
  const int gid = blockIdx.x % ngroups, rest = blockIdx.x / ngroups;
  const int b = gid / p.Hkv, kvh = gid % p.Hkv;
  const int h = kvh * grp + rest % grp, qt = rest / grp;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), g = lane >> 5, ln = lane & 31;
  const int i0 = qt * C::BM + 32 * w;   // this wave's 32-row tile
  const int i = i0 + ln;
  const bool in_range = i < p.L;
  int kb = INT_MAX, ke = INT_MIN;       // the tile's blocks: keys kb .. ke (kb a multiple of 32)
  if (i0 < p.L) {
    int bs0 = max(0, p.row_klo[(size_t)b * p.L + i0] - p.k_origin);
    if (p.window >= 0) bs0 = max(bs0, p.q_off + i0 - p.window);
    const int e = min(p.q_off + min(i0 + 31, p.L - 1), p.S - 1);
    // A tile whose first band starts past its last key has no key at all (a
    // one-row padding tile at the end: band start S): no dK/dV item visits it,
    // so none of its blocks is written and none may be read.
    if (bs0 <= e) {
      kb = bs0 & ~31;
      ke = e;
    }
  }
  kb = __builtin_amdgcn_readfirstlane(kb);
  ke = __builtin_amdgcn_readfirstlane(ke);
  const bool w_any = kb <= ke;
  if (lane == 0) { red[w][0] = w_any ? kb : INT_MAX; red[w][1] = w_any ? ke + 1 : INT_MIN; }
  __syncthreads();
  int kstart = INT_MAX, kend = INT_MIN;
#pragma unroll
  for (int x = 0; x < C::NW; ++x) { kstart = min(kstart, red[x][0]); kend = max(kend, red[x][1]); }
  kstart = __builtin_amdgcn_readfirstlane(kstart);
  kend = __builtin_amdgcn_readfirstlane(kend);

  const int bh = b * p.Hkv + kvh;
  const T* __restrict__ kbase = reinterpret_cast<const T*>(p.kv.k[0]) + (size_t)bh * p.S * D;
  // this lane's row in the tile's 32 x 32 dS blocks (see the dK/dV item's store)
  const int ds_nb = p.ds_w >> 5, ds_ntq = (p.L + 31) >> 5;
  const T* __restrict__ drow = reinterpret_cast<const T*>(p.dsbuf) +
                               ((size_t)(b * p.Hq + h) * ds_ntq + min(i0, p.L - 1) / 32) * ds_nb * 1024 + ln * 32;
  const TileDma<T, C::BN, D, C::NW> dma;
  const TileAccess<T, TL> acc(ln, lane);
  const KvPair<T, C::BN> pair = KV == kKvConcat ? KvPair<T, C::BN>() : KvPair<T, C::BN>(p.kv, bh, kstart, kend, D);
  auto load = [&](T* Ks, int j0) {
    if constexpr (KV == kKvConcat) {
      // unseen copies (nb_device.h): the loop's wait and barrier at the top of
      // each tile order the reads; a copy the compiler saw would make it wait
      // for the next tile's copies and dS loads before this tile's reads
      dma.issue_unseen(Ks, kbase + (size_t)j0 * D, min(C::BN, p.S - j0));
    } else {
      if (pair.ok) pair.load_k(dma, j0, Ks);   // uniform
      else kv_tile_load<T, C::BN, D, C::NW, false>(dma, p.kv, bh, j0, min(C::BN, p.S - j0), Ks, nullptr);
    }
  };
  // The B-operand fragments of one tile as stored: one load per 16 keys (the
  // lane's eight keys are contiguous, ds_slot), issued a tile ahead and used
  // only after the next top-of-tile wait, so nothing consumes them early.  The
  // block index is clamped to the row tile's own blocks (always in bounds); a
  // block outside the wave's range is replaced by zeros where it is used.
  constexpr int NM = C::BN / 16;
  auto ds_load = [&](F* raw, int j0) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int blk = min(max((j0 + 32 * (m >> 1) - kb) >> 5, 0), ds_nb - 1);
      raw[m] = __builtin_nontemporal_load(reinterpret_cast<const F*>(drow + blk * 1024 + 16 * (m & 1) + 8 * g));   // (read once)
    }
  };
  // zeros for blocks outside the wave's range (uniform), for rows past L and
  // for keys past S (the dK/dV items never wrote them)
  const bool rows_all = __builtin_amdgcn_readfirstlane(wave_min_i(in_range ? 1 : 0)) != 0;
  auto ds_mask = [&](F* fr, const F* raw, int j0) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int jw = j0 + 32 * (m >> 1);
      fr[m] = (jw >= kb && jw <= ke) ? raw[m] : F{};
    }
    if (!rows_all || j0 + C::BN > p.S) {   // uniform: the last row tile or the last key tile
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int k0 = j0 + 32 * (m >> 1) + 16 * (m & 1) + 4 * g;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (!in_range || k0 + (t & 3) + 8 * (t >> 2) >= p.S) fr[m][t] = to_elem<T>(0.f);
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) oacc[d] = f32x16{};
  constexpr int ND = D / 32;
  auto compute = [&](const T* Ks, const F* raw, int j0) __attribute__((always_inline)) {
    if (!w_any || j0 > ke || j0 + C::BN <= kb) return;
    F fr[NM];
    ds_mask(fr, raw, j0);
    lds_mfma_pipeline<NM * ND, C::AHEAD, F>(
        [&](int x) { return acc.col(Ks, x % ND, x / ND); },
        [&](int x, const F& a) { oacc[x % ND] = mma(a, fr[x / ND], oacc[x % ND]); });
  };
  F f0[NM], f1[NM];
  if (kstart < kend) {
    load(K0, kstart);
    ds_load(f0, kstart);
  }
  for (int j0 = kstart; j0 < kend; j0 += 2 * C::BN) {
    wait_global();
    __syncthreads();
    if (j0 + C::BN < kend) {
      load(K1, j0 + C::BN);
      ds_load(f1, j0 + C::BN);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(K0, f0, j0);
    if (j0 + C::BN >= kend) break;
    wait_global();
    __syncthreads();
    if (j0 + 2 * C::BN < kend) {
      load(K0, j0 + 2 * C::BN);
      ds_load(f0, j0 + 2 * C::BN);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(K1, f1, j0 + C::BN);
  }

  if constexpr (RowStage<T, C::NW, D>::ON) {
    if (p.dq_mode == kDqStore) {
      __syncthreads();   // every wave is done with the K tiles the staging overwrites
      T* const base = reinterpret_cast<T*>(p.dq) + (((size_t)b * p.Hq + h) * p.L + i0) * D;
      stage_rows_in<T, D>(&sm.st.r[w][0][0], oacc, p.scale);
      stage_rows_store<T, D>(&sm.st.r[w][0][0], base, D, min(32, p.L - i0));
      return;
    }
  }
  if (!in_range || (!w_any && p.dq_mode == kDqAddF32)) return;   // (no key: nothing to add)
  const size_t qrow = ((size_t)b * p.Hq + h) * p.L + i;
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int dd = 32 * d + 8 * rq + 4 * g;
      const float v0 = oacc[d][4 * rq] * p.scale, v1 = oacc[d][4 * rq + 1] * p.scale;
      const float v2 = oacc[d][4 * rq + 2] * p.scale, v3 = oacc[d][4 * rq + 3] * p.scale;
      if (p.dq_mode == kDqStore) {
        store_quad<T>(reinterpret_cast<T*>(p.dq) + qrow * D + dd, v0, v1, v2, v3);
      } else {
        f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.dq) + qrow * D + dd);
        f32x4 x = f32x4{v0, v1, v2, v3};
        if (p.dq_mode == kDqAddF32) {
          const f32x4 a = *dst;
          x = f32x4{a[0] + x[0], a[1] + x[1], a[2] + x[2], a[3] + x[3]};
        }
        *dst = x;
      }
    }
  }
}

// ---------------------------------------------------------------- Delta

// Delta_i = dO_i . O_i for every row (b, h, i), with O the stored value plus
// its saved rounding residual (fp32-accurate); 0 for padding rows.  Every lane
// reads 16 bytes of a row per tensor (D / 8 lanes per bf16 row, D / 4 per
// float32 row) and handles IT rows, all of whose loads are issued before any
// arithmetic, so each lane keeps 2 x IT 16-byte loads and IT residual loads in
// flight; the lanes of a row reduce with shuffles.  (Eight rows per workgroup
// with 4- to 16-byte loads launched one workgroup per 12 KB moved and
// measured about half the HBM rate; workgroups of 512 threads measured 5 %
// faster than 256 on the sliding layer, 1024 and 128 slower.)
constexpr int kPrepNT = 512;          // threads of the prep kernel's workgroups
template <typename T, int D>
struct DeltaCfg {
  // elements per load: 16 bytes, or more where a row would need more than a wave
  static constexpr int V = (16 / (int)sizeof(T)) * 64 >= D ? 16 / (int)sizeof(T) : D / 64;
  static constexpr int LPR = D / V;               // lanes per row
  static constexpr int RPI = 64 / LPR;            // rows of a wave per load round
  static constexpr int IT = D >= 512 ? 2 : D >= 256 ? 1 : 2;   // load rounds in flight (measured per head dim)
  static constexpr int ROWS = (kPrepNT / 64) * RPI * IT;   // rows per workgroup
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "a row's lanes tile the wave");
};

template <typename T, int D>
__device__ __forceinline__ void delta_rows(const BwdParams& p, int wg) {
  typedef DeltaCfg<T, D> C;
  typedef T VE __attribute__((ext_vector_type(C::V)));   // one 16-byte (or wider) load
  typedef int8_t VR __attribute__((ext_vector_type(C::V)));   // the residual codes of the same elements
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sub = lane % C::LPR, rsub = lane / C::LPR;
  const long long n_rows = (long long)p.B * p.Hq * p.L;
  // (bf16: O plus its saved residual codes, nb_device.h: resid_value; float32 O is exact)
  const bool with_resid = sizeof(T) == 2 && p.o_lo != nullptr;
  VE dv[C::IT], ov[C::IT];
  VR lv[C::IT];
  long long row[C::IT];
#pragma unroll
  for (int r = 0; r < C::IT; ++r) {
    row[r] = (long long)wg * C::ROWS + (w * C::IT + r) * C::RPI + rsub;
    const long long rr = row[r] < n_rows ? row[r] : n_rows - 1;
    const size_t e0 = (size_t)rr * D + (size_t)sub * C::V;
    dv[r] = *reinterpret_cast<const VE*>(reinterpret_cast<const T*>(p.dout) + e0);
    ov[r] = *reinterpret_cast<const VE*>(reinterpret_cast<const T*>(p.o) + e0);
    lv[r] = with_resid ? *reinterpret_cast<const VR*>(reinterpret_cast<const int8_t*>(p.o_lo) + e0) : VR{};
  }
#pragma unroll
  for (int r = 0; r < C::IT; ++r) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < C::V; ++e) {
      float o = to_f32(ov[r][e]);
      if constexpr (sizeof(T) == 2) {
        if (with_resid) o += resid_value(lv[r][e], ov[r][e]);
      }
      part += to_f32(dv[r][e]) * o;
    }
#pragma unroll
    for (int o = C::LPR / 2; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (row[r] < n_rows && sub == 0) {
      const int i = (int)(row[r] % p.L), b = (int)(row[r] / ((long long)p.Hq * p.L));
      const bool real = p.row_klo[(size_t)b * p.L + i] - p.k_origin <= p.q_off + i;
      p.delta[row[r]] = real ? part : 0.f;
    }
  }
}

// ---------------------------------------------------------------- work order

// Items of both passes sorted by decreasing work, ties in decreasing item
// order, in one workgroup (bitonic sort of (work, index) keys in LDS; more than
// kOrderMax items keep the natural order):
//   dK/dV: (batch row, key tile) -> number of 32-row query tiles whose bands
//          reach the tile, counted exactly as the pass counts them (binary
//          search over the nondecreasing band starts);
//   dQ:    (batch row, query tile) -> key range of its rows, from the first
//          row's band start to the last row's position (an estimate when the
//          first rows are padding -- the order only affects speed).
// Also empties the work queues of the backward kernel.
constexpr int kOrderMax = 2048;       // items sorted in LDS
constexpr int kOrderBandMax = 2048;   // query-tile band starts staged in LDS

template <int BK, int BQ, int BM>
__device__ void work_order(const BwdParams& p, int modes, unsigned long long* keys, int* bst) {
  const int tid = threadIdx.x;
  const int off = p.q_off;
  if (tid < kNumCounters) p.counters[tid] = 0;  // work queues and the deferred-item list start empty
  if (modes & 1) {
    const int n_kt = (p.S + BK - 1) / BK;
    const int n = p.B * n_kt;
    if (n > kOrderMax) {
      for (int i = tid; i < n; i += kPrepNT) p.order[i] = i;
    } else {
      const int n_q_tiles = (p.L + BQ - 1) / BQ;
      // band start of each query tile's first row (nondecreasing along a row)
      auto band_start_g = [&](int b, int t) {
        const int r = t * BQ;
        const int bq = max(0, p.row_klo[(size_t)b * p.L + r] - p.k_origin);
        return p.window >= 0 ? max(bq, off + r - p.window) : bq;
      };
      const bool staged = p.B * n_q_tiles <= kOrderBandMax;
      if (staged)
        for (int x = tid; x < p.B * n_q_tiles; x += kPrepNT) bst[x] = band_start_g(x / n_q_tiles, x % n_q_tiles);
      __syncthreads();
      int N = 1;
      while (N < n) N <<= 1;
      for (int i = tid; i < N; i += kPrepNT) {
        unsigned long long key = ~0ull;  // padding sorts last
        if (i < n) {
          const int b = i / n_kt, kt = i % n_kt;
          const int jmax = min(kt * BK + BK, p.S) - 1;
          const int t_first = max(0, kt * BK - off) / BQ;
          int lo = t_first, hi = n_q_tiles;  // first tile in [lo, hi) whose band starts after jmax
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            const int bsm = staged ? bst[b * n_q_tiles + mid] : band_start_g(b, mid);
            if (bsm <= jmax) lo = mid + 1;
            else hi = mid;
          }
          key = work_key((unsigned)(lo - t_first), i, n);
        }
        keys[i] = key;
      }
      order_by_work<kPrepNT>(keys, n, N, p.order);
    }
  }
  if (modes & 2) {
    const int n_qt = (p.L + BM - 1) / BM;
    const int n = p.B * n_qt;
    if (n > kOrderMax) {
      for (int i = tid; i < n; i += kPrepNT) p.qorder[i] = i;
    } else {
      int N = 1;
      while (N < n) N <<= 1;
      for (int i = tid; i < N; i += kPrepNT) {
        unsigned long long key = ~0ull;
        if (i < n) {
          const int b = i / n_qt, qt = i % n_qt;
          const int r0 = qt * BM, r1 = min(p.L, r0 + BM) - 1;
          int bq = max(0, p.row_klo[(size_t)b * p.L + r0] - p.k_origin);
          if (p.window >= 0) bq = max(bq, off + r0 - p.window);
          key = work_key((unsigned)max(0, min(off + r1 + 1, p.S) - bq), i, n);
        }
        keys[i] = key;
      }
      order_by_work<kPrepNT>(keys, n, N, p.qorder);
    }
  }
}

// The prep launch: workgroup 0 computes the work orders (dispatched first, so
// the serial sort overlaps the streaming), workgroups 1 .. gridDim.x - 1 form
// Delta (DeltaCfg::ROWS rows each); a grid of one workgroup computes the
// orders only.
// Owner o is attended iff some real key of its range [off[o], off[o + 1]) lies
// at or after its batch row's kcov_lo (the first key any segment covers): one
// workgroup of NT threads per owner.
template <int NT>
__device__ __forceinline__ void owner_flag(const OwnerParams& p, int o) {
  const int a = p.off[o], e = p.off[o + 1];
  int found = 0;
  for (int b = 0; b < p.B && !found; ++b) {
    const int lo = max(a, p.kcov_lo[b]);
    for (int jj = lo + (int)threadIdx.x; jj < e; jj += NT) {
      if (p.folded[(size_t)b * p.S + jj] > 0) { found = 1; break; }
    }
    found = __syncthreads_or(found);
  }
  if (threadIdx.x == 0) p.attended[o] = found ? 1 : 0;
}

// OWN: the last p.own.n_owner workgroups compute the owner flags (a separate
// instance, so the Delta workgroups of the other keep their short prologue).
template <typename T, int D, int BK, int BQ, int BM, bool OWN>
__global__ __launch_bounds__(kPrepNT) void bwd_prep_kernel(BwdParams p, int modes) {
  __shared__ unsigned long long keys[kOrderMax];
  __shared__ int bst[kOrderBandMax];
  if (blockIdx.x == 0) {
    work_order<BK, BQ, BM>(p, modes, keys, bst);
    return;
  }
  if constexpr (OWN) {
    const int first_owner = gridDim.x - p.own.n_owner;
    if ((int)blockIdx.x >= first_owner) {
      owner_flag<kPrepNT>(p.own, blockIdx.x - first_owner);
      return;
    }
  }
  delta_rows<T, D>(p, blockIdx.x - 1);
}

size_t dkdv_order_elems(int B, int S) { return (size_t)B * ((S + 31) / 32); }
size_t dq_order_elems(int B, int L) { return (size_t)B * ((L + 31) / 32); }
size_t dq_cross_elems(int B, int Hq, int L) { return (size_t)B * Hq * ((L + 31) / 32); }

// ---------------------------------------------------------------- backward kernel

template <typename T, int D>
union BwdSmemBoth {
  DkvSmem<T, D> kv;
  DkvStage<T, D> kst;
  DqSmem<T, D> q;
  DqStage<T, D> qst;
};
template <typename T, int D>
union BwdSmemKvOnly {
  DkvSmem<T, D> kv;
  DkvStage<T, D> kst;
};
template <typename T, int D>
union BwdSmemQOnly {
  DqSmem<T, D> q;
  DqStage<T, D> qst;
};
template <typename T, int D, int MODE>
struct BwdSmemFor {
  typedef typename std::conditional<MODE == 1, BwdSmemKvOnly<T, D>,
                                    typename std::conditional<MODE == 2, BwdSmemQOnly<T, D>,
                                                              BwdSmemBoth<T, D>>::type>::type type;
};

// A persistent grid (one workgroup per CU) drains the items of the selected
// passes (MODE bit 0: dK/dV, bit 1: dQ) from kNumQueues queues; workgroup w
// serves queue w % NQ, which holds the flat items f = q, q + NQ, ...  The flat
// list is the dK/dV items (longest first) followed by the dQ items (longest
// first), each with the kv head fastest: with 8 queues -- one per XCD, as
// consecutive workgroups land on consecutive XCDs -- every kv head stays on one
// XCD, whose L2 then holds the K/V and Q/dO rows its items share.  Running
// both passes in one grid lets the shorter dQ items fill the tail of the dK/dV
// items.  Which workgroup computes an item never changes the result.
template <typename T, int D, int MODE, int KV, bool AC = false>
__global__ __launch_bounds__((BwdShape<T, D>::NT), (BwdShape<T, D>::OCC)) void bwd_kernel(BwdParams p) {
  static_assert(DkvCfg<T, D>::NT == BwdShape<T, D>::NT && DqCfg<T, D>::NT == BwdShape<T, D>::NT,
                "one block shape for both passes");
  // (a pass that runs alone needs only its own LDS: at D = 512 the dK/dV pass
  // runs alone, and a float32 dQ item's tiles would not fit beside nothing)
  __shared__ typename BwdSmemFor<T, D, MODE>::type sm;
  auto dkdv = [&](int f) {
    if constexpr (MODE != 2) dkdv_item<T, D, KV != kKvConcat, MODE == 1, AC>(p, sm.kv, sm.kst, f);
  };
  const int n_kv = (MODE & 1) ? p.B * ((p.S + DkvCfg<T, D>::BK - 1) / DkvCfg<T, D>::BK) * p.Hkv : 0;
  const int n_q = (MODE & 2) ? p.B * ((p.L + DqCfg<T, D>::BM - 1) / DqCfg<T, D>::BM) * p.Hq : 0;
  const int total = n_kv + n_q;
  const int nq = min(kNumQueues, (int)gridDim.x);
  const int qcls = blockIdx.x % nq;
  int* const slot = reinterpret_cast<int*>(&sm);  // the fetched item, between items only
  for (;;) {
    if (threadIdx.x == 0) *slot = qcls + nq * atomicAdd(&p.counters[qcls], 1);
    __syncthreads();
    const int f = *slot;
    __syncthreads();  // every thread has the item before the item reuses the LDS
    if (f >= total) break;
    if constexpr (MODE == 1) {
      dkdv(f);
    } else if constexpr (MODE == 2) {
      dq_item<T, D, KV>(p, sm.q, sm.qst, f);
    } else {
      if (f < n_kv) dkdv(f);
      else dq_item<T, D, KV>(p, sm.q, sm.qst, f - n_kv);
    }
    __syncthreads();  // this item's LDS is dead before the next fetch
  }
}

// The dQ items the chunk-table backward deferred (their key ranges touch three
// or more chunks), taken from p.cross in the order they were appended.
template <typename T, int D>
__global__ __launch_bounds__((BwdShape<T, D>::NT), (BwdShape<T, D>::OCC)) void bwd_dq_cross_kernel(BwdParams p) {
  __shared__ BwdSmemQOnly<T, D> sm;
  int* const slot = reinterpret_cast<int*>(&sm);  // the fetched item, between items only
  for (;;) {
    if (threadIdx.x == 0) {
      const int x = atomicAdd(&p.counters[kCrossNext], 1);
      *slot = x < p.counters[kCrossCount] ? p.cross[x] : -1;
    }
    __syncthreads();
    const int f = *slot;
    __syncthreads();
    if (f < 0) break;
    dq_item<T, D, kKvAny>(p, sm.q, sm.qst, f);
    __syncthreads();
  }
}

// Delta (when with_delta) and the work orders of the passes in `modes`.
template <typename T, int D>
static hipError_t launch_prep_t(const BwdParams& p, bool with_delta, int modes, hipStream_t s) {
  typedef DkvCfg<T, D> CK;
  typedef DqCfg<T, D> CQ;
  static_assert(CK::BK >= 32 && CQ::BM >= 32, "the work-order arrays are sized for tiles of >= 32");
  const long long rows = (long long)p.B * p.Hq * p.L;
  constexpr int RW = DeltaCfg<T, D>::ROWS;
  const unsigned n_delta = with_delta ? (unsigned)((rows + RW - 1) / RW) : 0u;
  if (p.own.n_owner > 0)
    hipLaunchKernelGGL((bwd_prep_kernel<T, D, CK::BK, CK::BQ, CQ::BM, true>), dim3(n_delta + 1 + p.own.n_owner),
                       dim3(kPrepNT), 0, s, p, modes);
  else
    hipLaunchKernelGGL((bwd_prep_kernel<T, D, CK::BK, CK::BQ, CQ::BM, false>), dim3(n_delta + 1), dim3(kPrepNT), 0,
                       s, p, modes);
  return hipGetLastError();
}

// The persistent backward kernel, with the dK/dV items' copy placement
// (dkdv_item, AC): role A issues every copy in the in-step schedules when the
// neighbourhood has no left window.
template <typename T, int D, int MODE, int KV>
static void launch_bwd_kernel(const BwdParams& p, dim3 grid, hipStream_t s) {
  if constexpr ((MODE & 1) && !DkvCfg<T, D>::SKEW && D <= 128) {
    if (p.window < 0) {
      hipLaunchKernelGGL((bwd_kernel<T, D, MODE, KV, true>), grid, dim3(BwdShape<T, D>::NT), 0, s, p);
      return;
    }
  }
  hipLaunchKernelGGL((bwd_kernel<T, D, MODE, KV>), grid, dim3(BwdShape<T, D>::NT), 0, s, p);
}

template <typename T, int D, int MODE>
static hipError_t launch_main_t(const BwdParams& p, hipStream_t s) {
  const long long n_kv = (MODE & 1) ? (long long)p.B * ((p.S + DkvCfg<T, D>::BK - 1) / DkvCfg<T, D>::BK) * p.Hkv : 0;
  const long long n_q = (MODE & 2) ? (long long)p.B * ((p.L + DqCfg<T, D>::BM - 1) / DqCfg<T, D>::BM) * p.Hq : 0;
  dim3 grid((unsigned)std::min<long long>(n_kv + n_q, (long long)device_cu_count() * BwdShape<T, D>::OCC));
  // the chunk-table variants exist for the full backward only (the split
  // passes take the concatenated neighbourhood)
  const bool concat = p.kv.n == 1 && p.kv.start[0] == 0 && p.kv.rows[0] == p.S;
  if constexpr (MODE == 3) {
    if (!concat && p.dsbuf != nullptr) {   // dK/dV items storing dS, then dQ = dS K, both through the table
      const long long n_kv1 = (long long)p.B * ((p.S + DkvCfg<T, D>::BK - 1) / DkvCfg<T, D>::BK) * p.Hkv;
      dim3 grid1((unsigned)std::min<long long>(n_kv1, (long long)device_cu_count() * BwdShape<T, D>::OCC));
      hipLaunchKernelGGL((bwd_kernel<T, D, 1, kKvPair>), grid1, dim3(BwdShape<T, D>::NT), 0, s, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      dim3 grid2((unsigned)((p.L + DqsCfg<T, D>::BM - 1) / DqsCfg<T, D>::BM) * p.Hq * p.B);
      hipLaunchKernelGGL((dq_ds_kernel<T, D, kKvPair>), grid2, dim3(DqsCfg<T, D>::NT), 0, s, p);
      return hipGetLastError();
    }
    if (!concat) {
      launch_bwd_kernel<T, D, MODE, kKvPair>(p, grid, s);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess || !kv_may_need_general(p.kv, p.window, DqCfg<T, D>::BM, DqCfg<T, D>::BN)) return e;
      dim3 grid2((unsigned)std::min<long long>(n_q, (long long)device_cu_count() * BwdShape<T, D>::OCC));
      hipLaunchKernelGGL((bwd_dq_cross_kernel<T, D>), grid2, dim3(BwdShape<T, D>::NT), 0, s, p);
      return hipGetLastError();
    }
  }
  if constexpr (MODE == 3) {
    if (p.dsbuf != nullptr) {   // dK/dV items storing dS, then dQ = dS K
      const long long n_kv1 = (long long)p.B * ((p.S + DkvCfg<T, D>::BK - 1) / DkvCfg<T, D>::BK) * p.Hkv;
      dim3 grid1((unsigned)std::min<long long>(n_kv1, (long long)device_cu_count() * BwdShape<T, D>::OCC));
      hipLaunchKernelGGL((bwd_kernel<T, D, 1, kKvConcat>), grid1, dim3(BwdShape<T, D>::NT), 0, s, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      dim3 grid2((unsigned)((p.L + DqsCfg<T, D>::BM - 1) / DqsCfg<T, D>::BM) * p.Hq * p.B);
      hipLaunchKernelGGL((dq_ds_kernel<T, D, kKvConcat>), grid2, dim3(DqsCfg<T, D>::NT), 0, s, p);
      return hipGetLastError();
    }
  }
  launch_bwd_kernel<T, D, MODE, kKvConcat>(p, grid, s);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_t(const BwdParams& p, int what, hipStream_t s) {
  hipError_t e = hipSuccess;
  if constexpr (D >= 512) {
    // The global layers' head dim: the dK/dV items store dS and dQ = dS K runs
    // as its own GEMM (a dQ item recomputing S and dP would not fit a wave);
    // one concatenated K/V buffer.
    const bool concat = p.kv.n == 1 && p.kv.start[0] == 0 && p.kv.rows[0] == p.S;
    switch (what) {
      case kBwdPrep:
        return launch_prep_t<T, D>(p, true, 3, s);
      case kBwdOrders:
        return launch_prep_t<T, D>(p, false, 3, s);
      case kBwdMain: {
        if (p.dsbuf == nullptr || !concat) return hipErrorInvalidValue;
        const long long n_kv = (long long)p.B * ((p.S + DkvCfg<T, D>::BK - 1) / DkvCfg<T, D>::BK) * p.Hkv;
        dim3 grid1((unsigned)std::min<long long>(n_kv, (long long)device_cu_count() * BwdShape<T, D>::OCC));
        hipLaunchKernelGGL((bwd_kernel<T, D, 1, kKvConcat>), grid1, dim3(BwdShape<T, D>::NT), 0, s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        dim3 grid2((unsigned)((p.L + DqsCfg<T, D>::BM - 1) / DqsCfg<T, D>::BM) * p.Hq * p.B);
        hipLaunchKernelGGL((dq_ds_kernel<T, D, kKvConcat>), grid2, dim3(DqsCfg<T, D>::NT), 0, s, p);
        return hipGetLastError();
      }
    }
    return hipErrorInvalidValue;
  } else {
  switch (what) {
    case kBwdPrep:   // Delta + work orders of both passes
      return launch_prep_t<T, D>(p, true, 3, s);
    case kBwdOrders:   // the work orders alone (Delta already in the workspace)
      return launch_prep_t<T, D>(p, false, 3, s);
    case kBwdMain:
      return launch_main_t<T, D, 3>(p, s);
    case kBwdDq:     // Delta + the dQ order, then the dQ pass alone
      e = launch_prep_t<T, D>(p, true, 2, s);
      return e != hipSuccess ? e : launch_main_t<T, D, 2>(p, s);
    case kBwdDkdv:   // the dK/dV pass alone (Delta from an earlier dQ / prep call)
      e = launch_prep_t<T, D>(p, false, 1, s);
      return e != hipSuccess ? e : launch_main_t<T, D, 1>(p, s);
  }
  return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const BwdParams& p, int D, bool f32, int what, hipStream_t s) {
  if (f32) {
    if (D == 64) return launch_t<float, 64>(p, what, s);
    if (D == 128) return launch_t<float, 128>(p, what, s);
    if (D == 256) return launch_t<float, 256>(p, what, s);
    if (D == 512) return launch_t<float, 512>(p, what, s);
  } else {
    if (D == 64) return launch_t<bf16, 64>(p, what, s);
    if (D == 128) return launch_t<bf16, 128>(p, what, s);
    if (D == 256) return launch_t<bf16, 256>(p, what, s);
    if (D == 512) return launch_t<bf16, 512>(p, what, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- owner flags

// attended[o] = 1 iff some batch row has a covered key in chunk o: a key j is
// covered iff j >= kcov_lo[b] and folded[b, j] > 0 (every covered key is
// attended by at least one real query row, see the segment builder).
__global__ __launch_bounds__(256) void owner_flags_kernel(OwnerParams p) { owner_flag<256>(p, blockIdx.x); }

// dK/dV rows of chunk buffers outside the neighbourhood ([0, start) and
// [start + len, rows) of every (batch, kv head)): exact zeros, as for keys no
// query attends.
__global__ __launch_bounds__(256) void kv_zero_outside_kernel(KvChunks c, int BH, int row_vecs) {
  const int x = blockIdx.y;
  const int len = c.off[x + 1] - c.off[x];
  const int rows = c.rows[x], st = c.start[x];
  const int outside = rows - len;
  if (outside <= 0) return;
  const size_t n = (size_t)BH * outside * row_vecs;
  uint4* dk = reinterpret_cast<uint4*>(c.dk[x]);
  uint4* dv = reinterpret_cast<uint4*>(c.dv[x]);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t vec = i % row_vecs, rr = i / row_vecs;
    const int bh = (int)(rr / outside);
    int r = (int)(rr % outside);
    if (r >= st) r += len;
    const size_t o = ((size_t)bh * rows + r) * row_vecs + vec;
    dk[o] = uint4{0u, 0u, 0u, 0u};
    dv[o] = uint4{0u, 0u, 0u, 0u};
  }
}

hipError_t launch_kv_zero_outside(const KvChunks& c, int BH, int row_bytes, hipStream_t s) {
  int64_t most = 0;
  for (int x = 0; x < c.n; ++x) most = std::max<int64_t>(most, (int64_t)c.rows[x] - (c.off[x + 1] - c.off[x]));
  if (most == 0) return hipSuccess;
  const int row_vecs = row_bytes / 16;
  const int64_t need = ((int64_t)BH * most * row_vecs + 255) / 256;
  dim3 grid((unsigned)std::min<int64_t>(need, 1024), (unsigned)c.n);
  hipLaunchKernelGGL(kv_zero_outside_kernel, grid, dim3(256), 0, s, c, BH, row_vecs);
  return hipGetLastError();
}

hipError_t launch_owner_flags(const OwnerParams& p, hipStream_t s) {
  hipLaunchKernelGGL(owner_flags_kernel, dim3(p.n_owner), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace nb
