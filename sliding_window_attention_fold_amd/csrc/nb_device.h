// Device-side building blocks shared by the nbattn HIP kernels (gfx950 only).
//
// Matrix-core atom: one 32x32 output tile with a contraction of 16, computed by
// v_mfma_f32_32x32x16_bf16 for bfloat16 and by eight v_mfma_f32_32x32x2_f32 for
// the float32 debug path.  Both read their operands in the same lane layout, so
// every kernel is written once over the element type:
//
//   A (32 x 16):  lane l holds row (l % 32), contraction slots 8*(l/32) + t, t < 8
//   B (16 x 32):  lane l holds column (l % 32), contraction slots 8*(l/32) + t
//   C (32 x 32):  lane l holds column (l % 32); accumulator r holds row
//                 8*(r/4) + 4*(l/32) + (r%4)
//
// (measured on the device with a lane-layout check against a host matmul).
//
// A product whose A or B operand is a previous accumulator (softmax
// probabilities) takes its contraction index from the accumulator rows, which
// within a 16-slot step of a 32-row tile are  kappa(m, g, t) =
// 16*m + 8*(t/4) + 4*g + (t%4)  for step m, lane group g = l/32 and slot t.  The
// operand read from LDS must then place element kappa(m,g,t) at slot 8*g + t of
// step m, i.e. within every aligned 16-element group the 4-element quads 1 and 2
// trade places.  `perm16` is that position map (an involution).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nb {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// Softmax reference lag (log2 units): the running exponent reference moves
// when a row maximum exceeds it by more than this.  It is 0: the reference is
// the exact running maximum, so the key holding a row's maximum gets the
// unnormalised probability 2^0 = 1, which bf16 represents exactly.  With a lag,
// that probability is 2^x for some 0 < x <= lag and is rounded (up to 2^-9
// relative) before the P.V product; the backward recomputes P exactly, so
// Delta = dO . O then misses by that rounding times dO . v of the dominant key,
// and in a row dominated by one key dS = P (dP - Delta) is a small difference
// of large terms: rows of outlier scores were measured outside the 2e-2
// tolerance of dQ with a lag of 8.
constexpr float kRefLag = 0.0f;

// Wave index within the workgroup, as a wave-uniform (scalar) value: LDS
// destinations of the async copies must be uniform, and without the hint the
// compiler wraps every copy in a waterfall loop.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// 2^x with the hardware instruction (inputs are <= kRefLag or -inf here).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mma(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], c, 0, 0, 0);
  return c;
}

// Position of element e inside its aligned 16-element group after quads 1 and 2 swap.
__device__ __forceinline__ constexpr int perm16(int e) {
  const int q = (e >> 2) & 3;
  const int nq = (q == 1) ? 2 : (q == 2) ? 1 : q;
  return (e & ~15) | (nq << 2) | (e & 3);
}

// Row held by accumulator r of a 32x32 tile for lane group g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

template <typename T> __device__ __forceinline__ T to_elem(float x);
template <> __device__ __forceinline__ bf16 to_elem<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float to_elem<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

// Eight accumulators (slots 8*half .. 8*half+7 of a 32x32 tile) as an operand fragment.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type acc_to_frag(const f32x16& c, int half) {
  typename Frag<T>::type f;
#pragma unroll
  for (int t = 0; t < 8; ++t) f[t] = to_elem<T>(c[8 * half + t]);
  return f;
}

// 16-byte (bf16) / 32-byte (f32) fragment loads and stores.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type load_frag(const T* p) {
  return *reinterpret_cast<const typename Frag<T>::type*>(p);
}

template <typename T>
__device__ __forceinline__ typename Frag<T>::type zero_frag() {
  typename Frag<T>::type f;
#pragma unroll
  for (int t = 0; t < 8; ++t) f[t] = to_elem<T>(0.f);
  return f;
}

// Four consecutive elements.
template <typename T> struct Quad;
template <> struct Quad<bf16> { typedef bf16x4 type; };
template <> struct Quad<float> { typedef f32x4 type; };

template <typename T>
__device__ __forceinline__ void store_quad(T* p, float a, float b, float c, float d) {
  typename Quad<T>::type v;
  v[0] = to_elem<T>(a); v[1] = to_elem<T>(b); v[2] = to_elem<T>(c); v[3] = to_elem<T>(d);
  *reinterpret_cast<typename Quad<T>::type*>(p) = v;
}

// The saved rounding residual of a bf16 output, for the backward's Delta: one
// signed byte per element, r = a - bf16(a) in units of 1/254 of the stored
// value's ulp.  |r| <= ulp / 2, so the code lies in [-127, 127]; decoded, the
// stored value plus the residual carries about 17 significant bits (the error
// is at most ulp / 508), half the bytes of a bf16 residual (about 16 bits).
// Encoder and decoder take the ulp from the stored value's exponent field
// (subnormals and zero: the subnormal ulp 2^-133).
__device__ __forceinline__ int resid_ulp_exp(bf16 v) {
  const unsigned be = (__builtin_bit_cast(unsigned short, v) >> 7) & 0xFFu;
  return (int)(be > 1u ? be : 1u) - 127 - 7;
}
__device__ __forceinline__ uint32_t resid_code(float a, bf16 v) {
  const float x = rintf(ldexpf(a - (float)v, -resid_ulp_exp(v)) * 254.f);
  return (uint32_t)(int32_t)fminf(fmaxf(x, -127.f), 127.f) & 0xFFu;
}
__device__ __forceinline__ float resid_value(int8_t q, bf16 v) {
  return ldexpf((float)q * (1.f / 254.f), resid_ulp_exp(v));
}

// This lane's index in its wave, from an instruction the compiler cannot move:
// values derived from it are formed where they are used, not hoisted out of
// the loops before that point to sit in registers across them.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The value lane l ^ 32 holds (the other half of the wave), through
// v_permlane32_swap: no LDS round trip and no wait on outstanding LDS reads.
// The swap trades the upper half of its first operand with the lower half of
// its second, so with x in both, lanes 0..31 find their partner in the second
// result and lanes 32..63 in the first.
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

}  // namespace nb

namespace nb {

// Bytes of padding after every LDS row: keeps 16-byte alignment and moves
// consecutive rows onto different banks.
constexpr int kLdsPadBytes = 16;

template <typename T> struct Pad { static constexpr int elems = kLdsPadBytes / sizeof(T); };

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Rows of a result leave through LDS (bf16): a lane's accumulators hold four
// columns of one row, so stored directly a store instruction writes 16 bytes
// to each of 32 rows (32 cache lines for 512 bytes); staged and read back as
// 16-byte row pieces, an instruction writes whole row segments.  NWS waves
// stage 32 rows of W columns each, rows padded by 16 bytes (they stay 16-byte
// aligned).
//
// Bank layout (64 banks of 4 bytes).  Writers: lanes 0..31 hold rows 0..31 at
// the same 8-byte half of a 16-byte piece (lanes 32..63 the other half), so
// rows 16..31 keep the two halves of every piece swapped; with the 16-byte pad
// the 64 lanes of a 4-byte write (the residual codes) then cover the 64 banks
// once, which removed those writes' conflicts.  An 8-byte write down 32 rows
// measured about twice the LDS cycles of a contiguous one with or without the
// swap.  Readers: a row of W columns is LPR pieces, read by LPR lanes; where
// the 16 lanes of one 16-byte read span several rows (LPR < 16), those rows
// sit LPR physical rows apart, in different banks.
template <typename T, int NWS, int W>
struct RowStage {
  static constexpr bool ON = sizeof(T) == 2;
  static constexpr int RS = W + 8;
  __attribute__((aligned(1024))) T r[ON ? NWS : 1][ON ? 32 : 1][ON ? RS : 1];
};
// Physical staging row of row r (0..31) for rows of LPR 16-byte pieces.  For r0
// a multiple of 64 / LPR and rl < 64 / LPR it is additive:
// stage_row(r0 + rl) = stage_row(r0) + stage_row(rl).
template <int LPR>
__device__ __forceinline__ constexpr int stage_row(int r) {
  if constexpr (LPR >= 16) {
    return r;
  } else {
    constexpr int P = 16 / LPR;
    return (r & 16) | ((r & 15) / P) | ((r % P) * LPR);
  }
}
// A staged 16-byte piece of row r as written by stage_rows_in / stage_codes_in,
// halves back in order when hi (r >= 16; constant in the unrolled loops below).
__device__ __forceinline__ u32x4 stage_piece(const void* p, bool hi) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return hi ? u32x4{v[2], v[3], v[0], v[1]} : v;
}
// One wave's 32 x W block (lane: row ln, columns 32 d + 8 rq + 4 g .. + 3 of
// block d, values x[d][4 rq + e] * sc) written to its staging rows st.
// Wave-local: LDS operations of one wave complete in order, so the read-back
// below sees every lane's writes without a barrier.
template <typename T, int W, typename Acc>
__device__ __forceinline__ void stage_rows_in(T* st, const Acc& x, float sc) {
  typedef typename Quad<T>::type Q4;
  constexpr int RS = W + 8;
  const int lane = lane_here(), ln = lane & 31, g = lane >> 5, h = ln >> 4;
  T* const dst = st + stage_row<W / 8>(ln) * RS + 4 * (g ^ h);
#pragma unroll
  for (int d = 0; d < W / 32; ++d) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      Q4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = to_elem<T>(x[d][4 * rq + e] * sc);
      *reinterpret_cast<Q4*>(dst + 32 * d + 8 * rq) = v;
    }
  }
}
// The staged rows r < nrows stored as 16-byte pieces: row r at base + r * ld
// elements (base wave-uniform, so each store takes a scalar base and a 32-bit
// lane offset).
template <typename T, int W>
__device__ __forceinline__ void stage_rows_store(const T* st, T* base, size_t ld, int nrows) {
  constexpr int RS = W + 8, LPR = W / 8, RPI = 64 / LPR;
  const int lane = lane_here(), rl = lane / LPR, c = 8 * (lane % LPR);
  const uint32_t voff = (uint32_t)((rl * ld + c) * sizeof(T));
  const T* const src = st + stage_row<LPR>(rl) * RS + c;
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const u32x4 v = stage_piece(src + stage_row<LPR>(r0) * RS, r0 >= 16);
    char* const row = reinterpret_cast<char*>(base + r0 * ld);
    if (r0 + rl < nrows) *reinterpret_cast<u32x4*>(row + voff) = v;
  }
}
// As above, with each row's address from row_ptr(r) (rows not evenly spaced).
template <typename T, int W, typename RowPtr>
__device__ __forceinline__ void stage_rows_store_at(const T* st, int nrows, RowPtr row_ptr) {
  constexpr int RS = W + 8, LPR = W / 8, RPI = 64 / LPR;
  const int lane = lane_here(), rl = lane / LPR, c = 8 * (lane % LPR);
  const T* const src = st + stage_row<LPR>(rl) * RS + c;
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + rl;
    const u32x4 v = stage_piece(src + stage_row<LPR>(r0) * RS, r0 >= 16);
    if (r < nrows) *reinterpret_cast<u32x4*>(row_ptr(r) + c) = v;
  }
}
// The residual codes of one wave's 32 x W bf16 block (values x[d][4 rq + e] * sc
// as in stage_rows_in) staged as bytes: rows of W bytes padded by 16, in the
// layout above (a lane's 4 codes at byte 32 d + 8 rq + 4 g of its row, the
// 8-byte halves of each 16-byte piece swapped in rows 16..31).
template <int W, typename Acc>
__device__ __forceinline__ void stage_codes_in(uint8_t* st, const Acc& x, float sc) {
  constexpr int RS = W + 16;
  const int lane = lane_here(), ln = lane & 31, g = lane >> 5, sw = 8 * (ln >> 4);
  uint8_t* const dst = st + stage_row<W / 16>(ln) * RS + 4 * g;
#pragma unroll
  for (int d = 0; d < W / 32; ++d) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = x[d][4 * rq + e] * sc;
        word |= resid_code(a, (bf16)a) << (8 * e);
      }
      *reinterpret_cast<uint32_t*>(dst + 32 * d + 8 * rq + ((rq & 1) ? -sw : sw)) = word;
    }
  }
}
// The staged code rows r < nrows stored as 16-byte pieces at base + r * ld bytes.
template <int W>
__device__ __forceinline__ void stage_codes_store(const uint8_t* st, uint8_t* base, size_t ld, int nrows) {
  constexpr int RS = W + 16, LPR = W / 16, RPI = 64 / LPR;
  const int lane = lane_here(), rl = lane / LPR, c = 16 * (lane % LPR);
  const uint32_t voff = (uint32_t)(rl * ld + c);
  const uint8_t* const src = st + stage_row<LPR>(rl) * RS + c;
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const u32x4 v = stage_piece(src + stage_row<LPR>(r0) * RS, r0 >= 16);
    if (r0 + rl < nrows) *reinterpret_cast<u32x4*>(base + r0 * ld + voff) = v;
  }
}

// ---------------------------------------------------------------------------
// LDS tiles.  A tile holds ROWS rows of a row-major [*, D] matrix, row-major in
// LDS with no padding; the 16-byte chunks of each row are XOR-swizzled by a
// function of the row (period 16 rows) so that both the row reads of an MFMA
// operand and the transpose reads are free of bank conflicts.
// ---------------------------------------------------------------------------
template <typename T, int ROWS, int D>
struct Tile {
  static constexpr int EPC = 16 / sizeof(T);     // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;            // chunks per row (>= 8)
  static constexpr int ELEMS = ROWS * D;
  static constexpr int BLOCKS = ROWS * CPR / 64; // 1 KB blocks (one DMA instruction each)
  static_assert(CPR >= 8 && (CPR & (CPR - 1)) == 0, "row must be >= 8 power-of-two chunks");
  static_assert(ROWS * CPR % 64 == 0, "tile must be whole 1 KB blocks");
  // LDS has 64 banks of 4 bytes.  A 16-byte row read serves 16 lanes per
  // cycle (rows r..r+15 at one chunk): swz must be a bijection on 16
  // consecutive rows.  A transpose read serves 32 lanes per cycle (4
  // consecutive rows x one aligned 64-byte group of 4 chunks): the 4 rows must
  // land on different 4-chunk groups.  Rows of 8 chunks (128 bytes) pair up
  // per 256-byte bank line, hence the separate form.
  __device__ static __forceinline__ constexpr int swz(int r) {
    return CPR >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  // element offset of logical chunk lc of row r
  __device__ static __forceinline__ int off(int r, int lc) { return r * D + ((lc ^ swz(r)) * EPC); }
};

#define NB_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))
#define NB_LOCAL(p) ((__attribute__((address_space(3))) void*)(p))

// Asynchronous copy of rows [0, ROWS) of src (row stride D) into a tile with
// global_load_lds (no registers involved).  Rows at or beyond nrows repeat row
// nrows-1: finite values the kernels always mask out.  Each wave moves whole
// 1 KB blocks: lane l of block blk fills physical chunk blk*64 + l.
template <typename T, int ROWS, int D, int NW>
__device__ __forceinline__ void dma_tile(T* lds, const T* __restrict__ src, int nrows) {
  typedef Tile<T, ROWS, D> TL;
  const int w = wave_id(), l = threadIdx.x & 63;
#pragma unroll
  for (int x = 0; x < (TL::BLOCKS + NW - 1) / NW; ++x) {
    const int blk = w + x * NW;
    if (TL::BLOCKS % NW != 0 && blk >= TL::BLOCKS) break;
    const int P = blk * 64 + l;
    const int r = P / TL::CPR, pc = P % TL::CPR;
    const int lc = pc ^ TL::swz(r);
    const T* g = src + (size_t)min(r, nrows - 1) * D + lc * TL::EPC;
    __builtin_amdgcn_global_load_lds(NB_GLOBAL(g), NB_LOCAL(lds + blk * 64 * TL::EPC), 16, 0, 0);
  }
}

// The same copy through a buffer resource: the tile's base lives in scalar
// registers and each lane keeps the byte offsets of its chunks (loop
// invariant), so issuing a full tile costs one instruction per 1 KB block and
// no vector arithmetic.  Rows at or beyond nrows repeat row nrows-1 (uniform
// slow path for the last, partial tile).
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format

// ---------------------------------------------------------------------------
// Copies into LDS issued through inline asm ("unseen" copies).  The compiler
// does not know these instructions write LDS, so it adds no waits of its own:
// where a ring's slot index is a run-time value it cannot tell a copy's LDS
// destination from the slot a later LDS read uses, and would wait for every
// copy in flight before each such read -- including the copies just issued
// for later steps, which serialises the ring.  The caller orders every LDS
// read of a destination after its copies with wait_global / wait_global_le
// (and a barrier where other waves read it).  The instructions write no
// register; M0 is set inside the asm and declared clobbered.
// ---------------------------------------------------------------------------
// Raw buffer descriptor words (base, stride 0, num_records bytes, kBufferWord3).
__device__ __forceinline__ u32x4 buffer_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, (uint32_t)kBufferWord3};
}
// LDS byte address of a (generic) pointer to __shared__ memory: the low 32
// bits of a flat address in the LDS aperture are the LDS offset.  (An
// address-space cast of a run-time pointer here tripped the backend.)
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }
// 16 bytes per lane from rsrc + voff into LDS at lds_byte + 16 * lane (wave-uniform lds_byte).
__device__ __forceinline__ void unseen_copy16(const u32x4& rsrc, uint32_t lds_byte, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_byte)), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
// 4 bytes per lane from gaddr into LDS at lds_byte + 4 * lane.
__device__ __forceinline__ void unseen_copy4(const void* gaddr, uint32_t lds_byte) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_byte)), "v"(gaddr)
      : "memory", "m0");
}


template <typename T, int ROWS, int D, int NW>
struct TileDma {
  typedef Tile<T, ROWS, D> TL;
  static constexpr int PER = (TL::BLOCKS + NW - 1) / NW;
  static constexpr int RB = D * (int)sizeof(T);  // row bytes
  uint32_t voff[PER];
  __device__ __forceinline__ TileDma() {
    const int w = wave_id(), l = threadIdx.x & 63;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int P = (w + x * NW) * 64 + l;
      const int r = P / TL::CPR, pc = P % TL::CPR;
      voff[x] = (uint32_t)(r * RB + ((pc ^ TL::swz(r)) * 16));
    }
  }
  // number of copies one call of issue() makes from this wave
  __device__ __forceinline__ int count() const {
    const int w = wave_id();
    int c = 0;
#pragma unroll
    for (int x = 0; x < PER; ++x) c += (TL::BLOCKS % NW == 0 || w + x * NW < TL::BLOCKS) ? 1 : 0;
    return c;
  }
  // Tile rows [r_lo, r_hi) only, from src = the source row of tile row r_lo
  // (rows at or beyond nrows repeat row nrows - 1); other lanes sit idle.  A
  // tile whose rows come from several buffers is copied range by range.
  __device__ __forceinline__ void issue_rows(T* lds, const T* __restrict__ src, int r_lo, int r_hi, int nrows) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int w = wave_id(), l = threadIdx.x & 63;
    typedef __attribute__((address_space(3))) void lds_void;
    const int span = min(r_hi, nrows) - r_lo;   // source rows read
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, span * RB, kBufferWord3);
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int blk = w + x * NW;
      const int r = (blk * 64 + l) / TL::CPR;
      if ((TL::BLOCKS % NW == 0 || blk < TL::BLOCKS) && r >= r_lo && r < r_hi) {
        const uint32_t o = voff[x] - (uint32_t)((r_lo + r - min(r, nrows - 1)) * RB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + blk * 64 * TL::EPC), 16, o, 0, 0, 0);
      }
    }
#endif
  }
  // All ROWS tile rows, rows [0, n0) from srcA (the source row of tile row 0)
  // and rows [n0, ROWS) from srcB (the source row of tile row n0), 0 < n0 < ROWS.
  // A lane's tile row is its offset's row (offsets stay below RB past the row
  // start), so one compare against n0 * RB picks the source.
  __device__ __forceinline__ void issue_split(T* lds, const T* __restrict__ srcA, const T* __restrict__ srcB,
                                              int n0) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int w = wave_id();
    typedef __attribute__((address_space(3))) void lds_void;
    const uint32_t cut = (uint32_t)(n0 * RB);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)srcA, (short)0, n0 * RB, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)srcB, (short)0, (ROWS - n0) * RB, kBufferWord3);
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int blk = w + x * NW;
      if (TL::BLOCKS % NW == 0 || blk < TL::BLOCKS) {
        lds_void* dst = (lds_void*)(lds + blk * 64 * TL::EPC);
        if (voff[x] < cut) __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, voff[x], 0, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, voff[x] - cut, 0, 0, 0);
      }
    }
#endif
  }
  // issue() through unseen copies (see unseen_copy16).
  __device__ __forceinline__ void issue_unseen(T* lds, const T* __restrict__ src, int nrows) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int w = wave_id(), l = threadIdx.x & 63;
    const uint32_t lb = lds_addr(lds);
    const u32x4 rs = buffer_words(src, (uint32_t)(min(nrows, ROWS) * RB));
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int blk = w + x * NW;
      uint32_t o = voff[x];
      if (nrows < ROWS) {
        const int r = (blk * 64 + l) / TL::CPR;
        o -= (uint32_t)((r - min(r, nrows - 1)) * RB);
      }
      if (TL::BLOCKS % NW == 0 || blk < TL::BLOCKS) unseen_copy16(rs, lb + (uint32_t)(blk * 64 * TL::EPC * sizeof(T)), o);
    }
#endif
  }
  __device__ __forceinline__ void issue(T* lds, const T* __restrict__ src, int nrows) const {
    // The buffer-resource type exists only for the device target; the host
    // pass (which only needs the kernels' launch stubs) sees an empty body.
#if defined(__HIP_DEVICE_COMPILE__)
    const int w = wave_id(), l = threadIdx.x & 63;
    typedef __attribute__((address_space(3))) void lds_void;
    if (nrows >= ROWS) {
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, ROWS * RB, kBufferWord3);
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int blk = w + x * NW;
        if (TL::BLOCKS % NW == 0 || blk < TL::BLOCKS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + blk * 64 * TL::EPC), 16, voff[x], 0, 0, 0);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nrows * RB, kBufferWord3);
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int blk = w + x * NW;
        const int r = (blk * 64 + l) / TL::CPR;
        const uint32_t o = voff[x] - (uint32_t)((r - min(r, nrows - 1)) * RB);
        if (TL::BLOCKS % NW == 0 || blk < TL::BLOCKS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + blk * 64 * TL::EPC), 16, o, 0, 0, 0);
      }
    }
#endif
  }
};

// Asynchronous copy of n <= 64 consecutive 4-byte words (one wave; lanes >= n
// repeat word n-1).  The destination must hold 64 words.
template <bool UNSEEN = false>
__device__ __forceinline__ void dma_words(void* lds, const void* __restrict__ src, int n) {
  const int l = threadIdx.x & 63;
  const char* g = reinterpret_cast<const char*>(src) + 4 * min(l, n - 1);
  if constexpr (UNSEEN) unseen_copy4(g, lds_addr(lds));
  else __builtin_amdgcn_global_load_lds(NB_GLOBAL(g), NB_LOCAL(lds), 4, 0, 0);
}

// Scheduling hints: interleave N MFMAs each preceded by R LDS reads, so that
// only a couple of operand fragments are live at a time (with one wave per
// SIMD the scheduler otherwise hoists every read and runs out of registers).
template <int N, int R>
__device__ __forceinline__ void interleave_lds_mfma() {
#pragma unroll
  for (int x = 0; x < N; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
  }
}

// Software-pipelined form: the first AHEAD groups of R reads are issued up
// front, then each MFMA is followed by the reads AHEAD MFMAs ahead of it, so
// the LDS latency of an operand is covered by the MFMAs issued in between.
template <int N, int R, int AHEAD>
__device__ __forceinline__ void pipeline_lds_mfma() {
  static_assert(AHEAD >= 1 && AHEAD <= N, "read-ahead must be within the product");
  __builtin_amdgcn_sched_group_barrier(0x100, R * AHEAD, 0);
#pragma unroll
  for (int x = 0; x < N - AHEAD; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// Explicit software pipeline of N (operand read, MFMA) pairs: the reads of
// the first A operands are issued up front and each MFMA k is issued together
// with the read of operand k + A.  Scheduling barriers pin that order, so an
// operand's LDS latency is covered by the A MFMAs issued before its use; A + 1
// fragments are live at a time.
template <int N, int A, typename F, typename ReadFn, typename MmaFn>
__device__ __forceinline__ void lds_mfma_pipeline(ReadFn&& rd, MmaFn&& mm) {
  static_assert(A >= 1 && A <= N, "read-ahead must be within the product");
  F buf[A];
#pragma unroll
  for (int x = 0; x < A; ++x) buf[x] = rd(x);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    const F cur = buf[k % A];
    if (k + A < N) buf[k % A] = rd(k + A);
    mm(k, cur);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Wait until this wave's global reads (including copies into LDS) have landed.
__device__ __forceinline__ void wait_global() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Waits until at most n (wave-uniform, 0 <= n <= 31; larger n waits for 31) of
// this wave's vector-memory operations are outstanding.  They complete in
// issue order, so this waits for everything but the n most recent.
__device__ __forceinline__ void wait_global_le(int n) {
  // vmcnt is bits 3:0 and 15:14 of the operand; expcnt and lgkmcnt left at their maxima
#define NB_VMCNT(c) __builtin_amdgcn_s_waitcnt(0x0F70 | ((c) & 15) | (((c) >> 4) << 14))
  switch (n) {
    case 0: NB_VMCNT(0); break;    case 1: NB_VMCNT(1); break;    case 2: NB_VMCNT(2); break;
    case 3: NB_VMCNT(3); break;    case 4: NB_VMCNT(4); break;    case 5: NB_VMCNT(5); break;
    case 6: NB_VMCNT(6); break;    case 7: NB_VMCNT(7); break;    case 8: NB_VMCNT(8); break;
    case 9: NB_VMCNT(9); break;    case 10: NB_VMCNT(10); break;  case 11: NB_VMCNT(11); break;
    case 12: NB_VMCNT(12); break;  case 13: NB_VMCNT(13); break;  case 14: NB_VMCNT(14); break;
    case 15: NB_VMCNT(15); break;  case 16: NB_VMCNT(16); break;  case 17: NB_VMCNT(17); break;
    case 18: NB_VMCNT(18); break;  case 19: NB_VMCNT(19); break;  case 20: NB_VMCNT(20); break;
    case 21: NB_VMCNT(21); break;  case 22: NB_VMCNT(22); break;  case 23: NB_VMCNT(23); break;
    case 24: NB_VMCNT(24); break;  case 25: NB_VMCNT(25); break;  case 26: NB_VMCNT(26); break;
    case 27: NB_VMCNT(27); break;  case 28: NB_VMCNT(28); break;  case 29: NB_VMCNT(29); break;
    case 30: NB_VMCNT(30); break;  default: NB_VMCNT(31); break;
  }
#undef NB_VMCNT
}

// Precomputed readers for bf16 tiles.  The XOR swizzle only touches the low 4
// chunk bits, so every operand address is one of a few per-lane bases plus a
// compile-time offset; keeping just those bases live (instead of letting the
// compiler hoist one address per fragment) saves ~100 registers per kernel.
//
// RowReader: fragments (r0 + 32*sb, 16*kk + 8*g .. +7) for the lane's row r0.
template <typename TL>
struct RowReader {
  static constexpr int NB = (TL::CPR / 2 < 8) ? TL::CPR / 2 : 8;
  static constexpr int RB = TL::CPR * 16;  // row bytes
  int base[NB];
  __device__ __forceinline__ RowReader(int r0, int g, int byte0 = 0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) base[j] = byte0 + 2 * TL::off(r0, 2 * j + g);
  }
  __device__ __forceinline__ bf16x8 read(const bf16* lds, int sb, int kk) const {
    const int byte = base[kk % NB] + (kk / NB) * (2 * NB * 16) + sb * 32 * RB;
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(lds) + byte);
  }
};

// ColReader: the transposed fragments frag_col(dblk, m) of a bf16 tile.
template <typename TL>
struct ColReader {
  static constexpr int NB = (TL::CPR / 4 < 4) ? TL::CPR / 4 : 4;
  static constexpr int RB = TL::CPR * 16;
  int lo[NB], hi[NB];
  __device__ __forceinline__ ColReader(int lane, int byte0 = 0) {
    const int g = lane >> 5, s = lane & 15, half = (lane >> 4) & 1;
    const int r = 4 * g + (s >> 2);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int d = 32 * j + 16 * half + 4 * (s & 3);
      lo[j] = byte0 + 2 * (TL::off(r, d >> 3) + (d & 7));
      hi[j] = byte0 + 2 * (TL::off(r + 8, d >> 3) + (d & 7));
    }
  }
  __device__ __forceinline__ bf16x8 read(const bf16* lds, int dblk, int m) const {
    typedef __attribute__((address_space(3))) bf16x4 lds_b4;
    const int extra = (dblk / NB) * (NB * 4 * 16) + m * 16 * RB;
    const char* c = reinterpret_cast<const char*>(lds);
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(c + lo[dblk % NB] + extra));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(c + hi[dblk % NB] + extra));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
};

// Operand fragment along a tile row: elements (r, 16*kk + 8*g .. +7).
template <typename T, typename TL>
__device__ __forceinline__ typename Frag<T>::type frag_row(const T* lds, int r, int kk, int g) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const typename Frag<T>::type*>(lds + TL::off(r, 2 * kk + g));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(lds + TL::off(r, 4 * kk + 2 * g));
    const f32x4 b = *reinterpret_cast<const f32x4*>(lds + TL::off(r, 4 * kk + 2 * g + 1));
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// Operand fragment across tile rows, for a product whose other operand comes
// from accumulator rows: the lane's operand row is column d = 32*dblk + lane%32
// of the tile, and slot t of step m holds tile row kappa(m, g, t) (see the top
// of this file).  bf16: two ds_read_b64_tr_b16 per fragment -- within each
// 16-lane group, lane i receives element i%4 of the 8-byte pieces the lanes
// i/4 + 4u (u = 0..3) address, as slot u.  float: eight scalar LDS reads.
template <typename T, typename TL>
__device__ __forceinline__ typename Frag<T>::type frag_col(const T* lds, int dblk, int m, int lane) {
  const int g = lane >> 5;
  if constexpr (sizeof(T) == 2) {
    typedef __attribute__((address_space(3))) bf16x4 lds_b4;
    const int s = lane & 15, half = (lane >> 4) & 1;
    const int r = 16 * m + 4 * g + (s >> 2);
    const int d = 32 * dblk + 16 * half + 4 * (s & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(lds + TL::off(r, d >> 3) + (d & 7)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(lds + TL::off(r + 8, d >> 3) + (d & 7)));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    const int d = 32 * dblk + (lane & 31);
    f32x8 f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int r = 16 * m + 8 * (t >> 2) + 4 * g + (t & 3);
      f[t] = lds[TL::off(r, d / TL::EPC) + d % TL::EPC];
    }
    return f;
  }
}

// The same two readers with one and two address registers instead of NB and
// 2*NB.  The swizzle only permutes 16-byte chunks inside a row, and a tile
// starts on a 1 KB boundary with rows of at least 256 bytes, so a lane's
// address for fragment j is its base with a constant XORed into bits 5..7
// (row reads) or 6..7 (transposed reads): one v_xor per read in place of a
// register per fragment, for kernels short of registers to read ahead with.
template <typename TL>
struct RowReaderX {
  static constexpr int RB = TL::CPR * 16;
  static_assert(RB >= 256 && TL::CPR >= 16, "one row must span whole 256-byte bank lines");
  int b;   // row r0, chunk bits g ^ swz(r0)
  __device__ __forceinline__ RowReaderX(int r0, int g) : b(r0 * RB + 16 * (g ^ TL::swz(r0))) {}
  __device__ __forceinline__ bf16x8 read(const bf16* lds, int sb, int kk) const {
    typedef __attribute__((address_space(3))) const bf16x8 lds_b8;
    const uint32_t a = ((lds_addr(lds) + (uint32_t)b) ^ (uint32_t)(32 * (kk % 8))) + 256u * (kk / 8) + sb * 32 * RB;
    return *reinterpret_cast<lds_b8*>((uintptr_t)a);
  }
};
template <typename TL>
struct ColReaderX {
  static constexpr int NB = 4;
  static constexpr int RB = TL::CPR * 16;
  static_assert(RB >= 256 && TL::CPR >= 16, "one row must span whole 256-byte bank lines");
  int lo, hi;   // rows r and r + 8 at d block 0 (see ColReader)
  __device__ __forceinline__ ColReaderX(int lane) {
    const int g = lane >> 5, s = lane & 15, half = (lane >> 4) & 1;
    const int r = 4 * g + (s >> 2);
    const int u = 2 * half + ((s >> 1) & 1);   // the chunk within a 64-byte group
    lo = r * RB + 16 * (u ^ TL::swz(r)) + 8 * (s & 1);
    hi = (r + 8) * RB + 16 * (u ^ TL::swz(r + 8)) + 8 * (s & 1);
  }
  __device__ __forceinline__ bf16x8 read(const bf16* lds, int dblk, int m) const {
    typedef __attribute__((address_space(3))) bf16x4 lds_b4;
    const uint32_t base = lds_addr(lds);
    const uint32_t sw = 64u * (dblk % NB), extra = (dblk / NB) * (NB * 4 * 16) + m * 16 * RB;
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(uintptr_t)(((base + lo) ^ sw) + extra));
    const bf16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(uintptr_t)(((base + hi) ^ sw) + extra));
    return bf16x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
  }
};
// A TileAccess through the X readers (bf16, rows of at least 256 bytes).
template <typename TL>
struct TileAccessX {
  RowReaderX<TL> rr;
  ColReaderX<TL> cr;
  __device__ __forceinline__ TileAccessX(int r0, int lane) : rr(r0, lane >> 5), cr(lane) {}
  __device__ __forceinline__ bf16x8 row(const bf16* lds, int sb, int kk) const { return rr.read(lds, sb, kk); }
  __device__ __forceinline__ bf16x8 col(const bf16* lds, int dblk, int m) const { return cr.read(lds, dblk, m); }
};

// Operand access to a tile for one lane: rows r0 + 32*sb along D, and the
// transposed fragments; bf16 through the precomputed readers, float (debug
// path) through the generic element reads.
template <typename T, typename TL> struct TileAccess;

template <typename TL>
struct TileAccess<bf16, TL> {
  RowReader<TL> rr;
  ColReader<TL> cr;
  // row_byte0 / col_byte0: constant byte offsets (from the pointer later passed
  // to row() / col()) folded into the per-lane bases
  __device__ __forceinline__ TileAccess(int r0, int lane, int row_byte0 = 0, int col_byte0 = 0)
      : rr(r0, lane >> 5, row_byte0), cr(lane, col_byte0) {}
  __device__ __forceinline__ bf16x8 row(const bf16* lds, int sb, int kk) const { return rr.read(lds, sb, kk); }
  __device__ __forceinline__ bf16x8 col(const bf16* lds, int dblk, int m) const { return cr.read(lds, dblk, m); }
};

template <typename TL>
struct TileAccess<float, TL> {
  int r0, lane, rb0, cb0;
  __device__ __forceinline__ TileAccess(int r0_, int lane_, int row_byte0 = 0, int col_byte0 = 0)
      : r0(r0_), lane(lane_), rb0(row_byte0 / 4), cb0(col_byte0 / 4) {}
  __device__ __forceinline__ f32x8 row(const float* lds, int sb, int kk) const {
    return frag_row<float, TL>(lds + rb0, r0 + 32 * sb, kk, lane >> 5);
  }
  __device__ __forceinline__ f32x8 col(const float* lds, int dblk, int m) const {
    return frag_col<float, TL>(lds + cb0, dblk, m, lane);
  }
};

// ---------------------------------------------------------------------------
// Work orders: items sorted by decreasing work, ties by decreasing index.  A
// key carries both, (2^32 - 1 - work) << 32 | (n - 1 - item), so an ascending
// sort of the keys gives the order.
__device__ __forceinline__ unsigned long long work_key(unsigned work, int i, int n) {
  return ((unsigned long long)(0xFFFFFFFFu - work) << 32) | (unsigned)(n - 1 - i);
}
// Bitonic sort of keys[0, N) in LDS (N a power of two, entries past n padded
// with ~0) by the NT threads of the workgroup, then out[0, n) = the items in
// key order.  Every thread of the workgroup calls it.
template <int NT>
__device__ void order_by_work(unsigned long long* keys, int n, int N, int* out) {
  const int tid = threadIdx.x;
  __syncthreads();
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < N; i += NT) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long a = keys[i], c = keys[l];
          if ((a > c) == ((i & k) == 0)) {
            keys[i] = c;
            keys[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < n; i += NT) out[i] = n - 1 - (int)(unsigned)(keys[i] & 0xFFFFFFFFu);
  __syncthreads();
}

}  // namespace nb
