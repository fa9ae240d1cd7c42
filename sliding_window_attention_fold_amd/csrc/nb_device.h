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

// Store four values rounded to T and, when lo != nullptr, the rounding residuals
// (value - stored value, rounded to T): hi + lo carries ~16 significant bits for bf16.
template <typename T>
__device__ __forceinline__ void store_quad_split(T* hi, T* lo, float a, float b, float c, float d) {
  typename Quad<T>::type v, r;
  v[0] = to_elem<T>(a); v[1] = to_elem<T>(b); v[2] = to_elem<T>(c); v[3] = to_elem<T>(d);
  *reinterpret_cast<typename Quad<T>::type*>(hi) = v;
  if (lo != nullptr) {
    r[0] = to_elem<T>(a - to_f32(v[0])); r[1] = to_elem<T>(b - to_f32(v[1]));
    r[2] = to_elem<T>(c - to_f32(v[2])); r[3] = to_elem<T>(d - to_f32(v[3]));
    *reinterpret_cast<typename Quad<T>::type*>(lo) = r;
  }
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

// Copy ROWS x D elements of a row-major global matrix (rows row0.., row
// stride D) into LDS rows of pitch PITCH.  Rows at or beyond nrows are zero.
template <typename T, int ROWS, int D, int PITCH, int NT>
__device__ __forceinline__ void stage_rows(T* __restrict__ lds, const T* __restrict__ src, int nrows) {
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                 // chunks per row
  constexpr int TOTAL = ROWS * CPR;
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
#pragma unroll
  for (int c = threadIdx.x; c < TOTAL; c += NT) {
    const int r = c / CPR, col = (c % CPR) * EPC;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < nrows) v = *reinterpret_cast<const u32x4*>(src + (size_t)r * D + col);
    *reinterpret_cast<u32x4*>(lds + r * PITCH + col) = v;
  }
}

// Copy ROWS x D elements of a row-major global matrix into LDS transposed:
// element (r, d) goes to lds[d * TPITCH + perm16(r)], so that 16-byte reads at
// column 16*m + 8*g return the rows a probability accumulator holds for step m
// and lane group g.  Rows at or beyond nrows are zero.  ROWS % 16 == 0.
template <typename T, int ROWS, int D, int TPITCH, int NT>
__device__ __forceinline__ void stage_rows_transposed(T* __restrict__ lds, const T* __restrict__ src,
                                                      int nrows) {
  typedef typename Frag<T>::type F;
  typedef typename Quad<T>::type Q4;
  constexpr int RG = ROWS / 4;                 // groups of 4 rows
  constexpr int CG = D / 8;                    // groups of 8 columns
  constexpr int TOTAL = RG * CG;
#pragma unroll
  for (int gi = threadIdx.x; gi < TOTAL; gi += NT) {
    const int rg = gi % RG, cg = gi / RG;
    const int r0 = 4 * rg, c0 = 8 * cg;
    F x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = (r0 + e < nrows) ? load_frag<T>(src + (size_t)(r0 + e) * D + c0) : zero_frag<T>();
    const int col = perm16(r0);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      Q4 v;
      v[0] = x[0][d]; v[1] = x[1][d]; v[2] = x[2][d]; v[3] = x[3][d];
      *reinterpret_cast<Q4*>(lds + (c0 + d) * TPITCH + col) = v;
    }
  }
}

}  // namespace nb
