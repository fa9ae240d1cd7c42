// Neighbourhood K/V access through the chunk table (KvChunks): tile copies for
// the forward and dQ loops, row pointers for the dK/dV item.
#pragma once

#include <limits.h>

#include "nb_device.h"
#include "nb_kernels.h"

namespace nb {

enum KvWhich { kK = 0, kV = 1, kDK = 2, kDV = 3 };

// Pointer to the row of neighbourhood key j (batch b, kv head: bh = b * Hkv + h)
// in chunk buffer `which`.  One pass over the chunks with uniform indices, so a
// per-lane key needs no indexed parameter loads.
template <typename T>
__device__ __forceinline__ T* kv_row(const KvChunks& c, int which, int bh, int j, int D) {
  auto base = [&](int y) -> void* {
    return which == kK ? const_cast<void*>(c.k[y]) : which == kV ? const_cast<void*>(c.v[y])
         : which == kDK ? c.dk[y] : c.dv[y];
  };
  void* p = base(0);
  size_t r = (size_t)bh * c.rows[0] + c.start[0] + j;
  for (int y = 1; y < c.n; ++y) {
    if (j >= c.off[y]) {
      p = base(y);
      r = (size_t)bh * c.rows[y] + c.start[y] + (j - c.off[y]);
    }
  }
  return reinterpret_cast<T*>(p) + r * D;
}

// Rows of neighbourhood keys [j0, j1] (uniform bounds) in buffer `which` with
// uniform state when they lie in at most two chunks: key j's row is
// (j < cut ? base0 : base1) + j * D, each base shifted by its chunk's first
// key.  ok is false (kv_row then) when the keys touch three or more chunks.
template <typename T>
struct KvSpan {
  T* base0;
  T* base1;
  int cut;
  bool ok;

  __device__ __forceinline__ KvSpan(const KvChunks& c, int which, int bh, int j0, int j1, int D) {
    size_t r0, r1;
    const int x0 = kv_locate(c, bh, j0, &r0);
    const int x1 = kv_locate(c, bh, j1, &r1);
    auto base = [&](int y) -> T* {
      return reinterpret_cast<T*>(which == kK ? const_cast<void*>(c.k[y]) : which == kV ? const_cast<void*>(c.v[y])
                                  : which == kDK ? c.dk[y] : c.dv[y]);
    };
    ok = x1 <= x0 + 1;
    cut = x1 > x0 ? c.off[x1] : INT_MAX;
    base0 = base(x0) + ((long long)r0 - j0) * D;
    base1 = base(x1) + ((long long)r1 - j1) * D;
  }
  __device__ __forceinline__ T* row(int j, int D) const { return (j < cut ? base0 : base1) + (size_t)j * D; }
};

// Copies neighbourhood keys [j0, j0 + ROWS) of K and V into the tiles Ks, Vs
// (rows at or beyond nv repeat row nv - 1): one buffer-resource copy per chunk
// the tile touches (usually one).  WITH_V false: K alone (Vs unused).
template <typename T, int ROWS, int D, int NW, bool WITH_V = true>
__device__ __forceinline__ void kv_tile_load(const TileDma<T, ROWS, D, NW>& dma, const KvChunks& c, int bh, int j0,
                                             int nv, T* Ks, T* Vs) {
  int j = j0;
  while (j < j0 + nv) {   // uniform
    size_t row;
    const int x = kv_locate(c, bh, j, &row);
    const int e = (x + 1 < c.n) ? min(c.off[x + 1], j0 + nv) : j0 + nv;
    const int r_hi = (e == j0 + nv) ? ROWS : e - j0;
    dma.issue_rows(Ks, reinterpret_cast<const T*>(c.k[x]) + row * D, j - j0, r_hi, nv);
    if constexpr (WITH_V) dma.issue_rows(Vs, reinterpret_cast<const T*>(c.v[x]) + row * D, j - j0, r_hi, nv);
    j = e;
  }
}

// K/V rows of a key range [kstart, kend), copied ROWS keys per tile from
// kstart on, when it touches at most two chunks, x0 and x0 + 1, with scalar
// state only: bases shifted so that base + j * D is key j's row in its chunk;
// `cut` is the first key of the second chunk (INT_MAX when there is one) and
// cap the key past which the last chunk has no rows (copies repeat its last row
// there).  The tile holding `cut` takes rows from both chunks; ok is false (the
// general lookup is needed) when the range touches three or more chunks or the
// second chunk ends inside that tile.
template <typename T, int ROWS>
struct KvPair {
  const T* k0;
  const T* v0;
  const T* k1;
  const T* v1;
  int cut, cap;
  bool ok;

  __device__ __forceinline__ KvPair() : k0(nullptr), v0(nullptr), k1(nullptr), v1(nullptr), cut(INT_MAX), cap(0), ok(true) {}
  __device__ __forceinline__ KvPair(const KvChunks& c, int bh, int kstart, int kend, int D) {
    size_t r0 = 0, r1 = 0;
    int x0 = 0, x1 = 0;
    if (kstart < kend) {
      x0 = kv_locate(c, bh, kstart, &r0);
      x1 = kv_locate(c, bh, kend - 1, &r1);
    }
    const long long s0 = ((long long)r0 - kstart) * D;
    k0 = reinterpret_cast<const T*>(c.k[x0]) + s0;
    v0 = reinterpret_cast<const T*>(c.v[x0]) + s0;
    cap = c.off[x0 + 1];
    cut = INT_MAX;
    k1 = k0;
    v1 = v0;
    ok = x1 <= x0 + 1;
    if (x1 == x0 + 1) {
      cut = cap;
      const long long s1 = ((long long)r1 - (kend - 1)) * D;
      k1 = reinterpret_cast<const T*>(c.k[x1]) + s1;
      v1 = reinterpret_cast<const T*>(c.v[x1]) + s1;
      cap = c.off[x1 + 1];
      const int split = (cut - kstart) % ROWS;   // rows of the first chunk in the tile holding cut
      if (split != 0 && cut - split + ROWS > cap) ok = false;
    }
  }

  // Keys [j0, j0 + ROWS) (a tile of the range) into the tiles Ks, Vs.
  template <int D, int NW>
  __device__ __forceinline__ void load(const TileDma<T, ROWS, D, NW>& dma, int j0, T* Ks, T* Vs) const {
    if (j0 + ROWS <= cut) {
      const int nv = min(ROWS, cap - j0);   // (cap = cut when two chunks: a full tile)
      dma.issue(Ks, k0 + (size_t)j0 * D, nv);
      dma.issue(Vs, v0 + (size_t)j0 * D, nv);
    } else if (j0 >= cut) {
      const int nv = min(ROWS, cap - j0);
      dma.issue(Ks, k1 + (size_t)j0 * D, nv);
      dma.issue(Vs, v1 + (size_t)j0 * D, nv);
    } else {
      dma.issue_split(Ks, k0 + (size_t)j0 * D, k1 + (size_t)cut * D, cut - j0);
      dma.issue_split(Vs, v0 + (size_t)j0 * D, v1 + (size_t)cut * D, cut - j0);
    }
  }

  // The same tile of K alone.
  template <int D, int NW>
  __device__ __forceinline__ void load_k(const TileDma<T, ROWS, D, NW>& dma, int j0, T* Ks) const {
    if (j0 + ROWS <= cut) dma.issue(Ks, k0 + (size_t)j0 * D, min(ROWS, cap - j0));
    else if (j0 >= cut) dma.issue(Ks, k1 + (size_t)j0 * D, min(ROWS, cap - j0));
    else dma.issue_split(Ks, k0 + (size_t)j0 * D, k1 + (size_t)cut * D, cut - j0);
  }
};

// Whether some block of `rows` consecutive query rows may need the general
// lookup (see KvPair; tiles of `tile` keys): a row's band spans at most
// window + 1 keys, so a block's range spans at most rows + window keys and
// touches three chunks only if an interior chunk is shorter than that (no
// window: any length); the second chunk ends inside a tile only if some chunk
// after the first is shorter than a tile.
inline bool kv_may_need_general(const KvChunks& c, int window, int rows, int tile) {
  for (int x = 1; x < c.n; ++x)
    if (c.off[x + 1] - c.off[x] < tile) return true;
  if (c.n < 3) return false;
  if (window < 0) return true;
  for (int x = 1; x + 1 < c.n; ++x)
    if (c.off[x + 1] - c.off[x] < rows + window) return true;
  return false;
}

}  // namespace nb
