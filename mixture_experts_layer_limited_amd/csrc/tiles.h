// Tile lists of the grouped GEMMs, written by one work-group of 1024 threads
// (the tile-list kernel, and the one-work-group permutation of small batches).
#pragma once

#include "kernels.h"

namespace moe {

// Group g's rows are [first[g], first[g + 1]), g < G <= 1024; both arrays in
// LDS, scan has 1024 entries and every thread of the block must call.  Group g
// is split into c_g = ceil(rows / bm) m-tiles of near-equal size; a list holds
// every (m-tile, n-tile) pair, group by group, n-tile by n-tile, with the c_g
// m-tiles of one n-tile next to each other.  Neighbouring entries run at the
// same time on the same XCD (see xcd_remap), so the m-tiles that share a
// weight tile read it from that XCD's L2 instead of from HBM.
// Entry: {group, first row, end row, n-tile}; *n_tiles = sum_g c_g * ntn.  A
// second list with the same m-tiles and another n-tile count (ntn2 > 0) comes
// from the same scan.
__device__ inline void write_tile_lists(int* scan, const int* first, int G, const TileLists& t) {
  const int e = threadIdx.x;
  const int cnt = e < G ? (first[e + 1] - first[e] + t.bm - 1) / t.bm : 0;
  scan[e] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = e >= o ? scan[e - o] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  // one work item per (group, n-tile): its c_g m-tiles are entries
  // (scan[g] - c_g) * nn + nt * c_g + i, i < c_g
  for (int list = 0; list < 2; ++list) {
    const int nn = list ? t.ntn2 : t.ntn;
    int4* out = list ? t.tiles2 : t.tiles;
    if (nn <= 0) break;
    const int total = scan[1023] * nn;
    // this thread's items w = x * nn + nt = e, e + 1024, ..., stepped without
    // a division per item
    const int dx = 1024 / nn, dnt = 1024 - dx * nn;
    int x = e / nn, nt = e - x * nn;
    while (x < G) {
      const int c = scan[x] - (x > 0 ? scan[x - 1] : 0);
      const int r0 = first[x], n = first[x + 1] - r0;
      const int base = (scan[x] - c) * nn + nt * c;
      if (c > 0) {
        // m-tile i: rows [r0 + floor(i n / c), r0 + floor((i + 1) n / c)), with
        // floor(i n / c) = i q + floor(i r / c) for n = q c + r, stepped in i
        const int q = n / c, r = n - q * c;
        int lo = r0, acc = 0;
        for (int i = 0; i < c; ++i) {
          int hi = lo + q;
          acc += r;
          if (acc >= c) {
            acc -= c;
            ++hi;
          }
          out[base + i] = make_int4(x, lo, hi, nt);
          lo = hi;
        }
      }
      x += dx;
      nt += dnt;
      if (nt >= nn) {
        nt -= nn;
        ++x;
      }
    }
    if (e == 0) *(list ? t.n_tiles2 : t.n_tiles) = total;
  }
}

}  // namespace moe
