// Host-side check of the fused variant's pass-2 work decomposition (span_piece in
// flce_internal.hpp): for many problem shapes, row heights, piece widths and workgroup counts, in
// both dealing modes, every cell (row of token tiles x vocabulary tile) is covered by exactly one
// piece of exactly one workgroup, and every piece lies inside the grid and is at most bnmax wide.
// Spans must also give every workgroup the same number of cells to within one per segment it
// touches.  Prints "PASS pass2 <cases>" and exits 0, or prints the first failure and exits 1.
#include "flce_internal.hpp"

#include <algorithm>
#include <cstdio>
#include <vector>

int main() {
  long cases = 0;
  // token tiles: small, around multiples of the row heights, and the long-context 512; vocabulary
  // tiles: small and the Llama-2 / Llama-3 / Qwen3 vocabularies (125, 501, 594) and their neighbours
  const int tms[] = {1, 2, 3, 4, 5, 6, 7, 8, 9, 15, 16, 17, 31, 32, 33, 64, 65, 127, 512};
  const int tvs[] = {1, 2, 3, 5, 7, 8, 9, 10, 15, 16, 17, 20, 31, 33, 63, 64, 125, 126, 255, 500, 501, 594, 627};
  for (int tm : tms)
    for (int tv : tvs)
      for (int bm : {8, 4, 2})
        for (int bnmax : {1, 2, 3, 5, 6, 12, 24})
          for (int gmax : {1, 7, 255, 256})
            for (int blocks : {0, 1}) {
              if (tm == 512 && bnmax < 5) continue;   // the long-context rows with realistic pieces only
              flce::SpanPlan sp;
              sp.blocks = blocks;
              sp.R = (tm + bm - 1) / bm;
              sp.tv = tv;
              sp.S = flce::span_supers(tv);
              sp.gm = std::max(1, 16 / bm);
              sp.bnmax = bnmax;
              const int64_t units = blocks ? (int64_t)sp.R * ((tv + bnmax - 1) / bnmax) : (int64_t)sp.R * tv;
              sp.G = (int)std::min<int64_t>(gmax, units);
              if (sp.S < 1 || sp.S > 8 || (sp.S > 1 && (sp.S - 1) * ((tv + sp.S - 1) / sp.S) >= tv)) {
                std::printf("FAIL empty super-range tv=%d S=%d\n", tv, sp.S);
                return 1;
              }
              std::vector<int> cover((size_t)sp.R * tv, 0);
              int lo = 1 << 30, hi = 0;
              for (int L = 0; L < sp.G; ++L) {
                int r = 0, v0 = 0, n = 0, cells = 0;
                for (int k = 0; flce::span_piece(sp, L, k, r, v0, n); ++k) {
                  if (n < 1 || n > bnmax || r < 0 || r >= sp.R || v0 < 0 || v0 + n > tv) {
                    std::printf("FAIL piece tm=%d tv=%d bm=%d bnmax=%d G=%d blocks=%d L=%d: row %d tiles %d+%d\n", tm,
                                tv, bm, bnmax, sp.G, blocks, L, r, v0, n);
                    return 1;
                  }
                  for (int k = 0; k < n; ++k) cover[(size_t)r * tv + v0 + k]++;
                  cells += n;
                }
                lo = std::min(lo, cells);
                hi = std::max(hi, cells);
              }
              for (size_t i = 0; i < cover.size(); ++i)
                if (cover[i] != 1) {
                  std::printf("FAIL cell %zu covered %d times: tm=%d tv=%d bm=%d bnmax=%d G=%d blocks=%d\n", i,
                              cover[i], tm, tv, bm, bnmax, sp.G, blocks);
                  return 1;
                }
              // spans with at least one segment per workgroup: one run per workgroup, equal to within
              // the rounding of one segment's split (the segment widths differ by at most one tile
              // except the last super-range, which may be narrower)
              const int NS = sp.S * sp.R;
              if (!blocks && sp.G >= NS && hi - lo > (tv + sp.S - 1) / sp.S) {
                std::printf("FAIL unbalanced spans tm=%d tv=%d bm=%d G=%d: %d..%d cells\n", tm, tv, bm, sp.G, lo, hi);
                return 1;
              }
              ++cases;
            }
  std::printf("PASS pass2 %ld\n", cases);
  return 0;
}
