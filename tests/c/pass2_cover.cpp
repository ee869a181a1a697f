// Host-side check of the fused variant's pass-2 work dealing (StepPlan, step_block, step_items and
// grid_item in flce_internal.hpp): for many launch shapes, block shapes, step sizes and workgroup
// groupings, every block of the plane is in exactly one step, every logits tile (Z kernel) and every
// dx / dW tile product (P kernel) of a step's blocks is dealt to exactly one workgroup, each item
// decodes to a tile inside its block, and a group's workgroups get the same number of items to
// within one per block.  Prints "PASS pass2 <cases>" and exits 0, or the first failure and exits 1.
#include "flce_internal.hpp"

#include <algorithm>
#include <cstdio>
#include <vector>

static int fail(const char* what, int tm, int tv, int bt, int bv, int slots, int groups, int gsize) {
  std::printf("FAIL %s: tm=%d tv=%d bt=%d bv=%d slots=%d groups=%d gsize=%d\n", what, tm, tv, bt, bv, slots, groups,
              gsize);
  return 1;
}

int main() {
  long cases = 0;
  const int tms[] = {1, 2, 3, 7, 8, 15, 16, 17, 31, 33, 64, 65, 512};
  const int tvs[] = {1, 2, 5, 12, 16, 17, 63, 125, 126, 501, 594};
  const int ths[] = {3, 16};
  for (int tm : tms)
    for (int tv : tvs)
      for (int bt : {1, 4, 16})
        for (int bv : {1, 5, 16})
          for (int slots : {3, 48, 1000})
            for (int groups : {1, 8})
              for (int gsize : {7, 32})
                for (int th : ths) {
                  if (tm == 512 && (bt < 16 || bv < 16)) continue;   // long-context rows: the real shape only
                  flce::StepPlan sp;
                  sp.tm = tm;
                  sp.tv = tv;
                  sp.bt = std::min(bt, tm);
                  sp.bv = std::min(bv, tv);
                  sp.blocks_v = (tv + sp.bv - 1) / sp.bv;
                  sp.groups = groups;
                  sp.gsize = gsize;
                  sp.th = th;
                  const int blocks = ((tm + sp.bt - 1) / sp.bt) * sp.blocks_v;
                  std::vector<int> zcov((size_t)tm * tv, 0);
                  std::vector<int> pcov_dx((size_t)tm * th, 0), pcov_dw((size_t)tv * th, 0);
                  for (int first = 0; first < blocks; first += slots) {
                    sp.first = first;
                    sp.count = std::min(slots, blocks - first);
                    for (int kind = 0; kind < 2; ++kind) {
                      std::vector<int> per((size_t)groups * gsize, 0);
                      for (int g = 0; g < groups; ++g)
                        for (int w = 0; w < gsize; ++w) {
                          auto visit = [&](int j, int q) {
                            int mt0, vt0, nt, nv;
                            flce::step_block(sp, j, mt0, vt0, nt, nv);
                            per[(size_t)g * gsize + w]++;
                            if (kind == 0) {
                              int mi, nj;
                              flce::grid_item(q, nt, nv, 4, mi, nj);
                              if (mi < 0 || mi >= nt || nj < 0 || nj >= nv) return;
                              zcov[(size_t)(mt0 + mi) * tv + vt0 + nj]++;
                            } else if (q < nt * th) {
                              int mi, hb;
                              flce::grid_item(q, nt, th, 4, mi, hb);
                              if (mi < 0 || mi >= nt || hb < 0 || hb >= th) return;
                              pcov_dx[(size_t)(mt0 + mi) * th + hb]++;
                            } else {
                              int nj, hb;
                              flce::grid_item(q - nt * th, nv, th, 4, nj, hb);
                              if (nj < 0 || nj >= nv || hb < 0 || hb >= th) return;
                              // a vocabulary tile's dW products: one per token block containing it
                              pcov_dw[(size_t)(vt0 + nj) * th + hb]++;
                            }
                          };
                          if (kind == 0) flce::step_items<false>(sp, g, w, visit);
                          else flce::step_items<true>(sp, g, w, visit);
                        }
                      // balance inside each group: within one item per block the group holds
                      for (int g = 0; g < groups; ++g) {
                        const int nb = (sp.count - g + groups - 1) / groups;
                        const auto b = per.begin() + (size_t)g * gsize;
                        const int lo = *std::min_element(b, b + gsize), hi = *std::max_element(b, b + gsize);
                        if (nb > 0 && hi - lo > nb) return fail("unbalanced group", tm, tv, bt, bv, slots, groups, gsize);
                      }
                    }
                  }
                  const int token_blocks = (tm + sp.bt - 1) / sp.bt;
                  for (int c : zcov)
                    if (c != 1) return fail("logits tile not dealt exactly once", tm, tv, bt, bv, slots, groups, gsize);
                  for (int c : pcov_dx)
                    if (c != sp.blocks_v) return fail("dx product count", tm, tv, bt, bv, slots, groups, gsize);
                  for (int c : pcov_dw)
                    if (c != token_blocks) return fail("dW product count", tm, tv, bt, bv, slots, groups, gsize);
                  ++cases;
                }
  std::printf("PASS pass2 %ld\n", cases);
  return 0;
}
