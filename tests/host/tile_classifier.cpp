// Host driver for the tile classifier of the attention kernels: the mask
// helpers of fa_device.h (make_mask, rect_state, full_tiles_below,
// TileWalk, query_hull, set_instance_kind) compiled for the CPU, so that
// tests/test_tile_classifier.py can check them pair by pair against the
// oracle's predicate.
//
// Reads cases from stdin, one per line:
//   kind Sq Skv shift kv wl wr TQ TK TKW view
// (view 1: the causal view the bf16 tile loops take of a TTT mask, i.e.
// set_instance_kind<MK_TTT>).  For each case it prints
//   C <case index>
//   S qa s_0 s_1 ...      rect_state of query block [qa, qa+TQ) against
//                         every key tile [t*TK, t*TK+TK), t < ceil(Skv/TK)
//   W qa t_0 t_1 ...      the tiles TileWalk visits for that block
//   F qa f                full_tiles_below(m, qa, TK)
//   H k0 lo hi            query_hull of key block [k0, k0+TKW)
#include <cstdio>

#include "fa_device.h"

using namespace fa;

int main() {
  int kind, Sq, Skv, shift, kv, wl, wr, TQ, TK, TKW, view;
  int idx = 0;
  while (scanf("%d %d %d %d %d %d %d %d %d %d %d", &kind, &Sq, &Skv, &shift, &kv, &wl, &wr, &TQ, &TK, &TKW,
               &view) == 11) {
    MaskB m = make_mask(kind, shift, Sq, Skv, kv, wl, wr);
    if (view == 1) set_instance_kind<MK_TTT>(m);
    printf("C %d\n", idx++);
    const int ntk = (Skv + TK - 1) / TK;
    for (int qa = 0; qa < Sq; qa += TQ) {
      const int qb = qa + TQ < Sq ? qa + TQ : Sq;
      printf("S %d", qa);
      for (int t = 0; t < ntk; ++t) printf(" %d", rect_state(m, t * TK, t * TK + TK, qa, qb));
      printf("\nW %d", qa);
      TileWalk w;
      int guard = 0;
      for (w.start(m, qa, qb, TK); w.valid() && guard <= 4 * ntk + 4; w.next(m, qa, qb, TK), ++guard)
        printf(" %d", w.t);
      printf("\nF %d %d\n", qa, full_tiles_below(m, qa, TK));
    }
    for (int k0 = 0; k0 < Skv; k0 += TKW) {
      int lo, hi;
      query_hull(m, k0, k0 + TKW < Skv ? k0 + TKW : Skv, lo, hi);
      printf("H %d %d %d\n", k0, lo, hi);
    }
  }
  return 0;
}
