// Host driver for the tail-split planning and work decomposition of the
// attention kernels (attn_tiles.h), used by tests/test_split_plan.py.
// Reads commands from stdin, one per line, and prints one answer line each:
//   plan PER_XCD SLOTS NST_MAX CAP MIN_STAGES MAX_K -> n_full rem k
//   items PER_XCD N_FULL REM K       -> for every workgroup w of the launch,
//                                       "L piece slot" (one line per w, then "end")
//   tile PER_XCD N_FULL REM K SLOT   -> the logical tile of split slot SLOT
//   stages NST PIECE K               -> s0 s1
#include "attn_tiles.h"

#include <cstdio>
#include <cstring>

int main() {
  char cmd[16];
  while (std::scanf("%15s", cmd) == 1) {
    if (!std::strcmp(cmd, "plan")) {
      int per_xcd, slots, nst, cap, min_stages, max_k;
      if (std::scanf("%d %d %d %d %d %d", &per_xcd, &slots, &nst, &cap, &min_stages, &max_k) != 6) return 1;
      const t2va::SplitArgs sp = t2va::plan_split(per_xcd, slots, nst, (size_t)cap, min_stages, max_k);
      std::printf("%d %d %d\n", sp.n_full, sp.rem, sp.k);
    } else if (!std::strcmp(cmd, "items")) {
      t2va::SplitArgs sp;
      int per_xcd;
      sp.pbank = 0;
      if (std::scanf("%d %d %d %d", &per_xcd, &sp.n_full, &sp.rem, &sp.k) != 4) return 1;
      const int grid = 8 * (sp.n_full + sp.rem * sp.k);
      for (int w = 0; w < grid; ++w) {
        const t2va::SplitItem it = t2va::split_item(w, per_xcd, sp);
        std::printf("%d %d %d\n", it.L, it.piece, it.slot);
      }
      std::printf("end\n");
    } else if (!std::strcmp(cmd, "tile")) {
      t2va::SplitArgs sp;
      int per_xcd, slot;
      sp.pbank = 0;
      if (std::scanf("%d %d %d %d %d", &per_xcd, &sp.n_full, &sp.rem, &sp.k, &slot) != 5) return 1;
      std::printf("%d\n", t2va::split_tile(slot, per_xcd, sp));
    } else if (!std::strcmp(cmd, "stages")) {
      int nst, piece, k, s0, s1;
      if (std::scanf("%d %d %d", &nst, &piece, &k) != 3) return 1;
      t2va::piece_stages(nst, piece, k, s0, s1);
      std::printf("%d %d\n", s0, s1);
    } else {
      return 1;
    }
    std::fflush(stdout);
  }
  return 0;
}
