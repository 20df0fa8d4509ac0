// Host check of the fused step kernel's LDS layout and gather rule
// (csrc/step_layout.h): for every block-table width and every candidate
// count it allows, every gathered slot lies in the block-table row, the
// passes cover every candidate, and the regions the gate phase uses are
// disjoint and inside the V tiles.  Prints "ok" and exits 0, else the first
// violation and exits 1.
#include <cstdio>
#include <vector>

#include "step_layout.h"

using namespace sas::step_layout;

int main() {
  long checked = 0;
  for (int max_blocks = 1; max_blocks <= kMaxBlocks; ++max_blocks) {
    // regions for this width (the kernel's arrays)
    const long keys_end = kKeysOff + 4L * (max_blocks > kPass ? max_blocks : kPass);
    const long bt_end = kBtOff + 4L * max_blocks;
    if (keys_end > kBtOff || bt_end > kVsOff || kVsOff + kVsBytes > kVTilesBytes) {
      std::printf("layout overlap at max_blocks %d\n", max_blocks);
      return 1;
    }
  }
  std::vector<unsigned char> seen;
  for (int n = 0; n < kMaxBlocks; ++n) {  // candidates; the row has max_blocks >= n + 1 entries
    seen.assign(n + 1, 0);
    // the kernel gathers pass 0 always, then one pass per further 512 candidates
    for (int base = 0; base == 0 || base < n; base += kPass) {
      for (int u = 0; u < kKeysPerGroup; ++u) {
        for (int grp = 0; grp < kGroups; ++grp) {
          const int slot = gather_slot(base, u, grp, n);
          if (slot < 0 || slot > n) {
            std::printf("slot %d out of the row (n %d, base %d, u %d, group %d)\n", slot, n, base, u, grp);
            return 1;
          }
          seen[slot] = 1;
          ++checked;
        }
      }
    }
    for (int c = 0; c < n; ++c)
      if (!seen[c]) {
        std::printf("candidate %d of %d never gathered\n", c, n);
        return 1;
      }
  }
  std::printf("ok %ld gathers\n", checked);
  return 0;
}
