// LDS layout of the fused decode step's gate phase and the rule by which its
// gate-key gathers pick a candidate slot.  Plain constexpr C++ with no HIP
// headers, so that a host program can check the layout and replay the rule
// for every sequence length (tests/step_layout_check.cpp).
#pragma once

namespace sas {
namespace step_layout {

constexpr int kMaxBlocks = 16384;    // block-table columns (SAS_MAX_BLOCKS)
constexpr int kGroups = 32;          // 16-lane groups of the 512-thread workgroup
constexpr int kKeysPerGroup = 16;    // gate keys per group per gather pass
constexpr int kPass = kGroups * kKeysPerGroup;  // candidates per gather pass (512)
constexpr int kMaxGroup = 16;        // query heads per KV head
constexpr int kGateDim = 128;
constexpr int kVTilesBytes = 8 * 64 * 288;  // the 8 waves' V tiles the gate phase lives in

// byte offsets inside the V tiles: score keys (uint32, max(max_blocks, 512)
// entries: the select reads 512 whatever the count), the block-table row
// (int32, max_blocks entries), the per-head gate-query rows (fp32 [16][128])
constexpr int kKeysOff = 0;
constexpr int kKeysBytes = 4 * (kMaxBlocks > kPass ? kMaxBlocks : kPass);
constexpr int kBtOff = kKeysOff + kKeysBytes;
constexpr int kBtBytes = 4 * kMaxBlocks;
constexpr int kVsOff = kBtOff + kBtBytes;
constexpr int kVsBytes = 4 * kMaxGroup * kGateDim;
static_assert(kKeysOff + kKeysBytes <= kBtOff, "score keys overlap the block-table row");
static_assert(kBtOff + kBtBytes <= kVsOff, "block-table row overlaps the gate queries");
static_assert(kVsOff + kVsBytes <= kVTilesBytes, "gate phase exceeds the V tiles");
static_assert(kKeysOff % 16 == 0 && kBtOff % 16 == 0 && kVsOff % 16 == 0, "16-byte LDS accesses");

// Candidate slot whose page lane group grp gathers as key u of the pass that
// starts at candidate base, with n candidates (the blocks before the local
// block n).  A slot past the candidates reads the local block's page, slot
// n, which is in the row (n < max_blocks) and which the score keys, kept in
// their own array, never overwrite.
constexpr int gather_slot(int base, int u, int grp, int n) {
  return base + kGroups * u + grp < n ? base + kGroups * u + grp : n;
}

}  // namespace step_layout
}  // namespace sas
