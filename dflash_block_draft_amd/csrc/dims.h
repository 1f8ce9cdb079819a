// Sizes the kernels are specialised for, as plain constants (no device code), so
// host-side checks can include them too.
#pragma once

namespace dflash {

// Head dimensions the kernels are specialised for (Kimi K3 MLA: qk_nope 128,
// head-shared qk_rope 64, v 128; DSpark page, KimiK3DSparkAttention attributes).
constexpr int kDn = 128;
constexpr int kDr = 64;
constexpr int kDqk = kDn + kDr;
constexpr int kDv = 128;

// Attention tile (queries x keys).  Must match DFLASH_TILE_M / DFLASH_TILE_N.
constexpr int kTileM = 128;
constexpr int kTileN = 64;

}  // namespace dflash
