// Stage layout and global -> LDS copy plan of the backward's dK/dV kernel, as
// plain constexpr integer code (no device code), so that a host-side check can
// walk the plan and confirm every byte the kernel reads lands from its source.
#pragma once

#include <stdint.h>

#include "dims.h"

namespace dflash {

constexpr int kQC = 32;                         // queries per dK/dV chunk
constexpr int kKB = 128;                        // keys per dK/dV workgroup
// LDS row strides (bytes): row + 16
constexpr int kSQ = kDqk * 2 + 16;              // 400: q / k rows
constexpr int kSO = kDv * 2 + 16;               // 272: dout / v rows
constexpr int kSQT = kQC * 2 + 16;              // 80:  transposed q / dout rows (32 queries)
constexpr int kSKT = kTileN * 2 + 16;           // 144: transposed k rows (64 keys)

// dK/dV stage: Q, dO, Q^T, dO^T, lse2, D, visibility words (2 k-tiles x 32 rows),
// each region rounded up to whole 1 KiB blocks: one block is one buffer -> LDS copy
// instruction (64 lanes x 16 bytes), and no instruction spans two sources.
constexpr int kA_Q = 0;                          // 32 rows x 400 B in 13 blocks
constexpr int kA_O = kA_Q + 13 * 1024;           // 32 rows x 272 B in 9 blocks
constexpr int kA_QT = kA_O + 9 * 1024;           // 192 rows x 80 B = 15 blocks
constexpr int kA_OT = kA_QT + 15 * 1024;         // 128 rows x 80 B = 10 blocks
constexpr int kA_L = kA_OT + 10 * 1024;          // 32 floats
constexpr int kA_D = kA_L + 1024;                // 32 floats
constexpr int kA_B = kA_D + 1024;                // [2 k-tiles][32 rows] uint64
constexpr int kA_Stage = kA_B + 1024;            // 50 blocks
constexpr int kA_Blocks = kA_Stage / 1024;
constexpr int kA_Stages = 3;                     // chunks in flight: the next two while one is computed
constexpr int kA_PerWave = (kA_Blocks + 3) / 4;  // copy instructions per wave and stage: 13 (the last wave 11)
static_assert(kQC * kSQ <= 13 * 1024 && kQC * kSO <= 9 * 1024 && kDqk * kSQT == 15 * 1024 && kDv * kSQT == 10 * 1024,
              "dK/dV stage regions");
static_assert(kA_Stages * kA_Stage <= 160 * 1024, "LDS budget");

// Copy plan of the dK/dV stage: block `blk` (0..49) of a stage, lane l: the source
// region, the lane's byte offset inside it (fixed for the kernel; the chunk moves
// the uniform offset) -- padding chunks of a row and lanes past a region's rows
// re-read a valid chunk of the same row / region, landing in LDS padding.
enum : int { kRegQ, kRegO, kRegQT, kRegOT, kRegL, kRegD, kRegB };
constexpr int a_region(int blk) {
  return blk < 13 ? kRegQ : blk < 22 ? kRegO : blk < 37 ? kRegQT : blk < 47 ? kRegOT : blk - 47 + kRegL;
}
constexpr uint32_t a_voff(int blk, int lane, int Lqp) {
  switch (a_region(blk)) {
    case kRegQ: {
      const int j = blk * 64 + lane, row = j / 25, col = j % 25;
      return row >= kQC ? 0u : static_cast<uint32_t>(row * (kDqk * 2) + (col < 24 ? col : 0) * 16);
    }
    case kRegO: {
      const int j = (blk - 13) * 64 + lane, row = j / 17, col = j % 17;
      return row >= kQC ? 0u : static_cast<uint32_t>(row * (kDv * 2) + (col < 16 ? col : 0) * 16);
    }
    case kRegQT: case kRegOT: {
      const int j = (blk - (blk < 37 ? 22 : 37)) * 64 + lane, row = j / 5, col = j % 5;
      return static_cast<uint32_t>(row) * Lqp * 2 + (col < 4 ? col : 0) * 16;
    }
    case kRegL: case kRegD: return lane < 8 ? lane * 16u : 0u;
    default:  // visibility words: lanes 0..15 the first k-tile's 32 rows, 16..31 the second's
      return lane < 16 ? lane * 16u : lane < 32 ? 1024u + (lane - 16) * 16u : 0u;
  }
}
// the chunk's uniform offset into region reg: q0 its first query, tile the byte
// offset of the visibility words of (its q-tile, the workgroup's first k-tile),
// c the chunk's index in its q-tile
constexpr uint32_t a_soff(int reg, uint32_t q0, uint32_t tile, int c) {
  return reg == kRegQ ? q0 * (kDqk * 2) : reg == kRegO ? q0 * (kDv * 2)
       : reg == kRegQT || reg == kRegOT ? q0 * 2 : reg == kRegB ? tile + static_cast<uint32_t>(c) * (kQC * 8) : q0 * 4;
}

}  // namespace dflash
