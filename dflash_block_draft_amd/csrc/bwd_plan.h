// Staging layout of the backward's dK/dV kernel, as plain constexpr integer code
// (no device code), so that a host-side check can replay every global -> LDS
// copy and confirm that each operand read of the compute finds its bytes.
//
// The kernel walks 32-query chunks.  Chunk j's data is split in two parts: the
// F part (q and dout rows, the rows' exponent offsets and -D, the transposed
// visibility words) feeds the scores of chunk j in step j - 1; the T part (the
// transposed q and dout) feeds dV of chunk j, whose operands are read from the
// end of step j - 1 on, and dK of chunk j in step j.  Both parts of chunk j are
// copied in step j - 3: the F ring has three slots, the T ring four.
//
// Every row region is stored as 1 KiB blocks of 16 rows x 64 bytes with the four
// 16-byte pieces of a row permuted by the row (piece p at position p ^ swz(row)),
// so the 16-byte operand reads of 16 lanes hit distinct banks without padding,
// and every region is a whole number of blocks that the four waves split evenly.
#pragma once

#include <stdint.h>

#include "dims.h"

namespace dflash {

constexpr int kQC = 32;                          // queries per chunk
constexpr int kKB = 128;                         // keys per workgroup (two k-tiles)
constexpr int kKvWaves = 4;

// F slot: q rows (32 x 384 B), dout rows (32 x 256 B), then two 1 KiB blocks:
// LD (the chunk's 32 exponent offsets -lse*log2(e), then its 32 values -D) and
// the visibility words of the two k-tiles (64 keys x 32 query bits each)
constexpr int kF_Q = 0;
constexpr int kF_O = kF_Q + kQC * kDqk * 2;      // 12288
constexpr int kF_LD = kF_O + kQC * kDv * 2;      // 20480
constexpr int kF_B = kF_LD + 1024;               // 21504
constexpr int kF_Slot = kF_B + 1024;             // 22528
// T slot: transposed q (192 rows x 64 B), transposed dout (128 rows x 64 B)
constexpr int kT_QT = 0;
constexpr int kT_OT = kT_QT + kDqk * kQC * 2;    // 12288
constexpr int kT_Slot = kT_OT + kDv * kQC * 2;   // 20480
constexpr int kFSlots = 3;
constexpr int kTSlots = 4;

// copy instructions per wave and step: 3 q, 2 dout, LD, words (F); 3 q^T, 2 dout^T (T)
constexpr int kCopiesPerStep = 12;

// position of 16-byte piece p of row r inside its 64-byte block row
constexpr int swz(int r) { return (r >> 2) & 3; }

// LDS byte of (row, byte x) of a row region whose rows are `width` bytes wide
constexpr int region_byte(int row, int x, int width) {
  return ((row >> 4) * (width / 64) + x / 64) * 1024 + (row & 15) * 64 + ((((x & 63) >> 4) ^ swz(row)) << 4) +
         (x & 15);
}

// ---- copy plan: instruction j (0..11) of wave w.  Lane l writes 16 bytes at
// LDS byte dst_base(w, j) + 16 l of its slot; the source is region src_region(j)
// at byte voff(w, j, l) + the step's uniform offset (q0 the chunk's first query):
//   q: q0 * 384; dout: q0 * 256; LD: q0 * 8 (64 floats per chunk); words: q0 * 8
//   (256 bytes per chunk and k-tile, k-tiles nqt * 1024 bytes apart); q^T and
//   dout^T: q0 * 2 (rows Lqp * 2 bytes apart).
// A lane with nothing to copy reads past the end of every resource (zeros, no
// traffic) into an unused part of the block.
enum : int { kSrcQ, kSrcO, kSrcLD, kSrcB, kSrcQT, kSrcOT };
constexpr uint32_t kPastEnd = 0x80000000u;       // beyond every resource (the host bounds them by 2^31 bytes)

constexpr int src_region(int j) {
  return j < 3 ? kSrcQ : j < 5 ? kSrcO : j == 5 ? kSrcLD : j == 6 ? kSrcB : j < 10 ? kSrcQT : kSrcOT;
}
constexpr bool f_part(int j) { return j < 7; }
// LDS destination of instruction j of wave w, relative to its slot (F or T)
constexpr int dst_base(int w, int j) {
  return j < 3 ? kF_Q + (3 * w + j) * 1024
       : j < 5 ? kF_O + (2 * w + j - 3) * 1024
       : j == 5 ? kF_LD
       : j == 6 ? kF_B
       : j < 10 ? kT_QT + (3 * w + j - 7) * 1024
       : kT_OT + (2 * w + j - 10) * 1024;
}
// block blk of a region of `width`-byte rows, lane l: (row, byte of the row)
constexpr int blk_row(int blk, int l, int width) { return 16 * (blk / (width / 64)) + (l >> 2); }
constexpr int blk_x(int blk, int l, int width) {
  return (blk % (width / 64)) * 64 + (((l & 3) ^ swz(blk_row(blk, l, width))) << 4);
}
constexpr uint32_t voff(int w, int j, int l, int Lqp, int nqt) {
  switch (src_region(j)) {
    case kSrcQ: {
      const int blk = 3 * w + j;
      return static_cast<uint32_t>(blk_row(blk, l, 384) * 384 + blk_x(blk, l, 384));
    }
    case kSrcO: {
      const int blk = 2 * w + j - 3;
      return static_cast<uint32_t>(blk_row(blk, l, 256) * 256 + blk_x(blk, l, 256));
    }
    case kSrcLD: return l < 16 ? static_cast<uint32_t>(l) * 16u : kPastEnd;
    case kSrcB:
      return l < 16 ? static_cast<uint32_t>(l) * 16u
           : l < 32 ? static_cast<uint32_t>(nqt) * 1024u + static_cast<uint32_t>(l - 16) * 16u : kPastEnd;
    case kSrcQT: {
      const int blk = 3 * w + j - 7;
      return static_cast<uint32_t>(blk_row(blk, l, 64)) * static_cast<uint32_t>(Lqp) * 2u +
             static_cast<uint32_t>(blk_x(blk, l, 64));
    }
    default: {
      const int blk = 2 * w + j - 10;
      return static_cast<uint32_t>(blk_row(blk, l, 64)) * static_cast<uint32_t>(Lqp) * 2u +
             static_cast<uint32_t>(blk_x(blk, l, 64));
    }
  }
}

// ---- reads of the compute (lane l: li = l % 32, hi = l / 32), LDS byte in the slot
// S = Q K^T, operand chunk s (dims 16s .. 16s+15): row li, bytes 32s + 16hi .. +16
constexpr int rd_q(int s, int li, int hi) { return kF_Q + region_byte(li, 32 * s + 16 * hi, 384); }
// dP = dO V^T, operand chunk s (dims 16s ..)
constexpr int rd_o(int s, int li, int hi) { return kF_O + region_byte(li, 32 * s + 16 * hi, 256); }
// dK += dS^T Q: Q^T row 32nt + li, positions 16kk + 8hi .. +8 of the chunk's 32 (relabelled) queries
constexpr int rd_qt(int nt, int kk, int li, int hi) { return kT_QT + region_byte(32 * nt + li, 32 * kk + 16 * hi, 64); }
constexpr int rd_ot(int nt, int kk, int li, int hi) { return kT_OT + region_byte(32 * nt + li, 32 * kk + 16 * hi, 64); }
// four consecutive floats: queries 8g + 4hi .. +3 (accumulator rows 4g .. 4g+3)
constexpr int rd_nl(int g, int hi) { return kF_LD + (8 * g + 4 * hi) * 4; }
constexpr int rd_nd(int g, int hi) { return kF_LD + 128 + (8 * g + 4 * hi) * 4; }
// the visibility word (32 query bits) of key kl (0..63) of k-tile t of the workgroup
constexpr int rd_word(int t, int kl) { return kF_B + t * 256 + kl * 4; }

}  // namespace dflash
