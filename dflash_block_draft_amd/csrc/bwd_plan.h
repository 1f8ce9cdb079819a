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

// ======================================================================== dQ
// The dQ kernel walks the 32-key steps of its q-tile's tile list (two per
// 64-key tile).  Step m's data is split in two parts: the F part (k_nope and
// k_rope rows, v rows, and the tile's visibility words: 128 queries x 64 bits)
// feeds S^T and dP^T of step m, computed in step m - 1, whose first K operands
// are read at the end of step m - 2; the T part (the transposed k_nope and
// k_rope of the step's 32 keys) feeds dQ of step m in step m.  F(m) is copied in
// step m - 4 (ring of four slots), T(m) in step m - 2 (ring of three).
constexpr int kQ_KN = 0;                         // 32 rows x 256 B
constexpr int kQ_KR = kQ_KN + 32 * kDn * 2;      // 32 rows x 128 B   (8192)
constexpr int kQ_V = kQ_KR + 32 * kDr * 2;       // 32 rows x 256 B   (12288)
constexpr int kQ_B = kQ_V + 32 * kDv * 2;        // 128 x 8 B          (20480)
constexpr int kQF_Slot = kQ_B + 1024;            // 21504
constexpr int kQ_KTN = 0;                        // 128 rows x 64 B
constexpr int kQ_KTR = kQ_KTN + kDn * 64;        // 64 rows x 64 B     (8192)
constexpr int kQT_Slot = kQ_KTR + kDr * 64;      // 12288
constexpr int kQFSlots = 4;
constexpr int kQTSlots = 3;
// copy instructions per wave and step: 2 k_nope, 1 k_rope, 2 v, words (F); 2 k_nope^T, 1 k_rope^T (T)
constexpr int kQCopiesPerStep = 9;

// copy plan: instruction j (0..8) of wave w; the step's uniform offsets (key0 its
// first key): k_nope and v: key0 * 256; k_rope: key0 * 128; words: the tile's
// 1 KiB; transposed rows: key0 * 2 (rows Lkp * 2 bytes apart)
enum : int { kSrcKN, kSrcKR, kSrcV, kSrcBits, kSrcKTN, kSrcKTR };
constexpr int q_src_region(int j) {
  return j < 2 ? kSrcKN : j == 2 ? kSrcKR : j < 5 ? kSrcV : j == 5 ? kSrcBits : j < 8 ? kSrcKTN : kSrcKTR;
}
constexpr bool q_f_part(int j) { return j < 6; }
constexpr int q_dst_base(int w, int j) {
  return j < 2 ? kQ_KN + (2 * w + j) * 1024
       : j == 2 ? kQ_KR + w * 1024
       : j < 5 ? kQ_V + (2 * w + j - 3) * 1024
       : j == 5 ? kQ_B
       : j < 8 ? kQ_KTN + (2 * w + j - 6) * 1024
       : kQ_KTR + w * 1024;
}
constexpr uint32_t q_voff(int w, int j, int l, int Lkp) {
  switch (q_src_region(j)) {
    case kSrcKN: {
      const int blk = 2 * w + j;
      return static_cast<uint32_t>(blk_row(blk, l, 256) * 256 + blk_x(blk, l, 256));
    }
    case kSrcKR: return static_cast<uint32_t>(blk_row(w, l, 128) * 128 + blk_x(w, l, 128));
    case kSrcV: {
      const int blk = 2 * w + j - 3;
      return static_cast<uint32_t>(blk_row(blk, l, 256) * 256 + blk_x(blk, l, 256));
    }
    case kSrcBits: return static_cast<uint32_t>(l) * 16u;
    case kSrcKTN: {
      const int blk = 2 * w + j - 6;
      return static_cast<uint32_t>(blk_row(blk, l, 64)) * static_cast<uint32_t>(Lkp) * 2u +
             static_cast<uint32_t>(blk_x(blk, l, 64));
    }
    default:
      return static_cast<uint32_t>(blk_row(w, l, 64)) * static_cast<uint32_t>(Lkp) * 2u +
             static_cast<uint32_t>(blk_x(w, l, 64));
  }
}
// reads (lane l: li = l % 32, hi = l / 32)
// S^T = K Q^T, A operand chunk s (dims 16s ..): key row li
constexpr int rd_k(int s, int li, int hi) {
  return s < kDn / 16 ? kQ_KN + region_byte(li, 32 * s + 16 * hi, kDn * 2)
                      : kQ_KR + region_byte(li, 32 * (s - kDn / 16) + 16 * hi, kDr * 2);
}
// dP^T = V dO^T, A operand chunk s
constexpr int rd_v(int s, int li, int hi) { return kQ_V + region_byte(li, 32 * s + 16 * hi, kDv * 2); }
// dQ^T += K^T dS^T: K^T row d = 32mt + li, positions 16kk + 8hi .. +8 of the step's 32 (relabelled) keys
constexpr int rd_kt(int mt, int kk, int li, int hi) {
  return 32 * mt + li < kDn ? kQ_KTN + region_byte(32 * mt + li, 32 * kk + 16 * hi, 64)
                            : kQ_KTR + region_byte(32 * mt + li - kDn, 32 * kk + 16 * hi, 64);
}
// the visibility word (64 key bits) of query row ql (0..127) of the tile
constexpr int rd_qword(int ql) { return kQ_B + ql * 8; }

}  // namespace dflash
