// Host-side launchers of the gfx950 kernels (internal to the library; the
// public interface is include/dflash_mla.h).  Arguments reaching these have
// already been validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

struct AttnBf16Args {
  const uint16_t* q;      // [B,H,Lq,192] bf16
  const uint16_t* kn;     // [B,H,Lk,128] bf16
  const uint16_t* kr;     // [B,Lk,64]    bf16
  const uint16_t* v;      // [B,H,Lk,128] bf16
  const void* mask;       // [B,1,Lq,Lk] f32/bf16 or null
  uint16_t* out;          // [B,H,Lq,128] bf16
  const uint8_t* classes; // [B,nqt,nkt]  (null when mask is null)
  const int32_t* counts;  // [B*nqt]
  const int32_t* lists;   // [B*nqt, nkt]
  const int32_t* order;   // [B*nqt]
  const uint64_t* bits;   // [B*nqt*nkt, 128] visibility words of class-2 tiles
  int B, H, Lq, Lk, nqt, nkt;
  float scale;            // softmax scale (natural units)
  int mask_bf16;          // 1: mask is bf16, 0: f32
  float* lse;             // [B,H,Lq] f32 natural-log row normaliser (-inf: dead row), or null
  // key-range split: work item (b, q-tile, h) is cut into nsplit contiguous runs of
  // its tile list; with nsplit > 1 each run writes its normalised output (bf16,
  // RNE) and its row normaliser (f32) to part_o [nsplit,B,H,Lq,128] / part_lse
  // [nsplit,B,H,Lq] instead of out / lse, and launch_attn_combine merges them
  int nsplit;
  uint16_t* part_o;
  float* part_lse;
};

// out / lse of a split forward from its partial results (fixed order over the splits)
struct AttnCombineArgs {
  const uint16_t* part_o; const float* part_lse;
  uint16_t* out; float* lse;   // lse may be null
  int64_t rows;                // B*H*Lq
  int nsplit;
};

struct AttnF32Args {
  const float* q; const float* kn; const float* kr; const float* v;
  const float* mask;      // [B,1,Lq,Lk] f32 or null
  float* out;
  float* lse;             // [B,H,Lq] or null
  int B, H, Lq, Lk;
  float scale;
};

struct OccupancyArgs {
  const void* mask; int mask_bf16;
  int B, Lq, Lk, nqt, nkt;
  uint8_t* classes; int32_t* counts; int32_t* lists; int32_t* order;
  uint64_t* bits;   // [B*nqt*nkt, kTileM]: bit k of row r = entry (r, k) is +-0 (class-2 tiles only)
  uint32_t* sync;   // one counter: list workgroups done (zeroed by the classify pass)
  // DFlash block structure (block occupancy only): row b, query i in block j = i / bs
  // sees context key k <= anchors[b*A + j], k < ctx_valid[b], and noise keys of block j
  const int32_t* anchors; const int32_t* ctx_valid;  // [B, A], [B] or null (= ctx)
  int A, bs, ctx;
};

// Attention backward (bf16).  Workspace arrays are padded: Lqp = nqt*128 queries,
// Lkp = nkt*64 keys.  The transposed copies hold, per 16-entry group, entry
// 16g + k at position 16g + k with bits 2 and 3 of k swapped (the order in which
// an MFMA accumulator's rows become the next MFMA's reduction index).
struct AttnBwdArgs {
  const uint16_t* q; const uint16_t* kn; const uint16_t* kr; const uint16_t* v;
  const uint16_t* out; const uint16_t* dout;
  const void* mask; int mask_bf16;
  const float* lse;                       // [B,H,Lq]
  uint16_t* dq; uint16_t* dkn; uint16_t* dkr; uint16_t* dv;
  const uint8_t* classes; const int32_t* counts; const int32_t* lists; const int32_t* order;
  const uint64_t* bits;                   // tile map (null classes: every tile visible, no lists)
  uint16_t* qT;                           // [B*H, 192, Lqp]
  uint16_t* doT;                          // [B*H, 128, Lqp]
  uint16_t* knT;                          // [B*H, 128, Lkp]
  uint16_t* krT;                          // [B, 64, Lkp]
  float* rope_part;                       // [B*H, Lk, 64] per-head k_rope gradients
  float* ld;                              // [B*H, Lqp/32, 64]: per 32-query chunk, -lse*log2(e) (-inf for
                                          //   dead or padded rows), then -D
  uint32_t* bitsT;                        // [B, nkt, nqt, 4, 64] visibility of class-2 tiles by key: word
                                          //   (c, k) bit i = query 32c + i of the q-tile sees key k
  int B, H, Lq, Lk, nqt, nkt, Lqp, Lkp;
  float scale;
};

struct ExpandArgs {                   // fp32 expand
  const void* latent; const void* w;  // [B,Lk,R], [H*256,R]
  void* kn; void* v;                  // [B,H,Lk,128] each
  int B, Lk, R, H;
};

// Linear layer y = a W^T (bf16, fp32 accumulation) for the projections around
// the attention.  Rows m = b * (T1 + T2) + t come from a1[b, t] (t < T1) or
// a2[b, t - T1]; both [.., K] row-major.  Optional RMSNorm of the rows on load
// (stats_in: per-row partial sums of squares of the producer's bf16 outputs,
// stats_parts per row, over K entries; gamma [K]).  Optional statistics out:
// per-row partial sums of squares of the bf16 outputs over each 128-column tile
// of columns [0, Nstat), stats_out [M, Nstat / 128] (Nstat a multiple of 128).
constexpr int kLinearPlain = 0;   // y1 [M, N]
constexpr int kLinearSplit = 1;   // y1 [M, N1] (columns < N1), y2 [M, N - N1]
constexpr int kLinearHeads = 2;   // y1 [B, N / D, T1 + T2, D]
constexpr int kLinearKV = 3;      // per head h = n / 256: y1 = k_nope [B, N/256, T, 128] (n % 256 < 128), y2 = v
constexpr int kLinearHeadsT = 4;  // y1 [B, N / D, D, Lt] (time innermost), time index as for kLinearHeads
struct LinearArgs {
  const uint16_t* a1; const uint16_t* a2;
  int B, T1, T2, K;
  const uint16_t* w; int N;
  const float* stats_in; int stats_parts; const uint16_t* gamma; float eps;
  int mode; uint16_t* y1; uint16_t* y2; int N1; int D;
  float* stats_out; int Nstat;
  // head-major modes: time index of row t of batch row b is off(b) + t in a time
  // axis of Lt entries (Lt = 0: T1 + T2 and no offset); off(b) = clamp(row_off[b], 0, off_max)
  const int32_t* row_off; int off_max; int Lt;
  float* split_part;                 // set by the launcher for split-K runs: [splits, M, N] fp32
};

// In-place qk-norm + yarn RoPE of rows of a head-major tensor x [B, H, Lt, d]:
// rows t0(b) .. t0(b) + T - 1 with t0(b) = clamp(row_off[b], 0, off_max) (0 without
// row_off); position of row t0(b) + t is t0(b) + t.  d = 128.
struct NormRopeArgs {
  uint16_t* x; int B, H, Lt, T;
  const int32_t* row_off; int off_max;
  int rows_local;                         // 1: rows 0 .. T-1 (positions still t0(b) + t)
  const uint16_t* gamma; float eps;
  double inv_freq[64];                    // yarn inverse frequency of each rotary pair (fp64, from the host)
  float mscale;                           // cos / sin scale of yarn
};

// Block attention of the GQA draft: q [B, Hq, bs, d]; k cache [B, Hkv, Lmax, d];
// v cache transposed [B, Hkv, d, Lmax]; row b sees keys < clamp(ctx_len[b], 0, Lmax - bs) + bs.
struct GqaAttnArgs {
  const uint16_t* q; const uint16_t* k; const uint16_t* vt; uint16_t* out;
  const int32_t* ctx_len;
  int B, Hq, Hkv, bs, Lmax, splits, tiles_per_split;
  float scale;
  float* part_o; float* part_ml;        // [B*Hkv, splits, 64, 128], [B*Hkv, splits, 64, 2]
};

// y = RMSNorm(x) with statistics from the producer: y[m] = bf16(bf16(x[m] * r_m) * gamma).
struct RmsApplyArgs {
  const uint16_t* x; uint16_t* y; int64_t M; int N;
  const float* stats; int parts; const uint16_t* gamma; float eps;
};

// scratch (may be null): fp32 space for split-K partials; the launcher splits K
// across workgroups (then reduces the partials in order) when the output tiles
// alone cannot fill the chip and the scratch holds linear_split_bytes(a) bytes.
hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t s, float* scratch = nullptr, size_t scratch_bytes = 0);
size_t linear_split_bytes(const LinearArgs& a);
constexpr int kLinearMaxSplits = 16;
hipError_t launch_norm_rope_bf16(const NormRopeArgs& a, hipStream_t s);
hipError_t launch_gqa_attn_bf16(const GqaAttnArgs& a, hipStream_t s);
hipError_t launch_rms_apply_bf16(const RmsApplyArgs& a, hipStream_t s);
hipError_t launch_attn_bf16(const AttnBf16Args& a, hipStream_t s);
hipError_t launch_attn_combine(const AttnCombineArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnF32Args& a, hipStream_t s);
hipError_t launch_occupancy(const OccupancyArgs& a, hipStream_t s);
// The same tile map from the block structure (anchors, ctx_valid, bs) instead of a dense mask.
hipError_t launch_block_occupancy(const OccupancyArgs& a, hipStream_t s);
// Rewrite the lists so every k-tile is visited (empty tiles as class 3); debug/verification mode.
hipError_t launch_lists_all_tiles(const OccupancyArgs& a, hipStream_t s);
hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t s);
// dK, dV and the per-head k_rope parts (with the transposed visibility words they read)
hipError_t launch_bwd_dkdv(const AttnBwdArgs& a, hipStream_t s);
// dQ
hipError_t launch_bwd_dq(const AttnBwdArgs& a, hipStream_t s);
hipError_t launch_expand_f32(const ExpandArgs& a, hipStream_t s);

}  // namespace dflash
