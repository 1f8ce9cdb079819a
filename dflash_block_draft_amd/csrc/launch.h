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
};

struct AttnF32Args {
  const float* q; const float* kn; const float* kr; const float* v;
  const float* mask;      // [B,1,Lq,Lk] f32 or null
  float* out;
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

struct ExpandArgs {
  const void* latent; const void* w;  // [B,Lk,R], [H*256,R]
  void* kn; void* v;                  // [B,H,Lk,128] each
  int B, Lk, R, H;
};

hipError_t launch_attn_bf16(const AttnBf16Args& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnF32Args& a, hipStream_t s);
hipError_t launch_occupancy(const OccupancyArgs& a, hipStream_t s);
// The same tile map from the block structure (anchors, ctx_valid, bs) instead of a dense mask.
hipError_t launch_block_occupancy(const OccupancyArgs& a, hipStream_t s);
// Rewrite the lists so every k-tile is visited (empty tiles as class 3); debug/verification mode.
hipError_t launch_lists_all_tiles(const OccupancyArgs& a, hipStream_t s);
hipError_t launch_expand_bf16(const ExpandArgs& a, hipStream_t s);
hipError_t launch_expand_f32(const ExpandArgs& a, hipStream_t s);

}  // namespace dflash
