/*
 * dflash_mla.h -- C ABI of the MI355X (gfx950) DFlash/DSpark draft MLA attention.
 *
 * What the library computes (NeMo AutoModel documentation pages
 * "speculative.dflash.draft_kimi_k3" and "speculative.dspark.draft_kimi_k3"):
 * the draft's non-causal MLA attention.  Queries are the num_anchors*block_size
 * noise-block tokens; keys and values span [target-hidden context | noise
 * block] (KimiK3DSparkAttention.forward: the context is concatenated before the
 * noise block).  Every query head has its own K/V, because kv_b_proj emits one
 * qk_nope_head_dim + v_head_dim slice per head (KimiK3DFlashAttention class
 * text: no GQA group repeat).  A key is [k_nope (per head) | k_rope (one per
 * token, shared by all heads; NoPE, so no rotary -- module text of the DFlash
 * page)].  The softmax scale is q_head_dim ** -0.5 (KimiK3DSparkAttention
 * attributes).  The dense additive mask [batch, 1, Lq, ctx + Lq] is added to
 * the scores unchanged (KimiK3DFlashAttention.forward); the Lq x Lk score
 * matrix is never materialised (same passage: it is too large to afford).
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are device memory owned by the caller, contiguous, in the
 *    layouts stated per call, and 16-byte aligned.  The library allocates no
 *    memory and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously on it; a kernel fault surfaces at the caller's
 *    next synchronisation.  Calls on different streams are independent as long
 *    as they do not share a workspace.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    non-OK status means nothing was launched (except DFLASH_ERR_HIP, which
 *    reports a failed launch).  dflash_last_error() gives a readable reason.
 *  - No C++ exception crosses this interface.
 *  - Results are bitwise deterministic from run to run (no atomics in any
 *    reduction; the work schedule does not change which lane sums what).
 */
#ifndef DFLASH_MLA_H
#define DFLASH_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are int-sized in C and C++ alike.  C++ code sees them with a fixed
 * underlying type int, so any int a C caller passes (e.g. an unknown dtype the
 * library must reject) is a valid value there too, not undefined behaviour. */
#ifdef __cplusplus
#define DFLASH_ENUM_BASE : int
#else
#define DFLASH_ENUM_BASE
#endif

typedef enum dflash_status DFLASH_ENUM_BASE {
  DFLASH_OK = 0,
  DFLASH_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, non-positive size, bad scale, aliasing, bad flags */
  DFLASH_ERR_UNSUPPORTED = 2,  /* head dims or dtype combination the library does not implement */
  DFLASH_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  DFLASH_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} dflash_status;

typedef enum dflash_dtype DFLASH_ENUM_BASE {
  DFLASH_F32 = 0,
  DFLASH_BF16 = 1
} dflash_dtype;

/* Attention tile: queries per tile x keys per tile.  The mask-occupancy map
 * classifies tiles of exactly this shape. */
#define DFLASH_TILE_M 128
#define DFLASH_TILE_N 64

/* Tile classes stored in the occupancy map (one byte per tile). */
#define DFLASH_TILE_EMPTY 0   /* every mask entry is exactly -inf: the tile is skipped            */
#define DFLASH_TILE_ZERO 1    /* every mask entry is +0 or -0: no mask load, no mask add          */
#define DFLASH_TILE_BINARY 2  /* only +-0 and -inf, both present: a 64-bit visibility word per    */
                              /* row is stored in the workspace and applied instead of the values */
#define DFLASH_TILE_MIXED 3   /* anything else: the mask values are loaded and added              */

/* dflash_mla_attn flags */
#define DFLASH_ATTN_REUSE_TILE_MAP 0x1u  /* skip the occupancy pass: the workspace already holds
                                            the map of this same mask (e.g. the next draft layer,
                                            which receives the same mask) */
#define DFLASH_ATTN_NO_TILE_SKIP 0x2u    /* debug/verification: visit every tile, treating empty
                                            tiles as mixed; the result is bitwise identical.  The
                                            workspace lists are left covering every tile, so a later
                                            REUSE_TILE_MAP call on it also visits every tile */
#define DFLASH_ATTN_CHECK_ONLY 0x4u      /* validate the arguments and return; launch nothing */
#define DFLASH_ATTN_SPLIT_KEYS 0x8u      /* BF16: when the (batch, q-tile, head) grid is small, cut
                                            each q-tile's key tiles into 2, 4 or 8 runs processed
                                            in parallel and merged in a fixed order (the pages'
                                            softmax, regrouped: results equal the unsplit call's up
                                            to bf16 rounding of each run's weights and output;
                                            still deterministic run to run).  The
                                            workspace must then hold
                                            dflash_mla_attn_split_workspace_bytes(B, H, Lq, Lk).
                                            Ignored together with NO_TILE_SKIP. */

/* Human-readable name of a status. Never NULL. */
const char* dflash_status_string(dflash_status status);

/* Reason for the last non-OK status returned on the calling thread ("" if none). */
const char* dflash_last_error(void);

/*
 * kv_b_proj expansion of the compressed KV latent into per-head k_nope and v.
 * Pages: DFlash page, KimiK3DFlashAttention class text ("kv_b_proj produces
 * num_attention_heads slices of qk_nope_head_dim + v_head_dim"); DSpark page,
 * KimiK3DSparkAttention (kv_b_proj, kv_lora_rank); Kimi K3 model page, MLA
 * context-parallel forward (the latent is kv_lora_rank values per token besides
 * the head-shared rope part, and is expanded locally).
 *
 *   k_nope[b,h,t,e] = sum_r latent[b,t,r] * w_kv_b[h*(Dn+Dv) + e,      r]   (e < Dn)
 *   v     [b,h,t,e] = sum_r latent[b,t,r] * w_kv_b[h*(Dn+Dv) + Dn + e, r]   (e < Dv)
 *
 * latent  [B, Lk, R]          dtype dt   (the kv_b_proj input, already normed)
 * w_kv_b  [H*(Dn+Dv), R]      dtype dt   (Linear weight, out x in, no bias)
 * k_nope  [B, H, Lk, Dn]      dtype dt   (written)
 * v       [B, H, Lk, Dv]      dtype dt   (written)
 * Accumulation is fp32; bf16 outputs are rounded to nearest even.
 * Supported: Dn == 128, Dv == 128, R a positive multiple of 32, dt F32 or BF16.
 * Outputs must not overlap each other or the inputs.
 */
dflash_status dflash_mla_latent_expand(const void* latent, const void* w_kv_b,
                                       void* k_nope, void* v,
                                       int64_t B, int64_t Lk, int64_t R, int64_t H,
                                       int64_t Dn, int64_t Dv, dflash_dtype dt,
                                       void* stream);

/*
 * Bytes of device workspace dflash_mla_attn / dflash_mla_mask_occupancy need for
 * a masked call of this shape (the occupancy map, the per-q-tile lists of
 * non-empty k-tiles and the schedule).  0 if any size is not positive.
 */
size_t dflash_mla_attn_workspace_bytes(int64_t B, int64_t Lq, int64_t Lk);

/*
 * Bytes of workspace a BF16 dflash_mla_attn / dflash_mla_attn_lse /
 * dflash_mla_attn_blocks call with DFLASH_ATTN_SPLIT_KEYS needs: the tile map
 * (same layout and offsets as dflash_mla_attn_workspace_bytes) followed by the
 * fp32 partial outputs of the key-range runs, [S, B, H, Lq, Dv] and [S, B, H, Lq],
 * S in {1, 2, 4, 8} chosen from the shape (S = 1: the map size alone, no split).
 * 0 if any size is not positive or the sizes overflow.
 */
size_t dflash_mla_attn_split_workspace_bytes(int64_t B, int64_t H, int64_t Lq, int64_t Lk);

/*
 * Where the occupancy results sit inside the workspace, so a caller can read
 * them back (all offsets in bytes from the workspace start; any output pointer
 * may be NULL):
 *   classes  uint8  [B, n_q_tiles, n_k_tiles]   DFLASH_TILE_* per tile
 *   counts   int32  [B, n_q_tiles]              non-empty k-tiles per q-tile
 *   lists    int32  [B, n_q_tiles, n_k_tiles]   first counts[] entries: k-tile index | class << 24,
 *                                               in increasing k order
 *   order    int32  [B * n_q_tiles]             (b * n_q_tiles + q-tile) by decreasing count,
 *                                               ties by increasing index
 *   bits     uint64 [B, n_q_tiles, n_k_tiles, DFLASH_TILE_M]   for DFLASH_TILE_BINARY tiles only:
 *                                               bit k of row r is set iff mask entry
 *                                               (qt*M + r, kt*N + k) is +-0 (rows/columns past
 *                                               the mask read 0); other tiles' words are unspecified
 * After bits the workspace holds one private counter the occupancy pass uses.
 * n_q_tiles = ceil(Lq / DFLASH_TILE_M), n_k_tiles = ceil(Lk / DFLASH_TILE_N).
 */
dflash_status dflash_mla_tile_map_layout(int64_t B, int64_t Lq, int64_t Lk,
                                         int64_t* n_q_tiles, int64_t* n_k_tiles,
                                         size_t* classes_offset, size_t* counts_offset,
                                         size_t* lists_offset, size_t* order_offset,
                                         size_t* bits_offset);

/*
 * The mask-occupancy pass alone: classify every DFLASH_TILE_M x DFLASH_TILE_N
 * tile of the additive mask and build the lists/schedule in the workspace.
 * Tile of (b, qt, kt): rows [qt*M, min(qt*M+M, Lq)), columns [kt*N, min(kt*N+N, Lk))
 * of mask[b, 0]; entries outside the mask do not count.  Classes compare bit
 * patterns: exactly -inf is "masked"; +0/-0 is "zero"; everything else,
 * including NaN, +inf and large finite negatives, is a "value" and makes the
 * tile DFLASH_TILE_MIXED.
 *
 * additive_mask [B, 1, Lq, Lk] in mask_dt (F32 or BF16).
 * The pages pass the same mask to every draft layer (DFlash page,
 * KimiK3DFlashDecoderLayer.forward), so the result can be reused across layers
 * with DFLASH_ATTN_REUSE_TILE_MAP.
 */
dflash_status dflash_mla_mask_occupancy(const void* additive_mask, dflash_dtype mask_dt,
                                        int64_t B, int64_t Lq, int64_t Lk,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Non-causal draft MLA attention (DFlash page, KimiK3DFlashAttention.forward;
 * DSpark page, KimiK3DSparkAttention.forward).  For batch b, head h, query i:
 *
 *   s_j = scale * (q[b,h,i,:Dn] . k_nope[b,h,j,:] + q[b,h,i,Dn:] . k_rope_shared[b,j,:])
 *         + additive_mask[b,0,i,j]
 *   out[b,h,i,:] = sum_j softmax_j(s) * v[b,h,j,:]
 *
 * q             [B, H, Lq, Dn+Dr]  dtype dt  (q_nope then q_rope)
 * k_nope        [B, H, Lk, Dn]     dtype dt
 * k_rope_shared [B, Lk, Dr]        dtype dt  (one per token, shared by every head)
 * v             [B, H, Lk, Dv]     dtype dt
 * additive_mask [B, 1, Lq, Lk]     mask_dt, or NULL (= every key visible)
 * out           [B, H, Lq, Dv]     dtype dt  (written; must not overlap any input)
 * scale         finite and > 0; the pages' value is (Dn + Dr) ** -0.5.
 *
 * Supported: Dn == 128, Dr == 64, Dv == 128;
 *   (dt, mask_dt) in {(F32, F32), (BF16, F32), (BF16, BF16)};
 *   a BF16 call takes at most 2^23 - 1 keys (one (b, h) slice of k_nope or v
 *   within 2^31 bytes: the kernel addresses it through a 32-bit buffer range),
 *   else UNSUPPORTED.
 * BF16: QK^T and PV run as bf16 MFMA with fp32 accumulation and an online
 *   softmax in fp32; the probabilities are rounded to bf16 for PV; out is
 *   rounded to nearest even.  F32: fp32 arithmetic throughout.
 * A query row whose every score is -inf returns 0 (the pages do not define it).
 * Mask semantics: only exactly -inf hides a key; finite values, however large,
 *   are added; +inf/NaN entries propagate NaN into that row as the plain
 *   definition does.
 * Workspace (BF16 with a mask): at least dflash_mla_attn_workspace_bytes(B, Lq, Lk)
 *   bytes, 256-byte aligned; unused (may be NULL/0) when the mask is NULL or dt is F32.
 * flags: any of DFLASH_ATTN_REUSE_TILE_MAP, DFLASH_ATTN_NO_TILE_SKIP, DFLASH_ATTN_CHECK_ONLY,
 *   DFLASH_ATTN_SPLIT_KEYS (BF16; ignored by F32).  With SPLIT_KEYS on a shape that
 *   splits, the workspace is required (also without a mask): NULL or smaller than
 *   dflash_mla_attn_split_workspace_bytes returns WORKSPACE.
 * additive_mask NULL with DFLASH_ATTN_REUSE_TILE_MAP (BF16 only): the tile map
 *   already in the workspace alone decides which keys each query sees -- e.g. a
 *   map from dflash_mla_block_occupancy, which makes this the block-structure
 *   attention with any of the entry points (with lse, backward).  Such a map
 *   must come from a 0 / -inf visibility (classes empty / zero / binary); tiles of
 *   general values, which need the mask, are then read as all visible.
 *   NO_TILE_SKIP is rejected there (INVALID_ARG), as is F32.
 */
dflash_status dflash_mla_attn(const void* q, const void* k_nope, const void* k_rope_shared,
                              const void* v, const void* additive_mask, void* out,
                              int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                              int64_t Dn, int64_t Dr, int64_t Dv, float scale,
                              dflash_dtype dt, dflash_dtype mask_dt,
                              void* workspace, size_t workspace_bytes,
                              uint32_t flags, void* stream);

/*
 * dflash_mla_attn that also writes, for every (b, h, i), the natural-log row
 * normaliser lse[b,h,i] = log(sum_j exp(s_j)) (f32, [B, H, Lq]; -inf for a row
 * with no finite score), which the backward takes instead of recomputing the
 * softmax statistics.  In the BF16 path the sum adds the fp32 probabilities,
 * except on key steps of the exact path (a tile with general mask values, a
 * ragged key tail, a row's first visible step), where it adds the bf16-rounded
 * probabilities the kernel applies in PV.  Each probability is within a
 * relative 2^-9 of its rounding, so exp(s_j - lse) are within about 2^-9 of
 * both the exact softmax weights and the normalised weights that produced out.
 * lse must be 4-byte aligned and overlap nothing else; other
 * arguments, limits and errors as dflash_mla_attn.
 */
dflash_status dflash_mla_attn_lse(const void* q, const void* k_nope, const void* k_rope_shared,
                                  const void* v, const void* additive_mask, void* out, float* lse,
                                  int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                  int64_t Dn, int64_t Dr, int64_t Dv, float scale,
                                  dflash_dtype dt, dflash_dtype mask_dt,
                                  void* workspace, size_t workspace_bytes, uint32_t flags,
                                  void* stream);

/*
 * dflash_mla_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation with no workspace argument.  The tile map of a masked
 * BF16 call goes to a static device array of DFLASH_NO_ALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends; the
 * call allocates nothing.  Shapes whose map needs more
 * (dflash_mla_attn_workspace_bytes(B, Lq, Lk) > DFLASH_NO_ALLOC_SCRATCH_BYTES,
 * e.g. B * ceil(Lq/128) * ceil(Lk/64) beyond about 31,000 tiles) return
 * UNSUPPORTED.  flags: only DFLASH_ATTN_NO_TILE_SKIP and DFLASH_ATTN_CHECK_ONLY
 * (REUSE_TILE_MAP and SPLIT_KEYS return INVALID_ARG).  The current device must be
 * the stream's.  Every call on one GPU uses the same scratch and leaves its map
 * there: calls that overlap on one GPU (different streams, or threads) race and
 * must be serialised by the caller; calls in order on one stream are safe.
 * Other arguments, limits and errors as dflash_mla_attn.
 */
#define DFLASH_NO_ALLOC_SCRATCH_BYTES (32u << 20)
dflash_status dflash_mla_attn_no_alloc(const void* q, const void* k_nope, const void* k_rope_shared,
                                       const void* v, const void* additive_mask, void* out,
                                       int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                       int64_t Dn, int64_t Dr, int64_t Dv, float scale,
                                       dflash_dtype dt, dflash_dtype mask_dt,
                                       uint32_t flags, void* stream);

/*
 * Bytes of device workspace dflash_mla_attn_bwd needs (0 for invalid sizes).  It
 * begins with the forward's tile map in the dflash_mla_tile_map_layout layout,
 * so one workspace of this size serves the forward (dflash_mla_attn_lse) and then
 * the backward with DFLASH_ATTN_REUSE_TILE_MAP.
 */
size_t dflash_mla_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Lq, int64_t Lk);

/*
 * Gradients of dflash_mla_attn with respect to q, k_nope, k_rope_shared and v.
 * The draft is trained (DFlash page, KimiK3DFlashDraftModel: the DFlash trainer;
 * DSpark page, module text: speculative-decoding training).  With
 * p_ij = exp(s_ij - lse_i) and D_i = sum_d dout[i,d] * out[i,d]:
 *
 *   ds_ij = p_ij * (dout_i . v_j - D_i)
 *   dq_i = scale * sum_j ds_ij [k_nope_j | k_rope_j]    dv_j = sum_i p_ij dout_i
 *   dk_nope_j = scale * sum_i ds_ij q_i[:Dn]
 *   dk_rope_shared[b,j] = scale * sum_h sum_i ds_ij q_i[Dn:]   (summed over heads)
 *
 * Inputs (not modified): q, k_nope, k_rope_shared, v, additive_mask as in
 * dflash_mla_attn; out [B,H,Lq,Dv] and lse [B,H,Lq] f32 as written by
 * dflash_mla_attn_lse for the same inputs; dout [B,H,Lq,Dv] (gradient of out).
 * Outputs (written): dq [B,H,Lq,Dn+Dr], dk_nope [B,H,Lk,Dn], dk_rope_shared
 * [B,Lk,Dr], dv [B,H,Lk,Dv], all dtype dt.  Rows with lse = -inf (no visible
 * key) pass no gradient; hidden entries (mask -inf) have p = 0.  The mask gets
 * no gradient.
 * Supported: dt = BF16 (F32 returns UNSUPPORTED), mask_dt F32 or BF16, Dn 128,
 *   Dr 64, Dv 128, B * H <= 65535, at most 2^24 - 1 key tiles, and Lq and Lk
 *   (rounded up to 128 / 64) at most 2^31 / 384 (one (batch, head) slice of an
 *   operand within 2 GiB).  bf16 MFMA with
 *   fp32 accumulation; p and ds are rounded to bf16 as MFMA operands; outputs
 *   rounded to nearest even.  Deterministic: no atomics, dk_rope summed over
 *   heads in head order.
 * Workspace: at least dflash_mla_attn_bwd_workspace_bytes(B, H, Lq, Lk) bytes,
 *   256-byte aligned, not overlapping any tensor.  flags: 0, or
 *   DFLASH_ATTN_REUSE_TILE_MAP when the workspace already holds the tile map of
 *   this mask (a forward call on the same workspace); with additive_mask NULL and
 *   REUSE_TILE_MAP the map alone decides visibility, as for dflash_mla_attn
 *   (the block-structure path: dflash_mla_block_occupancy on this workspace first).
 * Errors: INVALID_ARG (NULL or misaligned pointers, sizes <= 0, bad scale, unknown
 *   flags, overlapping buffers), UNSUPPORTED, WORKSPACE, HIP.
 */
dflash_status dflash_mla_attn_bwd(const void* q, const void* k_nope, const void* k_rope_shared,
                                  const void* v, const void* additive_mask, const void* out,
                                  const void* dout, const float* lse, void* dq, void* dk_nope,
                                  void* dk_rope_shared, void* dv, int64_t B, int64_t H, int64_t Lq,
                                  int64_t Lk, int64_t Dn, int64_t Dr, int64_t Dv, float scale,
                                  dflash_dtype dt, dflash_dtype mask_dt, void* workspace,
                                  size_t workspace_bytes, uint32_t flags, void* stream);

/*
 * ---- Projections on either side of the attention (bf16 only) ----
 *
 * The draft's MLA uses Q-LoRA and a compressed KV latent with fp32-variance
 * RMSNorms (DFlash page, module text; DSpark page, KimiK3DSparkAttention
 * attributes q_a_proj, q_a_layernorm, q_b_proj, kv_a_proj_with_mqa,
 * kv_a_layernorm, kv_b_proj), and the target context is projected by fc and
 * normed once per step (DSpark page, KimiK3DSparkModel._forward_backbone).
 * Linear weights are [out, in] row-major (PyTorch Linear).  RMSNorm:
 *   rmsnorm(x)[k] = bf16( bf16(x[k] * rsqrt(mean_j(x[j]^2) + eps)) * gamma[k] ),
 * with the mean over the row in fp32 of the bf16 values.  Matrix products run as
 * bf16 MFMA with fp32 accumulation and round their outputs to bf16.  The norms
 * are fused: the producing product writes per-row partial sums of squares, and
 * the consuming product normalises its operand rows as it loads them.
 * All tensors are contiguous device memory, 16-byte aligned; outputs and the
 * workspace must not overlap any other buffer.  Errors: INVALID_ARG (NULL or
 * misaligned pointers, sizes <= 0, eps < 0 or not finite, overlaps),
 * UNSUPPORTED (divisibility below, sizes beyond int32), WORKSPACE, HIP.
 */

/* Workspace for one projection chain: an intermediate of [rows, width] bf16 plus
 * its row statistics.  context_project: (B*ctx, hidden); q_project:
 * (B*Lq, q_lora_rank); kv_project: (B*(ctx+Lq), R).  0 for invalid sizes. */
size_t dflash_mla_projection_workspace_bytes(int64_t rows, int64_t width);

/* out[b,t,:] = rmsnorm(target_hidden[b,t,:] . w_fc^T) with weight gamma [hidden]:
 * target_hidden [B, ctx, K_in], w_fc [hidden, K_in], out [B, ctx, hidden].
 * K_in a multiple of 32, hidden a multiple of 128. */
dflash_status dflash_mla_context_project(const void* target_hidden, const void* w_fc, const void* gamma,
                                         float eps, void* out, int64_t B, int64_t ctx, int64_t K_in,
                                         int64_t hidden, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* q[b,h,t,:] = (rmsnorm(x[b,t,:] . w_q_a^T) . w_q_b^T)[h*Dqk : (h+1)*Dqk]:
 * x [B, Lq, hidden], w_q_a [q_lora_rank, hidden], gamma_q [q_lora_rank],
 * w_q_b [H*Dqk, q_lora_rank], q [B, H, Lq, Dqk] (the layout dflash_mla_attn
 * takes; within a head, q_nope then q_rope).  hidden a multiple of 32,
 * q_lora_rank of 128, Dqk of 4. */
dflash_status dflash_mla_q_project(const void* x, const void* w_q_a, const void* gamma_q, float eps,
                                   const void* w_q_b, void* q, int64_t B, int64_t Lq, int64_t hidden,
                                   int64_t q_lora_rank, int64_t H, int64_t Dqk, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Keys and values of the draft attention over [context | noise]:
 *   h = [ctx_hidden[b] ; noise_hidden[b]]         ([ctx + Lq, hidden] per batch row)
 *   c = h . w_kv_a^T                               ([.., R + Dr])
 *   k_rope_shared[b,t,:] = c[t, R:]                ([B, ctx+Lq, Dr], head-shared)
 *   latent = rmsnorm(c[t, :R]) with gamma_kv [R]
 *   k_nope, v = kv_b_proj(latent) as dflash_mla_latent_expand ([B, H, ctx+Lq, 128] each)
 * ctx_hidden [B, ctx, hidden] (NULL allowed when ctx == 0), noise_hidden
 * [B, Lq, hidden], w_kv_a [R + Dr, hidden], w_kv_b [H*(Dn+Dv), R].
 * hidden a multiple of 32, R of 128, Dr of 4, Dn = Dv = 128. */
dflash_status dflash_mla_kv_project(const void* ctx_hidden, const void* noise_hidden, const void* w_kv_a,
                                    const void* gamma_kv, float eps, const void* w_kv_b, void* k_nope,
                                    void* k_rope_shared, void* v, int64_t B, int64_t ctx, int64_t Lq,
                                    int64_t hidden, int64_t R, int64_t Dr, int64_t H, int64_t Dn, int64_t Dv,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * ---- The MHA/GQA DFlash draft (Modular MAX page, pipelines.architectures.dflash_kimi_k25) ----
 *
 * A DFlash draft for a Kimi K2.5 target whose own attention is MHA/GQA with
 * DeepSeek-yarn RoPE and qk-norm; the context's keys and values are written once
 * into a bf16 cache (DFlashKimiK25.materialize) and each block then attends
 * non-causally to that cache plus itself (DFlashKimiK25.forward_block).
 *
 * Cache layout (caller-owned, bf16): k_cache [B, Hkv, Lmax, 128]; v_cache_t
 * [B, Hkv, 128, Lmax] (V transposed: keys contiguous per dimension, so the
 * attention reads V^T operands without transposing).  Lmax a multiple of 8.
 * rope: host array of 7 floats {theta, factor, original_max_position,
 * beta_fast, beta_slow, mscale, mscale_all_dim}; yarn inverse frequencies
 * blend 1/theta^(2i/128) and that divided by factor with a linear ramp between
 * the correction dimensions of beta_fast and beta_slow rotations, and cos/sin
 * are scaled by m(factor, mscale) / m(factor, mscale_all_dim), m(s, x) =
 * 0.1 x ln s + 1 (1 for s <= 1).  RoPE pairs dimension i with i + 64
 * (rotate-half).  qk-norm: RMSNorm over the 128 dims of every head
 * (fp32 variance; weight [128]) before RoPE.  Projections are bf16 MFMA with
 * fp32 accumulation (weights [out, in]); the attention uses scale `scale`.
 * head_dim must be 128.  Errors as for the projections.
 */

/* k_cache[b, :, t] = RoPE(qk-norm(ctx_hidden[b, t] . w_k^T)) at position t, and
 * v_cache_t[b, :, :, t] = ctx_hidden[b, t] . w_v^T, for t < Lc (<= Lmax).
 * ctx_hidden [B, Lc, hidden], w_k / w_v [Hkv * 128, hidden], gamma_k [128]. */
dflash_status dflash_gqa_materialize(const void* ctx_hidden, const void* w_k, const void* w_v,
                                     const void* gamma_k, float eps, const float* rope, void* k_cache,
                                     void* v_cache_t, int64_t B, int64_t Lc, int64_t Lmax, int64_t hidden,
                                     int64_t Hkv, int64_t head_dim, void* stream);

/* Workspace bytes of dflash_gqa_forward_block (the block's q and the split-K
 * partials); 0 for invalid sizes. */
size_t dflash_gqa_workspace_bytes(int64_t B, int64_t bs, int64_t Hq, int64_t Hkv, int64_t Lmax);

/* One draft block per batch row: with c = clamp(ctx_len[b], 0, Lmax - bs)
 * (ctx_len: int32 [B], device) and positions c + i for block token i:
 *   q = RoPE(qk-norm(blk_hidden . w_q^T)) per head            ([B, Hq, bs, 128])
 *   the block's k, v (as dflash_gqa_materialize) are written into the caches at
 *   times c .. c + bs - 1
 *   out[b, h, i] = softmax_j(scale * q . k_cache[b, h / (Hq/Hkv), j]) v_j over the
 *   keys j < c + bs (the context and the whole block: non-causal)
 * blk_hidden [B, bs, hidden], w_q [Hq * 128, hidden], gamma_q / gamma_k [128],
 * out [B, Hq, bs, 128] bf16.  Hq a multiple of Hkv and (Hq / Hkv) * bs <= 64.
 * The caches are modified (the block's rows); calls on overlapping caches race. */
dflash_status dflash_gqa_forward_block(const void* blk_hidden, const void* w_q, const void* w_k,
                                       const void* w_v, const void* gamma_q, const void* gamma_k, float eps,
                                       const float* rope, void* k_cache, void* v_cache_t,
                                       const int32_t* ctx_len, void* out, int64_t B, int64_t bs, int64_t Lmax,
                                       int64_t hidden, int64_t Hq, int64_t Hkv, int64_t head_dim, float scale,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * The tile map of the DFlash block mask computed from the block structure itself
 * instead of a dense mask: no mask bytes are read.  Row b, query i belongs to
 * block j = i / block_size and sees context key k (k < ctx) iff
 * k <= anchors[b, j] and k < ctx_valid[b], and noise key ctx + m iff
 * m / block_size == j (its own block, non-causally).  This is the block
 * structure the dense additive mask of the DFlash page (KimiK3DFlashAttention.forward)
 * carries; the resulting map equals dflash_mla_mask_occupancy of the 0 / -inf
 * mask with that visibility.
 *
 * anchors    int32 [B, A], device, 4-byte aligned: the context position each block
 *            is anchored at (any value; one below 0 hides the whole context)
 * ctx_valid  int32 [B], device, or NULL (= ctx); values are clamped to [0, ctx]
 * Lq = A * block_size, Lk = ctx + Lq; the workspace is sized and laid out as for
 * dflash_mla_attn_workspace_bytes(B, Lq, Lk) / dflash_mla_tile_map_layout.
 * Errors: INVALID_ARG (NULL or misaligned anchors, B/A/block_size <= 0, ctx < 0,
 * workspace overlapping anchors/ctx_valid), UNSUPPORTED (Lk beyond int32 or
 * 2^24 - 1 key tiles), WORKSPACE, HIP.
 */
dflash_status dflash_mla_block_occupancy(const int32_t* anchors, const int32_t* ctx_valid,
                                         int64_t B, int64_t A, int64_t block_size, int64_t ctx,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * dflash_mla_attn for the DFlash block mask given by its structure (see
 * dflash_mla_block_occupancy): out equals dflash_mla_attn with the dense 0 / -inf
 * additive mask of that structure, bitwise.  Lq = A * block_size, Lk = ctx + Lq;
 * tensors as for dflash_mla_attn.  BF16 only (F32 returns UNSUPPORTED).  The
 * workspace is required.  flags: 0 or any of DFLASH_ATTN_REUSE_TILE_MAP (the
 * workspace holds the map of this same structure, e.g. for the next draft layer)
 * and DFLASH_ATTN_SPLIT_KEYS (as for dflash_mla_attn: then the result equals the
 * dense-mask call with SPLIT_KEYS bitwise, and the workspace must hold
 * dflash_mla_attn_split_workspace_bytes).
 */
dflash_status dflash_mla_attn_blocks(const void* q, const void* k_nope, const void* k_rope_shared,
                                     const void* v, const int32_t* anchors, const int32_t* ctx_valid,
                                     void* out, int64_t B, int64_t H, int64_t A, int64_t block_size,
                                     int64_t ctx, int64_t Dn, int64_t Dr, int64_t Dv, float scale,
                                     dflash_dtype dt, void* workspace, size_t workspace_bytes,
                                     uint32_t flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_MLA_H */
