/*
 * mmdit.h - C ABI of the joint video-audio attention hot path for MI355X (gfx950).
 *
 * What the calls compute comes from the pages on SkyReels-V4 (a dual-stream
 * MMDiT that generates video and audio together) and on Prism (dynamic
 * block-sparse attention for joint video-audio DiTs at 2K):
 *   - mmdit_rope3d            time-shifted 3D rotary embedding of Q and K;
 *   - mmdit_joint_attn        softmax attention, joint over [video|audio|text] or
 *                             any query set against any key set (video->text);
 *   - mmdit_av_cross_attn     bidirectional audio<->video cross-attention;
 *   - mmdit_block_sparse_attn mean-pooled block scores, hybrid top-k/top-p block
 *                             selection, attention over the selected blocks;
 *   - mmdit_joint_attn_fwd    mmdit_joint_attn that also returns the per-query
 *                             log-sum-exp a training step keeps for the backward;
 *   - mmdit_joint_attn_bwd    gradients of that attention with respect to q, k, v;
 *   - mmdit_block_sparse_attn_fwd / _bwd  the same pair for the block-sparse
 *                             attention (selection held fixed in the backward).
 *
 * Conventions shared by every call
 *   Layout     Q, K, V and O are contiguous [tokens][heads][head_dim] (head_dim
 *              fastest).  Device pointers must be 16-byte aligned.  Inputs are
 *              bf16 (MMDIT_BF16) or fp32 (MMDIT_FP32); attention outputs are
 *              always fp32.
 *   Ownership  The caller owns every buffer, the workspace included (its size
 *              comes from mmdit_workspace_bytes).  The library allocates and
 *              frees nothing and keeps no state besides a thread-local error
 *              string.
 *   Streams    `stream` is a hipStream_t passed as void* (NULL = the default
 *              stream).  Device calls enqueue kernels and return at once;
 *              results are ready when the stream is.
 *   Errors     Every argument is checked on the host before anything is
 *              enqueued: a non-OK status means nothing was enqueued.  A failed
 *              launch returns MMDIT_ERR_HIP.  Faults inside a kernel surface at
 *              the caller's next synchronisation.  Nothing throws across the
 *              ABI.  mmdit_last_error() describes the last non-OK status of the
 *              calling thread.
 *   Scale      softmax_scale multiplies <q, k> inside the softmax; it must be
 *              finite and >= 0, and 0 selects 1/sqrt(head_dim).
 *   Outputs    Outputs are overwritten, never accumulated into, and must not
 *              alias inputs.  mmdit_rope3d works in place on Q and K.
 *   Threads    Calls are reentrant; concurrent calls must not share a workspace.
 */
#ifndef MMDIT_H
#define MMDIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MMDIT_ABI_VERSION 4
#define MMDIT_MAX_SEGMENTS 16

typedef enum {
    MMDIT_OK = 0,
    MMDIT_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size or parameter */
    MMDIT_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement     */
    MMDIT_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required      */
    MMDIT_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed      */
} mmdit_status;

typedef enum { MMDIT_FP32 = 0, MMDIT_BF16 = 1 } mmdit_dtype;

typedef enum { MMDIT_SEG_VIDEO = 0, MMDIT_SEG_AUDIO = 1, MMDIT_SEG_TEXT = 2 } mmdit_seg_kind;

typedef enum {
    MMDIT_OP_JOINT_ATTN = 0,
    MMDIT_OP_AV_CROSS_ATTN = 1,
    MMDIT_OP_BLOCK_SPARSE_ATTN = 2,
    MMDIT_OP_JOINT_ATTN_BWD = 3,
    MMDIT_OP_BLOCK_SPARSE_ATTN_BWD = 4,
    MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE = 5,
    MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE_BWD = 6,
    MMDIT_OP_JOINT_ATTN_ROPE = 7
} mmdit_op;

/* One run of tokens of one modality inside a [tokens][heads][head_dim] buffer.
 * VIDEO: `count` = T*H*W tokens of frames t0 .. t0+T-1 in raster (t, h, w)
 *        order; conditioning latents are a VIDEO segment with negative t0
 *        (SkyReels-V4 analysis, workflow step 1 and novelty 4: negative
 *        temporal indices mark conditioning latents).
 * AUDIO: token j sits at temporal position j * t_scale and h = w = 0, so it is
 *        turned by the video's temporal bands only; t_scale = 21/218 lines 218
 *        audio tokens up with 21 frames (novelty 5; trdm.cn article, 2.2).
 * TEXT:  not rotated (the pages give text no positions). */
typedef struct {
    int32_t kind;          /* mmdit_seg_kind */
    int64_t offset;        /* first token of the segment */
    int64_t count;         /* number of tokens */
    int32_t t0, T, H, W;   /* VIDEO only */
    double t_scale;        /* AUDIO only */
} mmdit_segment;

/* RoPE geometry.  head_dim = d_t + d_h + d_w, each slice even; slices sit in
 * t, h, w order and rotate adjacent pairs (2i, 2i+1) of the slice by angle
 * p_axis * theta^(-2i/d_axis).  With the vectorised kernel every slice width
 * must be a multiple of 8. */
typedef struct {
    int32_t heads, head_dim;
    int32_t d_t, d_h, d_w;
    double theta;
    const mmdit_segment* segs;
    int32_t n_segs;        /* 1 .. MMDIT_MAX_SEGMENTS, non-overlapping */
    int64_t n_tokens;      /* tokens in the Q / K buffers */
} mmdit_rope_desc;

/* Block-sparse geometry (Prism page, "Ideas clave" and "Metodo" section 3):
 * macro-zones zone[3] = {Z_T, Z_H, Z_W} cut into uniform blocks block[3];
 * blocks are numbered zone by zone in raster order, raster inside a zone.
 * Each query block keeps the longer of its top_k most probable key blocks and
 * the smallest probability-ordered prefix whose mass reaches top_p (ties go
 * to the lower block id). */
typedef struct {
    int32_t zone[3];
    int32_t block[3];
    int32_t top_k;         /* >= 0 */
    double top_p;          /* in [0, 1]; >= 1 keeps every block */
    int32_t wait_limit;    /* 0 (use this): the default bound of the attention
                              kernel's internal waits, 2^18 sleeps of about 64
                              cycles.  1 .. 2^18 lowers it, for tests of the
                              failure path: a wait that reaches the bound gives
                              up, and the rows of the query blocks its workgroup
                              serves (o rows, lse entries) are written as NaN. */
} mmdit_sparse_desc;

/* ---- host-only calls (no GPU needed) ------------------------------------- */

int32_t mmdit_abi_version(void);

/* Text of the calling thread's last non-OK status ("" if none).  The pointer
 * stays valid until the thread's next failing library call. */
const char* mmdit_last_error(void);

/* Number of floats the RoPE table for `desc` needs, or 0 if desc is invalid. */
size_t mmdit_rope3d_table_floats(const mmdit_rope_desc* desc);

/* Fill `host_table` (mmdit_rope3d_table_floats(desc) floats, caller-owned host
 * memory) with (cos, sin) pairs: angles in fp64, rounded to fp32.  Per segment
 * in order: VIDEO -> [T][d_t/2] then [H][d_h/2] then [W][d_w/2] pairs for
 * positions t0.., 0.., 0..; AUDIO -> [count][d_t/2] pairs for j * t_scale;
 * TEXT -> nothing.  The caller copies the table to device memory. */
mmdit_status mmdit_rope3d_build_table(const mmdit_rope_desc* desc, float* host_table);

/* Workspace bytes `op` needs for these sizes (0 if none).  JOINT_ATTN: n_q, n_kv
 * as in mmdit_joint_attn (also for mmdit_joint_attn_fwd).  JOINT_ATTN_BWD: as
 * in mmdit_joint_attn_bwd.  AV_CROSS_ATTN: n_q = n_video, n_kv = n_audio.
 * BLOCK_SPARSE_ATTN and BLOCK_SPARSE_ATTN_BWD: n_q = n_kv = T*H*W and `sp`
 * gives the block geometry.  BLOCK_SPARSE_ATTN_ADAPTIVE and
 * BLOCK_SPARSE_ATTN_ADAPTIVE_BWD: n_q = T*H*W; n_kv, dtype and `sp` are not
 * read. */
size_t mmdit_workspace_bytes(int32_t op, int64_t n_q, int64_t n_kv, int32_t heads,
                             int32_t head_dim, int32_t dtype, const mmdit_sparse_desc* sp);

/* Host-side tile table of a content-adaptive grid (see
 * mmdit_block_sparse_attn_adaptive for the tiling): for the zone shape codes
 * zone_shape [T*H*W/512] (host memory, a forward call's output copied back),
 * tile s (nt = T*H*W/64 tiles) holds the tokens tile_base[s] + offset(r),
 * r = 0..63 in raster order over a box of 2^(d & 3) x 2^((d >> 2) & 3) x
 * 2^((d >> 4) & 3) tokens along (t, h, w), d = tile_dims[s], offset(r) =
 * (a*H + b)*W + c for the box coordinates (a, b, c) of r; tile_block[s] is the
 * tile's block.  The same arithmetic the library's kernels use.  Output arrays
 * are host memory of nt entries and may be NULL.  T, H, W must be multiples
 * of 8; codes above 15 are rejected. */
mmdit_status mmdit_adaptive_tile_table(int32_t T, int32_t H, int32_t W, const uint8_t* zone_shape,
                                       int32_t* tile_base, uint8_t* tile_dims, int32_t* tile_block);

/* ---- device calls (async on `stream`) ------------------------------------- */

/* Time-shifted 3D RoPE, in place on q and k ([n_tokens][heads][head_dim]).
 * Sources: SkyReels-V4 analysis (paper.rainbus.top 2602.21818), workflow step 1,
 * novelties 4 and 5; trdm.cn SkyReels-V4 article, section 2.2.
 * dev_table: device copy of mmdit_rope3d_build_table's output for `desc`.
 * Math is fp32 on the stored values; bf16 results are rounded to nearest even.
 * Tokens outside every VIDEO/AUDIO segment are neither read nor written. */
mmdit_status mmdit_rope3d(const mmdit_rope_desc* desc, const float* dev_table,
                          void* q, void* k, int32_t dtype, void* stream);

/* O[i] = sum_j softmax_j(softmax_scale * <q_i, k_j>) v_j per head, no mask.
 * Sources: SkyReels-V4 analysis, workflow step 3 (joint self-attention over
 * video/audio and text tokens; video queries text embeddings); trdm.cn
 * article, section 2.1.  Joint self-attention passes the same concatenated
 * [cond|video|audio|text] buffer as q, k and v with n_q = n_kv; video->text
 * passes video queries and text keys.
 * q [n_q][heads][head_dim], k and v [n_kv][heads][head_dim] in `dtype`,
 * o [n_q][heads][head_dim] fp32.  head_dim 64 or 128.  bf16: Q K^T on bf16
 * matrix cores, fp32 online softmax, P V on fp16 matrix cores (P in (0, 2^8]
 * rounded to fp16; V scaled per head by a power of two 2^e that puts its
 * largest magnitude in [2^14, 2^15), so its conversion is exact for every
 * entry within 2^-28 of that maximum and nothing overflows; O is scaled back
 * by 2^-e), fp32 accumulation; fp32: fp32 throughout.  n_q >= 0 (0 is a
 * no-op), n_kv >= 1. */
mmdit_status mmdit_joint_attn(const void* q, int64_t n_q, const void* k, const void* v,
                              int64_t n_kv, int32_t heads, int32_t head_dim, int32_t dtype,
                              float softmax_scale, float* o, void* ws, size_t ws_bytes,
                              void* stream);

/* Bytes of the per-GPU scratch array of mmdit_joint_attn_noalloc (64 MiB). */
#define MMDIT_NOALLOC_SCRATCH_BYTES (64u << 20)

/* mmdit_joint_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and output, bit for bit, with the workspace taken from
 * a fixed scratch array of MMDIT_NOALLOC_SCRATCH_BYTES that the library's
 * code object holds on each GPU it runs on until the process ends.  The call
 * allocates and frees nothing.  Sizes whose workspace
 * (mmdit_workspace_bytes(MMDIT_OP_JOINT_ATTN, ...)) exceeds the scratch are
 * rejected with MMDIT_ERR_WORKSPACE before anything is enqueued: with 24 heads
 * of 128 that is up to about 10900 keys (the 5850-token joint block, the
 * video->text and video->audio shapes).  The first call on a device looks up
 * the array's address there (the calling thread's current device, which must
 * own `stream`).  Every call on a GPU shares its one array, and nothing in it
 * needs to start cleared: calls that overlap on one GPU (concurrent streams,
 * threads) race and give wrong results; serialise them.  Arguments as for
 * mmdit_joint_attn. */
mmdit_status mmdit_joint_attn_noalloc(const void* q, int64_t n_q, const void* k, const void* v,
                                      int64_t n_kv, int32_t heads, int32_t head_dim, int32_t dtype,
                                      float softmax_scale, float* o, void* stream);

/* The joint self-attention of one dual-stream block with its RoPE fused in:
 * o = mmdit_joint_attn(R(q), R(k), v) where R is mmdit_rope3d's rotation for
 * `desc` (n_q = n_kv = desc->n_tokens, heads and head_dim from desc), and the
 * rotated tensors themselves, bit for bit those mmdit_rope3d writes, in q_rot
 * and k_rot for the block's audio<->video cross-attention.  Sources:
 * SkyReels-V4 analysis, workflow steps 1 and 3 (time-shifted 3D RoPE of the
 * video/audio tokens, then joint self-attention and the cross-attentions in
 * every block); trdm.cn article, sections 2.1-2.2.
 * The fusion: the pass that stages V for the P V products also rotates K and
 * writes it to k_rot (or the workspace), and the attention kernel rotates
 * each Q row in registers as it loads it (storing it to q_rot), so the
 * separate RoPE pass and one read of Q disappear.
 * q, k, v [n_tokens][heads][head_dim] bf16 (unrotated q and k are left
 * unchanged), o fp32; q_rot, k_rot bf16 of the same shape, 16-byte aligned,
 * each either NULL (not wanted) or disjoint from q, k, v, o, each other and
 * the workspace.  dev_table: the device copy of mmdit_rope3d_build_table's
 * output for desc.  bf16 only (MMDIT_ERR_UNSUPPORTED for fp32).  Workspace:
 * mmdit_workspace_bytes(MMDIT_OP_JOINT_ATTN_ROPE, n_tokens, n_tokens, heads,
 * head_dim, MMDIT_BF16, NULL). */
mmdit_status mmdit_joint_attn_rope(const mmdit_rope_desc* desc, const float* dev_table, const void* q,
                                   const void* k, const void* v, int32_t dtype, float softmax_scale, float* o,
                                   void* q_rot, void* k_rot, void* ws, size_t ws_bytes, void* stream);

/* mmdit_joint_attn for a training step: the same output o, plus
 * lse [heads][n_q] fp32, the natural log of sum_j exp(softmax_scale * <q_i, k_j>)
 * per head and query, which mmdit_joint_attn_bwd takes to rebuild the
 * attention probabilities.  Sources: SkyReels-V4 analysis, workflow step 4
 * (the joint model is trained with a flow-matching objective); Prism page,
 * "Resultados" (training-step time of the attention at 2K).  Arguments and
 * workspace as in mmdit_joint_attn; lse is caller-owned device memory,
 * 4-byte aligned, and must not alias o or an input (may be NULL only when
 * n_q == 0). */
mmdit_status mmdit_joint_attn_fwd(const void* q, int64_t n_q, const void* k, const void* v,
                                  int64_t n_kv, int32_t heads, int32_t head_dim, int32_t dtype,
                                  float softmax_scale, float* o, float* lse, void* ws, size_t ws_bytes,
                                  void* stream);

/* Gradients of O = softmax(softmax_scale * Q K^T) V per head (sources as for
 * mmdit_joint_attn_fwd).  With P the attention probabilities, rebuilt from q,
 * k and lse, and d_o the gradient of the loss with respect to O:
 *   dv = P^T d_o,  dS = P o (d_o v^T - D),  D_i = <d_o_i, o_i>,
 *   dq = softmax_scale * dS k,  dk = softmax_scale * dS^T q.
 * q, k, v, n_q, n_kv, heads, head_dim, dtype and softmax_scale as passed to
 * mmdit_joint_attn_fwd; o [n_q][heads][head_dim] fp32 and lse [heads][n_q]
 * fp32 are its outputs; d_o [n_q][heads][head_dim] in `dtype`.
 * dq [n_q][heads][head_dim], dk and dv [n_kv][heads][head_dim] fp32, written
 * (not accumulated), must not overlap each other or any input.  bf16: the
 * five products on bf16 matrix cores (P and dS rounded to bf16) with fp32
 * accumulation; fp32: fp32 throughout.  n_q == 0 gives dk = dv = 0.
 * Deterministic: the same inputs give bitwise the same gradients.
 * Workspace: mmdit_workspace_bytes(MMDIT_OP_JOINT_ATTN_BWD, ...). */
mmdit_status mmdit_joint_attn_bwd(const void* q, int64_t n_q, const void* k, const void* v,
                                  int64_t n_kv, int32_t heads, int32_t head_dim, int32_t dtype,
                                  float softmax_scale, const float* o, const float* lse, const void* d_o,
                                  float* dq, float* dk, float* dv, void* ws, size_t ws_bytes, void* stream);

/* Both directions of the audio<->video cross-attention of one block.
 * Sources: SkyReels-V4 analysis, workflow step 3 and novelty 2 (bidirectional
 * audio-video cross-attention in every layer); trdm.cn article, section 2.2.
 * o_video[n_video] = attention(q_v, k_a, v_a)   (video queries, audio keys)
 * o_audio[n_audio] = attention(q_a, k_v, v_v)   (audio queries, video keys)
 * The video side includes conditioning-frame tokens.  Shapes as in
 * mmdit_joint_attn; the two outputs are fp32 and must not alias. */
mmdit_status mmdit_av_cross_attn(const void* q_v, const void* k_v, const void* v_v,
                                 int64_t n_video, const void* q_a, const void* k_a,
                                 const void* v_a, int64_t n_audio, int32_t heads,
                                 int32_t head_dim, int32_t dtype, float softmax_scale,
                                 float* o_video, float* o_audio, void* ws, size_t ws_bytes,
                                 void* stream);

/* Block-sparse video self-attention over a T x H x W raster grid.
 * Source: Prism page (xyznot.com 2610.05416), "Ideas clave" (macro-zones,
 * hybrid top-k/top-p) and "Metodo" section 3 (mean-pooled block
 * representatives, block probabilities, S_i = TopK(P_i,k) u TopP(P_i,p),
 * online-softmax attention over S_i only).
 * Steps: fp64 block means of Q and K; fp64 logits <Qbar_i, Kbar_j> *
 * softmax_scale (taken as double: the selection is decided in fp64) and their
 * row softmax P_i; selection as described for
 * mmdit_sparse_desc; attention of every query over the tokens of its block's
 * selected key blocks.
 * q, k, v [T*H*W][heads][head_dim] bf16; o same shape fp32.
 * sel_mask [heads][nb][ceil(nb/32)] uint32: bit j%32 of word j/32 set iff key
 * block j is selected; sel_count [heads][nb] int32 = number of selected blocks.
 * Either may be NULL if not wanted.  T, H, W must be multiples of the zone,
 * the zone of the block; block volume 64; head_dim 128; at most 32768 blocks
 * per head (MMDIT_ERR_UNSUPPORTED beyond).
 * The attention kernel's internal waits are bounded (sp->wait_limit): a wait
 * that times out never hangs the call; the rows of the query blocks its
 * workgroup serves come out as NaN, never as plausible wrong values.  The same
 * holds for every block-sparse forward call below (the adaptive call uses the
 * default bound).
 * V enters the P V products as fp16 after a per-head power-of-two prescale
 * (exact; no range limit on V), as in mmdit_joint_attn. */
mmdit_status mmdit_block_sparse_attn(const void* q, const void* k, const void* v, int32_t T,
                                     int32_t H, int32_t W, int32_t heads, int32_t head_dim,
                                     const mmdit_sparse_desc* sp, double softmax_scale, float* o,
                                     uint32_t* sel_mask, int32_t* sel_count, void* ws,
                                     size_t ws_bytes, void* stream);

/* mmdit_block_sparse_attn for a training step: the same o and selection, plus
 * lse [heads][T*H*W] fp32, the natural log of sum_j exp(softmax_scale *
 * <q_i, k_j>) over the keys of the query's selected blocks.  Sources: Prism
 * page, "Metodo" section 3 (attention over S_i only) and "Resultados"
 * (training-step time of the sparse attention at 2K).  sel_mask is required
 * here: mmdit_block_sparse_attn_bwd takes it.  Other arguments and workspace
 * as in mmdit_block_sparse_attn; lse is 4-byte aligned and aliases nothing. */
mmdit_status mmdit_block_sparse_attn_fwd(const void* q, const void* k, const void* v, int32_t T, int32_t H,
                                         int32_t W, int32_t heads, int32_t head_dim, const mmdit_sparse_desc* sp,
                                         double softmax_scale, float* o, float* lse, uint32_t* sel_mask,
                                         int32_t* sel_count, void* ws, size_t ws_bytes, void* stream);

/* Per-token Euclidean norms: out[t] = sqrt(sum_c x[t][c]^2) for t < n, x fp32
 * [n][width] (width a multiple of 4, x 16-byte aligned), out fp32 [n], fp32
 * sums.  Source: Prism page, "Metodo" section 1 (a = ||h_hat||_2 of the
 * audio->video cross-attention output, cached for the next layer's block
 * shapes); with x = the o_video of mmdit_av_cross_attn ([n_video][heads *
 * head_dim]) it gives that layer's a_norm for mmdit_block_sparse_attn_adaptive.
 * n == 0 does nothing; out must not overlap x. */
mmdit_status mmdit_token_norms(const float* x, int64_t n, int64_t width, float* out, void* stream);

/* Block-sparse video self-attention with content-adaptive 3D block shapes.
 * Sources: Prism page (xyznot.com 2610.05416), "Ideas clave" (8x8x8
 * macro-zones, dual-guidance variation indicator, 16 candidate shapes of 64,
 * 128 or 256 tokens) and "Metodo" sections 1-3.
 * Per zone m, in fp64: sigma2_d = mean over the heads*head_dim channels of the
 * variance, over the 8 positions along axis d, of the mean of v over the
 * other two axes; E = sum_d sigma2_d; rho = E / max_m E; the volume B is 64 if
 * rho >= 0.5, 128 if rho >= 0.25, else 256; abar = (zone mean of a_norm) / (its
 * largest zone mean); r_d and vhat_d are the shares of sigma2_d and of the same
 * directional variance of a_norm (0 for a zero total); g_d = r_d + abar vhat_d +
 * 1e-6; l*_d = -log2(g_d)/2 + (log2 B + sum log2(g)/2) / 3; the shape is the
 * candidate of volume B nearest to l* (log2 edges, Euclidean, ties to the first
 * in candidate order).  Candidates: the boxes with edges in {2, 4, 8}; code
 * 0..6 volume 64: (2,4,8) (2,8,4) (4,2,8) (4,4,4) (4,8,2) (8,2,4) (8,4,2); 7..12
 * volume 128: (2,8,8) (4,4,8) (4,8,4) (8,2,8) (8,4,4) (8,8,2); 13..15 volume 256:
 * (4,8,8) (8,4,8) (8,8,4), as (b_T, b_H, b_W).
 * Blocks are numbered zone by zone (zones in raster order), in raster order of
 * their position inside the zone; the block means of q and k, the fp64 block
 * probabilities and the top-k / top-p selection over blocks are those of
 * mmdit_block_sparse_attn with these blocks; every query attends to the
 * tokens of its block's selected blocks.
 * Tiles: each zone is 8 tiles of 64 tokens; a block of B tokens is B/64
 * consecutive tiles (the block's longest edge halved, first of t, h, w among
 * equals, once per factor 2; tiles in raster order inside the block).
 * a_norm [T*H*W] fp32: per-token norms of the previous layer's audio->video
 * cross-attention output (mmdit_token_norms), or NULL for no audio guidance.
 * q, k, v [T*H*W][heads][head_dim] bf16; o fp32, lse [heads][T*H*W] fp32 or
 * NULL (as for mmdit_block_sparse_attn_fwd).  Optional outputs (NULL if not
 * wanted): zone_shape [nz] uint8 candidate codes (nz = T*H*W / 512);
 * tile_block [nt] int32 block id of each tile (nt = T*H*W / 64); n_blocks [1]
 * int32 number of blocks; sel_mask [heads][nt][ceil(nt/32)] uint32, row i
 * (tile i) has bit j set iff tile j's block is selected by tile i's block;
 * sel_count [heads][nt] int32 selected blocks of tile i's block.  T, H, W must
 * be multiples of 8, nz <= 4096, head_dim 128.  Workspace:
 * mmdit_workspace_bytes(MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE, T*H*W, 0, heads,
 * head_dim, MMDIT_BF16, NULL). */
mmdit_status mmdit_block_sparse_attn_adaptive(const void* q, const void* k, const void* v, const float* a_norm,
                                              int32_t T, int32_t H, int32_t W, int32_t heads, int32_t head_dim,
                                              int32_t top_k, double top_p, double softmax_scale, float* o,
                                              float* lse, uint8_t* zone_shape, int32_t* tile_block,
                                              int32_t* n_blocks, uint32_t* sel_mask, int32_t* sel_count, void* ws,
                                              size_t ws_bytes, void* stream);

/* Gradients of mmdit_block_sparse_attn_adaptive with its shapes and selection
 * held fixed (both are piecewise constant in the inputs): the gradients of
 * masked softmax attention over the selected tile pairs, as
 * mmdit_block_sparse_attn_bwd states them.  Sources: Prism page, "Metodo"
 * sections 1-3 and "Resultados" (training-step time of the sparse attention).
 * q, k, v, T, H, W, heads, head_dim and softmax_scale as passed to the
 * forward; o and lse (required) are its outputs, zone_shape [T*H*W/512] and
 * sel_mask (tile level) likewise.  d_o [T*H*W][heads][head_dim] bf16; dq, dk,
 * dv fp32, written, 16-byte aligned, overlapping nothing.  The uniform sparse
 * backward's passes run over the forward's 64-token tiles, each tile's tokens
 * found in place in the raster tensors from its first token and shape (a
 * tile table built from zone_shape); nothing is permuted.  Deterministic.
 * Workspace:
 * mmdit_workspace_bytes(MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE_BWD, T*H*W, 0,
 * heads, head_dim, MMDIT_BF16, NULL). */
mmdit_status mmdit_block_sparse_attn_adaptive_bwd(const void* q, const void* k, const void* v, int32_t T, int32_t H,
                                                  int32_t W, int32_t heads, int32_t head_dim, double softmax_scale,
                                                  const float* o, const float* lse, const void* d_o,
                                                  const uint8_t* zone_shape, const uint32_t* sel_mask, float* dq,
                                                  float* dk, float* dv, void* ws, size_t ws_bytes, void* stream);

/* Gradients of the block-sparse attention with its selection held fixed (the
 * selection is piecewise constant in q and k): for every query i and key j of
 * a selected block pair, P_ij = exp(softmax_scale * <q_i, k_j> - lse_i), and
 * with D_i = <d_o_i, o_i>:
 *   dv_j = sum_i P_ij d_o_i,   dS_ij = P_ij (<d_o_i, v_j> - D_i),
 *   dq_i = softmax_scale * sum_j dS_ij k_j,  dk_j = softmax_scale * sum_i dS_ij q_i,
 * sums over the selected pairs only.  Sources as for
 * mmdit_block_sparse_attn_fwd.  q, k, v, T, H, W, heads, head_dim, sp (its
 * zone and block geometry) and softmax_scale as passed to the forward; o,
 * lse and sel_mask are its outputs; d_o [T*H*W][heads][head_dim] bf16.  dq,
 * dk, dv [T*H*W][heads][head_dim] fp32, written (not accumulated), 16-byte
 * aligned, must not overlap each other or any input.  bf16 products with
 * fp32 accumulation; deterministic.  Workspace:
 * mmdit_workspace_bytes(MMDIT_OP_BLOCK_SPARSE_ATTN_BWD, ...). */
mmdit_status mmdit_block_sparse_attn_bwd(const void* q, const void* k, const void* v, int32_t T, int32_t H,
                                         int32_t W, int32_t heads, int32_t head_dim, const mmdit_sparse_desc* sp,
                                         double softmax_scale, const float* o, const float* lse, const void* d_o,
                                         const uint32_t* sel_mask, float* dq, float* dk, float* dv, void* ws,
                                         size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MMDIT_H */
