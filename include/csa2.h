/*
 * csa2.h -- C ABI of the CSA2 (Compressed Sparse Attention 2) decode/prefill hot path
 * for AMD MI355X (gfx950).
 *
 * What the path computes (sources cited by page and section):
 *   [summary] picx.dev whiteboard summary "DeepSeek-V4.1-Flash: Pushing the Limits of KV
 *             Cache Compression", Methodology > Architecture Components:
 *             item 2 (CSA2: Full / Reindex / Reuse modes), item 5 (FP4 main KV cache);
 *             Introduction (global branch + local sliding-window branch).
 *   [blog]    cyber-feed.org repost of the blog article of the same title, introduction
 *             (sparse attention covering the whole context combined with SWA).
 * Per query row: an indexer scores the visible compressed entries, a Top-K selects a
 * set, the attention gathers the selected entries from an MXFP4 cache (E2M1 codes, one
 * E8M0 scale per 32 channels), dequantizes them in registers and runs softmax attention
 * over them; a bf16 sliding-window branch attends over the last tokens.  Readings of the
 * points the pages leave open (indexer form, scale format, tie-break, branch outputs):
 *   score[t, j] = sum_h w_idx[t, h] * max(0, q_idx[t, h, :] . k_idx[j, :])
 *   Top-K order: descending score, ascending index; output ascending, -1 padded
 *   global key  = [dequant(latent) (512) ; rope (64)], value = dequant(latent) (512),
 *                 shared by all heads; logit = sm_scale * q . key
 *   the two branches are returned separately as (o, lse) pairs.
 *
 * Conventions (all entry points):
 *   - Every call is asynchronous on `stream` (a hipStream_t of the current device;
 *     NULL = the null stream).  No host synchronisation, no device allocation: the caller
 *     owns all memory, including the workspace, whose size csa2_workspace_bytes()
 *     returns.  The SWA branch runs on a library-owned stream of the current device
 *     (one per host thread, created on first use), forked from `stream` and joined back
 *     into it with events before the call returns; work queued on `stream` afterwards
 *     sees every output.  Fork and join are capturable.  For fewer than 256 rows with
 *     H == H_kv the branch runs on persistent workgroups, one per CU, on at most half the
 *     device's CUs (128 on MI355X), and the global branch's attention is planned for the
 *     CUs left (csa2_plan_cus).
 *   - "device" pointers are device memory and must be 16-byte aligned.
 *   - bf16 tensors are raw 16-bit patterns; all layouts are dense row-major.
 *   - Paged caches: 64 entries per page; entry j of sequence b lives in physical row
 *     page_table[b * max_pages + j / 64] * 64 + j % 64 of every per-entry plane.
 *   - Arguments are validated on the host before any HIP call; a failure returns a
 *     status and sets a thread-local message (csa2_last_error) and launches nothing.
 *     Device contents are preconditions, not checked: indices in [0, n_vis) or -1,
 *     page-table entries of visible entries in [0, n_pages), finite inputs.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 3

#define CSA2_D_LAT 512   /* latent channels per entry (MXFP4) */
#define CSA2_D_ROPE 64   /* rope channels per entry (bf16) */
#define CSA2_D_Q 576     /* query head dim of the global branch */
#define CSA2_D_IDX 64    /* indexer query/key dim (bf16) */
#define CSA2_D_SWA 128   /* sliding-window head dim (bf16) */
#define CSA2_PAGE 64     /* entries per page */
#define CSA2_MAX_H_I 16  /* indexer heads */
#define CSA2_MAX_K 65536 /* Top-K size */
/* Main-KV cache formats (kv_format): E2M1 codes (256 B per entry) with
 *   CSA2_KV_MXFP4:     one E8M0 scale per 32 channels (kv_scl [*, 16]; OCP MXFP4), or
 *   CSA2_KV_FP4_E4M3:  one E4M3 scale per 16 channels (kv_scl [*, 32]), the literal
 *                      format of [summary] item 5 (largest magnitude 6 x 448 = 2688). */
#define CSA2_KV_MXFP4 0
#define CSA2_KV_FP4_E4M3 1
/* Main-KV row layout (kv_row_bytes, row_bytes): the byte distance between consecutive cache
 * rows, the same in all three planes (codes, rope, scales).
 *   0: dense planes, each its own array: codes 256 B, rope 128 B, scales 16 B (E8M0) or
 *      32 B (E4M3) per row;
 *   otherwise a multiple of 16, at least the entry's bytes (400 with E8M0 scales, 416 with
 *      E4M3 scales), at most CSA2_MAX_ROW_BYTES: the planes interleave, every entry's three
 *      parts in one row, e.g. kv_lat = base, kv_rope = base + 256, kv_scl = base + 384 with
 *      row bytes 400 (the packed row layout).  The plane pointers must then be 16-byte
 *      aligned, and the caller keeps the three parts of a row apart.
 * With packed rows the attention gathers each selected entry from one row instead of three
 * arrays (one DRAM page rather than three): faster when the picks are scattered and the
 * attention has the whole device, no faster when it shares the memory with other work. */
#define CSA2_MAX_ROW_BYTES 4096

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,        /* a required pointer is NULL */
  CSA2_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  CSA2_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned */
  CSA2_ERR_MODE = 4,        /* bad layer-group schedule or a buffer the mode forbids */
  CSA2_ERR_WORKSPACE = 5,   /* workspace NULL/misaligned or smaller than required */
  CSA2_ERR_UNSUPPORTED = 6, /* valid request this build does not implement */
  CSA2_ERR_HIP = 7          /* a HIP call failed; csa2_last_error has HIP's message */
} csa2_status;

typedef enum {
  CSA2_FULL = 0,
  CSA2_REINDEX = 1,
  CSA2_REUSE = 2,
  CSA2_REINDEX_POOL = 3  /* Reindex that searches the first Full layer's candidate pool */
} csa2_mode;

/* Operation codes for csa2_workspace_bytes. */
enum {
  CSA2_OP_INDEX_TOPK = 1,
  CSA2_OP_SPARSE_ATTN = 2,
  CSA2_OP_LAYER_GROUP = 3,
  CSA2_OP_INDEX_TOPK_POOL = 4
};
#define CSA2_POOL_BLOCK 8      /* entries per candidate-pool block (aligned) */
#define CSA2_POOL_MAX_SEL 2048 /* selections that seed a pool: 2048 blocks x 8 positions */
#define CSA2_POOL_MAX_K 8192   /* Top-K size of a pooled search */

/* Indexer scoring + Top-K ([summary] Architecture Components, item 2: Full and Reindex
 * layers compute fresh Top-K indices from the indexer key).
 * For each row t: scores the entries j < n_vis[t] of sequence seq_id[t], selects
 * min(K, n_vis[t]) of them by (score desc, index asc) and writes them to
 * idx_out[t, 0:K] in ascending order, -1 in the unused tail. */
typedef struct csa2_index_args {
  int32_t T;          /* query rows, >= 0 */
  int32_t B;          /* sequences (rows of page_table), >= 1 */
  int32_t H_I;        /* indexer heads, 1..16 */
  int32_t K;          /* selected entries per row, 1..CSA2_MAX_K */
  int32_t max_pages;  /* page_table row stride; n_vis[t] <= max_pages * 64 */
  int32_t n_pages;    /* physical pages in k_idx */
  const void* q_idx;           /* device bf16 [T, H_I, 64] */
  const float* w_idx;          /* device f32  [T, H_I] */
  const void* k_idx;           /* device bf16 [n_pages, 64, 64] (one 64-d key per entry) */
  const int32_t* page_table;   /* device i32  [B, max_pages] */
  const int32_t* seq_id;       /* device i32  [T], in [0, B) */
  const int32_t* n_vis;        /* device i32  [T], visible entries, 0..max_pages*64 */
  int32_t* idx_out;            /* device i32  [T, K] (output) */
} csa2_index_args;

/* Hierarchical sparse indexer ([summary] Architecture Components, item 3: the first Full
 * layer's selection defines a candidate pool of up to 2,048 blocks x 8 positions, and the
 * later Reindex layers search only that pool, so their cost stops growing with context).
 * Reading of the block: an aligned run of CSA2_POOL_BLOCK entry positions, block b =
 * {8b .. 8b+7}.  For each row t the pool is the union of the blocks that hold an entry of
 * sel[t, 0:K_sel], cut to the n_vis[t] visible entries.  The layer's own indexer (ix.q_idx,
 * ix.w_idx, ix.k_idx, same score as csa2_index_topk) scores every pool entry, and the
 * min(ix.K, pool size) best by (score desc, index asc) go to ix.idx_out[t, 0:ix.K] in
 * ascending order, -1 in the unused tail.  Per row the indexer keys read are at most
 * 8 * K_sel (16,384 entries, 2 MiB at K_sel = 2048), whatever the context length. */
typedef struct csa2_pool_args {
  csa2_index_args ix;          /* the searching layer's indexer, shapes and output; ix.K in
                                  1..CSA2_POOL_MAX_K */
  const int32_t* sel;          /* device i32 [T, K_sel]: the pool-building selection (e.g. a
                                  Full layer's idx_out): entries in [0, n_vis[t]) in strictly
                                  ascending order, then -1 to the end of the row */
  int32_t K_sel;               /* 1..CSA2_POOL_MAX_SEL */
} csa2_pool_args;

/* Sparse global attention over the selected FP4 entries plus the bf16 sliding-window
 * branch ([summary] Architecture Components, items 2 and 5; Introduction).
 * Global branch, per row t and head h (entries of sequence seq_id[t]):
 *   logit_j = sm_scale * (q[t,h,0:512] . v_j + q[t,h,512:576] . rope_j),  j in idx[t,:],
 *   v_j = e2m1(code) * 2^(scale - 127)  (low nibble = even channel),
 *   o[t,h,:] = sum_j softmax(logit)_j v_j,  lse[t,h] = log sum_j exp(logit_j);
 *   no valid index: o = 0, lse = -inf.
 * SWA branch (skipped when q_swa is NULL, then every SWA pointer must be NULL):
 *   keys/values at positions [swa_start[t], swa_start[t] + swa_len[t]) of sequence
 *   seq_id[t], KV head h * H_kv / H, logit = sm_scale_swa * q_swa . k;
 *   o_swa = softmax-weighted values (128-d), lse_swa; empty window: 0 / -inf.
 * Numerics: the latent q.k on the MX-scaled fp4 x fp8 matrix path (the bf16 query split
 * into two fp8 parts; CSA2_KV_MXFP4) or in fp16 MFMA with the bf16 query rounded to fp16
 * (CSA2_KV_FP4_E4M3: exact for query magnitudes in [2^-14, 65504]); rope q.k in bf16 MFMA;
 * the probability-value product in fp16 MFMA with fp32 accumulation (dequantized values
 * are exact in fp16 for E8M0 scale bytes 104..140, i.e. |v| <= 49152, and for every E4M3
 * scale -- the pages bound KV magnitudes by ~22.6); softmax and outputs in fp32. */
typedef struct csa2_attn_args {
  int32_t T;          /* query rows */
  int32_t B;          /* sequences */
  int32_t H;          /* query heads: 16, 32, 64 or 128 */
  int32_t K;          /* index slots per row, 1..CSA2_MAX_K */
  int32_t max_pages;
  int32_t n_pages;
  const void* q;               /* device bf16 [T, H, 576] */
  const uint8_t* kv_lat;       /* device u8   [n_pages, 64, 256] E2M1 codes */
  const uint8_t* kv_scl;       /* device u8   [n_pages, 64, 16]  E8M0 scales */
  const void* kv_rope;         /* device bf16 [n_pages, 64, 64] */
  const int32_t* page_table;   /* device i32  [B, max_pages] */
  const int32_t* seq_id;       /* device i32  [T] */
  const int32_t* idx;          /* device i32  [T, K] entry indices or -1 */
  float sm_scale;              /* logit scale, e.g. 1/sqrt(576) */
  float* o;                    /* device f32 [T, H, 512] (output) */
  float* lse;                  /* device f32 [T, H]      (output, natural log) */
  /* sliding-window branch */
  int32_t H_kv;                /* SWA KV heads, H % H_kv == 0, H / H_kv <= 8 */
  int32_t L_swa;               /* SWA buffer positions per sequence */
  const void* q_swa;           /* device bf16 [T, H, 128] or NULL */
  const void* swa_k;           /* device bf16 [B, L_swa, H_kv, 128] */
  const void* swa_v;           /* device bf16 [B, L_swa, H_kv, 128] */
  const int32_t* swa_start;    /* device i32 [T] */
  const int32_t* swa_len;      /* device i32 [T], window length, start+len <= L_swa */
  float sm_scale_swa;          /* e.g. 1/sqrt(128) */
  float* o_swa;                /* device f32 [T, H, 128] (output) */
  float* lse_swa;              /* device f32 [T, H]      (output) */
  int32_t kv_format;           /* CSA2_KV_MXFP4 (kv_scl [n_pages, 64, 16]) or
                                  CSA2_KV_FP4_E4M3 (kv_scl [n_pages, 64, 32]) */
  int32_t kv_row_bytes;        /* main-KV row layout: 0 = dense planes, else the bytes
                                  between rows of every plane (see CSA2_MAX_ROW_BYTES) */
} csa2_attn_args;

/* One layer of a Full / Reindex / Reuse group ([summary] Architecture Components,
 * item 2).  Full: own main KV planes + own indexer (q_idx, w_idx, k_idx) -> idx_out.
 * Reindex: main KV of the nearest preceding Full layer, own indexer -> idx_out.
 * Reuse: main KV of the nearest preceding Full layer and the indices of the nearest
 * preceding Full/Reindex layer; it must leave every indexer/KV/idx_out field NULL.
 * Reindex-pool: a Reindex layer whose Top-K searches only the candidate pool of layer 0's
 * selection (see csa2_index_topk_pool; needs K <= CSA2_POOL_MAX_SEL).
 * Every layer has its own q, SWA caches and outputs. */
typedef struct csa2_layer_desc {
  int32_t mode;                /* csa2_mode */
  const void* q;               /* bf16 [T, H, 576] */
  const void* q_swa;           /* bf16 [T, H, 128] or NULL (then no SWA for this layer) */
  const void* q_idx;           /* bf16 [T, H_I, 64]  (Full, Reindex) */
  const float* w_idx;          /* f32  [T, H_I]      (Full, Reindex) */
  const void* k_idx;           /* bf16 [n_pages, 64, 64] (Full, Reindex) */
  const uint8_t* kv_lat;       /* Full only */
  const uint8_t* kv_scl;       /* Full only */
  const void* kv_rope;         /* Full only */
  const void* swa_k;           /* bf16 [B, L_swa, H_kv, 128] */
  const void* swa_v;
  int32_t* idx_out;            /* i32 [T, K] (Full, Reindex; output) */
  float* o;                    /* f32 [T, H, 512] */
  float* lse;                  /* f32 [T, H] */
  float* o_swa;                /* f32 [T, H, 128] */
  float* lse_swa;              /* f32 [T, H] */
} csa2_layer_desc;

/* Shapes and per-row metadata shared by the layers of a group. */
typedef struct csa2_group_args {
  int32_t T, B, H, H_I, K, H_kv, L_swa, max_pages, n_pages;
  const int32_t* page_table;   /* [B, max_pages] */
  const int32_t* seq_id;       /* [T] */
  const int32_t* n_vis;        /* [T] */
  const int32_t* swa_start;    /* [T] */
  const int32_t* swa_len;      /* [T] */
  float sm_scale, sm_scale_swa;
  int32_t kv_format;           /* format of every Full layer's main-KV planes */
  int32_t kv_row_bytes;        /* row layout of every Full layer's main-KV planes (as in
                                  csa2_attn_args) */
} csa2_group_args;

/* Indexer scoring + Top-K.  Workspace: csa2_workspace_bytes(CSA2_OP_INDEX_TOPK, a).
 * CSA2_ERR_UNSUPPORTED: at most 64 rows with max_pages * 64 above 16,777,216 entries (few
 * long rows are split into 4096-entry chunks, at most 4096 of them per row). */
csa2_status csa2_index_topk(const csa2_index_args* a, void* ws, size_t ws_bytes, void* stream);

/* Hierarchical-indexer search of a candidate pool (scoring + Top-K over the pool).
 * Workspace: csa2_workspace_bytes(CSA2_OP_INDEX_TOPK_POOL, a). */
csa2_status csa2_index_topk_pool(const csa2_pool_args* a, void* ws, size_t ws_bytes,
                                 void* stream);
/* Sparse FP4 global attention + SWA.  Workspace: csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, a)
 * (may be 0, then ws may be NULL). */
csa2_status csa2_sparse_attn_fp4(const csa2_attn_args* a, void* ws, size_t ws_bytes,
                                 void* stream);

/* A Full/Reindex/Reuse layer group, layers run in order on `stream`; L[0] must be Full.
 * Workspace: csa2_workspace_bytes(CSA2_OP_LAYER_GROUP, g). */
csa2_status csa2_layer_group(const csa2_layer_desc* L, int32_t n_layers,
                             const csa2_group_args* g, void* ws, size_t ws_bytes,
                             void* stream);

/* The layer group without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, semantics, kernels and results as csa2_layer_group; the
 * workspace is instead a fixed array of CSA2_NOALLOC_SCRATCH_BYTES in the library's device
 * code, one per device, held until the process ends.  The first call on a device (with it
 * current) takes the array's address and makes the device's side stream; after that no
 * call allocates anything.  Errors: CSA2_ERR_WORKSPACE when the group needs more workspace
 * than the array holds (csa2_workspace_bytes(CSA2_OP_LAYER_GROUP, g) above the limit: every
 * decode group of up to 64 rows x 32,768 entries, 32 x 65,536 or 4 x 262,144 fits; a
 * 4096-row prefill does not), CSA2_ERR_HIP when the set-up fails; otherwise as
 * csa2_layer_group.  All calls on one device share its array (and its side stream), whose
 * contents persist between calls: calls that overlap on one device, from several host
 * threads or streams, race and must be serialized by the caller. */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
csa2_status csa2_layer_group_noalloc(const csa2_layer_desc* L, int32_t n_layers,
                                     const csa2_group_args* g, void* stream);

/* MXFP4 cache write ([summary] Architecture Components, item 5): quantizes `rows` fp32
 * latent rows x [rows, 512] into physical rows dst_row[r] of the planes
 * lat [*, 256] and scl [*, 16] (OCP MX: shared exponent floor(log2 max|x|) - 2 over each
 * 32-channel block, clamped to [-127, 127]; elements rounded to E2M1 to nearest, ties to
 * the even code, saturating at 6; sign kept on zeros).  dst_row NULL = rows 0..rows-1.
 * row_bytes: the row layout of lat and scl (0 = dense planes; see CSA2_MAX_ROW_BYTES);
 * only the codes and scale bytes of the written rows change.  Inputs must be finite. */
csa2_status csa2_mxfp4_quantize(const float* x, int64_t rows, uint8_t* lat, uint8_t* scl,
                                const int64_t* dst_row, int32_t row_bytes, void* stream);

/* KV append: one compressed cache entry from each block of CSA2_APPEND_TOKENS raw tokens,
 * written straight into the paged cache planes (a Full layer computing its own KV:
 * [summary] Architecture Components, item 1, Eq. 1 -- the global KV entries are projections
 * C = H W^KV with companion projections Z = H W^Z -- and item 2; [card] block-based
 * sequence compression; 4:1 compression).  The pages print no pooling formula; the reading
 * here, per channel ch of entry e over its block's tokens i:
 *   y[e, ch] = sum_i softmax_i(z[e, i, ch]) * c[e, i, ch]
 * computed in fp32.  Channels 0..511 of y are written as MXFP4 to kv_lat/kv_scl (the
 * csa2_mxfp4_quantize rule), channels 512..575 as bf16 (round to nearest even) to kv_rope;
 * with c_idx, the 64-d indexer key is pooled the same way and written as bf16 to k_idx.
 * Inputs must be finite.  Rows dst_row[e] (NULL = 0..n-1) of every written plane are
 * overwritten; distinct entries must have distinct rows. */
#define CSA2_APPEND_TOKENS 4
typedef struct csa2_append_args {
  int64_t n;                   /* entries, >= 0 */
  const float* c;              /* device f32 [n, 4, 576] token projections (latent ; rope) */
  const float* z;              /* device f32 [n, 4, 576] pooling logits */
  const float* c_idx;          /* device f32 [n, 4, 64] indexer-key projections, or NULL */
  const float* z_idx;          /* device f32 [n, 4, 64] their logits; NULL iff c_idx is */
  const int64_t* dst_row;      /* device i64 [n] physical cache rows, or NULL */
  uint8_t* kv_lat;             /* device u8   [rows, 256] (output) */
  uint8_t* kv_scl;             /* device u8   [rows, 16]  (output) */
  void* kv_rope;               /* device bf16 [rows, 64]  (output) */
  void* k_idx;                 /* device bf16 [rows, 64]  (output); NULL iff c_idx is */
  int32_t kv_row_bytes;        /* row layout of kv_lat, kv_scl and kv_rope (as in
                                  csa2_attn_args; MXFP4 scales) */
} csa2_append_args;
csa2_status csa2_kv_append(const csa2_append_args* a, void* stream);
/* Cache write in the CSA2_KV_FP4_E4M3 format ([summary] item 5, literal reading): rows
 * x [rows, 512] -> lat [*, 256] (as csa2_mxfp4_quantize) and scl [*, 32], one E4M3 byte per
 * 16 channels: s = E4M3(max|x| / 6), to nearest with ties to the even significand,
 * saturating at 448; each element |x| / s rounded to E2M1 (ties to the even code,
 * saturating at 6), sign kept; a scale that rounds to 0 gives (signed) zero codes.
 * dst_row and row_bytes (at least 416 when not 0) as for csa2_mxfp4_quantize.  Inputs
 * must be finite. */
csa2_status csa2_fp4e4m3_quantize(const float* x, int64_t rows, uint8_t* lat, uint8_t* scl,
                                  const int64_t* dst_row, int32_t row_bytes, void* stream);
/* Workspace bytes for an operation; args points to the op's argument struct
 * (csa2_index_args, csa2_attn_args, csa2_group_args or csa2_pool_args).  Returns 0 for
 * NULL args. */
size_t csa2_workspace_bytes(int32_t op, const void* args);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* csa2_last_error(void);
const char* csa2_status_string(csa2_status s);
int32_t csa2_abi_version(void);

/* Compute units of the current device that the launch plans (attention splits, the SWA
 * branch's persistent workgroups) and therefore csa2_workspace_bytes assume: queried once
 * per device (hipDeviceAttributeMultiprocessorCount) and cached for the process; 256 (one
 * MI355X) when no device can be queried.  Size a workspace with the device current that
 * the call will run on. */
int32_t csa2_plan_cus(void);

/* Kernel timing: while enabled, every kernel launch of the library records a start and a
 * stop event itself (hipExtLaunchKernel), and the elapsed time accumulates per kernel
 * name; the SWA branch then runs on the caller's stream after the global branch, so that
 * kernels do not overlap.  csa2_timing_read synchronizes on the recorded events, returns
 * the number of distinct kernels (at most `max`) with their names (NUL-terminated, 64
 * bytes each), launch counts and total milliseconds, and resets the totals. */
csa2_status csa2_timing_enable(int32_t on);
int32_t csa2_timing_read(char* names_64, int64_t* launches, double* total_ms, int32_t max);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
