// Internal declarations of the CSA2 gfx950 library: kernel parameter blocks, launchers
// and small device helpers.  Not part of the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// Start/stop events that the next kernel launch records itself (null = none): set by the
// host-side timing wrapper around a launcher while kernel timing is on.
extern thread_local hipEvent_t g_launch_events[2];
#define CSA2_LAUNCH(kernel, grid, block, stream, ...)                                        \
  hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ::csa2::g_launch_events[0],        \
                        ::csa2::g_launch_events[1], 0, __VA_ARGS__)

constexpr int kLat = 512;        // latent channels (E2M1 codes, 2 per byte)
constexpr int kLatBytes = 256;
constexpr int kScl = 16;         // E8M0 scale bytes per entry (one per 32 channels)
constexpr int kRope = 64;        // rope channels (bf16)
constexpr int kDq = 576;
constexpr int kDidx = 64;
constexpr int kDswa = 128;
constexpr int kPage = 64;

// ---------------------------------------------------------------- parameter blocks
struct IdxScoreParams {
  int T, H_I, max_pages, chunks;       // chunks = blocks per row
  int64_t key_stride;                  // u32 keys per row in the workspace
  const uint16_t* q_idx;               // [T, H_I, 64]
  const float* w_idx;                  // [T, H_I]
  const uint16_t* k_idx;               // [n_pages*64, 64]
  const int32_t* page_table;
  const int32_t* seq_id;
  const int32_t* n_vis;
  uint32_t* keys;                      // [T, key_stride] order-preserving keys
  uint32_t* clear;                     // optional: words zeroed by the first blocks
  int clear_words;
  uint32_t* trash;                     // row-tiled scoring: 1 KB that masked stores hit
  // pooled scoring (hierarchical indexer): score the 8-entry blocks of the selections
  // pool_sel [T, pool_K] instead of every visible entry; key slot 8i + o = entry o of the
  // block of selection i (chunks then counts workgroups of kPoolSelPerBlock selections)
  const int32_t* pool_sel = nullptr;
  int pool_K = 0;
};

struct TopkParams {
  int T, K;
  int64_t key_stride;
  const uint32_t* keys;
  const int32_t* n_vis;
  int32_t* idx_out;                    // [T, K]
  // chunked path (few long rows): workspace for per-row histograms, per-chunk candidate
  // counts, the digit found, and candidate keys and indices (a segment of kCkKeys per
  // chunk, laid out like the keys); null otherwise
  uint32_t* ck_hist;                   // [T, kCkHistWords]
  uint32_t* ck_counts;                 // [T, n_chunks]
  uint32_t* ck_sel;                    // [T, 8]
  uint32_t* ck_ckey = nullptr;         // [T, key_stride]
  int32_t* ck_cidx = nullptr;          // [T, key_stride]
  // pooled rows: keys are the 8 * pool_K slots of the pooled scoring; the output maps
  // slot 8i + o to entry 8 * (pool_sel[t, i] / 8) + o
  const int32_t* pool_sel = nullptr;
  int pool_K = 0;
};

// Top-K over few long rows runs chunked: rows longer than 65536 keys with at most
// kCkMaxRows rows are split into 4096-key chunks, one workgroup each (rows of at most
// kCkMaxChunks chunks).
constexpr int kCkKeys = 4096;
constexpr int kCkHistWords = 4096;
constexpr int kCkMaxRows = 64;
constexpr int kCkMaxChunks = 4096;
inline bool topk_chunked(int T, int64_t key_stride) {
  return key_stride > 65536 && T <= kCkMaxRows;
}
__host__ __device__ inline int64_t topk_chunks(int64_t key_stride) { return (key_stride + kCkKeys - 1) / kCkKeys; }

struct AttnParams {
  int T, H, K, max_pages, splits, per_split;   // per_split: idx slots per split
  int fmt = 0;                                  // 0: E8M0 per 32; 1: E4M3 per 16
  float sm_scale_log2;                          // sm_scale * log2(e)
  const uint16_t* q;                            // [T, H, 576]
  const uint8_t* kv_lat;
  const uint8_t* kv_scl;
  const uint16_t* kv_rope;
  const int32_t* page_table;
  const int32_t* seq_id;
  const int32_t* idx;                           // [T, K]
  float* o;                                     // final [T, H, 512] when splits == 1
  float* lse;
  float* o_part;                                // [T, splits, H, 512] when splits > 1
  float* lse_part;                              // [T, splits, H]
};

struct MergeParams {
  int T, H, splits;
  const float* o_part;
  const float* lse_part;
  float* o;
  float* lse;
};

struct SwaParams {
  int T, H, H_kv, L_swa;
  float sm_scale_log2;
  const uint16_t* q_swa;               // [T, H, 128]
  const uint16_t* k;                   // [B, L_swa, H_kv, 128]
  const uint16_t* v;
  const int32_t* seq_id;
  const int32_t* start;
  const int32_t* len;
  float* o;                            // [T, H, 128]
  float* lse;                          // [T, H]
  int wgs = 0;                         // > 0: that many one-per-CU workgroups (decode rows,
                                       // H == H_kv); 0: one per (row, KV head)
};

struct QuantParams {
  int64_t rows;
  const float* x;                      // [rows, 512]
  uint8_t* lat;
  uint8_t* scl;
  const int64_t* dst_row;              // may be null
};

struct AppendParams {
  int64_t n;                           // entries
  const float* c;                      // [n, 4, 576] token projections C
  const float* z;                      // [n, 4, 576] pooling logits Z
  const float* c_idx;                  // [n, 4, 64] or null
  const float* z_idx;                  // [n, 4, 64] or null
  const int64_t* dst_row;              // [n] physical rows, or null = 0..n-1
  uint8_t* lat;                        // [*, 256]
  uint8_t* scl;                        // [*, 16]
  uint16_t* rope;                      // [*, 64] bf16
  uint16_t* k_idx;                     // [*, 64] bf16, or null
};

// ---------------------------------------------------------------- launch geometry
constexpr int kIdxChunk = 2048;        // entries scored per workgroup (whole pages)
constexpr int kIdxGemmMinRows = 256;   // from this many rows, scoring runs row-tiled
static_assert(kCkMaxRows < kIdxGemmMinRows, "row-tiled scoring reuses the chunked Top-K area");
constexpr int kSwaTileMinRows = 256;   // from this many rows, SWA runs row-tiled on MFMA
constexpr int kTopkThreads = 1024;
constexpr int kPoolBlock = 8;          // entries per pool block (aligned)
constexpr int kPoolMaxSel = 2048;      // selections that may seed a pool
constexpr int kPoolMaxK = 8192;        // Top-K size over a pool (staged in LDS)
constexpr int kPoolSelPerWave = 32;    // selections per wave of the pooled scoring
constexpr int kPoolSelPerBlock = 4 * kPoolSelPerWave;   // per workgroup (4 waves)
inline int64_t pool_key_stride(int pool_K) { return ((int64_t)kPoolBlock * pool_K + 63) / 64 * 64; }

// Split plan of the attention launch: `splits` workgroups per row, each covering
// `per_split` (a multiple of 32, <= 2048) consecutive index slots, sized to fill `cus`
// CUs (a smaller budget never gives more splits).
constexpr int kNumCus = 256;
void attn_plan(int T, int H, int K, int* splits, int* per_split, int cus = kNumCus);

// The SWA branch beside the global one, for decode rows with H == H_kv: this many
// persistent one-per-CU workgroups (16 (row, KV head) units in flight each), or 0 for the
// one-workgroup-per-unit launch.  The attention beside it is planned for the other CUs.
constexpr int kSwaPMaxWgs = 128;
inline int swa_persist_wgs(int T, int H, int H_kv) {
  if (T <= 0 || T >= kSwaTileMinRows || H != H_kv) return 0;
  const int64_t w = ((int64_t)T * H_kv + 15) / 16;
  return (int)(w < kSwaPMaxWgs ? w : kSwaPMaxWgs);
}
// 64-head workgroups per (row, split) of the sparse attention kernel
inline int attn_head_groups(int H) { return H > 64 ? H / 64 : 1; }

// ---------------------------------------------------------------- launchers
// Each launcher enqueues one kernel on `s` and returns hipGetLastError().
hipError_t launch_idx_score(const IdxScoreParams& p, hipStream_t s);
hipError_t launch_topk(const TopkParams& p, hipStream_t s);
hipError_t launch_topk_chunked(const TopkParams& p, int pass, hipStream_t s);
hipError_t launch_sparse_attn(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_swa(const SwaParams& p, hipStream_t s);
hipError_t launch_quantize(const QuantParams& p, hipStream_t s);
hipError_t launch_kv_append(const AppendParams& p, hipStream_t s);
hipError_t launch_fp4e4m3_quantize(const QuantParams& p, hipStream_t s);

}  // namespace csa2
