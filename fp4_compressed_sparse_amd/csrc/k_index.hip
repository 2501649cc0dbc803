// Indexer scoring and Top-K selection for CSA2 on gfx950.
//
// Score ([summary] = picx.dev whiteboard summary "DeepSeek-V4.1-Flash: Pushing the Limits
// of KV Cache Compression", Methodology > Architecture Components, item 2: Full and Reindex
// layers compute fresh Top-K indices from the indexer key; the scoring form is the
// ReLU-gated multi-head indexer that the pages do not print, one 64-d key per entry):
//   s[t, j] = sum_h w[t, h] * max(0, q_idx[t, h, :] . k_idx[j, :])
// computed as a bf16 MFMA contraction (heads x 64) . (64 x 16 entries) with fp32
// accumulation, streaming each sequence's paged indexer keys once.
//
// Top-K: the K largest scores, ties to the lowest index, emitted in ascending index
// order, -1 padded.  Radix select over order-preserving u32 keys (digits of 12, 12 and
// 8 bits, or a 16-bit first digit in a window under the row maximum) finds the K-th key
// tau and how many keys equal to tau to keep; an ordered block-wide scan then compacts
// the selected indices in index order.  Rows of up to 64K
// entries are read once into registers; few longer rows spread over many workgroups in
// 4096-key chunks; many longer rows are streamed, one workgroup each, through a list of
// candidates above a sampled threshold.
//
// Pooled search (hierarchical indexer, [summary] item 3): the same scoring over the
// aligned 8-entry blocks that hold a Full layer's selection, then the register Top-K over
// those slots.
#include <type_traits>

#include "csa2_internal.h"
#include "csa2_device.h"
#include "csa2_swa_wave.h"

namespace csa2 {

constexpr int kIdxWaves = 4;
constexpr int kIdxPagesPerWave = kIdxChunk / kIdxWaves / kPage;   // pooled scoring, and the
static_assert(kIdxPagesPerWave <= 64, "one page-table entry per lane");   // most per wave

// Keys of one 64-entry page for the MFMA B operands.  MFMA pair u covers entries 16u ..
// 16u+15: in its first operand lane (g, n) holds entry 16u + n, channels [8g, 8g+8), in the
// second the same entry, channels [32+8g, 40+8g) (the query operands use the same channel
// order).  Loaded as is, every load instruction would read 64 bytes of each of 16 rows,
// and the rows' halves would reach HBM as separate 64-byte requests (measured: the decode
// scoring at 5.0 TB/s where a plain read of as many bytes runs at 6.6).  So each
// instruction reads 8 whole rows instead, 1 KB contiguous: instruction 2u rows 16u + e,
// 2u+1 rows 16u + 8 + e (e = n & 7), lane (g, n) taking the 16-byte piece g or 4 + g that
// idx_key_operands needs.  Every row of the page is read, visible or not (a page is whole
// in memory): the scores of rows past the visible count are never stored, and loads
// without a per-lane condition keep the loop free of branches, so that the wait for a page
// leaves the next page's loads in flight (with masked loads the compiler waited for all).
// Streamed once per step: non-temporal.
__device__ __forceinline__ void idx_load_page(const uint16_t* k_idx, int page, int n, int g,
                                              u32x4 (&kb)[8]) {
  const int e = n & 7;
  const int cA = (n < 8) ? g : 4 + g, cB = (n < 8) ? 4 + g : g;
  const uint16_t* pg = k_idx + (int64_t)page * kPage * kDidx;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    kb[2 * u] = ld_global_16_nt(pg + (16 * u + e) * kDidx + 8 * cA);
    kb[2 * u + 1] = ld_global_16_nt(pg + (16 * u + 8 + e) * kDidx + 8 * cB);
  }
}

// The loaded pieces of pair u -> its two MFMA operands.  Lane (g, n) holds, from
// instruction A (rows 16u + e) the piece (row 16u + e, channels 8cA..), from B (row 16u + 8
// + e, channels 8cB..).  First operand: lanes n < 8 keep A, lanes n >= 8 keep B.  Second:
// lane n takes the other instruction's piece of lane n ^ 8 of its 16-lane row (a DPP
// rotation by 8), which holds row 16u + n, channels 32 + 8g.
__device__ __forceinline__ void idx_key_operands(bool lo, const u32x4& a, const u32x4& b,
                                                 u32x4& k0, u32x4& k1) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    k0[d] = lo ? a[d] : b[d];
    const uint32_t y = lo ? b[d] : a[d];
    k1[d] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)y, 0x128, 0xf, 0xf, false);  // row_ror:8
  }
}

// Score one page: MFMA A = q_idx (rows = heads, zero-padded to 16), B = keys (columns =
// entries); the result of group u in lane (g, n) holds heads 4g..4g+3 of entry 16u + n.
// Each lane first sums its own four heads, then a reduce-scatter over the four lane groups
// (v_permlane32_swap pairs groups g and g+2, v_permlane16_swap groups g and g+1) leaves
// lane (g, n) with the whole sum of entry 16g + n, so the page's 64 keys go out in one
// store.
__device__ __forceinline__ float idx_score_64(const u32x4& qa0, const u32x4& qa1,
                                              const float (&w)[4], const u32x4 (&kb)[8],
                                              int n) {
  float su[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    u32x4 k0, k1;
    idx_key_operands(n < 8, kb[2 * u], kb[2 * u + 1], k0, k1);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa0), as_bf16x8(k0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa1), as_bf16x8(k1), acc, 0, 0, 0);
    float s = w[0] * relu_f32(acc[0]);
    s += w[1] * relu_f32(acc[1]);
    s += w[2] * relu_f32(acc[2]);
    s += w[3] * relu_f32(acc[3]);
    su[u] = s;
  }
  // lanes 0..31 (g = 0, 1) gather groups u = 0, 1 from g + 2; lanes 32..63 gather u = 2, 3
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(su[0]), __float_as_uint(su[2]), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(su[1]), __float_as_uint(su[3]), false, false);
  const float ha = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float hb = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  // then each row g keeps group u = g from rows g and g ^ 1
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(ha), __float_as_uint(hb), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// One workgroup scores 4 PPW consecutive pages of one row, each wave a run of PPW whole
// pages.  The wave resolves its pages' physical numbers once (one page-table entry per
// lane, broadcast by shuffle) and keeps the next page's 8 KB of keys in flight while it
// scores the current one; the run's keys are stored at its end.
// PPW pages per wave (8, or 4 when a row set too small to fill the CUs needs more waves).
template <int PPW>
__device__ __forceinline__ void idx_score_block(const IdxScoreParams& p, int blk) {
  constexpr int kPerWave = PPW * kPage;
  static_assert(PPW <= kIdxPagesPerWave, "register budget");
  const int t = blk / p.chunks;
  const int c = blk - t * p.chunks;
  const int nv = p.n_vis[t];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j_begin = (c * kIdxWaves + wave) * kPerWave;
  if (j_begin >= nv) return;                 // wave-uniform; no block barriers below
  const int j_end = min(j_begin + kPerWave, nv);
  const int npages = (j_end - j_begin + kPage - 1) / kPage;
  const int b = p.seq_id[t];
  const int n = lane & 15, g = lane >> 4;

  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages + j_begin / kPage;
  const int my_page = (lane < npages) ? pt[lane] : 0;

  u32x4 qa0 = {0u, 0u, 0u, 0u}, qa1 = {0u, 0u, 0u, 0u};
  if (n < p.H_I) {
    const uint16_t* qp = p.q_idx + ((int64_t)t * p.H_I + n) * kDidx + 8 * g;
    qa0 = ld_global_16(qp);
    qa1 = ld_global_16(qp + 32);
  }
  float w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    w[i] = (h < p.H_I) ? p.w_idx[(int64_t)t * p.H_I + h] : 0.f;
  }
  uint32_t* keys = p.keys + (int64_t)t * p.key_stride + j_begin;

  const int span = j_end - j_begin;           // valid entries of page pi: span - 64*pi
  auto valid_in = [&](int pi) { return min(kPage, span - kPage * pi); };
  // The scores stay in registers until the last page: a store inside the loop would sit
  // among the memory operations that each page's wait counts, so every page would also
  // wait for the previous page's store to be acknowledged.
  // Every wave runs all PPW pages, its last page again in place of those past its run
  // (scores not stored): straight-line code, so each page's wait leaves the next page's
  // loads in flight.
  float sc[PPW];
  u32x4 buf[2][8];
  const int last = npages - 1;
  idx_load_page(p.k_idx, __shfl(my_page, 0), n, g, buf[0]);
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    if (pi + 1 < PPW)
      idx_load_page(p.k_idx, __shfl(my_page, min(pi + 1, last)), n, g, buf[(pi + 1) & 1]);
    sc[pi] = idx_score_64(qa0, qa1, w, buf[pi & 1], n);
  }
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi)
    if (pi < npages && 16 * g + n < valid_in(pi)) keys[kPage * pi + 16 * g + n] = float_key(sc[pi]);
}

// zero a workspace area for the Top-K that follows (every workgroup of the launch takes part)
__device__ __forceinline__ void idx_clear(const IdxScoreParams& p) {
  for (int i = (int)(blockIdx.x * 256 + threadIdx.x); i < p.clear_words; i += (int)gridDim.x * 256)
    p.clear[i] = 0u;
}

template <int PPW>
__global__ __launch_bounds__(256) void idx_score_kernel(IdxScoreParams p) {
  idx_clear(p);
  idx_score_block<PPW>(p, (int)blockIdx.x + p.block0);
}

// The same scoring with a small SWA branch of the same rows in one launch (no second stream,
// so no fork and join events): workgroups 0 .. swa_blocks-1 run the window attention, one
// (row, KV head) unit per wave in turn, and the rest score.  The branch's bytes are a small
// share of the scoring's, so it costs the launch little.
template <int PPW>
__global__ __launch_bounds__(256) void idx_score_swa_kernel(IdxScoreParams p, SwaParams w,
                                                           int swa_blocks) {
  idx_clear(p);
  if ((int)blockIdx.x < swa_blocks) {                // workgroup-uniform
    swa_wave_units<1>(w, (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6), swa_blocks * 4);
    return;
  }
  idx_score_block<PPW>(p, (int)blockIdx.x - swa_blocks + p.block0);
}

// ---------------------------------------------------------------- pooled scoring
// Hierarchical indexer ([summary] Architecture Components, item 3): a Reindex layer scores
// only the candidate pool, the aligned 8-entry blocks that hold the selected entries of
// the Full layer.  The selections of a row are ascending with -1 at the tail, so entries
// sharing a block are neighbours: selection i owns key slots 8i .. 8i+7 of the row, which
// hold the block's scores when i is the first selection in its block and 0 (no candidate)
// otherwise.  Slot order is entry order, so the Top-K's lowest-slot tie-break keeps the
// lowest entry.  Each wave takes kPoolSelPerWave consecutive selections, one per lane
// (block row and visible count resolved once), and scores them in groups of 64 slots; a
// group is scored like a 64-entry page whose rows come 8 at a time from 8 lanes' blocks.
// The next group's 8 KB of keys is in flight while the current one is scored; the keys are
// stored after the last group.
__global__ __launch_bounds__(256) void idx_pool_score_kernel(IdxScoreParams p) {
  const int t = blockIdx.x / p.chunks;
  const int c = blockIdx.x - t * p.chunks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i0 = c * kPoolSelPerBlock + wave * kPoolSelPerWave;   // first of this wave
  if (i0 >= p.pool_K) return;                        // wave-uniform; no block barriers
  const int nv = p.n_vis[t];
  const int b = p.seq_id[t];
  const int n = lane & 15, g = lane >> 4;
  const int32_t* sel = p.pool_sel + (int64_t)t * p.pool_K;
  const int i = i0 + lane;
  const int j = (lane < kPoolSelPerWave && i < p.pool_K) ? sel[i] : -1;
  int prev = __shfl_up(j, 1);
  if (lane == 0) prev = (i0 > 0) ? sel[i0 - 1] : -1;
  const bool first = j >= 0 && j < nv && (prev < 0 || (prev >> 3) != (j >> 3));
  int brow = 0, bvis = 0;        // physical row of the block's entry 0; its visible entries
  if (first) {
    const int blk = j >> 3;
    brow = p.page_table[(int64_t)b * p.max_pages + (blk >> 3)] * kPage + kPoolBlock * (blk & 7);
    bvis = min(kPoolBlock, nv - kPoolBlock * blk);
  }

  u32x4 qa0 = {0u, 0u, 0u, 0u}, qa1 = {0u, 0u, 0u, 0u};
  if (n < p.H_I) {
    const uint16_t* qp = p.q_idx + ((int64_t)t * p.H_I + n) * kDidx + 8 * g;
    qa0 = ld_global_16(qp);
    qa1 = ld_global_16(qp + 32);
  }
  float w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int h = 4 * g + q;
    w[q] = (h < p.H_I) ? p.w_idx[(int64_t)t * p.H_I + h] : 0.f;
  }
  uint32_t* keys = p.keys + (int64_t)t * p.key_stride + kPoolBlock * (int64_t)i0;
  const int ngroups = min(kPoolSelPerWave / 8, (p.pool_K - i0 + 7) / 8);

  // group v, MFMA pair u: column n is entry n & 7 of the block of selection 8v + 2u +
  // (n >> 3) of this wave; as in idx_load_page, instruction 2u reads the block of selection
  // 8v + 2u whole (1 KB) and 2u+1 that of 8v + 2u + 1, idx_key_operands then forms the
  // operands
  auto load_group = [&](int v, u32x4 (&kb)[8]) {
    const int e = n & 7;
    const int cA = (n < 8) ? g : 4 + g, cB = (n < 8) ? 4 + g : g;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sA = 8 * v + 2 * u, sB = sA + 1;
      const int rowA = __shfl(brow, sA) + e, rowB = __shfl(brow, sB) + e;
      kb[2 * u] = ld_global_16(p.k_idx + (int64_t)rowA * kDidx + 8 * cA);
      kb[2 * u + 1] = ld_global_16(p.k_idx + (int64_t)rowB * kDidx + 8 * cB);
    }
  };
  // lane (g, n) holds slot 16g + n of the group: entry n & 7 of selection 8v + 2g + (n >> 3);
  // the keys are stored after the last group (no store among the loads' waits)
  constexpr int kGroups = kPoolSelPerWave / 8;
  float sc[kGroups];
  u32x4 buf[2][8];
  // all kGroups groups, straight-line (a group past the wave's selections reads rows 0..7
  // and is not stored), so that each group's wait leaves the next group's loads in flight
  load_group(0, buf[0]);
#pragma unroll
  for (int v = 0; v < kGroups; ++v) {
    if (v + 1 < kGroups) load_group(v + 1, buf[(v + 1) & 1]);
    sc[v] = idx_score_64(qa0, qa1, w, buf[v & 1], n);
  }
#pragma unroll
  for (int v = 0; v < kGroups; ++v) {
    if (v < ngroups) {
      const bool ok = (n & 7) < __shfl(bvis, 8 * v + 2 * g + (n >> 3));
      keys[64 * v + 16 * g + n] = ok ? float_key(sc[v]) : 0u;
    }
  }
}

// ---------------------------------------------------------------- Top-K
// Radix select over 32-bit keys in three digit passes (bits 31..20, 19..8, 7..0).  The
// shared helpers below work on one row per workgroup of kTopkThreads threads.
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kHistBins = 4096;

struct TopkShared {
  uint32_t hist[kHistBins];
  uint32_t wave_tot[kTopkWaves];
  uint32_t digit, remaining;
};

// Given the histogram of the current digit (among keys matching the prefix so far) and
// `remaining` = rank (1-based, from the top) of the wanted key among them, find the digit
// holding that key and the rank left inside it.  Thread t owns bins 4t .. 4t+3.
__device__ __forceinline__ void topk_find_digit(TopkShared& sh, uint32_t remaining) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = sh.hist[4 * tid + e];
  const uint32_t tot = c[0] + c[1] + c[2] + c[3];
  uint32_t suf = tot;                              // inclusive suffix sum within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(suf, o);
    if (lane + o < 64) suf += y;
  }
  if (lane == 0) sh.wave_tot[wave] = suf;
  __syncthreads();
  uint32_t above = suf - tot;                      // keys in bins of higher threads
  for (int w = wave + 1; w < kTopkWaves; ++w) above += sh.wave_tot[w];
#pragma unroll
  for (int e = 3; e >= 0; --e) {
    if (above < remaining && above + c[e] >= remaining) {
      sh.digit = (uint32_t)(4 * tid + e);
      sh.remaining = remaining - above;
    }
    above += c[e];
  }
  __syncthreads();
}

// Ordered compaction of one tile of 4 x kTopkThreads keys: thread t holds the tile's keys
// 4t..4t+3 (valid[e] marks real keys), whose indices are idx[e].  Output position of a
// selected key i: (#keys > tau before i) + min(#keys == tau before i, need_eq).
__device__ __forceinline__ void topk_emit_tile(TopkShared& sh, const uint32_t kv[4],
                                               const bool valid[4], const int idx[4],
                                               uint32_t tau, uint32_t need_eq,
                                               uint32_t& gt_base, uint32_t& eq_base,
                                               int32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t cg = 0u, ce = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    cg += (valid[e] && kv[e] > tau);
    ce += (valid[e] && kv[e] == tau);
  }
  const uint32_t packed = cg | (ce << 16);
  uint32_t incl = packed;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  uint32_t wave_off = 0u, tile_tot = 0u;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t x = sh.wave_tot[w];
    wave_off += (w < wave) ? x : 0u;
    tile_tot += x;
  }
  const uint32_t excl = wave_off + incl - packed;
  uint32_t gtb = gt_base + (excl & 0xffffu);
  uint32_t eqb = eq_base + (excl >> 16);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (!valid[e]) continue;
    if (kv[e] > tau) {
      out[gtb + min(eqb, need_eq)] = idx[e];
      ++gtb;
    } else if (kv[e] == tau) {
      if (eqb < need_eq) out[gtb + eqb] = idx[e];
      ++eqb;
    }
  }
  gt_base += tile_tot & 0xffffu;
  eq_base += tile_tot >> 16;
  __syncthreads();                                 // wave_tot is reused by the next tile
}

__device__ __forceinline__ uint32_t topk_digit(uint32_t k, int pass) {
  return pass == 0 ? (k >> 20) : (pass == 1 ? ((k >> 8) & 0xfffu) : (k & 0xffu));
}
__device__ __forceinline__ uint32_t topk_prefix_mask(int pass) {
  return pass == 0 ? 0u : (pass == 1 ? 0xfff00000u : 0xffffff00u);
}
__device__ __forceinline__ uint32_t topk_place(uint32_t d, int pass) {
  return pass == 0 ? (d << 20) : (pass == 1 ? (d << 8) : d);
}

// Exclusive prefix sum over the wave of small per-lane counts (< 2^BITS) and the wave
// total, from one ballot per count bit (no LDS traffic).
template <int BITS>
__device__ __forceinline__ uint32_t wave_prefix_small(uint32_t v, uint32_t& total) {
  const uint64_t below = (1ull << (threadIdx.x & 63)) - 1ull;
  uint32_t pre = 0u, tot = 0u;
#pragma unroll
  for (int bit = 0; bit < BITS; ++bit) {
    const uint64_t m = __ballot((v >> bit) & 1u);
    pre += (uint32_t)__popcll(m & below) << bit;
    tot += (uint32_t)__popcll(m) << bit;
  }
  total = tot;
  return pre;
}

constexpr uint32_t kNoDigit = 0xffffffffu;

// Wave 0 locates the digit holding the `remaining`-th key (from the top) in a 4096-bin
// histogram: lane l first sums bins 64l .. 64l+63, a suffix scan over lanes picks the
// lane whose range holds the rank, then the wave scans that lane's 64 bins in parallel.
// A histogram of fewer than `remaining` keys yields kNoDigit.
__device__ __forceinline__ void topk_find_digit_w0(const uint32_t* hist, uint32_t remaining,
                                                   uint32_t* s_digit, uint32_t* s_rem) {
  const int lane = threadIdx.x & 63;
  const u32x4* h4 = reinterpret_cast<const u32x4*>(hist + 64 * lane);
  uint32_t tot = 0u;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const u32x4 v = h4[q];
    tot += v[0] + v[1] + v[2] + v[3];
  }
  // suffix sums: keys in lanes >= l
  const uint32_t incl = wave_incl_scan(tot);
  const uint32_t all = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  if (all < remaining) {                                       // wave-uniform
    if (lane == 0) *s_digit = kNoDigit;
    return;
  }
  const uint32_t suf = all - incl + tot;
  const uint32_t above = suf - tot;
  const uint64_t hit = __ballot(above < remaining && suf >= remaining);
  const int L = (int)__builtin_ctzll(hit);                     // exactly one lane
  const uint32_t above_L = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
  const uint32_t rem2 = remaining - above_L;
  // bins of lane L, highest first: lane l takes bin 64L + 63 - l
  const uint32_t c = hist[64 * L + 63 - lane];
  const uint32_t incl2 = wave_incl_scan(c);                    // keys in bins above, incl.
  const uint64_t hit2 = __ballot(incl2 - c < rem2 && incl2 >= rem2);
  const int l2 = (int)__builtin_ctzll(hit2);
  if (lane == l2) {
    *s_digit = (uint32_t)(64 * L + 63 - l2);
    *s_rem = rem2 - (incl2 - c);
  }
}

// Pooled rows: the row is the 8 * pool_K key slots of the pooled scoring (0 = no
// candidate), at most 4096 * NR of them.  Thread t keeps slots [4NR t, 4NR (t+1)) in
// registers, so the row is read from memory once and one block-wide scan orders the
// output.  When at most K slots hold a candidate all of them are taken; slots map back to
// entries.
template <int NR>
__global__ __launch_bounds__(kTopkThreads) void topk_pool_kernel(TopkParams p) {
  constexpr int KPT = 4 * NR;                        // keys per thread
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][kHistBins];
  __shared__ uint32_t s_digit, s_rem;
  __shared__ uint32_t s_wtot[kTopkWaves];
  const int t = blockIdx.x;
  const int n = kPoolBlock * p.pool_K;
  const int K = p.K;
  int32_t* out = p.idx_out + (int64_t)t * K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* psel = p.pool_sel + (int64_t)t * p.pool_K;
  auto entry_of = [&](int slot) { return kPoolBlock * (psel[slot >> 3] >> 3) + (slot & 7); };
  // keys below n are >= float_key(-inf) > 0; 0 marks the slots past n
  const uint32_t* keys = p.keys + (int64_t)t * p.key_stride;
  const int i0 = KPT * tid;
  uint32_t kv[KPT];
  if (i0 + KPT <= n) {
    const u32x4* k4 = reinterpret_cast<const u32x4*>(keys + i0);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const u32x4 v = k4[r];
      kv[4 * r] = v[0]; kv[4 * r + 1] = v[1]; kv[4 * r + 2] = v[2]; kv[4 * r + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < KPT; ++e) kv[e] = (i0 + e < n) ? keys[i0 + e] : 0u;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) hist[0][4 * tid + e] = 0u;

  // Digit schedule.  Scores of one row mostly share the sign and the top exponent bits, so
  // a first digit over bits 31..20 would pile them into a few bins (and the histogram
  // atomics onto a few addresses).  When at least K keys share the top 4 bits of the row
  // maximum, the K-th key is among them: take that nibble as a fixed prefix and digits
  // over bits 27..16, 15..4, 3..0; otherwise bits 31..20, 19..8, 7..0.
  uint32_t kmax = 0u;
#pragma unroll
  for (int e = 0; e < KPT; ++e) kmax = max(kmax, kv[e]);
  kmax = wave_max_u32(kmax);
  if (lane == 0) s_wtot[wave] = kmax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) kmax = max(kmax, s_wtot[w]);
  uint32_t ctop = 0u, cnz = 0u;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    ctop += (kv[e] != 0u && (kv[e] >> 28) == (kmax >> 28));
    cnz += (kv[e] != 0u);
  }
  uint32_t ctot, nzt = 0u;
  (void)wave_prefix_small<7>(ctop, ctot);
  (void)wave_prefix_small<7>(cnz, nzt);
  __syncthreads();                                   // everyone has read the maxima
  if (lane == 0) s_wtot[wave] = ctot | (nzt << 16);  // each part <= 64 * 64
  __syncthreads();
  uint32_t wsum = 0u;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) wsum += s_wtot[w];
  const uint32_t n_cand = wsum >> 16;                // slots holding a candidate
  ctop = wsum & 0xffffu;                             // (rows hold <= 16384 slots)
  const bool take_all = n_cand <= (uint32_t)K;
  const bool narrow = ctop >= (uint32_t)K;
  // take_all: tau = 0 with no ties to keep selects every candidate
  uint32_t prefix = (narrow && !take_all) ? (kmax & 0xf0000000u) : 0u;
  uint32_t remaining = take_all ? 0u : (uint32_t)K;
  __syncthreads();                                   // s_wtot is reused below
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    if (take_all) break;                             // block-uniform
    const int shift = narrow ? (pass == 0 ? 16 : (pass == 1 ? 4 : 0)) : (pass == 0 ? 20 : (pass == 1 ? 8 : 0));
    const int width = narrow ? (pass == 2 ? 4 : 12) : (pass == 2 ? 8 : 12);
    const uint32_t pmask = ~((2u << (shift + width - 1)) - 1u);   // bits above the digit
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* h = hist[pass & 1];
#pragma unroll
    for (int e = 0; e < KPT; ++e)
      if (kv[e] != 0u && (kv[e] & pmask) == prefix) atomicAdd(&h[(kv[e] >> shift) & dmask], 1u);
    // the other buffer is free: clear it for the next pass
#pragma unroll
    for (int e = 0; e < 4; ++e) hist[(pass + 1) & 1][4 * tid + e] = 0u;
    __syncthreads();
    if (wave == 0) topk_find_digit_w0(h, remaining, &s_digit, &s_rem);
    __syncthreads();
    prefix |= s_digit << shift;
    remaining = s_rem;
  }
  const uint32_t tau = prefix, need_eq = remaining;

  // ---- ordered compaction: position = (#greater before) + min(#equal before, need_eq).
  // Each thread marks its keys above and at tau in bit masks, so the emission walks only
  // the selected keys (about K / n of them).
  uint64_t gtm = 0u, eqm = 0u;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    gtm |= (uint64_t)(kv[e] > tau) << e;
    eqm |= (uint64_t)(kv[e] == tau) << e;
  }
  const uint32_t cg = (uint32_t)__popcll(gtm), ce = (uint32_t)__popcll(eqm);
  uint32_t wg, we;
  const uint32_t pg = wave_prefix_small<7>(cg, wg);
  const uint32_t pe = wave_prefix_small<7>(ce, we);
  if (lane == 0) s_wtot[wave] = wg | (we << 16);
  __syncthreads();
  uint32_t off = 0u;
  for (int w = 0; w < wave; ++w) off += s_wtot[w];
  const uint32_t gtb = (off & 0xffffu) + pg;         // keys above tau before this thread
  const uint32_t eqb = (off >> 16) + pe;             // keys at tau before this thread
  // the first need_eq keys at tau (in index order) are selected
  uint32_t r = min(sub_sat_u32(need_eq, eqb), ce);
  uint64_t sel = gtm;
  while (r--) {
    const uint64_t low = eqm & (0ull - eqm);
    sel |= low;
    eqm ^= low;
  }
  uint32_t pos = gtb + min(eqb, need_eq);
  // Stage the ordered output in the (now free) histogram space when it fits, so that the
  // row goes out in coalesced stores; else write it in place.
  const int n_out = take_all ? (int)n_cand : K;      // the rest is -1 padding
  if (K <= 2 * kHistBins) {
    int32_t* s_out = reinterpret_cast<int32_t*>(&hist[0][0]);
    while (sel) {
      s_out[pos++] = i0 + (int)__builtin_ctzll(sel);
      sel &= sel - 1;
    }
    __syncthreads();
    for (int i = tid; i < K; i += kTopkThreads) out[i] = (i < n_out) ? entry_of(s_out[i]) : -1;
  } else {
    while (sel) {
      out[pos++] = entry_of(i0 + (int)__builtin_ctzll(sel));
      sel &= sel - 1;
    }
    for (int i = n_out + tid; i < K; i += kTopkThreads) out[i] = -1;
  }
}

// Maximum over the wave by DPP (row steps, then the row carries, as in wave_incl_scan).
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Exclusive prefix over the wave's lanes, and the wave total, of NG per-lane counts of at
// most 4 each: three counts share one DPP scan in 10-bit fields (a field's total is at
// most 256, so no carry crosses into the next).
template <int NG>
__device__ __forceinline__ void wave_group_prefix(const uint32_t (&c)[NG], uint32_t (&pre)[NG],
                                                  uint32_t (&tot)[NG]) {
#pragma unroll
  for (int f = 0; f < NG; f += 3) {
    uint32_t pk = 0u;
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (f + j < NG) pk |= c[f + j] << (10 * j);
    const uint32_t incl = wave_incl_scan(pk);
    const uint32_t ex = incl - pk;
    const uint32_t all = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (f + j < NG) {
        pre[f + j] = (ex >> (10 * j)) & 0x3ffu;
        tot[f + j] = (all >> (10 * j)) & 0x3ffu;
      }
  }
}

// One digit pass over register-resident keys: keys whose bits above the digit equal
// `prefix` are counted into h; the other buffer is cleared for the pass after.
template <int KPT>
__device__ __forceinline__ void topk_reg_pass(const uint32_t (&kv)[KPT], uint32_t* h,
                                              uint32_t* h_next, int shift, int width,
                                              uint32_t& prefix, uint32_t& remaining,
                                              uint32_t* s_digit, uint32_t* s_rem) {
  const int tid = threadIdx.x;
  const uint32_t pmask = ~((2u << (shift + width - 1)) - 1u);   // bits above the digit
  const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
  for (int e = 0; e < KPT; ++e)
    if ((kv[e] & pmask) == prefix) atomicAdd(&h[(kv[e] >> shift) & dmask], 1u);
#pragma unroll
  for (int e = 0; e < 4; ++e) h_next[4 * tid + e] = 0u;
  __syncthreads();
  if (tid < 64) topk_find_digit_w0(h, remaining, s_digit, s_rem);
  __syncthreads();
  prefix |= *s_digit << shift;
  remaining = *s_rem;
}

// Keys of the boundary bin after the first digit, gathered for the last two digits.
constexpr int kRowList = 4096;

// Rows of at most 4096 * NR keys, one workgroup per row, the row read once into registers.
// Wave w holds keys [KPW w, KPW (w + 1)); its lane l holds the 4-key groups starting at
// KPW w + 256 r + 4 l (r < NR), so every load instruction reads 1 KB of consecutive keys.
// Digits: the first is bits 31..16 of the keys whose top 16 bits lie within 4095 of the
// row maximum's (for float scores, about 32 octaves below the maximum, in bins of 1/128
// octave).  When at least K keys fall in that window (the usual case) the K-th key is
// among them; the keys of its bin are gathered into an LDS list, where one wave finds bits
// 15..4 and 3..0.  Otherwise (or when the bin overflows the list) the remaining digits are
// passes over the registers: bits 31..20, 19..8, 7..0, or 15..4, 3..0.
// The list append also counts the second digit, so one wave finds it from the counts and
// the last digit on the list.  Compaction: when the list's last digit shows that every key
// equal to tau is kept (the usual case), the selection is the keys >= tau, marked in an
// LDS bitmap in entry order and written from it by contiguous runs per thread; otherwise
// from the lane-interleaved registers, with the ties at tau ranked in entry order.
// Slots past n_vis hold key 0, below every visible key (>= float_key(-inf) > 0); they can
// only be counted when the maximum is within the window of 0, and there are always K
// larger keys.
template <int NR>
__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(TopkParams p) {
  constexpr int KPT = 4 * NR;                        // keys per thread
  constexpr int KPW = 64 * KPT;                      // keys per wave
  typedef typename std::conditional<(KPT <= 32), uint32_t, uint64_t>::type Mask;
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][kHistBins];
  __shared__ uint32_t s_list[kRowList];
  __shared__ uint32_t s_bits[KPT * kTopkThreads / 32];   // selection bitmap (entry order)
  __shared__ uint32_t s_digit, s_rem, s_cnt, s_eqc;
  __shared__ uint32_t s_wtot[kTopkWaves];
  const int t = blockIdx.x;
  if (p.row_flags && !p.row_flags[t]) return;        // selected on the candidate path
  const int n = p.n_vis[t];
  const int K = p.K;
  int32_t* out = p.idx_out + (int64_t)t * K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n <= K) {                                      // every visible entry is selected
    for (int i = tid; i < K; i += kTopkThreads) out[i] = (i < n) ? i : -1;
    return;
  }
  const int wbase = KPW * wave;
  const uint32_t* keys = p.keys + (int64_t)t * p.key_stride + wbase + 4 * lane;
  uint32_t kv[KPT];
  if (wbase + KPW <= n) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(keys + 256 * r);
      kv[4 * r] = v[0]; kv[4 * r + 1] = v[1]; kv[4 * r + 2] = v[2]; kv[4 * r + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        kv[4 * r + e] = (wbase + 256 * r + 4 * lane + e < n) ? keys[256 * r + e] : 0u;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hist[0][4 * tid + e] = 0u;
    hist[1][4 * tid + e] = 0u;
  }
#pragma unroll
  for (int e = 0; e < KPT / 32 + (KPT < 32); ++e)
    if (KPT >= 32 || tid < KPT * kTopkThreads / 32) s_bits[(KPT >= 32 ? KPT / 32 : 1) * tid + e] = 0u;
  if (tid == 0) s_cnt = 0u;
  bool all_tied = false;                             // block-uniform: see the compaction
  uint32_t kmax = 0u;
#pragma unroll
  for (int e = 0; e < KPT; ++e) kmax = max(kmax, kv[e]);
  kmax = wave_max_u32_dpp(kmax);
  if (lane == 0) s_wtot[wave] = kmax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) kmax = max(kmax, s_wtot[w]);

  // first digit: bits 31..16 of the keys within 4095 below those of the maximum
  const int lo = (int)(kmax >> 16) - (kHistBins - 1);
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const int b = (int)(kv[e] >> 16) - lo;
    if (b >= 0) atomicAdd(&hist[0][b], 1u);
  }
  __syncthreads();
  if (wave == 0) topk_find_digit_w0(hist[0], (uint32_t)K, &s_digit, &s_rem);
  __syncthreads();
  uint32_t prefix, remaining;
  const uint32_t d0 = s_digit;
  if (d0 == kNoDigit) {                              // block-uniform; hist[1] is clear
    prefix = 0u;
    remaining = (uint32_t)K;
    topk_reg_pass(kv, hist[1], hist[0], 20, 12, prefix, remaining, &s_digit, &s_rem);
    topk_reg_pass(kv, hist[0], hist[1], 8, 12, prefix, remaining, &s_digit, &s_rem);
    topk_reg_pass(kv, hist[1], hist[0], 0, 8, prefix, remaining, &s_digit, &s_rem);
  } else {
    prefix = (uint32_t)(lo + (int)d0) << 16;
    remaining = s_rem;
    // gather the bin's keys (any order) into the list, counting their second digit (bits
    // 15..4) on the way (hist[1] is clear)
    Mask bm = 0u;
#pragma unroll
    for (int e = 0; e < KPT; ++e) bm |= (Mask)((kv[e] & 0xffff0000u) == prefix) << e;
    const uint32_t c = (uint32_t)__builtin_popcountll((uint64_t)bm);
    const uint32_t incl = wave_incl_scan(c);
    const uint32_t wt = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    uint32_t base = 0u;
    if (lane == 0 && wt != 0u) base = atomicAdd(&s_cnt, wt);
    uint32_t at = (uint32_t)__builtin_amdgcn_readlane((int)base, 0) + incl - c;
    if (bm) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t nib = (uint32_t)(bm >> (4 * r)) & 0xfu;
        if (nib) {                                   // the wave skips groups with no match
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((nib >> e) & 1u) {
              atomicAdd(&hist[1][(kv[4 * r + e] >> 4) & 0xfffu], 1u);
              if (at < (uint32_t)kRowList) s_list[at] = kv[4 * r + e];
              ++at;
            }
        }
      }
    }
    __syncthreads();
    const uint32_t L = s_cnt;
    if (L > (uint32_t)kRowList) {                    // block-uniform
      // the second digit from its counts, the last over the registers
#pragma unroll
      for (int e = 0; e < 4; ++e) hist[0][4 * tid + e] = 0u;
      if (wave == 0) topk_find_digit_w0(hist[1], remaining, &s_digit, &s_rem);
      __syncthreads();
      prefix |= s_digit << 4;
      remaining = s_rem;
      topk_reg_pass(kv, hist[0], hist[1], 0, 4, prefix, remaining, &s_digit, &s_rem);
    } else {
      if (wave == 0) {
        // bits 15..4 from their counts, bits 3..0 over the list
        topk_find_digit_w0(hist[1], remaining, &s_digit, &s_rem);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        prefix |= s_digit << 4;
        remaining = s_rem;
        // bits 3..0: 16 bins, bin 15 - l read by lane l
        if (lane < 16) hist[0][lane] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        for (uint32_t i = (uint32_t)lane; i < L; i += 64u) {
          const uint32_t k = s_list[i];
          if ((k & 0xfffffff0u) == prefix) atomicAdd(&hist[0][k & 0xfu], 1u);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const uint32_t cb = lane < 16 ? hist[0][15 - lane] : 0u;
        const uint32_t inc2 = wave_incl_scan(cb);   // keys in this bin and those above
        const uint64_t hit = __ballot(lane < 16 && inc2 - cb < remaining && inc2 >= remaining);
        const int l2 = (int)__builtin_ctzll(hit);
        if (lane == l2) {
          s_digit = prefix | (uint32_t)(15 - l2);
          s_rem = remaining - (inc2 - cb);
          s_eqc = cb;                                // keys equal to tau
        }
      }
      __syncthreads();
      prefix = s_digit;
      remaining = s_rem;
      all_tied = NR <= 8 && s_eqc == remaining;   // (the widest rows: register budget)
    }
  }
  const uint32_t tau = prefix, need_eq = remaining;

  if (all_tied) {
    // ---- every key at tau is kept, so the selection is the keys >= tau: marked in an LDS
    // bitmap in entry order, then thread t compacts entries [KPT t, KPT (t + 1)).
    Mask ge = 0u;
#pragma unroll
    for (int e = 0; e < KPT; ++e) ge |= (Mask)(kv[e] >= tau) << e;
    while (ge) {
      const int e = (int)__builtin_ctzll((uint64_t)ge);
      const int j = wbase + 256 * (e >> 2) + 4 * lane + (e & 3);
      atomicOr(&s_bits[j >> 5], 1u << (j & 31));
      ge &= ge - 1u;
    }
    __syncthreads();
    const int i0 = KPT * tid;
    uint64_t w;
    if constexpr (KPT == 64) w = (uint64_t)s_bits[2 * tid] | ((uint64_t)s_bits[2 * tid + 1] << 32);
    else if constexpr (KPT == 32) w = s_bits[tid];
    else w = (s_bits[i0 >> 5] >> (i0 & 31)) & ((1u << KPT) - 1u);
    const uint32_t c = (uint32_t)__builtin_popcountll(w);
    const uint32_t incl = wave_incl_scan(c);
    if (lane == 63) s_wtot[wave] = incl;
    __syncthreads();
    uint32_t at = incl - c;
#pragma unroll
    for (int v = 0; v < kTopkWaves; ++v) at += (v < wave) ? s_wtot[v] : 0u;
    // each thread's picks are consecutive in the output, so the stores stay near-coalesced
    while (w) {
      out[at++] = i0 + (int)__builtin_ctzll(w);
      w &= w - 1u;
    }
    return;
  }

  // ---- ordered compaction.  Entry order is (wave, group r, lane, key in group): wave
  // offsets come from per-wave totals, the rest from per-group prefixes over the lanes.
  Mask gtm = 0u, eqm = 0u;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    gtm |= (Mask)(kv[e] > tau) << e;
    eqm |= (Mask)(kv[e] == tau) << e;
  }
  const uint32_t cg = (uint32_t)__builtin_popcountll((uint64_t)gtm);
  const uint32_t ce = (uint32_t)__builtin_popcountll((uint64_t)eqm);
  const uint32_t both = wave_incl_scan(cg | (ce << 16));   // each part <= 64 * KPT <= 4096
  if (lane == 63) s_wtot[wave] = both;
  __syncthreads();
  uint32_t off_g = 0u, off_e = 0u, all_e = 0u;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t v = s_wtot[w];
    if (w < wave) {
      off_g += v & 0xffffu;
      off_e += v >> 16;
    }
    all_e += v >> 16;
  }
  Mask sel = gtm;
  if (all_e == need_eq) {                            // every key at tau is kept (usual)
    sel |= eqm;
  } else {                                           // the first need_eq keys at tau
    uint32_t c[NR], pre[NR], tot[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) c[r] = (uint32_t)__builtin_popcount((uint32_t)(eqm >> (4 * r)) & 0xfu);
    wave_group_prefix<NR>(c, pre, tot);
    uint32_t acc = off_e;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      uint32_t rk = acc + pre[r];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((eqm >> (4 * r + e)) & 1u) {
          if (rk < need_eq) sel |= (Mask)1 << (4 * r + e);
          ++rk;
        }
      acc += tot[r];
    }
  }
  uint32_t c[NR], pre[NR], tot[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) c[r] = (uint32_t)__builtin_popcount((uint32_t)(sel >> (4 * r)) & 0xfu);
  wave_group_prefix<NR>(c, pre, tot);
  uint32_t acc = off_g + min(off_e, need_eq);        // keys selected in the waves before
  // Stage the ordered output in the (now free) histogram space when it fits, so that the
  // row goes out in coalesced stores; else write it in place.
  if (K <= 2 * kHistBins) {
    int32_t* s_out = reinterpret_cast<int32_t*>(&hist[0][0]);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      uint32_t at = acc + pre[r];
      uint32_t nib = (uint32_t)(sel >> (4 * r)) & 0xfu;
      while (nib) {
        s_out[at++] = wbase + 256 * r + 4 * lane + (int)__builtin_ctz(nib);
        nib &= nib - 1u;
      }
      acc += tot[r];
    }
    __syncthreads();
    for (int i = tid; i < K; i += kTopkThreads) out[i] = s_out[i];
  } else {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      uint32_t at = acc + pre[r];
      uint32_t nib = (uint32_t)(sel >> (4 * r)) & 0xfu;
      while (nib) {
        out[at++] = wbase + 256 * r + 4 * lane + (int)__builtin_ctz(nib);
        nib &= nib - 1u;
      }
      acc += tot[r];
    }
  }
}

// Radix select of the `rank`-th largest of the first L keys of an LDS list over the first
// `passes` digits (3: the exact key and how many keys equal to it to keep; 2: the key with
// its low 8 bits cleared).  Block-wide (kTopkThreads threads).
__device__ __forceinline__ void topk_list_select(TopkShared& sh, const uint32_t* lkey, int L,
                                                 uint32_t rank, int passes, uint32_t& key,
                                                 uint32_t& keep) {
  const int tid = threadIdx.x;
  uint32_t pre = 0u, rem = rank;
#pragma unroll
  for (int ps = 0; ps < 3; ++ps) {
    if (ps == passes) break;                         // block-uniform
    const uint32_t pmask = topk_prefix_mask(ps);
#pragma unroll
    for (int e = 0; e < 4; ++e) sh.hist[4 * tid + e] = 0u;
    __syncthreads();
    for (int i = tid; i < L; i += kTopkThreads) {
      const uint32_t k = lkey[i];
      if ((k & pmask) == pre) atomicAdd(&sh.hist[topk_digit(k, ps)], 1u);
    }
    __syncthreads();
    topk_find_digit(sh, rem);
    pre |= topk_place(sh.digit, ps);
    rem = sh.remaining;
  }
  key = pre;
  keep = rem;
}

// The ordered emission from an LDS list that holds every key >= tau in index order.
__device__ __forceinline__ void topk_emit_list(TopkShared& sh, const uint32_t* lkey,
                                               const int32_t* lidx, int L, uint32_t tau,
                                               uint32_t need_eq, int32_t* out) {
  const int tid = threadIdx.x;
  uint32_t gt_base = 0u, eq_base = 0u;
  for (int b0 = 0; b0 < L; b0 += 4 * kTopkThreads) {
    uint32_t kv[4];
    bool valid[4];
    int idx[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = b0 + 4 * tid + e;
      valid[e] = i < L;
      kv[e] = valid[e] ? lkey[i] : 0u;
      idx[e] = valid[e] ? lidx[i] : 0;
    }
    topk_emit_tile(sh, kv, valid, idx, tau, need_eq, gt_base, eq_base, out);
  }
}

// Rows of any length, streamed from memory.  The first pass histograms the top digit (bits
// 31..20).  When the keys at or above the chosen digit fit in LDS (kTopkListCap), a second
// stream copies them, with their indices and in index order, into an LDS list; the last two
// digits are then found on the list and the emission walks the list: two streams of the row
// in all.  Otherwise the remaining digit passes and the emission each stream the row.
constexpr int kTopkListCap = 4096;

// Two workgroups per CU (8 waves per SIMD, so at most 64 VGPRs; 49 KB of LDS each): one
// row's stream then hides behind another's.  The register cap costs a few spills outside
// the streaming loop; prefill Top-K 921-948 -> 706-721 us.
__global__ __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_stream_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  __shared__ uint32_t s_lkey[kTopkListCap];
  __shared__ int32_t s_lidx[kTopkListCap];
  const int t = blockIdx.x;
  if (p.row_flags && !p.row_flags[t]) return;        // selected on the candidate path
  const int n = p.n_vis[t];
  const int K = p.K;
  int32_t* out = p.idx_out + (int64_t)t * K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n <= K) {
    for (int i = tid; i < K; i += kTopkThreads) out[i] = (i < n) ? i : -1;
    return;
  }
  const uint32_t* keys = p.keys + (int64_t)t * p.key_stride;
  const u32x4* k4 = reinterpret_cast<const u32x4*>(keys);
  auto load4 = [&](int i0, uint32_t (&kv)[4], bool (&valid)[4]) {
    if (i0 + 3 < n) {
      const u32x4 v = k4[i0 >> 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) { kv[e] = v[e]; valid[e] = true; }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        valid[e] = i0 + e < n;
        kv[e] = valid[e] ? keys[i0 + e] : 0u;
      }
    }
  };
  auto list_select = [&](int L, uint32_t rank, int passes, uint32_t& key, uint32_t& keep) {
    topk_list_select(sh, s_lkey, L, rank, passes, key, keep);
  };
  auto emit_list = [&](int L, uint32_t tau, uint32_t need_eq) {
    topk_emit_list(sh, s_lkey, s_lidx, L, tau, need_eq, out);
  };
  // The second stream: keys >= thr into the list in index order (at most kTopkListCap are
  // stored); returns how many there are.
  auto compact = [&](uint32_t thr) -> uint32_t {
    uint32_t base = 0u;
    constexpr int kAhead = 3;                        // tiles of loads in flight
    constexpr int kTile = 4 * kTopkThreads;
    uint32_t kn[kAhead][4];
    bool vn[kAhead][4];
#pragma unroll
    for (int a = 0; a < kAhead; ++a) load4(4 * tid + a * kTile, kn[a], vn[a]);
    for (int t0 = 0; t0 < n; t0 += kAhead * kTile) {
#pragma unroll
      for (int a = 0; a < kAhead; ++a) {             // static buffer index: no register moves
        const int tile = t0 + a * kTile;
        if (tile >= n) break;                        // block-uniform
        const int i0 = tile + 4 * tid;
        uint32_t f = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) f |= (uint32_t)(vn[a][e] && kn[a][e] >= thr) << e;
        uint32_t wtot;
        const uint32_t pre = wave_prefix_small<3>((uint32_t)__popc(f), wtot);
        if (lane == 0) sh.wave_tot[wave] = wtot;
        __syncthreads();
        uint32_t off = 0u, tot = 0u;
#pragma unroll
        for (int w = 0; w < kTopkWaves; ++w) {
          const uint32_t x = sh.wave_tot[w];
          off += (w < wave) ? x : 0u;
          tot += x;
        }
        uint32_t pos = base + off + pre;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((f >> e) & 1u) {
            if (pos < (uint32_t)kTopkListCap) {
              s_lkey[pos] = kn[a][e];
              s_lidx[pos] = i0 + e;
            }
            ++pos;
          }
        }
        base += tot;
        load4(i0 + kAhead * kTile, kn[a], vn[a]);    // past n: no load
        __syncthreads();                             // wave_tot is reused by the next tile
      }
    }
    return base;
  };

  // ---- sampled threshold.  A sample of the row (one 16-key segment in every `gap`, at
  // most kTopkListCap keys) goes to the list; its r-th largest key (to 24 bits), with r
  // chosen so that about 1.3 K + 8 n / sample keys of the row are expected at or above
  // it, becomes the threshold of a single full stream into the list.  When that stream holds at least
  // K and at most kTopkListCap keys, the exact selection runs on the list; otherwise the
  // passes below run as if no sample had been taken.
  {
    const int nseg = n >> 4;
    const int gap = (nseg + kTopkListCap / 16 - 1) / (kTopkListCap / 16);
    const int sseg = (nseg + gap - 1) / gap;         // sampled segments, <= kTopkListCap / 16
    const int ns = 16 * sseg;
    const uint32_t r = (uint32_t)((1.3 * (double)K * ns) / n) + 8u;
    if (nseg > 0 && r <= (uint32_t)ns) {
      // at most two segments' quarters per thread, both loads in flight at once
      const int q0 = tid >> 2, q1 = q0 + kTopkThreads / 4;
      u32x4 v0 = u32x4{0u, 0u, 0u, 0u}, v1 = u32x4{0u, 0u, 0u, 0u};
      if (q0 < sseg) v0 = k4[((int64_t)q0 * gap * 16 + 4 * (tid & 3)) >> 2];
      if (q1 < sseg) v1 = k4[((int64_t)q1 * gap * 16 + 4 * (tid & 3)) >> 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (q0 < sseg) s_lkey[16 * q0 + 4 * (tid & 3) + e] = v0[e];
        if (q1 < sseg) s_lkey[16 * q1 + 4 * (tid & 3) + e] = v1[e];
      }
      __syncthreads();
      uint32_t thr, unused;
      list_select(ns, r, 2, thr, unused);
      (void)unused;
      __syncthreads();                               // the sample is read by all
      const uint32_t L = compact(thr);
      if (L >= (uint32_t)K && L <= (uint32_t)kTopkListCap) {
        uint32_t tau, need_eq;
        list_select((int)L, (uint32_t)K, 3, tau, need_eq);
        emit_list((int)L, tau, need_eq);
        return;
      }
      __syncthreads();
    }
  }

  uint32_t prefix = 0u, remaining = (uint32_t)K;
  int pass = 0;
  for (; pass < 3; ++pass) {
    const uint32_t pmask = topk_prefix_mask(pass);
#pragma unroll
    for (int e = 0; e < 4; ++e) sh.hist[4 * tid + e] = 0u;
    __syncthreads();
    // four tiles of loads in flight per thread
    for (int i0 = 4 * tid; i0 < n; i0 += 16 * kTopkThreads) {
      uint32_t kv[4][4];
      bool valid[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) load4(i0 + 4 * kTopkThreads * u, kv[u], valid[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (valid[u][e] && (kv[u][e] & pmask) == prefix)
            atomicAdd(&sh.hist[topk_digit(kv[u][e], pass)], 1u);
    }
    __syncthreads();
    topk_find_digit(sh, remaining);
    prefix |= topk_place(sh.digit, pass);
    remaining = sh.remaining;
    if (pass == 0) {
      // keys at or above the top digit: K - rank of the K-th key in its bin, plus the bin
      const bool fits = (uint32_t)K - remaining + sh.hist[sh.digit] <= (uint32_t)kTopkListCap;
      __syncthreads();                               // read by all before the next pass clears
      if (fits) break;
    }
  }
  if (pass == 0) {
    // ---- second stream: keys with top digit >= d0 into the LDS list, in index order
    const uint32_t d0 = prefix >> 20;
    const int L = (int)compact(d0 << 20);            // = K - rank + hist[d0] <= cap
    // ---- the last two digits among the list's keys in bin d0
#pragma unroll
    for (int sub = 1; sub < 3; ++sub) {
      const uint32_t pmask = topk_prefix_mask(sub);
#pragma unroll
      for (int e = 0; e < 4; ++e) sh.hist[4 * tid + e] = 0u;
      __syncthreads();
      for (int i = tid; i < L; i += kTopkThreads) {
        const uint32_t k = s_lkey[i];
        if ((k & pmask) == prefix) atomicAdd(&sh.hist[topk_digit(k, sub)], 1u);
      }
      __syncthreads();
      topk_find_digit(sh, remaining);
      prefix |= topk_place(sh.digit, sub);
      remaining = sh.remaining;
    }
    emit_list(L, prefix, remaining);
    return;
  }
  uint32_t gt_base = 0u, eq_base = 0u;
  for (int base = 0; base < n; base += 4 * kTopkThreads) {
    const int i0 = base + 4 * tid;
    uint32_t kv[4];
    bool valid[4];
    int idx[4];
    load4(i0, kv, valid);
#pragma unroll
    for (int e = 0; e < 4; ++e) idx[e] = i0 + e;
    topk_emit_tile(sh, kv, valid, idx, prefix, remaining, gt_base, eq_base, out);
  }
}

// ---------------------------------------------------------------- sampled candidates
// Per row: the threshold of the sampled-candidate path, the top 24 bits of the r-th
// largest sampled key, r = 1.5 K nsv / n + 16 (nsv the row's valid samples).  One wave
// per row and no block barrier: the wave holds the row's (at most 4096) samples in
// registers, the first digit is bits 31..16 of the keys whose top 16 bits lie within 4095
// of the sample maximum's, the second bits 15..8 of the keys in the chosen bin.  A row
// with fewer than r valid samples, or fewer than r in the window, is flagged for the exact
// path.  Rows that select everything (n <= K) get threshold ~0 and no flag.
constexpr int kThrKeysPerLane = kSamplePages * kPage / 64;
__global__ __launch_bounds__(64) void topk_thr_kernel(TopkParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_digit, s_rem;
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const int n = p.n_vis[t];
  if (n <= p.K) {
    if (lane == 0) {
      p.thr[t] = 0xffffffffu;
      p.row_flags[t] = 0u;
    }
    return;
  }
  const int G = p.page_gap;
  const int nsp = ((n + kPage - 1) / kPage + G - 1) / G;   // sampled pages with visible keys
  const int ns = min(nsp, kSamplePages) * kPage;            // a multiple of 64
  // lane l holds keys 256 j + 4 l + e: 1 KB of consecutive keys per load instruction
  const uint32_t* keys = p.keys + (int64_t)t * p.key_stride + 4 * lane;
  uint32_t kv[kThrKeysPerLane];
#pragma unroll
  for (int j = 0; j < kThrKeysPerLane / 4; ++j) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (256 * j + 4 * lane < ns) v = *reinterpret_cast<const u32x4*>(keys + 256 * j);
    kv[4 * j] = v[0]; kv[4 * j + 1] = v[1]; kv[4 * j + 2] = v[2]; kv[4 * j + 3] = v[3];
  }
  u32x4* h4 = reinterpret_cast<u32x4*>(s_hist);
#pragma unroll
  for (int q = 0; q < kHistBins / 256; ++q) h4[64 * q + lane] = u32x4{0u, 0u, 0u, 0u};
  uint32_t c = 0u, kmax = 0u;
#pragma unroll
  for (int e = 0; e < kThrKeysPerLane; ++e) {
    c += (kv[e] != 0u);
    kmax = max(kmax, kv[e]);
  }
  const uint32_t nsv = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(c), 63);
  kmax = wave_max_u32_dpp(kmax);
  const uint32_t r = (uint32_t)((1.5 * (double)p.K * nsv) / n) + 16u;
  const int lo = (int)(kmax >> 16) - (kHistBins - 1);
  bool flag = r > nsv;                               // wave-uniform
  uint32_t thr = 0u;
  if (!flag) {
#pragma unroll
    for (int e = 0; e < kThrKeysPerLane; ++e) {
      const int b = (int)(kv[e] >> 16) - lo;
      if (kv[e] != 0u && b >= 0) atomicAdd(&s_hist[b], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    topk_find_digit_w0(s_hist, r, &s_digit, &s_rem);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const uint32_t d0 = s_digit;
    flag = d0 == kNoDigit;
    if (!flag) {
      const uint32_t top = (uint32_t)(lo + (int)d0);  // the bin's top 16 bits
      const uint32_t rem = s_rem;
#pragma unroll
      for (int q = 0; q < kHistBins / 256; ++q) h4[64 * q + lane] = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
      for (int e = 0; e < kThrKeysPerLane; ++e)
        if ((kv[e] >> 16) == top) atomicAdd(&s_hist[(kv[e] >> 8) & 0xffu], 1u);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      topk_find_digit_w0(s_hist, rem, &s_digit, &s_rem);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      thr = (top << 16) | (s_digit << 8);
    }
  }
  if (lane == 0) {
    p.thr[t] = flag ? 0u : thr;
    p.row_flags[t] = flag ? 1u : 0u;
  }
}

// Per row: the exact Top-K among the candidates (every key >= the row's threshold, chunk
// by chunk in entry order).  Rows flagged by the scoring (a chunk held more than kCandCap),
// or whose candidates number fewer than K or more than kCandList, are flagged here and left
// to the exact path.
// Two workgroups per CU (LDS under 80 KB, at most 64 VGPRs): each row's chain of
// block-wide steps hides behind another row's.
__global__ __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_cand_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  __shared__ uint32_t s_lkey[kCandList];
  __shared__ int32_t s_lidx[kCandList];
  __shared__ uint32_t s_off[kTopkThreads + 1];
  const int t = blockIdx.x;
  const int n = p.n_vis[t];
  const int K = p.K;
  int32_t* out = p.idx_out + (int64_t)t * K;
  const int tid = threadIdx.x;
  if (n <= K) {
    for (int i = tid; i < K; i += kTopkThreads) out[i] = (i < n) ? i : -1;
    return;
  }
  if (p.row_flags[t]) return;
  const int nch = (n + kGemmChunk - 1) / kGemmChunk;   // chunks holding visible entries
  // chunk offsets in the list: an exclusive scan of the counts (nch <= kTopkThreads chunks
  // per thread pass)
  uint32_t base = 0u;
  for (int c0 = 0; c0 < nch; c0 += kTopkThreads) {
    const int c = c0 + tid;
    const uint32_t v = c < nch ? p.cand_cnt[(int64_t)t * p.n_chunks + c] : 0u;
    const uint32_t incl = wave_incl_scan(v);
    if ((tid & 63) == 63) sh.wave_tot[tid >> 6] = incl;
    __syncthreads();
    uint32_t woff = 0u, tot = 0u;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      const uint32_t x = sh.wave_tot[w];
      woff += (w < (tid >> 6)) ? x : 0u;
      tot += x;
    }
    s_off[tid] = base + woff + incl - v;
    if (tid == kTopkThreads - 1) s_off[kTopkThreads] = base + tot;
    __syncthreads();
    // copy this pass's chunks into the list: list position i -> (chunk, slot) by a binary
    // search over the offsets, so that every thread issues all of its loads at once
    const uint32_t L_end = s_off[kTopkThreads];
    if (L_end <= (uint32_t)kCandList) {
      const int ncc = min(kTopkThreads, nch - c0);
      constexpr int kPer = kCandList / kTopkThreads;
      uint32_t kk[kPer];
      int32_t ii[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const uint32_t i = s_off[0] + (uint32_t)(tid + u * kTopkThreads);
        if (i < L_end) {
          int lo = 0, hi = ncc - 1;                  // last chunk whose offset <= i
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= i) lo = mid; else hi = mid - 1;
          }
          const int64_t src = ((int64_t)t * p.n_chunks + c0 + lo) * kCandCap + (i - s_off[lo]);
          kk[u] = p.cand_key[src];
          ii[u] = p.cand_idx[src];
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const uint32_t i = s_off[0] + (uint32_t)(tid + u * kTopkThreads);
        if (i < L_end) {
          s_lkey[i] = kk[u];
          s_lidx[i] = ii[u];
        }
      }
    }
    base += tot;
    __syncthreads();
  }
  const uint32_t L = base;
  if (L < (uint32_t)K || L > (uint32_t)kCandList) {
    if (tid == 0) p.row_flags[t] = 1u;
    return;
  }
  uint32_t tau, need_eq;
  topk_list_select(sh, s_lkey, (int)L, (uint32_t)K, 3, tau, need_eq);
  topk_emit_list(sh, s_lkey, s_lidx, (int)L, tau, need_eq, out);
}

hipError_t launch_topk_thr(const TopkParams& p, hipStream_t s) {
  CSA2_LAUNCH(topk_thr_kernel, dim3((unsigned)p.T), dim3(64), s, p);
  return hipGetLastError();
}

hipError_t launch_topk_cand(const TopkParams& p, hipStream_t s) {
  CSA2_LAUNCH(topk_cand_kernel, dim3((unsigned)p.T), dim3(kTopkThreads), s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- chunked Top-K
// Few long rows: the work of a row spreads over many CUs in 4096-key chunks, one
// workgroup of 256 threads each (16 keys per thread), in three launches:
//   1. histogram of the top digit (bits 31..20): chunk histograms in LDS, non-zero bins
//      added to the row's histogram in memory (zeroed by the scoring launch);
//   2. every chunk finds the digit d0 holding the K-th key from the row histogram and
//      copies its keys with top digit >= d0, and their indices, in index order, to its own
//      candidate segment, with a count;
//   3. one workgroup per row finds the last two digits among the candidates of bin d0 and
//      emits the selection chunk by chunk (candidate segments in chunk order are in index
//      order), each chunk's candidates one emission tile.
// Every key >= tau is a candidate, so the emission sees all it needs.
constexpr int kCkThreads = 256;
constexpr int kCkPerThread = kCkKeys / kCkThreads;   // 16

__device__ __forceinline__ void ck_load(const TopkParams& p, int t, int ch, int n,
                                        uint32_t (&kv)[kCkPerThread]) {
  const int i0 = ch * kCkKeys + kCkPerThread * (int)threadIdx.x;
  const uint32_t* keys = p.keys + (int64_t)t * p.key_stride;
  if (i0 + kCkPerThread <= n) {
    const u32x4* k4 = reinterpret_cast<const u32x4*>(keys + i0);
#pragma unroll
    for (int r = 0; r < kCkPerThread / 4; ++r) {
      const u32x4 v = k4[r];
      kv[4 * r] = v[0]; kv[4 * r + 1] = v[1]; kv[4 * r + 2] = v[2]; kv[4 * r + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kCkPerThread; ++e) kv[e] = (i0 + e < n) ? keys[i0 + e] : 0u;
  }
}

// 1: histogram of bits 31..20 of the chunk's keys, added to the row histogram
__global__ __launch_bounds__(kCkThreads) void topk_ck_hist_kernel(TopkParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistBins];
  const int nch = (int)topk_chunks(p.key_stride);
  const int t = blockIdx.x / nch, ch = blockIdx.x - t * nch;
  const int n = p.n_vis[t];
  if (n <= p.K || ch * kCkKeys >= n) return;         // uniform per workgroup
  uint32_t kv[kCkPerThread];
  ck_load(p, t, ch, n, kv);
  for (int i = threadIdx.x; i < kHistBins; i += kCkThreads) s_hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kCkPerThread; ++e)
    if (kv[e] != 0u) atomicAdd(&s_hist[kv[e] >> 20], 1u);
  __syncthreads();
  uint32_t* g = p.ck_hist + (int64_t)t * kCkHistWords;
  for (int i = threadIdx.x; i < kHistBins; i += kCkThreads) {
    const uint32_t c = s_hist[i];
    if (c) atomicAdd(&g[i], c);
  }
}

// 2: candidates of the chunk (top digit >= d0) in index order, and their count
__global__ __launch_bounds__(kCkThreads) void topk_ck_compact_kernel(TopkParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistBins];
  __shared__ uint32_t s_digit, s_rem;
  __shared__ uint32_t s_w[kCkThreads / 64];
  const int nch = (int)topk_chunks(p.key_stride);
  const int t = blockIdx.x / nch, ch = blockIdx.x - t * nch;
  const int n = p.n_vis[t];
  if (n <= p.K || ch * kCkKeys >= n) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kv[kCkPerThread];
  ck_load(p, t, ch, n, kv);                          // in flight while the digit is found
  for (int i = tid; i < kHistBins; i += kCkThreads)
    s_hist[i] = p.ck_hist[(int64_t)t * kCkHistWords + i];
  __syncthreads();
  if (tid < 64) topk_find_digit_w0(s_hist, (uint32_t)p.K, &s_digit, &s_rem);
  __syncthreads();
  const uint32_t d0 = s_digit;
  if (ch == 0 && tid == 0) {
    uint32_t* sel = p.ck_sel + (int64_t)t * 8;
    sel[0] = d0;
    sel[1] = s_rem;
  }
  const uint32_t thr = d0 << 20;
  uint32_t f = 0u;
#pragma unroll
  for (int e = 0; e < kCkPerThread; ++e) f |= (uint32_t)(kv[e] != 0u && kv[e] >= thr) << e;
  uint32_t wtot;
  const uint32_t pre = wave_prefix_small<5>((uint32_t)__popc(f), wtot);
  if (lane == 0) s_w[wave] = wtot;
  __syncthreads();
  uint32_t off = 0u, tot = 0u;
#pragma unroll
  for (int w = 0; w < kCkThreads / 64; ++w) {
    off += (w < wave) ? s_w[w] : 0u;
    tot += s_w[w];
  }
  const int64_t seg = (int64_t)t * p.key_stride + (int64_t)ch * kCkKeys;
  uint32_t pos = off + pre;
  const int i0 = ch * kCkKeys + kCkPerThread * tid;
#pragma unroll
  for (int e = 0; e < kCkPerThread; ++e) {
    if ((f >> e) & 1u) {
      p.ck_ckey[seg + pos] = kv[e];
      p.ck_cidx[seg + pos] = i0 + e;
      ++pos;
    }
  }
  if (tid == 0) p.ck_counts[(int64_t)t * nch + ch] = tot;
}

// 3: one workgroup per row: the last two digits among the candidates, then the emission.
// The candidates usually fit an LDS list: they are gathered there once (each thread takes
// list positions, finds their chunk by binary search over the chunks' offsets, and has all
// its loads in flight at once); otherwise the passes and the emission read the candidate
// segments in memory.
constexpr int kCkListCap = 8192;

__global__ __launch_bounds__(kTopkThreads) void topk_ck_select_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  __shared__ uint32_t s_cnt[kCkMaxChunks];
  __shared__ uint32_t s_off[kCkMaxChunks + 1];
  __shared__ uint32_t s_lkey[kCkListCap];
  __shared__ int32_t s_lidx[kCkListCap];
  const int t = blockIdx.x;
  const int n = p.n_vis[t];
  const int K = p.K;
  int32_t* out = p.idx_out + (int64_t)t * K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n <= K) {                                      // every visible entry is selected
    for (int i = tid; i < K; i += kTopkThreads) out[i] = (i < n) ? i : -1;
    return;
  }
  const int nch = (int)topk_chunks(p.key_stride);
  const int nrow = (n + kCkKeys - 1) / kCkKeys;      // chunks holding visible keys
  // counts and their exclusive prefix: thread tid owns chunks 4 tid .. 4 tid + 3
  uint32_t c4[4], own = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * tid + e;
    c4[e] = (c < nrow) ? p.ck_counts[(int64_t)t * nch + c] : 0u;
    own += c4[e];
  }
  const uint32_t incl = wave_incl_scan(own);
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  uint32_t before = incl - own, total = 0u;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t x = sh.wave_tot[w];
    before += (w < wave) ? x : 0u;
    total += x;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 4 * tid + e;
    if (c < nrow) {
      s_cnt[c] = c4[e];
      s_off[c] = before;
    }
    before += c4[e];
  }
  if (tid == 0) s_off[nrow] = total;
  const uint32_t* sel = p.ck_sel + (int64_t)t * 8;
  uint32_t prefix = sel[0] << 20, remaining = sel[1];
  const uint32_t* ckey = p.ck_ckey + (int64_t)t * p.key_stride;
  const int32_t* cidx = p.ck_cidx + (int64_t)t * p.key_stride;
  __syncthreads();                                   // s_cnt, s_off; wave_tot read by all
  const bool in_lds = total <= (uint32_t)kCkListCap;
  if (in_lds) {
    const int L = (int)total;
    for (int p0 = tid; p0 < L; p0 += 4 * kTopkThreads) {
      uint32_t kv[4];
      int iv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {                  // four loads of each kind in flight
        const int pos = p0 + u * kTopkThreads;
        if (pos < L) {
          int lo = 0, hi = nrow;                     // last chunk with s_off[c] <= pos
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_off[mid] <= (uint32_t)pos) lo = mid; else hi = mid;
          }
          const int64_t at = (int64_t)lo * kCkKeys + (pos - (int)s_off[lo]);
          kv[u] = ckey[at];
          iv[u] = cidx[at];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int pos = p0 + u * kTopkThreads;
        if (pos < L) {
          s_lkey[pos] = kv[u];
          s_lidx[pos] = iv[u];
        }
      }
    }
  }
#pragma unroll
  for (int sub = 1; sub < 3; ++sub) {
    const uint32_t pmask = topk_prefix_mask(sub);
#pragma unroll
    for (int e = 0; e < 4; ++e) sh.hist[4 * tid + e] = 0u;
    __syncthreads();                                 // (also: the list is written)
    if (in_lds) {
      for (int i = tid; i < (int)total; i += kTopkThreads) {
        const uint32_t k = s_lkey[i];
        if ((k & pmask) == prefix) atomicAdd(&sh.hist[topk_digit(k, sub)], 1u);
      }
    } else {
      for (int c = 0; c < nrow; ++c) {
        const int cnt = (int)s_cnt[c];
        for (int j = tid; j < cnt; j += kTopkThreads) {
          const uint32_t k = ckey[(int64_t)c * kCkKeys + j];
          if ((k & pmask) == prefix) atomicAdd(&sh.hist[topk_digit(k, sub)], 1u);
        }
      }
    }
    __syncthreads();
    topk_find_digit(sh, remaining);
    prefix |= topk_place(sh.digit, sub);
    remaining = sh.remaining;
  }
  uint32_t gt_base = 0u, eq_base = 0u;
  if (in_lds) {
    for (int b0 = 0; b0 < (int)total; b0 += 4 * kTopkThreads) {
      uint32_t kv[4];
      bool valid[4];
      int idx[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = b0 + 4 * tid + e;
        valid[e] = i < (int)total;
        kv[e] = valid[e] ? s_lkey[i] : 0u;
        idx[e] = valid[e] ? s_lidx[i] : 0;
      }
      topk_emit_tile(sh, kv, valid, idx, prefix, remaining, gt_base, eq_base, out);
    }
    return;
  }
  for (int c = 0; c < nrow; ++c) {                   // each chunk's candidates one tile
    const int cnt = (int)s_cnt[c];
    uint32_t kv[4];
    bool valid[4];
    int idx[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * tid + e;
      valid[e] = j < cnt;
      kv[e] = valid[e] ? ckey[(int64_t)c * kCkKeys + j] : 0u;
      idx[e] = valid[e] ? cidx[(int64_t)c * kCkKeys + j] : 0;
    }
    topk_emit_tile(sh, kv, valid, idx, prefix, remaining, gt_base, eq_base, out);
  }
}

// ---------------------------------------------------------------- scoring, many rows
// Many query rows over few sequences (prefill): a workgroup scores a tile of rows against a
// 2048-entry range, so each key page is read once per row tile instead of once per row.
// The (row, head) pairs form the MFMA's M dimension (heads padded to HP = 4, 8 or 16; 128
// pairs per wave in 8 blocks of 16), entries its N dimension and the 64 key channels its
// K dimension (two 32-channel steps, the eight blocks' chains interleaved); the head sum
// w . ReLU(.) runs on the accumulators.  Key pages arrive by LDS DMA into a ring of four,
// three pages ahead, chunk c (16 bytes) of key k at slot c ^ ((k >> 1) & 7), so that the 16
// lanes of an operand read hit distinct banks.  A wave's scores of a page pass through LDS
// and leave a page later as 256-byte row segments.  Every wave issues two DMA loads per page
// (pages past the end reload the last one), so one counter value names the page to wait
// for.  Rows of a tile that belong to different sequences are scored in one pass per
// sequence.
constexpr int kGemmRing = 4;
// 16-pair MFMA row blocks per wave: 4 (not 8) leaves registers for three waves per SIMD,
// which hide each other's barrier and epilogue time (prefill scoring 1332 -> 1093 us)
constexpr int kGemmBlocks = 4;
constexpr int kGemmWavesPerSimd = 3;
constexpr int kGemmPageBytes = kPage * kDidx * 2;

// Barrier with this wave's LDS accesses complete and no wait on vector memory (the key
// pages arrive by LDS DMA, awaited explicitly); `lds` counts as written by it.
__device__ __forceinline__ void dma_barrier(const void* lds) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : "v"(lds) : "memory");
}

// s_waitcnt vmcnt(N) for a compile-time N < 64 (other counters unrestricted)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// MODE (kGemmKeys, kGemmSample, kGemmCand): see IdxScoreParams.  A workgroup's chunk is 32
// pages of the "page space": page space page q is logical page q * G of the sequence (G =
// page_gap in sample mode, else 1), and its keys go to columns 64 q .. 64 q + 63.
template <int HP, int MODE>
__global__ __launch_bounds__(256, kGemmWavesPerSimd) void idx_gemm_kernel(IdxScoreParams p) {
  constexpr int RB = 16 / HP;            // rows per 16-pair MFMA block
  constexpr int NRB = kGemmBlocks;       // blocks per wave
  constexpr int RW = RB * NRB;           // rows per wave
  constexpr int RT = 4 * RW;             // rows per workgroup
  constexpr int S = RW / 4;              // stores per wave and page
  // the ring's pages are separate arrays, indexed statically, so that the compiler can tell
  // a page being read from the pages whose DMA is still in flight
  __shared__ __attribute__((aligned(16))) uint8_t s_pg0[kGemmPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_pg1[kGemmPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_pg2[kGemmPageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_pg3[kGemmPageBytes];
  __shared__ __attribute__((aligned(16))) float s_out[2][4][RW][kPage];
  __shared__ int s_seq[RT], s_nv[RT];
  __shared__ float s_thr[MODE == kGemmCand ? RT : 1];   // thresholds as scores
  __shared__ int s_any;

  for (int i = (int)(blockIdx.x * 256 + threadIdx.x); i < p.clear_words; i += (int)gridDim.x * 256)
    p.clear[i] = 0u;
  const int G = (MODE == kGemmSample) ? p.page_gap : 1;
  const int nrt = (p.T + RT - 1) / RT;
  const int rt = (int)blockIdx.x % nrt, ch = (int)blockIdx.x / nrt;   // an XCD's blocks share ch
  const int t0 = rt * RT, q0 = ch * (kGemmChunk / kPage);            // first page-space page
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const bool filtered = MODE == kGemmKeys && p.row_flags != nullptr;
  if (tid == 0) s_any = 0;
  __syncthreads();
  for (int i = tid; i < RT; i += 256) {
    const int t = t0 + i;
    s_seq[i] = t < p.T ? p.seq_id[t] : -1;
    s_nv[i] = t < p.T ? p.n_vis[t] : 0;
    if (MODE == kGemmCand) s_thr[i] = t < p.T ? key_float(p.thr[t]) : INFINITY;
    if (filtered && t < p.T && p.row_flags[t]) s_any = 1;
  }
  __syncthreads();
  if (filtered && !s_any) return;                    // no row of this tile needs the keys

  const int rw0 = wave * RW;                         // first tile row of the wave
  int prev = -1;
  for (;;) {
    // next sequence of the tile (in increasing id, the same in every lane) and the entries
    // its rows see
    int cur = INT32_MAX, nvmax = 0;
    for (int i = 0; i < RT; ++i) {
      const int sq = s_seq[i];
      if (sq > prev && sq < cur) cur = sq;
    }
    if (cur == INT32_MAX) break;
    for (int i = 0; i < RT; ++i)
      if (s_seq[i] == cur) nvmax = max(nvmax, s_nv[i]);
    cur = __builtin_amdgcn_readfirstlane(cur);
    prev = cur;
    // page-space pages holding visible entries of some row of this sequence, in this chunk
    const int vq = ((nvmax + kPage - 1) / kPage + G - 1) / G;
    const int np = __builtin_amdgcn_readfirstlane(min(max(vq - q0, 0), kGemmChunk / kPage));
    uint32_t cnt[S];                                   // kGemmCand: candidates so far, per row
#pragma unroll
    for (int r4 = 0; r4 < S; ++r4) cnt[r4] = 0u;
    if (np == 0) continue;

    // operands of this wave's rows (zero for rows of other sequences and padded heads)
    u32x4 qa[NRB][2];
    float wv[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int ra = rw0 + RB * rb + n / HP, ha = n % HP;
      const bool va = s_seq[ra] == cur && ha < p.H_I;
      const uint16_t* qp = p.q_idx + ((int64_t)(t0 + ra) * p.H_I + ha) * kDidx + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        qa[rb][ks] = va ? ld_global_16(qp + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rw0 + RB * rb + (4 * g + i) / HP, h = (4 * g + i) % HP;
        wv[rb][i] = (s_seq[r] == cur && h < p.H_I) ? p.w_idx[(int64_t)(t0 + r) * p.H_I + h] : 0.f;
      }
    }
    // store targets of this wave's rows (a row is written only where its sequence is
    // scored and its entries are visible; other lanes store to the sink)
    uint32_t* const sink = p.trash + 4 * lane;
    // physical pages of the range, one per lane (read once: a load in the page loop would
    // count among the operations the loop waits for)
    const int my_page =
        lane < np ? p.page_table[(int64_t)cur * p.max_pages + (int64_t)(q0 + lane) * G] : 0;
    // DMA of page pp (clamped to the last page) into ring slot `dst`: wave w moves keys
    // 16w .. 16w+15 (two 1 KB units)
    auto dma_page = [&](int pp, uint8_t* dst) {
      const int64_t prow = (int64_t)__shfl(my_page, min(pp, np - 1)) * kPage;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int k = 16 * wave + 8 * d + (lane >> 3);
        const int c = (lane & 7) ^ ((k >> 1) & 7);
        __builtin_amdgcn_global_load_lds(p.k_idx + (prow + k) * kDidx + 8 * c,
                                         dst + 1024 * (2 * wave + d), 16, 0, 0);
      }
    };
    // this wave's rows of page pp's scores (LDS buffer pp & 1), 256 bytes per row; masked
    // lanes store to the sink
    auto store_page = [&](int pp) {
      const int col = kPage * (q0 + pp) + 4 * n;       // key column of the lane's first entry
      const int e0 = kPage * (q0 + pp) * G + 4 * n;    // its entry
#pragma unroll
      for (int r4 = 0; r4 < S; ++r4) {
        const int rl = 4 * r4 + g;
        const int r = rw0 + rl;
        const f32x4 v = *reinterpret_cast<const f32x4*>(&s_out[pp & 1][wave][rl][4 * n]);
        u32x4 kk;
        if (MODE != kGemmCand) {
#pragma unroll
          for (int e = 0; e < 4; ++e) kk[e] = float_key(v[e]);
        }
        const bool row_ok = s_seq[r] == cur;
        if (MODE == kGemmKeys) {
          const bool ok = row_ok && e0 < s_nv[r];
          uint32_t* dst = ok ? p.keys + (int64_t)(t0 + r) * p.key_stride + col : sink;
          *reinterpret_cast<u32x4*>(dst) = kk;
        } else if (MODE == kGemmSample) {            // masked entries read as 0
#pragma unroll
          for (int e = 0; e < 4; ++e) kk[e] = (e0 + e < s_nv[r]) ? kk[e] : 0u;
          uint32_t* dst = row_ok ? p.keys + (int64_t)(t0 + r) * p.key_stride + col : sink;
          *reinterpret_cast<u32x4*>(dst) = kk;
        } else {
          // keys at or above the row's threshold, appended in entry order: the 16 lanes of
          // lane group g hold the row's 64 entries of the page, four each
          // !(score < threshold score) is key >= threshold key (the key map is monotone,
          // -0 and +0 share a key and compare equal, and a NaN score, whose key is above
          // every finite one, passes)
          const float th = s_thr[r];
          uint32_t f = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            f |= (uint32_t)(row_ok && e0 + e < s_nv[r] && !(v[e] < th)) << e;
          const uint32_t c = (uint32_t)__popc(f);
          const uint32_t incl = row16_incl_scan(c);
          const uint32_t tot = row16_last(incl);
          if (__ballot(f != 0u)) {                   // a wave-uniform test: mostly taken
            const int64_t base = ((int64_t)(t0 + r) * p.n_chunks + ch) * kCandCap;
            uint32_t pos = cnt[r4] + incl - c;
            while (f) {                              // the lane's candidates, in order
              const int e = __builtin_ctz(f);
              if (pos < (uint32_t)kCandCap) {
                p.cand_key[base + pos] = float_key(v[e]);
                p.cand_idx[base + pos] = e0 + e;
              }
              ++pos;
              f &= f - 1u;
            }
          }
          cnt[r4] += tot;
        }
      }
    };
    // One page: the stores of page pp-1, page pp's operands from slot `kp`, the DMA of page
    // pp+3 into slot `nx`, the MFMAs, and the wait for page pp+1.  The wait counts only the
    // loads issued after page pp+1's (those of pages pp+2 and pp+3): loads complete in
    // order, while stores may complete before earlier loads.
    auto page_step = [&](int pp, const uint8_t* kp, uint8_t* nx) {
      dma_barrier(s_pg0);                              // page pp in LDS, page pp-1 consumed
      if (pp > 0) store_page(pp - 1);
      u32x4 kv[4][2];                                  // all operands read before the DMA
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int k = 16 * kb + n;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          kv[kb][ks] = *reinterpret_cast<const u32x4*>(kp + 128 * k + 16 * ((4 * ks + g) ^ ((k >> 1) & 7)));
      }
      dma_page(pp + 3, nx);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int k = 16 * kb + n;
        f32x4 acc[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[rb][0]), as_bf16x8(kv[kb][0]),
                                                            f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[rb][1]), as_bf16x8(kv[kb][1]),
                                                            acc[rb], 0, 0, 0);
        float sc[NRB];                                 // this lane's heads, per block
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          sc[rb] = wv[rb][0] * relu_f32(acc[rb][0]);
          sc[rb] += wv[rb][1] * relu_f32(acc[rb][1]);
          sc[rb] += wv[rb][2] * relu_f32(acc[rb][2]);
          sc[rb] += wv[rb][3] * relu_f32(acc[rb][3]);
        }
        if (HP == 4) {                                 // lane group g is row g of the block
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) s_out[pp & 1][wave][RB * rb + g][k] = sc[rb];
        } else if (HP == 8) {
          // a row's heads sit in lane groups 2r and 2r + 1: one v_permlane16_swap of two
          // blocks' sums leaves groups 0 and 2 with block 2j's rows 0 and 1, groups 1 and 3
          // with block 2j + 1's (a reduce-scatter: no copy, every value written once)
#pragma unroll
          for (int j = 0; j < NRB / 2; ++j) {
            const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(sc[2 * j]),
                                                            __float_as_uint(sc[2 * j + 1]), false, false);
            const float v = __uint_as_float(c[0]) + __uint_as_float(c[1]);
            s_out[pp & 1][wave][RB * (2 * j + (g & 1)) + (g >> 1)][k] = v;
          }
        } else {
          // one row per block over all four lane groups: v_permlane32_swap pairs blocks 0, 2
          // and 1, 3 across groups g and g + 2, then v_permlane16_swap leaves group g with
          // block g's whole sum
          static_assert(HP != 16 || NRB == 4, "four blocks per wave at 16 heads");
          const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc[0]), __float_as_uint(sc[2]), false, false);
          const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc[1]), __float_as_uint(sc[3]), false, false);
          const float ha = __uint_as_float(a[0]) + __uint_as_float(a[1]);
          const float hb = __uint_as_float(b[0]) + __uint_as_float(b[1]);
          const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(ha), __float_as_uint(hb), false, false);
          s_out[pp & 1][wave][g][k] = __uint_as_float(c[0]) + __uint_as_float(c[1]);
        }
      }
      wait_vmem<4>();                                  // page pp+1 in LDS
    };
    dma_page(0, s_pg0);
    dma_page(1, s_pg1);
    dma_page(2, s_pg2);
    wait_vmem<4>();                                    // page 0
    for (int pp = 0; pp < np; pp += kGemmRing) {
      page_step(pp, s_pg0, s_pg3);
      if (pp + 1 >= np) break;
      page_step(pp + 1, s_pg1, s_pg0);
      if (pp + 2 >= np) break;
      page_step(pp + 2, s_pg2, s_pg1);
      if (pp + 3 >= np) break;
      page_step(pp + 3, s_pg3, s_pg2);
    }
    store_page(np - 1);
    if (MODE == kGemmCand && n == 0) {               // the rows' counts for this chunk
#pragma unroll
      for (int r4 = 0; r4 < S; ++r4) {
        const int r = rw0 + 4 * r4 + g;
        if (s_seq[r] == cur) {
          p.cand_cnt[(int64_t)(t0 + r) * p.n_chunks + ch] = cnt[r4];
          if (cnt[r4] > (uint32_t)kCandCap) p.row_flags[t0 + r] = 1u;
        }
      }
    }
    wait_vmem<0>();
    dma_barrier(s_pg0);                                // ring free for the next pass
  }
}

template <int MODE>
hipError_t launch_idx_gemm(const IdxScoreParams& p, unsigned blocks, hipStream_t s) {
  const int hp = p.H_I <= 4 ? 4 : (p.H_I <= 8 ? 8 : 16);
  if (hp == 4) CSA2_LAUNCH((idx_gemm_kernel<4, MODE>), dim3(blocks), dim3(256), s, p);
  else if (hp == 8) CSA2_LAUNCH((idx_gemm_kernel<8, MODE>), dim3(blocks), dim3(256), s, p);
  else CSA2_LAUNCH((idx_gemm_kernel<16, MODE>), dim3(blocks), dim3(256), s, p);
  return hipGetLastError();
}

hipError_t launch_idx_score(const IdxScoreParams& p, hipStream_t s) {
  if (p.T >= kIdxGemmMinRows && !p.pool_sel) {
    // page-space columns: key_stride (every page, or the packed sample)
    const int64_t nch = (p.key_stride + kGemmChunk - 1) / kGemmChunk;
    const int hp = p.H_I <= 4 ? 4 : (p.H_I <= 8 ? 8 : 16);
    const int rt = 4 * kGemmBlocks * (16 / hp);       // rows per workgroup
    const unsigned blocks = (unsigned)(((int64_t)p.T + rt - 1) / rt * nch);
    if (p.gemm_mode == kGemmSample) return launch_idx_gemm<kGemmSample>(p, blocks, s);
    if (p.gemm_mode == kGemmCand) return launch_idx_gemm<kGemmCand>(p, blocks, s);
    return launch_idx_gemm<kGemmKeys>(p, blocks, s);
  }
  const int64_t blocks = (p.block_end > 0 ? (int64_t)p.block_end : (int64_t)p.T * p.chunks) - p.block0;
  if (blocks <= 0) return hipSuccess;
  if (p.pool_sel) CSA2_LAUNCH(idx_pool_score_kernel, dim3((unsigned)blocks), dim3(256), s, p);
  else if (p.ppw == 4) CSA2_LAUNCH(idx_score_kernel<4>, dim3((unsigned)blocks), dim3(256), s, p);
  else CSA2_LAUNCH(idx_score_kernel<8>, dim3((unsigned)blocks), dim3(256), s, p);
  return hipGetLastError();
}

hipError_t launch_idx_score_swa(const IdxScoreParams& p, const SwaParams& w, int swa_blocks,
                                hipStream_t s) {
  const int64_t blocks = (int64_t)p.T * p.chunks + swa_blocks;
  if (p.ppw == 4) CSA2_LAUNCH(idx_score_swa_kernel<4>, dim3((unsigned)blocks), dim3(256), s, p, w, swa_blocks);
  else CSA2_LAUNCH(idx_score_swa_kernel<8>, dim3((unsigned)blocks), dim3(256), s, p, w, swa_blocks);
  return hipGetLastError();
}

// One launch of the chunked Top-K (1: top-digit histogram, 2: candidates, 3: selection and
// emission); the row histograms must be zero before launch 1.
hipError_t launch_topk_chunked(const TopkParams& p, int pass, hipStream_t s) {
  const unsigned blocks = (unsigned)((int64_t)p.T * topk_chunks(p.key_stride));
  const dim3 block(kCkThreads);
  switch (pass) {
    case 1: CSA2_LAUNCH(topk_ck_hist_kernel, dim3(blocks), block, s, p); break;
    case 2: CSA2_LAUNCH(topk_ck_compact_kernel, dim3(blocks), block, s, p); break;
    case 3: CSA2_LAUNCH(topk_ck_select_kernel, dim3((unsigned)p.T), dim3(kTopkThreads), s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.T), block(kTopkThreads);
  if (p.pool_sel) {                                  // at most 8 * kPoolMaxSel slots
    const int slots = kPoolBlock * p.pool_K;
    if (slots <= 4 * kTopkThreads) CSA2_LAUNCH((topk_pool_kernel<1>), grid, block, s, p);
    else if (slots <= 8 * kTopkThreads) CSA2_LAUNCH((topk_pool_kernel<2>), grid, block, s, p);
    else if (slots <= 16 * kTopkThreads) CSA2_LAUNCH((topk_pool_kernel<4>), grid, block, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  // key_stride bounds every row's n_vis; pick the register-resident variant that holds it
  const int64_t nr = (p.key_stride + 4 * kTopkThreads - 1) / (4 * kTopkThreads);
  if (nr <= 2) CSA2_LAUNCH((topk_row_kernel<2>), grid, block, s, p);
  else if (nr <= 4) CSA2_LAUNCH((topk_row_kernel<4>), grid, block, s, p);
  else if (nr <= 8) CSA2_LAUNCH((topk_row_kernel<8>), grid, block, s, p);
  else if (nr <= 16) CSA2_LAUNCH((topk_row_kernel<16>), grid, block, s, p);
  else if (!topk_chunked(p.T, p.key_stride)) CSA2_LAUNCH(topk_stream_kernel, grid, block, s, p);
  else return hipErrorInvalidValue;                  // chunked rows go through launch_topk_chunked
  return hipGetLastError();
}

}  // namespace csa2
