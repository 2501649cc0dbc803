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
// order, -1 padded.  Radix select over order-preserving u32 keys (4 passes of 8 bits)
// finds the K-th key tau and how many keys equal to tau to keep; an ordered block-wide
// scan then compacts the selected indices in index order.
#include "csa2_internal.h"
#include "csa2_device.h"

namespace csa2 {

constexpr int kIdxWaves = 4;
constexpr int kIdxPerWave = kIdxChunk / kIdxWaves;   // 256 entries per wave
constexpr int kIdxUnroll = 4;                         // 16-entry groups in flight per wave

// One workgroup scores kIdxChunk consecutive entries of one row; each wave takes 256 of
// them, 16 per MFMA pair.  MFMA A = q_idx (rows = heads, zero-padded to 16), B = keys
// (columns = entries).  The 64 key channels are split over the two MFMAs and the four
// lane groups g as channels [16g, 16g+8) and [16g+8, 16g+16); q uses the same split, so
// each lane loads 32 contiguous key bytes.
__global__ __launch_bounds__(256) void idx_score_kernel(IdxScoreParams p) {
  const int t = blockIdx.x / p.chunks;
  const int c = blockIdx.x - t * p.chunks;
  const int nv = p.n_vis[t];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j_begin = c * kIdxChunk + wave * kIdxPerWave;
  if (j_begin >= nv) return;                 // wave-uniform; no block barriers below
  const int j_end = min(j_begin + kIdxPerWave, nv);
  const int b = p.seq_id[t];
  const int n = lane & 15, g = lane >> 4;

  u32x4 qa0 = {0u, 0u, 0u, 0u}, qa1 = {0u, 0u, 0u, 0u};
  if (n < p.H_I) {
    const uint16_t* qp = p.q_idx + ((int64_t)t * p.H_I + n) * kDidx + 16 * g;
    qa0 = ld_global_16(qp);
    qa1 = ld_global_16(qp + 8);
  }
  float w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    w[i] = (h < p.H_I) ? p.w_idx[(int64_t)t * p.H_I + h] : 0.f;
  }
  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  uint32_t* keys = p.keys + (int64_t)t * p.key_stride;

  for (int j0 = j_begin; j0 < j_end; j0 += 16 * kIdxUnroll) {
    u32x4 kb0[kIdxUnroll], kb1[kIdxUnroll];
#pragma unroll
    for (int u = 0; u < kIdxUnroll; ++u) {
      const int j = j0 + 16 * u + n;
      if (j < j_end) {
        const int64_t row = (int64_t)pt[j >> 6] * kPage + (j & 63);
        const uint16_t* kp = p.k_idx + row * kDidx + 16 * g;
        kb0[u] = ld_global_16(kp);
        kb1[u] = ld_global_16(kp + 8);
      } else {
        kb0[u] = u32x4{0u, 0u, 0u, 0u};
        kb1[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kIdxUnroll; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa0), as_bf16x8(kb0[u]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa1), as_bf16x8(kb1[u]), acc, 0, 0, 0);
      // lane holds heads 4g..4g+3 of entry n
      float s = w[0] * fmaxf(acc[0], 0.f);
      s += w[1] * fmaxf(acc[1], 0.f);
      s += w[2] * fmaxf(acc[2], 0.f);
      s += w[3] * fmaxf(acc[3], 0.f);
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      const int j = j0 + 16 * u + n;
      if (g == 0 && j < j_end) keys[j] = float_key(s);
    }
  }
}

// One workgroup (1024 threads) per row.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  constexpr int NWAVE = kTopkThreads / 64;
  __shared__ uint32_t hist[NWAVE][256];
  __shared__ uint32_t s_digit, s_remaining;
  __shared__ uint32_t wave_tot[NWAVE];

  const int t = blockIdx.x;
  const int n = p.n_vis[t];
  const int K = p.K;
  int32_t* out = p.idx_out + (int64_t)t * K;
  const uint32_t* keys = p.keys + (int64_t)t * p.key_stride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (n <= K) {                       // every visible entry is selected
    for (int i = tid; i < K; i += kTopkThreads) out[i] = (i < n) ? i : -1;
    return;
  }

  // ---- radix select of the K-th largest key
  uint32_t prefix = 0u, pmask = 0u, remaining = (uint32_t)K;
  const int n4 = n >> 2;
  const u32x4* k4 = reinterpret_cast<const u32x4*>(keys);
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < NWAVE * 256; i += kTopkThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n4; i += kTopkThreads) {
      const u32x4 v = k4[i];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((v[e] & pmask) == prefix) atomicAdd(&hist[wave][(v[e] >> shift) & 255u], 1u);
    }
    for (int i = 4 * n4 + tid; i < n; i += kTopkThreads) {
      const uint32_t v = keys[i];
      if ((v & pmask) == prefix) atomicAdd(&hist[wave][(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t cnt[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t s = 0u;
        for (int w = 0; w < NWAVE; ++w) s += hist[w][4 * lane + e];
        cnt[e] = s;
      }
      const uint32_t tot = cnt[0] + cnt[1] + cnt[2] + cnt[3];
      uint32_t suf = tot;                                // inclusive suffix sum over lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(suf, o);
        if (lane + o < 64) suf += y;
      }
      uint32_t above = suf - tot;                        // keys in higher lanes' bins
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (above < remaining && above + cnt[e] >= remaining) {
          s_digit = (uint32_t)(4 * lane + e);
          s_remaining = remaining - above;
        }
        above += cnt[e];
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    remaining = s_remaining;
  }
  const uint32_t tau = prefix;        // K-th largest key
  const uint32_t need_eq = remaining; // keys equal to tau to keep (lowest indices first)

  // ---- ordered compaction: position = (#greater before) + min(#equal before, need_eq)
  uint32_t gt_base = 0u, eq_base = 0u;
  for (int base = 0; base < n; base += 4 * kTopkThreads) {
    const int i0 = base + 4 * tid;
    uint32_t kv[4];
    if (i0 + 3 < n) {
      const u32x4 v = k4[i0 >> 2];
      kv[0] = v[0]; kv[1] = v[1]; kv[2] = v[2]; kv[3] = v[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[e] = (i0 + e < n) ? keys[i0 + e] : 0u;
    }
    uint32_t cg = 0u, ce = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool valid = i0 + e < n;
      cg += (valid && kv[e] > tau);
      ce += (valid && kv[e] == tau);
    }
    const uint32_t packed = cg | (ce << 16);
    uint32_t incl = packed;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t wave_off = 0u, tile_tot = 0u;
    for (int w = 0; w < NWAVE; ++w) {
      const uint32_t x = wave_tot[w];
      wave_off += (w < wave) ? x : 0u;
      tile_tot += x;
    }
    const uint32_t excl = wave_off + incl - packed;
    uint32_t gtb = gt_base + (excl & 0xffffu);
    uint32_t eqb = eq_base + (excl >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e >= n) break;
      if (kv[e] > tau) {
        out[gtb + min(eqb, need_eq)] = i0 + e;
        ++gtb;
      } else if (kv[e] == tau) {
        if (eqb < need_eq) out[gtb + eqb] = i0 + e;
        ++eqb;
      }
    }
    gt_base += tile_tot & 0xffffu;
    eq_base += tile_tot >> 16;
    __syncthreads();
  }
}

hipError_t launch_idx_score(const IdxScoreParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.T * p.chunks;
  hipLaunchKernelGGL(idx_score_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)p.T), dim3(kTopkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace csa2
