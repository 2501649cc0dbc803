// Sparse global attention over the Top-K selected MXFP4 entries (CSA2 global branch) on
// gfx950.
//
// [summary] = picx.dev whiteboard summary "DeepSeek-V4.1-Flash: Pushing the Limits of KV
// Cache Compression", Methodology > Architecture Components: item 2 (CSA2 attends over
// the Top-K selected compressed entries), item 5 (FP4 main KV: E2M1 codes with shared
// power-of-two scales; read here as OCP MXFP4, one E8M0 scale per 32 channels).
// Every head of a row shares each entry (MLA-style latent): key = [latent ; rope] (576),
// value = latent (512).
//
// Kernel design (one workgroup per (row, split of the K slots), one wave per 16 heads):
//   gather   : the split's physical rows are resolved once into LDS; per 32-entry tile the
//              workgroup issues coalesced 16-byte loads of the latent codes, scales and
//              rope rows (next tile's loads in flight while the current one computes) and
//              stages the raw bytes in LDS.
//   QK^T     : S^T[entries x heads] on bf16 MFMA 16x16x32; the A operand (keys) is
//              dequantized in registers straight from the staged FP4 bytes with the
//              scaled-convert instruction (exact: e2m1 * 2^k is a bf16); the B operand is
//              the wave's 16 query heads held in registers for the whole kernel.
//   softmax  : online, per head, in the log2 domain, fp32.
//   PV       : O^T[channels x heads] += V^T P^T on fp16 MFMA 16x16x32 with fp32
//              accumulation.  V^T is dequantized once per tile into LDS (fp16, channel
//              major); P stays in registers (the S^T result layout is already the B
//              operand layout of the PV product, up to a permutation of the contraction
//              index applied to V^T alike).  fp16 rather than bf16 for P: bf16 rounding of
//              P alone would put the output's relative error near 1.7e-3.
// Splits write normalized partial outputs plus log2-sum-exp; a merge kernel combines them.
#include "csa2_internal.h"
#include "csa2_device.h"

namespace csa2 {

constexpr int kTE = 32;             // entries per tile
constexpr int kLatStride = 272;     // LDS bytes per staged latent row (256 + 16 pad)
constexpr int kRopeStride = 144;    // LDS bytes per staged rope row (128 + 16 pad)
constexpr int kVtStride = 72;       // LDS bytes per V^T channel row (32 fp16 + 8 pad)
constexpr int kMaxPerSplit = 2048;  // idx slots per split (LDS row table size)

void attn_plan(int T, int H, int K, int* splits, int* per_split) {
  (void)H;
  const int min_s = (K + kMaxPerSplit - 1) / kMaxPerSplit;
  const int max_s = max(1, (K + 2 * kTE - 1) / (2 * kTE));   // >= 2 tiles per split
  int s = (T > 0) ? (256 + T - 1) / T : 1;
  s = min(s, max_s);
  s = max(s, min_s);
  // whole tiles per split; the split count follows from the rounded slot count
  int per = (K + s - 1) / s;
  per = (per + kTE - 1) / kTE * kTE;
  *per_split = per;
  *splits = (K + per - 1) / per;
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void sparse_attn_kernel(AttnParams p) {
  constexpr int NT = 64 * NW;
  constexpr int LAT_PER_T = (kTE * 16 + NT - 1) / NT;
  constexpr int ROPE_PER_T = (kTE * 8 + NT - 1) / NT;
  constexpr int VT_ITEMS = (kTE / 4) * (kLat / 8);            // (entry quad, channel octet)
  constexpr int VT_PER_T = (VT_ITEMS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint8_t s_lat[kTE * kLatStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[kTE * kScl];
  __shared__ __attribute__((aligned(16))) uint8_t s_rope[kTE * kRopeStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_vt[kLat * kVtStride];
  __shared__ int32_t s_rows[kMaxPerSplit];

  const int t = blockIdx.x / p.splits;
  const int sp = blockIdx.x - t * p.splits;
  const int k0 = sp * p.per_split;
  const int k1 = min(k0 + p.per_split, p.K);
  const int nslots = max(k1 - k0, 0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int h = wave * 16 + n;

  // ---- resolve the split's physical rows once (-1 = empty slot)
  {
    const int b = p.seq_id[t];
    const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
    const int32_t* idx = p.idx + (int64_t)t * p.K + k0;
    const int ntile_slots = (nslots + kTE - 1) / kTE * kTE;
    for (int i = tid; i < ntile_slots; i += NT) {
      int32_t row = -1;
      if (i < nslots) {
        const int j = idx[i];
        if (j >= 0) row = pt[j >> 6] * kPage + (j & 63);
      }
      s_rows[i] = row;
    }
  }

  // ---- query heads as the QK^T B operand: lane (g, n) holds head h, channel slots of g
  u32x4 qb[18];
  {
    const uint16_t* qp = p.q + ((int64_t)t * p.H + h) * kDq;
#pragma unroll
    for (int s = 0; s < 16; ++s)
      qb[s] = ld_global_16(qp + 128 * (s >> 2) + 32 * g + 8 * (s & 3));
#pragma unroll
    for (int s = 0; s < 2; ++s) qb[16 + s] = ld_global_16(qp + kLat + 32 * s + 8 * g);
  }

  f32x4 acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  __syncthreads();
  const int ntiles = (nslots + kTE - 1) / kTE;

  u32x4 r_lat[LAT_PER_T], r_rope[ROPE_PER_T], r_scl = {0u, 0u, 0u, 0u};
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int r = 0; r < LAT_PER_T; ++r) {
      const int c = tid + NT * r;
      r_lat[r] = u32x4{0u, 0u, 0u, 0u};
      if (c < kTE * 16) {
        const int row = s_rows[tile * kTE + (c >> 4)];
        if (row >= 0) r_lat[r] = ld_global_16(p.kv_lat + (int64_t)row * kLatBytes + (c & 15) * 16);
      }
    }
#pragma unroll
    for (int r = 0; r < ROPE_PER_T; ++r) {
      const int c = tid + NT * r;
      r_rope[r] = u32x4{0u, 0u, 0u, 0u};
      if (c < kTE * 8) {
        const int row = s_rows[tile * kTE + (c >> 3)];
        if (row >= 0) r_rope[r] = ld_global_16(p.kv_rope + (int64_t)row * kRope + (c & 7) * 8);
      }
    }
    if (tid < kTE) {
      const int row = s_rows[tile * kTE + tid];
      r_scl = (row >= 0) ? ld_global_16(p.kv_scl + (int64_t)row * kScl) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < LAT_PER_T; ++r) {
      const int c = tid + NT * r;
      if (c < kTE * 16)
        *reinterpret_cast<u32x4*>(s_lat + (c >> 4) * kLatStride + (c & 15) * 16) = r_lat[r];
    }
#pragma unroll
    for (int r = 0; r < ROPE_PER_T; ++r) {
      const int c = tid + NT * r;
      if (c < kTE * 8)
        *reinterpret_cast<u32x4*>(s_rope + (c >> 3) * kRopeStride + (c & 7) * 16) = r_rope[r];
    }
    if (tid < kTE) *reinterpret_cast<u32x4*>(s_scl + tid * kScl) = r_scl;
  };

  if (ntiles > 0) load_tile(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    store_tile();
    __syncthreads();
    if (tile + 1 < ntiles) load_tile(tile + 1);

    // ---- V^T (fp16, channel-major) for the tile: item = (entry quad, channel octet)
#pragma unroll
    for (int r = 0; r < VT_PER_T; ++r) {
      const int it = tid + NT * r;
      if (it < VT_ITEMS) {
        const int eq = it & 7;            // entries 4eq .. 4eq+3
        const int co = it >> 3;           // channels 8co .. 8co+7
        uint32_t hv[4][4];                // [entry][channel pair] packed f16x2
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * eq + i;
          const uint32_t w = *reinterpret_cast<const uint32_t*>(s_lat + e * kLatStride + 4 * co);
          const float sc = e8m0_to_f32(s_scl[e * kScl + (co >> 2)]);
          fp4x8_to_f16_pairs(w, sc, hv[i]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          u32x2 lo, hi;   // channel 2k and 2k+1 of the octet, entries 4eq..4eq+3
          lo[0] = (hv[0][k] & 0xffffu) | (hv[1][k] << 16);
          lo[1] = (hv[2][k] & 0xffffu) | (hv[3][k] << 16);
          hi[0] = (hv[0][k] >> 16) | (hv[1][k] & 0xffff0000u);
          hi[1] = (hv[2][k] >> 16) | (hv[3][k] & 0xffff0000u);
          *reinterpret_cast<u32x2*>(s_vt + (8 * co + 2 * k) * kVtStride + 8 * eq) = lo;
          *reinterpret_cast<u32x2*>(s_vt + (8 * co + 2 * k + 1) * kVtStride + 8 * eq) = hi;
        }
      }
    }

    // ---- S^T = K Q^T for the tile (two 16-entry M-blocks)
    f32x4 sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int e = 16 * mb + n;
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      const u32x4 sc4 = *reinterpret_cast<const u32x4*>(s_scl + e * kScl);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x4 w4 = *reinterpret_cast<const u32x4*>(s_lat + e * kLatStride + 64 * q4 + 16 * g);
        const float sc = e8m0_to_f32((sc4[q4] >> (8 * g)) & 255u);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16(w4[r], sc),
                                                      as_bf16x8(qb[4 * q4 + r]), a, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4 rv = *reinterpret_cast<const u32x4*>(s_rope + e * kRopeStride + 64 * s + 16 * g);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rv), as_bf16x8(qb[16 + s]), a, 0, 0, 0);
      }
      sacc[mb] = a;
    }

    // ---- online softmax (lane: head n, entries 16mb + 4g + i)
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = s_rows[tile * kTE + 16 * mb + 4 * g + i] >= 0;
        const float v = ok ? sacc[mb][i] * p.sm_scale_log2 : -INFINITY;
        x[4 * mb + i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    __syncthreads();                      // V^T complete
    if (m_new != -INFINITY) {             // uniform across the workgroup (shared mask)
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      f16x8 pb;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(x[i] - m_new);
        psum += pv;
        pb[i] = (_Float16)pv;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] *= alpha;
      // ---- O^T += V^T P^T: A row = channel 16c + n, contraction slots of lane group g
      //      are entries 4g..4g+3 then 16+4g..16+4g+3 (the S^T result rows of this lane)
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        const uint8_t* vrow = s_vt + (16 * c + n) * kVtStride;
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(vrow + 8 * g);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(vrow + 32 + 8 * g);
        const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(va), pb, acc[c], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: normalize, write (partial) output and log2-sum-exp
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const float lse2 = (l_tot > 0.f) ? m_run + __log2f(l_tot) : -INFINITY;
  float* obase;
  if (p.splits == 1) {
    obase = p.o + ((int64_t)t * p.H + h) * kLat;
    if (g == 0) p.lse[(int64_t)t * p.H + h] = lse2 * 0.69314718055994530942f;
  } else {
    const int64_t slot = ((int64_t)t * p.splits + sp) * p.H + h;
    obase = p.o_part + slot * kLat;
    if (g == 0) p.lse_part[slot] = lse2;
  }
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const f32x4 v = acc[c] * inv;
    *reinterpret_cast<f32x4*>(obase + 16 * c + 4 * g) = v;
  }
}

// o = sum_s 2^(lse2_s - lse2) o_s, lse2 = log2 sum_s 2^lse2_s; one block per (row, head).
__global__ __launch_bounds__(128) void attn_merge_kernel(MergeParams p) {
  const int th = blockIdx.x;
  const int t = th / p.H, h = th - t * p.H;
  const int S = p.splits;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, p.lse_part[((int64_t)t * S + s) * p.H + h]);
  float* o = p.o + ((int64_t)t * p.H + h) * kLat;
  const int c = 4 * threadIdx.x;
  if (mx == -INFINITY) {
    *reinterpret_cast<f32x4*>(o + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (threadIdx.x == 0) p.lse[(int64_t)t * p.H + h] = -INFINITY;
    return;
  }
  float z = 0.f;
  for (int s = 0; s < S; ++s)
    z += __builtin_amdgcn_exp2f(p.lse_part[((int64_t)t * S + s) * p.H + h] - mx);
  const float lse2 = mx + __log2f(z);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const int64_t slot = ((int64_t)t * S + s) * p.H + h;
    const float wgt = __builtin_amdgcn_exp2f(p.lse_part[slot] - lse2);
    if (wgt > 0.f) acc += wgt * *reinterpret_cast<const f32x4*>(p.o_part + slot * kLat + c);
  }
  *reinterpret_cast<f32x4*>(o + c) = acc;
  if (threadIdx.x == 0) p.lse[(int64_t)t * p.H + h] = lse2 * 0.69314718055994530942f;
}

hipError_t launch_sparse_attn(const AttnParams& p, hipStream_t s) {
  const unsigned blocks = (unsigned)((int64_t)p.T * p.splits);
  switch (p.H / 16) {
    case 1: hipLaunchKernelGGL(sparse_attn_kernel<1>, dim3(blocks), dim3(64), 0, s, p); break;
    case 2: hipLaunchKernelGGL(sparse_attn_kernel<2>, dim3(blocks), dim3(128), 0, s, p); break;
    case 4: hipLaunchKernelGGL(sparse_attn_kernel<4>, dim3(blocks), dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL(sparse_attn_kernel<8>, dim3(blocks), dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((int64_t)p.T * p.H)), dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace csa2
