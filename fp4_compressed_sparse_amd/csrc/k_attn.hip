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
// One workgroup per (row, split of the K index slots).  Waves are (head group of 32 heads
// -- 16 when H = 16 --, half); with H = 64 that is 4 waves.
//   gather  : the split's physical rows are resolved once into LDS.  Each 32-entry tile
//             (8 KB codes, 4 KB rope, 0.5 KB scales) is fetched with coalesced 16-byte loads
//             into registers three tiles ahead, then written to LDS with an XOR swizzle of
//             the 16-byte slots so the operand reads below are bank-conflict free.
//   QK^T    : S^T[32 entries x 32 heads], split over the two waves of a head group by
//             channel half (288 of 576).  The latent part runs on the MXFP4 matrix path
//             (v_mfma_scale 16x16x128, A = the cached E2M1 codes with their own E8M0
//             block scales, dequantized inside the MFMA); the query enters as two fp8
//             (E4M3) parts with per-32-channel E8M0 scales, hi + lo, which reproduce the
//             bf16 query exactly.  The rope part is a bf16 MFMA.  The two partial sums
//             meet in LDS, so both waves hold the full S^T tile.
//   softmax : online, per head, log2 domain, fp32; the running maximum is raised only
//             when a tile exceeds it by more than 2^8 (fp16 P stays below 256).
//   PV      : O^T[256 channels x 32 heads] += V^T P^T on fp16 MFMA 16x16x32, fp32
//             accumulation; each wave owns one channel half.  V^T is dequantized once per
//             tile into LDS, channel-major, with entries stored in the order the P^T
//             operand already has in registers (the S^T result rows of a lane), so every
//             V^T operand is one 16-byte LDS read.  fp16 rather than bf16 for P: bf16
//             rounding of P alone would put the output's relative error near 1.7e-3.
// Splits write normalized partial outputs plus log2-sum-exp; a merge kernel combines them.
#include "csa2_internal.h"
#include "csa2_device.h"

namespace csa2 {

constexpr int kTE = 32;              // entries per tile
constexpr int kMaxPerSplit = 2048;   // idx slots per split (LDS row table size)
constexpr int kNPre = 3;             // tiles in flight in registers
// raw tile layout in LDS (bytes): codes [32][256], rope [32][128], scales [32][16]
constexpr int kRawLat = 0, kRawRope = 8192, kRawScl = 12288, kRawBytes = 12800;
constexpr int kChunks = 13;          // 1 KB load units per tile: 8 codes, 4 rope, 1 scales
constexpr int kVtStride = 80;        // LDS bytes per V^T channel row (32 fp16 + 16 pad)

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

// An all-zero row stands in for empty index slots (so staged tiles never hold garbage).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[256];

// Position of entry e of a tile in a V^T row: the P^T operand of lane group g carries
// entries 4g..4g+3 then 16+4g..16+4g+3, so contraction slots 8g..8g+7 map to those.
__device__ __forceinline__ int vt_pos(int e) {
  return (e < 16) ? (8 * (e >> 2) + (e & 3)) : (8 * ((e - 16) >> 2) + 4 + (e & 3));
}

template <int NHG, int NB>   // NHG head groups of 16*NB heads; waves = 2 * NHG
__global__ __launch_bounds__(128 * NHG) void sparse_attn_kernel(AttnParams p) {
  constexpr int HG = 16 * NB;                                 // heads per group
  constexpr int NW = 2 * NHG;
  constexpr int NT = 64 * NW;
  constexpr int CPW = (kChunks + NW - 1) / NW;                // load units per wave
  constexpr int VT_ITEMS = (kTE / 4) * (kLat / 8);            // (entry quad, channel octet)
  constexpr int VT_PER_T = (VT_ITEMS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint8_t s_raw[2][kRawBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_vt[kLat * kVtStride];
  __shared__ __attribute__((aligned(16))) f32x4 s_part[NW][2 * NB][64];
  __shared__ int32_t s_rows[kMaxPerSplit];

  const int t = blockIdx.x / p.splits;
  const int sp = blockIdx.x - t * p.splits;
  const int k0 = sp * p.per_split;
  const int nslots = max(min(k0 + p.per_split, p.K) - k0, 0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int hg = wave >> 1, half = wave & 1;       // head group; channel half
  const int ntiles = (nslots + kTE - 1) / kTE;

  // ---- resolve the split's physical rows once (-1 = empty slot)
  {
    const int b = p.seq_id[t];
    const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
    const int32_t* idx = p.idx + (int64_t)t * p.K + k0;
    for (int i = tid; i < ntiles * kTE; i += NT) {
      int32_t row = -1;
      if (i < nslots) {
        const int j = idx[i];
        if (j >= 0) row = pt[j >> 6] * kPage + (j & 63);
      }
      s_rows[i] = row;
    }
  }

  // ---- query operands of this wave (heads HG*hg + 16nb + n, channel half `half`)
  // Latent part, per 128-channel chunk kk of the half: the scaled MFMA pairs A lane group
  // gA (one 32-channel block 4kk + gA of an entry) with B lane group 2(gA&1) + (p >= 16),
  // byte p%16 + 16(gA>>1).  So B lane (g, n) carries channels 32(4kk + g/2) + 16(g&1) + [0,16)
  // in bytes 0..15 and the same run of block 4kk + g/2 + 2 in bytes 16..31; it supplies the
  // E8M0 scale of block 4kk + g.  Each block is scaled by 2^X, X = floor(log2 max|q|) - 7,
  // and split as hi = fp8(q 2^-X), lo = fp8(q 2^-X - hi): exact for every bf16 value within
  // 2^9 of the block maximum, and within 2^-16 of it below that.
  i32x8 qhi[NB][2], qlo[NB][2];
  int qsc[NB][2];
  u32x4 qrope[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint16_t* qp = p.q + ((int64_t)t * p.H + HG * hg + 16 * nb + n) * kDq;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int kk = 2 * half + k2;
      const int c0 = 32 * (4 * kk + (g >> 1)) + 16 * (g & 1);
      float x[2][16];
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const u32x4 v0 = ld_global_16(qp + c0 + 64 * run);
        const u32x4 v1 = ld_global_16(qp + c0 + 64 * run + 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[run][2 * e] = __uint_as_float(v0[e] << 16);
          x[run][2 * e + 1] = __uint_as_float(v0[e] & 0xffff0000u);
          x[run][8 + 2 * e] = __uint_as_float(v1[e] << 16);
          x[run][8 + 2 * e + 1] = __uint_as_float(v1[e] & 0xffff0000u);
        }
      }
      int X[2];
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        float am = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(x[run][e]));
        am = fmaxf(am, __shfl_xor(am, 16));          // the other half of the block
        const uint32_t ab = __float_as_uint(am);
        const int E = (int)(ab >> 23);
        X[run] = (ab == 0u) ? -127 : min(max((E ? E - 127 : -127) - 7, -127), 127);
      }
      // scale this lane supplies: block 4kk + g (g = 0: run 0 here, g = 3: run 1 here,
      // g = 1: run 0 of lane g = 3, g = 2: run 1 of lane g = 0)
      const int x0o = __shfl_xor(X[0], 32), x1o = __shfl_xor(X[1], 32);
      const int Xs = (g == 0) ? X[0] : (g == 3) ? X[1] : (g == 1) ? x0o : x1o;
      qsc[nb][k2] = Xs + 127;
      i32x8 hi, lo;
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const float inv = __uint_as_float((uint32_t)(127 - X[run]) << 23);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float y[4], r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = x[run][4 * d + e] * inv;
          int h = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          h = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], h, true);
          r[0] = y[0] - __builtin_amdgcn_cvt_f32_fp8(h, 0);
          r[1] = y[1] - __builtin_amdgcn_cvt_f32_fp8(h, 1);
          r[2] = y[2] - __builtin_amdgcn_cvt_f32_fp8(h, 2);
          r[3] = y[3] - __builtin_amdgcn_cvt_f32_fp8(h, 3);
          int l = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
          l = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], l, true);
          hi[4 * run + d] = h;
          lo[4 * run + d] = l;
        }
      }
      qhi[nb][k2] = hi;
      qlo[nb][k2] = lo;
    }
    qrope[nb] = ld_global_16(qp + kLat + 32 * half + 8 * g);
  }

  f32x4 acc[16][NB];
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
  }

  wait_vmem_all();                                   // Q operands are in registers
  __syncthreads();                                   // s_rows ready

  // ---- gather: load unit j of a tile = 1 KB, lane l moves 16 bytes
  //   j < 8      : codes of entries 4j + l/16, slot l%16 (16 B)
  //   8 <= j < 12: rope of entries 8(j-8) + l/8, slot l%8
  //   j == 12    : scales of entry l (lanes < 32)
  // Wave w owns units j = w + NW c.  Per unit the plane base, row stride, entry, source
  // offset and swizzled LDS slot are fixed for the whole kernel: resolve them once.
  const uint64_t zero_addr = reinterpret_cast<uint64_t>(g_zero_row);
  uint64_t u_base[CPW];
  int u_stride[CPW], u_entry[CPW], u_off[CPW], u_dst[CPW];
  bool u_live[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int j = wave + NW * c;
    u_live[c] = j < kChunks && (j < 12 || lane < 32);
    if (j < 8) {
      const int e = 4 * j + (lane >> 4);
      u_base[c] = reinterpret_cast<uint64_t>(p.kv_lat);
      u_stride[c] = kLatBytes;
      u_entry[c] = e;
      u_off[c] = 16 * (lane & 15);
      u_dst[c] = kRawLat + 256 * e + 16 * ((lane & 15) ^ (e & 15));
    } else if (j < 12) {
      const int e = 8 * (j - 8) + (lane >> 3);
      u_base[c] = reinterpret_cast<uint64_t>(p.kv_rope);
      u_stride[c] = 2 * kRope;
      u_entry[c] = e;
      u_off[c] = 16 * (lane & 7);
      u_dst[c] = kRawRope + 128 * e + 16 * ((lane & 7) ^ (e & 7));
    } else {
      u_base[c] = reinterpret_cast<uint64_t>(p.kv_scl);
      u_stride[c] = kScl;
      u_entry[c] = lane & 31;
      u_off[c] = 0;
      u_dst[c] = kRawScl + 16 * (lane & 31);
    }
  }
  u32x4 stg[kNPre][CPW];
  // every wave issues exactly CPW loads per tile, without branches (dead units and empty
  // slots read the zero row), so the compiler can count loads in flight across tiles
  auto load_tile = [&](int tile, u32x4 (&r)[CPW]) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int row = s_rows[tile * kTE + u_entry[c]];
      const uint64_t src = (row >= 0 && u_live[c])
          ? u_base[c] + (uint64_t)((int64_t)row * u_stride[c] + u_off[c]) : zero_addr;
      r[c] = ld_global_16_addr(src);
    }
  };
  auto store_tile = [&](const u32x4 (&r)[CPW], uint8_t* raw) {
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      if (u_live[c]) *reinterpret_cast<u32x4*>(raw + u_dst[c]) = r[c];
  };

#pragma unroll
  for (int b = 0; b < kNPre; ++b)
    if (b < ntiles) load_tile(b, stg[b]);
  if (ntiles > 0) store_tile(stg[0], s_raw[0]);
  __syncthreads();

  const float sc_log2 = p.sm_scale_log2;
  for (int i0 = 0; i0 < ntiles; i0 += kNPre) {
#pragma unroll
    for (int bb = 0; bb < kNPre; ++bb) {
      const int i = i0 + bb;
      if (i < ntiles) {
        const uint8_t* raw = s_raw[i & 1];
        // tile i's registers are in LDS: reuse them for tile i + kNPre
        if (i + kNPre < ntiles) load_tile(i + kNPre, stg[bb]);

        // ---- V^T (fp16, channel-major, entries at vt_pos order) for the tile
#pragma unroll
        for (int r = 0; r < VT_PER_T; ++r) {
          const int it = tid + NT * r;
          if (it < VT_ITEMS) {
            const int eq = it & 7;               // entries 4eq .. 4eq+3
            const int co = it >> 3;              // channels 8co .. 8co+7
            uint32_t hv[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int e = 4 * eq + k;
              const int slot = (co >> 2) ^ (e & 15);
              const uint32_t w = *reinterpret_cast<const uint32_t*>(
                  raw + kRawLat + 256 * e + 16 * slot + 4 * (co & 3));
              const float sc = e8m0_to_f32(raw[kRawScl + 16 * e + (co >> 2)]);
              fp4x8_to_f16_pairs(w, sc, hv[k]);
            }
            uint8_t* dst = s_vt + 8 * co * kVtStride + 2 * vt_pos(4 * eq);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              u32x2 lo, hi;   // channel 8co+2k and 8co+2k+1, entries 4eq..4eq+3
              lo[0] = __builtin_amdgcn_perm(hv[1][k], hv[0][k], 0x05040100u);
              lo[1] = __builtin_amdgcn_perm(hv[3][k], hv[2][k], 0x05040100u);
              hi[0] = __builtin_amdgcn_perm(hv[1][k], hv[0][k], 0x07060302u);
              hi[1] = __builtin_amdgcn_perm(hv[3][k], hv[2][k], 0x07060302u);
              *reinterpret_cast<u32x2*>(dst + (2 * k) * kVtStride) = lo;
              *reinterpret_cast<u32x2*>(dst + (2 * k + 1) * kVtStride) = hi;
            }
          }
        }

        // ---- partial S^T over this wave's channel half: [mb][nb], lane (g, n)
        f32x4 sacc[2][NB];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int e = 16 * mb + n;
          f32x4 a[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) a[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
          const u32x4 sc4 = *reinterpret_cast<const u32x4*>(raw + kRawScl + 16 * e);
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int kk = 2 * half + k2;
            const int chunk = 4 * kk + g;             // this lane's 32-channel block
            const u32x4 w4 = *reinterpret_cast<const u32x4*>(
                raw + kRawLat + 256 * e + 16 * (chunk ^ (e & 15)));
            const int ksc = (int)((sc4[kk] >> (8 * g)) & 255u);
            const i32x8 ka = {(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3], 0, 0, 0, 0};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              a[nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  ka, qhi[nb][k2], a[nb], 4, 0, 0, ksc, 0, qsc[nb][k2]);
              a[nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  ka, qlo[nb][k2], a[nb], 4, 0, 0, ksc, 0, qsc[nb][k2]);
            }
          }
          {
            const int chunk = 4 * half + g;
            const u32x4 rv = *reinterpret_cast<const u32x4*>(
                raw + kRawRope + 128 * e + 16 * (chunk ^ (e & 7)));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              a[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rv), as_bf16x8(qrope[nb]), a[nb], 0, 0, 0);
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) sacc[mb][nb] = a[nb];
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s_part[wave][NB * mb + nb][lane] = sacc[mb][nb];
        // the next tile's raw bytes (staged one round ago) go to the other buffer
        if (i + 1 < ntiles) store_tile(stg[(bb + 1) % kNPre], s_raw[(i + 1) & 1]);
        __syncthreads();                         // partial S, V^T and raw(i+1) visible

        // ---- full S^T = half 0 + half 1 (same order in both waves), online softmax
        float x[NB][8];
        float tmax[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) tmax[nb] = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const f32x4 o4 = s_part[wave ^ 1][NB * mb + nb][lane];
            const f32x4 tot = half ? (o4 + sacc[mb][nb]) : (sacc[mb][nb] + o4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const bool ok = s_rows[i * kTE + 16 * mb + 4 * g + k] >= 0;
              const float v = ok ? tot[k] * sc_log2 : -INFINITY;
              x[nb][4 * mb + k] = v;
              tmax[nb] = fmaxf(tmax[nb], v);
            }
          }
        f16x8 pb[NB];
        bool any_valid = false;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          tmax[nb] = fmaxf(tmax[nb], __shfl_xor(tmax[nb], 16));
          tmax[nb] = fmaxf(tmax[nb], __shfl_xor(tmax[nb], 32));
          any_valid |= tmax[nb] != -INFINITY;
        }
        if (any_valid) {                         // uniform: the tile mask is shared
          bool raise[NB], any_raise = false;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            raise[nb] = tmax[nb] > m_run[nb] + 8.f;
            any_raise |= raise[nb];
          }
          if (__ballot(any_raise)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const float al = raise[nb] ? __builtin_amdgcn_exp2f(m_run[nb] - tmax[nb]) : 1.f;
              m_run[nb] = raise[nb] ? tmax[nb] : m_run[nb];
              l_run[nb] *= al;
#pragma unroll
              for (int c = 0; c < 16; ++c) acc[c][nb] *= al;
            }
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            float ps = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(x[nb][k] - m_run[nb]);
              pb[nb][k] = ph;
              ps += (float)ph;
            }
            l_run[nb] += ps;
          }
          // ---- O^T += V^T P^T over this wave's 256 channels
          const uint8_t* vt = s_vt + (256 * half + n) * kVtStride + 16 * g;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const f16x8 va = as_f16x8(*reinterpret_cast<const u32x4*>(vt + 16 * c * kVtStride));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[c][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[nb], acc[c][nb], 0, 0, 0);
          }
        }
        __syncthreads();                         // V^T, s_part and raw(i) free again
      }
    }
  }

  // ---- epilogue: normalize, write (partial) output and log2-sum-exp
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l_tot = l_run[nb] + __shfl_xor(l_run[nb], 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const float lse2 = (l_tot > 0.f) ? m_run[nb] + log2f(l_tot) : -INFINITY;
    const int h = HG * hg + 16 * nb + n;
    float* obase;
    if (p.splits == 1) {
      obase = p.o + ((int64_t)t * p.H + h) * kLat;
      if (g == 0 && half == 0) p.lse[(int64_t)t * p.H + h] = lse2 * 0.69314718055994530942f;
    } else {
      const int64_t slot = ((int64_t)t * p.splits + sp) * p.H + h;
      obase = p.o_part + slot * kLat;
      if (g == 0 && half == 0) p.lse_part[slot] = lse2;
    }
#pragma unroll
    for (int c = 0; c < 16; ++c)
      *reinterpret_cast<f32x4*>(obase + 256 * half + 16 * c + 4 * g) = acc[c][nb] * inv;
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
  switch (p.H) {
    case 16: hipLaunchKernelGGL((sparse_attn_kernel<1, 1>), dim3(blocks), dim3(128), 0, s, p); break;
    case 32: hipLaunchKernelGGL((sparse_attn_kernel<1, 2>), dim3(blocks), dim3(128), 0, s, p); break;
    case 64: hipLaunchKernelGGL((sparse_attn_kernel<2, 2>), dim3(blocks), dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL((sparse_attn_kernel<4, 2>), dim3(blocks), dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((int64_t)p.T * p.H)), dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace csa2
