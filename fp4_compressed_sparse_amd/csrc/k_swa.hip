// Sliding-window attention branch of CSA2 on gfx950.
//
// [summary] = picx.dev whiteboard summary "DeepSeek-V4.1-Flash: Pushing the Limits of KV
// Cache Compression", Introduction (a global attention branch combined with local
// sliding-window attention); [blog] cyber-feed.org repost, introduction (SWA covering the
// local window).  Head h of row t attends over the bf16 keys/values at window positions
// [start, start + len) of its sequence, KV head h * H_kv / H.
//
// Decode-shaped work: one query vector per head against <= a few hundred keys is a
// matrix-vector product (about 1 flop per byte), so it runs on wavefront reductions, not
// MFMA.  Lane (g, d): token 4*quad + g, channels 8d .. 8d+7, so each 16-lane group reads
// one 256-byte key row contiguously.  Three forms:
//   swa_kernel<G>       one workgroup per (row, KV head) serves the G query heads that
//                       share the KV head, so each K/V byte is read once; waves take
//                       interleaved token quads with an online softmax, then merge
//                       through LDS (GQA decode rows);
//   swa_persist_kernel  H == H_kv decode rows beside the global branch: a fixed set of
//                       one-per-CU workgroups, one wave per (row, KV head) unit;
//   swa_tile_kernel     many rows (prefill): row tiles on MFMA.
#include "csa2_internal.h"
#include "csa2_device.h"
#include "csa2_swa_wave.h"

namespace csa2 {

constexpr int kSwaWaves = 4;
constexpr int kSwaUnroll = 4;   // token quads in flight per wave

template <int G>
__global__ __launch_bounds__(256) void swa_kernel(SwaParams p) {
  __shared__ float s_m[kSwaWaves][G];
  __shared__ float s_l[kSwaWaves][G];
  __shared__ __attribute__((aligned(16))) float s_o[kSwaWaves][G][kDswa];

  const int kh = blockIdx.x % p.H_kv;
  const int t = blockIdx.x / p.H_kv;
  const int b = p.seq_id[t];
  const int start = p.start[t];
  const int len = p.len[t];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, d = lane & 15;

  float q[G][8];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const u32x4 v = ld_global_16(p.q_swa + ((int64_t)t * p.H + kh * G + gi) * kDswa + 8 * d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[gi][2 * e] = __uint_as_float(v[e] << 16);
      q[gi][2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = -INFINITY;
    l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[gi][e] = 0.f;
  }

  const int64_t tok_stride = (int64_t)p.H_kv * kDswa;           // elements per position
  const int64_t base = (((int64_t)b * p.L_swa + start) * p.H_kv + kh) * kDswa + 8 * d;
  const int nq = (len + 3) >> 2;
  for (int q0 = wave; q0 < nq; q0 += kSwaWaves * kSwaUnroll) {
    u32x4 kv[kSwaUnroll], vv[kSwaUnroll];
#pragma unroll
    for (int u = 0; u < kSwaUnroll; ++u) {
      const int tok = 4 * (q0 + kSwaWaves * u) + g;
      if (tok < len) {
        kv[u] = ld_global_16_nt(p.k + base + tok * tok_stride);
        vv[u] = ld_global_16_nt(p.v + base + tok * tok_stride);
      } else {
        kv[u] = u32x4{0u, 0u, 0u, 0u};
        vv[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kSwaUnroll; ++u) {
      const int tok = 4 * (q0 + kSwaWaves * u) + g;
      float kf[8], vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = __uint_as_float(kv[u][e] << 16);
        kf[2 * e + 1] = __uint_as_float(kv[u][e] & 0xffff0000u);
        vf[2 * e] = __uint_as_float(vv[u][e] << 16);
        vf[2 * e + 1] = __uint_as_float(vv[u][e] & 0xffff0000u);
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(q[gi][e], kf[e], s);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if (tok < len) {
          const float x = s * p.sm_scale_log2;
          const float mn = fmaxf(m[gi], x);
          const float alpha = __builtin_amdgcn_exp2f(m[gi] - mn);
          const float pv = __builtin_amdgcn_exp2f(x - mn);
          l[gi] = l[gi] * alpha + pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[gi][e] = fmaf(o[gi][e], alpha, pv * vf[e]);
          m[gi] = mn;
        }
      }
    }
  }

  // merge the four token lanes groups (xor 16, 32), then the waves through LDS
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float mo = __shfl_xor(m[gi], off);
      const float lo = __shfl_xor(l[gi], off);
      const float mn = fmaxf(m[gi], mo);
      const float a = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[gi] - mn);
      const float bb = (mn == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
      l[gi] = l[gi] * a + lo * bb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float oo = __shfl_xor(o[gi][e], off);
        o[gi][e] = o[gi][e] * a + oo * bb;
      }
      m[gi] = mn;
    }
    if (lane == 0) {
      s_m[wave][gi] = m[gi];
      s_l[wave][gi] = l[gi];
    }
    if (g == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][gi][8 * d + e] = o[gi][e];
    }
  }
  __syncthreads();
  for (int it = threadIdx.x; it < G * kDswa; it += 256) {
    const int gi = it / kDswa, c = it - gi * kDswa;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSwaWaves; ++w) mx = fmaxf(mx, s_m[w][gi]);
    float z = 0.f, acc = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kSwaWaves; ++w) {
        const float wgt = __builtin_amdgcn_exp2f(s_m[w][gi] - mx);
        z += s_l[w][gi] * wgt;
        acc += s_o[w][gi][c] * wgt;
      }
    }
    const int64_t oh = (int64_t)t * p.H + kh * G + gi;
    p.o[oh * kDswa + c] = (z > 0.f) ? acc / z : 0.f;
    if (c == 0) p.lse[oh] = (z > 0.f) ? (mx + log2f(z)) * 0.69314718055994530942f : -INFINITY;
  }
}

// ---------------------------------------------------------------- beside the global branch
// The same decode-shaped work on a fixed set of workgroups (one per CU: the LDS the
// workgroup reserves keeps a second one off its CU), each of whose 16 waves takes whole
// (row, KV head) units in turn.  The branch then holds a bounded share of the CUs while
// the global branch's attention, whose workgroups each need a whole CU, runs on the rest,
// instead of waiting for the branch's many small workgroups to drain.  Each wave runs
// swa_wave_units (its non-temporal window loads displace less of what the global branch
// beside it keeps in the caches).
constexpr int kSwaPWaves = 16;
constexpr int kSwaPHold = 96 * 1024;    // LDS reserved per workgroup (more than half a CU's)

template <int G>
__global__ __launch_bounds__(64 * kSwaPWaves) void swa_persist_kernel(SwaParams p) {
  __shared__ uint8_t s_hold[kSwaPHold];
  if (p.T < 0) s_hold[threadIdx.x] = 0;             // never taken; keeps the reservation
  const int wave = threadIdx.x >> 6;
  swa_wave_units<G>(p, (int)blockIdx.x * kSwaPWaves + wave, (int)gridDim.x * kSwaPWaves);
}

// ---------------------------------------------------------------- many rows (prefill)
// Many query rows over few sequences: consecutive rows' windows overlap, so a workgroup
// takes a tile of 64 rows of one query head and walks the union of their windows in blocks
// of 32 key positions, each block staged once in LDS for all 64 rows.  Wave w owns rows
// 16w .. 16w+15 and runs on MFMA:
//   S^T = K Q^T    (bf16 16x16x32; lane (g, n) gets keys 4g..4g+3 and 16+4g..16+4g+3 of
//                   row n, which are exactly the eight keys its P^T operand carries)
//   O^T += V^T P^T (bf16 16x16x32 with P split as hi + lo, both bf16: the product is exact
//                   to about 2^-16 of P, with no range limit on V)
// Keys are masked per row to [start, start + len); the online softmax is per row, in the
// log2 domain, in fp32.  V^T is staged channel-major with its key slots in the order of
// the P^T operand.  Rows of a tile that belong to different sequences are handled in one
// pass per sequence.
constexpr int kSwaTileRows = 64;
constexpr int kSwaKB = 32;             // key positions per block
constexpr int kSwaVtStride = 80;       // LDS bytes per V^T channel row (32 bf16 + 16 pad)

// slot of key e (0..31) of a block in a V^T row: the P^T operand of lane group g carries
// keys 4g..4g+3 then 16+4g..16+4g+3
__device__ __forceinline__ int swa_vt_pos(int e) {
  return (e < 16) ? (8 * (e >> 2) + (e & 3)) : (8 * ((e - 16) >> 2) + 4 + (e & 3));
}

__global__ __launch_bounds__(256) void swa_tile_kernel(SwaParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][kSwaKB * kDswa * 2];        // 8 KB
  __shared__ __attribute__((aligned(16))) uint8_t s_vt[2][kDswa * kSwaVtStride];    // 10 KB
  __shared__ int s_seq[kSwaTileRows], s_st[kSwaTileRows], s_en[kSwaTileRows];

  const int ntiles = (p.T + kSwaTileRows - 1) / kSwaTileRows;
  const int tile = (int)blockIdx.x % ntiles, h = (int)blockIdx.x / ntiles;
  const int kh = h * p.H_kv / p.H;
  const int t0 = tile * kSwaTileRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  for (int i = tid; i < kSwaTileRows; i += 256) {
    const int t = t0 + i;
    const bool ok = t < p.T;
    s_seq[i] = ok ? p.seq_id[t] : -1;
    s_st[i] = ok ? p.start[t] : 0;
    s_en[i] = ok ? p.start[t] + p.len[t] : 0;
  }
  __syncthreads();

  const int rl = 16 * wave + n;                      // this lane's row within the tile
  const int row = t0 + rl;
  // Q^T operand: row n, channels 32c + 8g .. +7
  u32x4 qv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qv[c] = row < p.T ? ld_global_16(p.q_swa + ((int64_t)row * p.H + h) * kDswa + 32 * c + 8 * g)
                      : u32x4{0u, 0u, 0u, 0u};
  const int64_t tok_stride = (int64_t)p.H_kv * kDswa;   // elements per position

  int prev = -1;
  for (;;) {
    int cur = INT32_MAX;
    for (int i = 0; i < kSwaTileRows; ++i) {
      const int sq = s_seq[i];
      if (sq > prev && sq < cur) cur = sq;
    }
    if (cur == INT32_MAX) break;
    prev = cur;
    // union of the windows of this sequence's rows, clamped to the cache
    int lo = INT32_MAX, hi = 0;
    for (int i = 0; i < kSwaTileRows; ++i) {
      if (s_seq[i] == cur && s_en[i] > s_st[i]) {
        lo = min(lo, s_st[i]);
        hi = max(hi, s_en[i]);
      }
    }
    lo = max(lo, 0);
    hi = min(hi, p.L_swa);
    const int nblk = (hi > lo) ? (hi - lo + kSwaKB - 1) / kSwaKB : 0;
    const bool mine = s_seq[rl] == cur;
    const int rs = s_st[rl], re = min(s_en[rl], p.L_swa);
    const uint16_t* kbase = p.k + ((int64_t)cur * p.L_swa * p.H_kv + kh) * kDswa;
    const uint16_t* vbase = p.v + ((int64_t)cur * p.L_swa * p.H_kv + kh) * kDswa;

    // staging: threads 0..127 move V (unit: keys 4eq..4eq+3 x channels 8dq..8dq+7),
    // threads 128..255 move K (key u/4, chunks 4(u%4) .. +3)
    const int su = tid & 127;
    const bool stage_v = tid < 128;
    u32x4 st[4];
    auto load_block = [&](int b) {
      const int p0 = lo + kSwaKB * b;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = stage_v ? 4 * (su & 7) + i : (su >> 2);
        const int ch = stage_v ? 8 * (su >> 3) : 8 * (4 * (su & 3) + i);
        const int pos = p0 + key;
        st[i] = (pos < hi) ? ld_global_16((stage_v ? vbase : kbase) + (int64_t)pos * tok_stride + ch)
                           : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto store_block = [&](int buf) {
      if (stage_v) {
        const int eq = su & 7, dq = su >> 3;
        uint8_t* dst = s_vt[buf] + 8 * dq * kSwaVtStride + 2 * swa_vt_pos(4 * eq);
#pragma unroll
        for (int d = 0; d < 4; ++d) {       // channels 8dq + 2d, 8dq + 2d + 1
          u32x2 a, b;
          a[0] = __builtin_amdgcn_perm(st[1][d], st[0][d], 0x05040100u);
          a[1] = __builtin_amdgcn_perm(st[3][d], st[2][d], 0x05040100u);
          b[0] = __builtin_amdgcn_perm(st[1][d], st[0][d], 0x07060302u);
          b[1] = __builtin_amdgcn_perm(st[3][d], st[2][d], 0x07060302u);
          *reinterpret_cast<u32x2*>(dst + (2 * d) * kSwaVtStride) = a;
          *reinterpret_cast<u32x2*>(dst + (2 * d + 1) * kSwaVtStride) = b;
        }
      } else {
        const int key = su >> 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 4 * (su & 3) + i;
          *reinterpret_cast<u32x4*>(s_k[buf] + 256 * key + 16 * (c ^ (key & 15))) = st[i];
        }
      }
    };

    float m_run = -1.0e30f, l_run = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nblk > 0) {
      load_block(0);
      store_block(0);
    }
    __syncthreads();
    for (int b = 0; b < nblk; ++b) {
      const int buf = b & 1;
      if (b + 1 < nblk) load_block(b + 1);
      const int p0 = lo + kSwaKB * b;
      // ---- S^T for keys 16kb + 4g + i of row n
      float x[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        const int key = 16 * kb + n;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(s_k[buf] + 256 * key +
                                                           16 * ((4 * c + g) ^ (key & 15)));
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), as_bf16x8(qv[c]), s, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = p0 + 16 * kb + 4 * g + i;
          const bool ok = mine && pos >= rs && pos < re;
          x[4 * kb + i] = ok ? s[i] * p.sm_scale_log2 : -INFINITY;
        }
      }
      // ---- online softmax of row n (its 32 keys sit in lanes n, n+16, n+32, n+48)
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] *= alpha;
      bf16x8 phi, plo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(x[i] - m_run);
        l_run += pv;
        const __bf16 h16 = (__bf16)pv;
        phi[i] = h16;
        plo[i] = (__bf16)(pv - (float)h16);
      }
      // ---- O^T += V^T P^T, channels 16d + n rows of V^T
      const uint8_t* vt = s_vt[buf] + n * kSwaVtStride + 16 * g;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4*>(vt + 16 * d * kSwaVtStride));
        acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[d], 0, 0, 0);
        acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[d], 0, 0, 0);
      }
      if (b + 1 < nblk) store_block(buf ^ 1);
      __syncthreads();
    }
    // ---- rows of this sequence: normalize and write
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (mine && row < p.T) {
      const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
      float* o = p.o + ((int64_t)row * p.H + h) * kDswa + 4 * g;
#pragma unroll
      for (int d = 0; d < 8; ++d) *reinterpret_cast<f32x4*>(o + 16 * d) = acc[d] * inv;
      if (g == 0)
        p.lse[(int64_t)row * p.H + h] = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * 0.69314718055994530942f
                                                      : -INFINITY;
    }
  }
}

hipError_t launch_swa(const SwaParams& p, hipStream_t s) {
  if (p.T >= kSwaTileMinRows) {
    const unsigned blocks = (unsigned)((int64_t)(p.T + kSwaTileRows - 1) / kSwaTileRows * p.H);
    CSA2_LAUNCH(swa_tile_kernel, dim3(blocks), dim3(256), s, p);
    return hipGetLastError();
  }
  if (p.wgs > 0) {
    if (p.H != p.H_kv) return hipErrorInvalidValue;
    CSA2_LAUNCH(swa_persist_kernel<1>, dim3(p.wgs), dim3(64 * kSwaPWaves), s, p);
    return hipGetLastError();
  }
  const unsigned blocks = (unsigned)((int64_t)p.T * p.H_kv);
  switch (p.H / p.H_kv) {
    case 1: CSA2_LAUNCH(swa_kernel<1>, dim3(blocks), dim3(256), s, p); break;
    case 2: CSA2_LAUNCH(swa_kernel<2>, dim3(blocks), dim3(256), s, p); break;
    case 4: CSA2_LAUNCH(swa_kernel<4>, dim3(blocks), dim3(256), s, p); break;
    case 8: CSA2_LAUNCH(swa_kernel<8>, dim3(blocks), dim3(256), s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa2
