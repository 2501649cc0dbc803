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
// MFMA.  One workgroup per (row, KV head) serves the G query heads that share the KV head
// so each K/V byte is read once.  Lane (g, d): token 4*quad + g, channels 8d .. 8d+7, so
// each 16-lane group reads one 256-byte key row contiguously.  Waves take interleaved
// token quads with an online softmax, then merge through LDS.
#include "csa2_internal.h"
#include "csa2_device.h"

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
        kv[u] = ld_global_16(p.k + base + tok * tok_stride);
        vv[u] = ld_global_16(p.v + base + tok * tok_stride);
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

hipError_t launch_swa(const SwaParams& p, hipStream_t s) {
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
