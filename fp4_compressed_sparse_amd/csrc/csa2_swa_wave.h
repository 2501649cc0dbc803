// Device code shared by the persistent SWA kernel and the launch that runs the SWA branch
// beside the indexer scoring (one wave per (row, KV head) unit).
#pragma once

#include "csa2_internal.h"
#include "csa2_device.h"

namespace csa2 {

// One wave's share of the decode window attention (H == H_kv * G): units (row, KV head)
// first, first + stride, ...; lane (g, d) takes token 4*quad + g, channels 8d .. 8d+7, the
// four lane groups merge by shuffles and the wave writes the unit's outputs itself.  Window
// rows are read once: non-temporal loads.
constexpr int kSwaPUnroll = 4;          // token quads in flight per wave

template <int G>
__device__ __forceinline__ void swa_wave_units(const SwaParams& p, int first, int stride) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, d = lane & 15;
  const int units = p.T * p.H_kv;
  const int64_t tok_stride = (int64_t)p.H_kv * kDswa;          // elements per position
  for (int u = first; u < units; u += stride) {
    const int kh = u % p.H_kv, t = u / p.H_kv;
    const int b = p.seq_id[t], start = p.start[t], len = p.len[t];
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
    const int64_t base = (((int64_t)b * p.L_swa + start) * p.H_kv + kh) * kDswa + 8 * d;
    const int nq = (len + 3) >> 2;
    for (int q0 = 0; q0 < nq; q0 += kSwaPUnroll) {
      u32x4 kv[kSwaPUnroll], vv[kSwaPUnroll];
#pragma unroll
      for (int i = 0; i < kSwaPUnroll; ++i) {
        const int tok = 4 * (q0 + i) + g;
        if (tok < len) {
          kv[i] = ld_global_16_nt(p.k + base + tok * tok_stride);
          vv[i] = ld_global_16_nt(p.v + base + tok * tok_stride);
        } else {
          kv[i] = u32x4{0u, 0u, 0u, 0u};
          vv[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int i = 0; i < kSwaPUnroll; ++i) {
        const int tok = 4 * (q0 + i) + g;
        float kf[8], vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[2 * e] = __uint_as_float(kv[i][e] << 16);
          kf[2 * e + 1] = __uint_as_float(kv[i][e] & 0xffff0000u);
          vf[2 * e] = __uint_as_float(vv[i][e] << 16);
          vf[2 * e + 1] = __uint_as_float(vv[i][e] & 0xffff0000u);
        }
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
          float sc = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) sc = fmaf(q[gi][e], kf[e], sc);
          sc += __shfl_xor(sc, 1);
          sc += __shfl_xor(sc, 2);
          sc += __shfl_xor(sc, 4);
          sc += __shfl_xor(sc, 8);
          if (tok < len) {
            const float x = sc * p.sm_scale_log2;
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
    // merge the four token lane groups (xor 16, 32); every lane then holds the unit's state
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
      const int64_t oh = (int64_t)t * p.H + kh * G + gi;
      if (g == 0) {
        const float inv = (l[gi] > 0.f) ? 1.f / l[gi] : 0.f;
        f32x4 lo4, hi4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo4[e] = o[gi][e] * inv;
          hi4[e] = o[gi][4 + e] * inv;
        }
        f32x4* dst = reinterpret_cast<f32x4*>(p.o + oh * kDswa + 8 * d);
        dst[0] = lo4;
        dst[1] = hi4;
      }
      if (lane == 0)
        p.lse[oh] = (l[gi] > 0.f) ? (m[gi] + log2f(l[gi])) * 0.69314718055994530942f : -INFINITY;
    }
  }
}

}  // namespace csa2
