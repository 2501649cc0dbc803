// MXFP4 cache write for CSA2 on gfx950: fp32 latent rows -> E2M1 codes + E8M0 scales.
//
// [summary] = picx.dev whiteboard summary "DeepSeek-V4.1-Flash: Pushing the Limits of KV
// Cache Compression", Methodology > Architecture Components, item 5 (FP4 main KV cache in
// the OCP MXFP4 format).  OCP MX conversion: shared exponent floor(log2 max|x|) - 2 per
// 32-channel block (E2M1's largest exponent is 2), clamped to the E8M0 range; each element
// x * 2^-X rounded to the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}, halfway cases to the even
// code, saturating at 6; the sign bit is x's sign, zeros included.
//
// One wave per row: lane l owns channels 8l .. 8l+7 (one output dword), four lanes form a
// scale block.  All decisions are exact in fp32: the block maximum, the exponent read off
// its bit pattern, scaling by a power of two and comparisons against the grid midpoints.
#include "csa2_internal.h"
#include "csa2_device.h"

namespace csa2 {

// Lane l of a wave holds channels 8l .. 8l+7 of a row (x); four consecutive lanes form a
// 32-channel scale block.  Returns the E2M1 codes as one dword and the block's shared
// exponent X (scale byte X + 127).
__device__ __forceinline__ uint32_t mxfp4_encode_lane(const float (&x)[8], int& X) {
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));

  const uint32_t ab = __float_as_uint(amax);
  if (ab == 0u) {
    X = -127;
  } else {
    const int E = (int)(ab >> 23);
    const int fl = E ? E - 127 : (31 - __clz((int)(ab & 0x7fffffu))) - 149;   // floor(log2)
    X = min(max(fl - 2, -127), 127);
  }
  // 2^-X is a normal float for every X a finite input produces (X <= 125)
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);
  uint32_t word = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = fabsf(x[e]) * inv;
    uint32_t code = (y > 0.25f) + (y >= 0.75f) + (y > 1.25f) + (y >= 1.75f) + (y > 2.5f) +
                    (y >= 3.5f) + (y > 5.0f);
    code |= (__float_as_uint(x[e]) >> 31) << 3;
    word |= code << (4 * e);
  }
  return word;
}

__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(QuantParams p) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const int lane = threadIdx.x & 63;
  const f32x4* xp = reinterpret_cast<const f32x4*>(p.x + r * kLat + 8 * lane);
  const f32x4 a = xp[0], b = xp[1];
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  int X;
  const uint32_t word = mxfp4_encode_lane(x, X);
  const int64_t dst = p.dst_row ? p.dst_row[r] : r;
  *reinterpret_cast<uint32_t*>(p.lat + dst * p.lat_stride + 4 * lane) = word;
  if ((lane & 3) == 0) p.scl[dst * p.scl_stride + (lane >> 2)] = (uint8_t)(X + 127);
}

// ---------------------------------------------------------------- E4M3 scales per 16
// The literal format of [summary] item 5: E2M1 codes with one E4M3 scale per 16 channels
// (OCP FP8 E4M3: bias 7, subnormals m 2^-9, largest 448).  Scale s = E4M3(max|x| / 6),
// nearest with ties to the even significand, saturating at 448; each element |x| / s
// rounded to the E2M1 grid with ties to the even code, saturating at 6; the sign bit is x's
// sign; a scale that rounds to 0 leaves (signed) zeros.  Decisions are exact: max|x| / 6 is
// taken in fp64 (its rounding to E4M3 then equals the rounding of the exact quotient), and
// each element is compared with s times a grid midpoint, a product exact in fp32.
__device__ __forceinline__ uint32_t e4m3_round_rne(double q) {   // q >= 0
  if (q >= 448.0) return 0x7eu;
  if (q < 0.015625) return (uint32_t)__builtin_rint(q * 512.0);  // subnormals, 8 = 2^-6
  const int e = (int)((__double_as_longlong(q) >> 52) & 0x7ff) - 1023;   // floor(log2 q)
  double k = __builtin_rint(q * __longlong_as_double((long long)(1023 + 3 - e) << 52));
  int ee = e;
  if (k == 16.0) { k = 8.0; ee += 1; }
  if (ee > 8) return 0x7eu;
  return (uint32_t)(((ee + 7) << 3) | ((int)k - 8));
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const int e = (int)((b >> 3) & 15u), m = (int)(b & 7u);
  return e ? __uint_as_float((uint32_t)(e - 7 + 127) << 23) * (1.f + 0.125f * (float)m)
           : 0.001953125f * (float)m;
}

__global__ __launch_bounds__(256) void fp4e4m3_quantize_kernel(QuantParams p) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const int lane = threadIdx.x & 63;
  const f32x4* xp = reinterpret_cast<const f32x4*>(p.x + r * kLat + 8 * lane);
  const f32x4 a = xp[0], b = xp[1];
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));          // lanes 2k, 2k+1: one 16-channel group
  const uint32_t sb = e4m3_round_rne((double)amax / 6.0);
  const float s = e4m3_value(sb);
  uint32_t word = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = fabsf(x[e]);
    uint32_t code = (s > 0.f) ? (y > 0.25f * s) + (y >= 0.75f * s) + (y > 1.25f * s) +
                                    (y >= 1.75f * s) + (y > 2.5f * s) + (y >= 3.5f * s) +
                                    (y > 5.0f * s)
                              : 0u;
    code |= (__float_as_uint(x[e]) >> 31) << 3;
    word |= code << (4 * e);
  }
  const int64_t dst = p.dst_row ? p.dst_row[r] : r;
  *reinterpret_cast<uint32_t*>(p.lat + dst * p.lat_stride + 4 * lane) = word;
  if ((lane & 1) == 0) p.scl[dst * p.scl_stride + (lane >> 1)] = (uint8_t)sb;
}

hipError_t launch_fp4e4m3_quantize(const QuantParams& p, hipStream_t s) {
  const int64_t blocks = (p.rows + 3) / 4;
  CSA2_LAUNCH(fp4e4m3_quantize_kernel, dim3((unsigned)blocks), dim3(256), s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- KV append
// One cache entry from a block of 4 raw tokens ([summary] Architecture Components, item 1,
// Eq. 1: the global KV entries come from the projections C and Z of the encoder's hidden
// state; [card] block-based sequence compression, 4:1).  The pages print no pooling rule;
// the one read here is a softmax over the block's tokens per channel, the entry being the
// weighted sum of the tokens' C.  The pooled latent is written in MXFP4 (as above), the rope
// and indexer-key parts in bf16 (round to nearest even).
//
// One wave per entry: lane l pools latent channels 8l .. 8l+7, rope channel l and indexer
// channel l from the four tokens, in fp32.
__device__ __forceinline__ float pool4(const float (&z)[4], const float (&c)[4]) {
  const float m = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float w = __builtin_amdgcn_exp2f((z[i] - m) * 1.4426950408889634f);
    num = fmaf(w, c[i], num);
    den += w;
  }
  return num / den;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= p.n) return;
  const int lane = threadIdx.x & 63;
  constexpr int D = kLat + kRope;                    // channels per token
  const float* c = p.c + e * 4 * D;
  const float* z = p.z + e * 4 * D;
  // Latent loads read whole lines: each instruction 1 KB contiguous, lane l channels 4l ..
  // 4l+3 (h = 0) or 256 + 4l .. (h = 1).  (Eight channels per lane straight from memory put
  // 16-byte pieces 32 bytes apart, so every line reached HBM in 64-byte halves.)
  float cl[4][2][4], zl[4][2][4], cr[4], zr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 c4 = *reinterpret_cast<const f32x4*>(c + i * D + 256 * h + 4 * lane);
      const f32x4 z4 = *reinterpret_cast<const f32x4*>(z + i * D + 256 * h + 4 * lane);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cl[i][h][k] = c4[k];
        zl[i][h][k] = z4[k];
      }
    }
    cr[i] = c[i * D + kLat + lane];
    zr[i] = z[i * D + kLat + lane];
  }
  float yh[2][4];                                    // pooled channels 256h + 4l + k
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float zk[4] = {zl[0][h][k], zl[1][h][k], zl[2][h][k], zl[3][h][k]};
      const float ck[4] = {cl[0][h][k], cl[1][h][k], cl[2][h][k], cl[3][h][k]};
      yh[h][k] = pool4(zk, ck);
    }
  // the encoder's layout, lane l channels 8l .. 8l+7: lanes 2l' and 2l'+1 (l' = l mod 32)
  // of half l / 32
  const bool hi = lane >= 32;
  const int s0 = (2 * lane) & 63;
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int src = s0 + (k >> 2);
    const float a = __shfl(yh[0][k & 3], src), b = __shfl(yh[1][k & 3], src);
    y[k] = hi ? b : a;
  }
  int X;
  const uint32_t word = mxfp4_encode_lane(y, X);
  const int64_t dst = p.dst_row ? p.dst_row[e] : e;
  *reinterpret_cast<uint32_t*>(p.lat + dst * p.lat_stride + 4 * lane) = word;
  if ((lane & 3) == 0) p.scl[dst * p.scl_stride + (lane >> 2)] = (uint8_t)(X + 127);
  uint16_t* rope_row = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(p.rope) + dst * p.rope_stride);
  rope_row[lane] = bf16_rne(pool4(zr, cr));
  if (p.c_idx) {
    float ci[4], zi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ci[i] = p.c_idx[(e * 4 + i) * kDidx + lane];
      zi[i] = p.z_idx[(e * 4 + i) * kDidx + lane];
    }
    p.k_idx[dst * kDidx + lane] = bf16_rne(pool4(zi, ci));
  }
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t s) {
  const int64_t blocks = (p.n + 3) / 4;
  CSA2_LAUNCH(kv_append_kernel, dim3((unsigned)blocks), dim3(256), s, p);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantParams& p, hipStream_t s) {
  const int64_t blocks = (p.rows + 3) / 4;
  CSA2_LAUNCH(mxfp4_quantize_kernel, dim3((unsigned)blocks), dim3(256), s, p);
  return hipGetLastError();
}

}  // namespace csa2
