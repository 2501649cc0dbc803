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

__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(QuantParams p) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const int lane = threadIdx.x & 63;
  const f32x4* xp = reinterpret_cast<const f32x4*>(p.x + r * kLat + 8 * lane);
  const f32x4 a = xp[0], b = xp[1];
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));

  const uint32_t ab = __float_as_uint(amax);
  int X;
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
  const int64_t dst = p.dst_row ? p.dst_row[r] : r;
  *reinterpret_cast<uint32_t*>(p.lat + dst * kLatBytes + 4 * lane) = word;
  if ((lane & 3) == 0) p.scl[dst * kScl + (lane >> 2)] = (uint8_t)(X + 127);
}

hipError_t launch_quantize(const QuantParams& p, hipStream_t s) {
  const int64_t blocks = (p.rows + 3) / 4;
  CSA2_LAUNCH(mxfp4_quantize_kernel, dim3((unsigned)blocks), dim3(256), s, p);
  return hipGetLastError();
}

}  // namespace csa2
