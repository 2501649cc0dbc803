// Measured peaks of one MI355X (gfx950), for reading the library's kernels against: dense
// matrix-core (MFMA) throughput per operand type and LDS read bandwidth.  Each kernel runs
// a long loop of independent instructions from every SIMD of every CU and writes one value
// per thread at the end (so that nothing is optimized away); the host times it with HIP
// events.  Not part of the CSA2 C ABI: bench.py loads this library on its own.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kChains = 8;   // independent accumulators per wave: keeps the pipe full

// kind 0: bf16 16x16x32; 1: fp16 16x16x32; 2: scaled 16x16x128 fp8 x fp4 (the attention's
// QK^T form); 3: scaled 16x16x128 fp8 x fp8; 4: scaled 16x16x128 fp4 x fp4
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop(float* out, int iters, float seed) {
  // distinct starting values: chains that provably hold the same values would be merged
  // by the compiler into one dependent chain
  f32x4 acc[kChains];
  const float s = seed * (float)(threadIdx.x + 1);
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{s + c, s - c, s * c, (float)c};
  bf16x8 ab;
  f16x8 ah;
  i32x8 a8;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    ab[k] = (__bf16)(s + k);
    ah[k] = (_Float16)(s - k);
    a8[k] = (int)(0x3c3c3c3cu ^ (threadIdx.x * 0x01010101u) ^ k);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      if (KIND == 0) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, ab, acc[c], 0, 0, 0);
      if (KIND == 1) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, ah, acc[c], 0, 0, 0);
      if (KIND == 2)   // A fp4 (format 4), B fp8 E4M3 (format 0)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, a8, acc[c], 4, 0, 0, 127,
                                                                  0, 127);
      if (KIND == 3)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, a8, acc[c], 0, 0, 0, 127,
                                                                  0, 127);
      if (KIND == 4)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, a8, acc[c], 4, 4, 0, 127,
                                                                  0, 127);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) r += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// LDS read bandwidth: every thread reads 16 bytes per step from a 64 KB LDS image, lanes
// at consecutive 16-byte slots (no bank conflicts), the slot window moving each step.
__global__ __launch_bounds__(1024) void lds_loop(uint32_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[16384];
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) lds[i] = i * 2654435761u;
  __syncthreads();
  u32x4 x = {0u, 0u, 0u, 0u};
  const int base = threadIdx.x & 1023;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int slot = (base + 64 * (it * 8 + u)) & 4095;
      x ^= *reinterpret_cast<const u32x4*>(&lds[4 * slot]);
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

template <class F>
double time_ms(F&& launch, int reps) {
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.0;
  launch();                                  // warm-up
  (void)hipEventRecord(a, nullptr);
  for (int r = 0; r < reps; ++r) launch();
  (void)hipEventRecord(b, nullptr);
  (void)hipEventSynchronize(b);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return (hipGetLastError() == hipSuccess) ? ms / reps : -1.0;
}

}  // namespace

// Dense MFMA throughput in TFLOP/s for `kind` (see mfma_loop), with `blocks_per_cu` 4-wave
// workgroups on every CU; -1 on a HIP error.
extern "C" double csa2peak_mfma_tflops(int kind, int blocks_per_cu) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1.0;
  const int blocks = cus * blocks_per_cu, threads = 256, iters = 2048;
  float* out = nullptr;
  if (hipMalloc(&out, sizeof(float) * blocks * threads) != hipSuccess) return -1.0;
  double flop_per_mfma = 0.0;
  double ms = -1.0;
  switch (kind) {
    case 0: flop_per_mfma = 2.0 * 16 * 16 * 32;
      ms = time_ms([&] { mfma_loop<0><<<blocks, threads>>>(out, iters, 1.f); }, 5); break;
    case 1: flop_per_mfma = 2.0 * 16 * 16 * 32;
      ms = time_ms([&] { mfma_loop<1><<<blocks, threads>>>(out, iters, 1.f); }, 5); break;
    case 2: flop_per_mfma = 2.0 * 16 * 16 * 128;
      ms = time_ms([&] { mfma_loop<2><<<blocks, threads>>>(out, iters, 1.f); }, 5); break;
    case 3: flop_per_mfma = 2.0 * 16 * 16 * 128;
      ms = time_ms([&] { mfma_loop<3><<<blocks, threads>>>(out, iters, 1.f); }, 5); break;
    case 4: flop_per_mfma = 2.0 * 16 * 16 * 128;
      ms = time_ms([&] { mfma_loop<4><<<blocks, threads>>>(out, iters, 1.f); }, 5); break;
    default: break;
  }
  (void)hipFree(out);
  if (ms <= 0.0) return -1.0;
  const double flops = flop_per_mfma * kChains * iters * (threads / 64) * (double)blocks;
  return flops / (ms * 1e-3) / 1e12;
}

// LDS read bandwidth in TB/s over the whole device (one 1024-thread workgroup per CU); -1
// on a HIP error.
extern "C" double csa2peak_lds_tbs(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1.0;
  const int blocks = cus, threads = 1024, iters = 512;
  uint32_t* out = nullptr;
  if (hipMalloc(&out, sizeof(uint32_t) * blocks * threads) != hipSuccess) return -1.0;
  const double ms = time_ms([&] { lds_loop<<<blocks, threads>>>(out, iters); }, 5);
  (void)hipFree(out);
  if (ms <= 0.0) return -1.0;
  return 16.0 * 8 * iters * threads * (double)blocks / (ms * 1e-3) / 1e12;
}
