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
// One workgroup per (row, split of the K index slots, 64-head group) with twelve waves: four
// score waves and eight value waves, three waves per SIMD, so that one wave's LDS and VALU
// work hides behind the others' matrix work.  The query operands of a score wave and the
// accumulators of a value wave occupy the same registers.
//   gather  : the split's physical rows are resolved once into LDS.  Each 32-entry tile
//             (8 KB codes, 4 KB rope, 0.5 KB scales) goes straight from memory into a ring
//             of four LDS tiles by LDS DMA (16 bytes per lane, three tiles ahead), the lanes
//             fetching in an XOR-swizzled order of 16-byte slots so that the operand reads
//             below are bank-conflict free; no registers or LDS store instructions are spent
//             on staging.
//   QK^T    : score wave hb computes S^T[32 entries x 16 heads 16hb..] over all 576
//             channels.  The latent part runs on the MXFP4 matrix path (v_mfma_scale
//             16x16x128: A = the cached E2M1 codes with their own E8M0 block scales,
//             dequantized inside the MFMA); the query enters as two fp8 (E4M3) parts with
//             per-32-channel E8M0 scales, hi + lo, which reproduce the bf16 query exactly.
//             The rope part is bf16 MFMA.
//   softmax : online, per head, log2 domain, fp32, in the score wave; the running maximum
//             is raised only when a tile exceeds it by more than 2^12 (fp16 P <= 4096).
//             The wave publishes P (fp16) and, when it raised a maximum, the rescale factors.
//   PV      : value wave v accumulates O^T[64 channels 64v.. x all heads] += V^T P^T on
//             fp16 MFMA 16x16x32 with fp32 accumulation; each V^T operand (one 16-byte LDS
//             read) feeds every 16-head block.  V^T is dequantized once per tile into LDS
//             (fp16, channel-major, entries in the order the P^T operand has in registers)
//             by the value waves, one tile ahead.  fp16 rather than bf16 for P: bf16
//             rounding of P alone would put the output's relative error near 1.7e-3.
// Shared buffers are double-buffered by tile parity, so each tile needs one barrier.  Splits
// write normalized partial outputs plus log2-sum-exp, and a merge kernel combines them.
// Both kernels number their workgroups so that everything of a row runs on one XCD, whose
// L2 then serves the row's shared query and its partial outputs.
#include "csa2_internal.h"
#include "csa2_device.h"

namespace csa2 {

constexpr int kTE = 32;              // entries per tile
constexpr int kMaxPerSplit = 2048;   // idx slots per split (LDS row table size)
constexpr int kNPre = 2;             // loop unroll: the tile parity picks the P and V^T
                                     // buffers statically
constexpr int kRing = 4;             // raw tiles in LDS: one read, one ready, two in flight
constexpr float kRaise = 12.f;       // log2 headroom before the running maximum is raised
// raw tile layout in LDS (bytes): codes [32][256], rope [32][128], scales [32][16] (E8M0
// per 32 channels) or [32][32] (E4M3 per 16 channels)
constexpr int kRawLat = 0, kRawRope = 8192, kRawScl = 12288, kRawBytes = 13312;
constexpr int kChunks = 13;          // 1 KB load units per tile: 8 codes, 4 rope, 1 scales
constexpr int kRawSlot = kRawBytes + 1024;   // a raw tile and the 1 KB its dead loads fill
constexpr int kVtStride = 80;        // LDS bytes per V^T channel row (32 fp16 + 16 pad)

void attn_plan(int T, int H, int K, int* splits, int* per_split, int cus) {
  const int groups = attn_head_groups(H);
  const int min_s = (K + kMaxPerSplit - 1) / kMaxPerSplit;
  const int max_s = max(1, (K + 2 * kTE - 1) / (2 * kTE));   // >= 2 tiles per split
  cus = max(1, min(cus, kNumCus));
  // as many splits as fit the CUs in one round (a second round of a few workgroups would
  // cost a whole split's time)
  int s = (T > 0) ? max(1, cus / (T * groups)) : 1;
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

// LDS swizzle of a staged tile's codes: entry e's 16-byte slot c sits at slot
// c ^ (e & 15) ^ (e >> 4), so readers that take entries e and e + 16 in one access hit
// different banks.  (The map is its own inverse.)
__device__ __forceinline__ int lat_slot(int c, int e) { return c ^ (e & 15) ^ (e >> 4); }

// Barrier for the tile loop: this wave's LDS accesses are complete, no wait on vector
// memory (the raw tiles arrive by LDS DMA, whose completion the loading waves await
// explicitly).  The memory clobber keeps the compiler from moving LDS accesses across it;
// `raw` is passed so that the DMA-filled buffer counts as written by it.
__device__ __forceinline__ void tile_barrier(const void* raw) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : "v"(raw) : "memory");
}

// Position of entry e of a tile in a V^T row: the P^T operand of lane group g carries
// entries 4g..4g+3 then 16+4g..16+4g+3, so contraction slots 8g..8g+7 map to those.
__device__ __forceinline__ int vt_pos(int e) {
  return (e < 16) ? (8 * (e >> 2) + (e & 3)) : (8 * ((e - 16) >> 2) + 4 + (e & 3));
}

// Workgroup b of n runs on XCD b % 8; return the index of the b-th workgroup when XCD x
// takes the x-th contiguous range of [0, n).
__device__ __forceinline__ int xcd_linear(int b, int n) {
  const int q8 = n >> 3, r8 = n & 7;
  const int x = b & 7, slot = b >> 3;
  return (x < r8) ? x * (q8 + 1) + slot : r8 * (q8 + 1) + (x - r8) * q8 + slot;
}

// E4M3 scale byte -> (a power of two, for the conversions that apply a scale's exponent
// only, and the remaining significand 1 + m/8, or m for the subnormals m 2^-9)
__device__ __forceinline__ void e4m3_split(uint32_t b, float& pow2, _Float16& mant) {
  const int e = (int)((b >> 3) & 15u), m = (int)(b & 7u);
  pow2 = __uint_as_float((uint32_t)((e ? e - 7 : -9) + 127) << 23);
  mant = (_Float16)(e ? 1.f + 0.125f * (float)m : (float)m);
}

// 8 E2M1 codes times an E4M3 scale -> 4 packed f16 pairs (exact: at most 6 significant bits,
// magnitudes in [2^-10, 2688]).
__device__ __forceinline__ void fp4x8_e4m3_to_f16_pairs(uint32_t w, uint32_t sbyte,
                                                        uint32_t out[4]) {
  float pow2;
  _Float16 mant;
  e4m3_split(sbyte, pow2, mant);
  fp4x8_to_f16_pairs(w, pow2, out);
  const f16x2 mm = {mant, mant};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    out[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, out[k]) * mm);
}

// FMT 0: MXFP4 (E8M0 scale per 32 channels); FMT 1: FP4 with an E4M3 scale per 16 channels
template <int NHB, int FMT>   // NHB: 16-head blocks per workgroup, 1, 2 or 4 (blockIdx.y
__global__ __launch_bounds__(768) void sparse_attn_kernel(AttnParams p) {   // picks 64-head groups)
  constexpr int NW = 12;
  constexpr int NT = 64 * NW;
  constexpr int NV = 8;                              // value waves
  constexpr int CPW = (kChunks + NV - 1) / NV;       // load units per value wave and tile
  static_assert((kTE / 4) * (kLat / 8) == 64 * NV, "one V^T unit per value thread");

  // ring of raw tiles, each followed by 1 KB that dead loads write to
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kRing][kRawSlot];
  __shared__ __attribute__((aligned(16))) uint8_t s_vt[2][kLat * kVtStride];
  __shared__ __attribute__((aligned(16))) u32x4 s_p[2][NHB][64];     // P^T operands
  __shared__ float s_alpha[2][NHB][16];              // rescale factors of a raise
  __shared__ float s_l[NHB][16];
  __shared__ uint32_t s_flag[3];                     // per tile mod 3: blocks that raised
  __shared__ int32_t s_rows[kMaxPerSplit];
  __shared__ uint32_t s_tmask[kMaxPerSplit / kTE];

  // blockIdx.x -> (row, split): XCD x takes the x-th contiguous range of (row, split)
  const int lin = xcd_linear((int)blockIdx.x, p.T * p.splits);
  const int t = lin / p.splits;
  const int sp = lin - t * p.splits;
  const int k0 = sp * p.per_split;
  const int nslots = max(min(k0 + p.per_split, p.K) - k0, 0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int h0 = 16 * NHB * blockIdx.y;              // first head of this workgroup
  const int ntiles = (nslots + kTE - 1) / kTE;
  // the loops run whole groups of kNPre tiles (static buffer parity and staging slot, and
  // no path on which a tile of a group is skipped, so the compiler counts loads in flight
  // exactly); a padding tile has no valid entry
  const int ntiles2 = (ntiles + kNPre - 1) / kNPre * kNPre;
  // Roles: waves 0..3 score (one per SIMD, as waves go to the SIMDs in turn), waves 4..11
  // are value waves (two per SIMD).  Each role runs its own loop; both loops pass the same
  // barriers in the same order.
  const bool scorer_role = wave < 4;

  // ---- the score waves' query loads go out first, so that their latency overlaps the
  //      row resolution below
  const int hb = min(wave, NHB - 1);
  const uint16_t* qp = p.q + ((int64_t)t * p.H + h0 + 16 * hb + n) * kDq;
  u32x4 qraw[4][2][2], qrope0, qrope1;
  if (scorer_role && FMT == 1) {
    // FMT 1: per 128-channel chunk kk and step j, B lane (g, n) carries query channels
    // 32(4kk + g) + 8j .. +7, the channels A lane (g, n) dequantizes from the 16-byte code
    // slot of block 4kk + g (dword j)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        qraw[kk][j >> 1][j & 1] = ld_global_16(qp + 32 * (4 * kk + g) + 8 * j);
    qrope0 = ld_global_16(qp + kLat + 8 * g);
    qrope1 = ld_global_16(qp + kLat + 32 + 8 * g);
  } else if (scorer_role) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c0 = 32 * (4 * kk + (g >> 1)) + 16 * (g & 1);
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        qraw[kk][run][0] = ld_global_16(qp + c0 + 64 * run);
        qraw[kk][run][1] = ld_global_16(qp + c0 + 64 * run + 8);
      }
    }
    qrope0 = ld_global_16(qp + kLat + 8 * g);
    qrope1 = ld_global_16(qp + kLat + 32 + 8 * g);
  }

  // ---- resolve the split's physical rows once (-1 = empty slot); one validity bit per
  //      entry of each tile
  {
    const int b = p.seq_id[t];
    const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
    const int32_t* idx = p.idx + (int64_t)t * p.K + k0;
    for (int i = tid; i < ntiles2 * kTE; i += NT) {
      int32_t row = -1;
      if (i < nslots) {
        const int j = idx[i];
        if (j >= 0) row = pt[j >> 6] * kPage + (j & 63);
      }
      s_rows[i] = row;
      const uint64_t bal = __ballot(row >= 0);      // 64 slots = two tiles per wave step
      if (lane == 0) s_tmask[i >> 5] = (uint32_t)bal;
      if (lane == 32) s_tmask[i >> 5] = (uint32_t)(bal >> 32);
    }
    if (tid < 3) s_flag[tid] = 0u;
  }
  __syncthreads();                                   // s_rows ready

  // V^T (fp16, channel-major, entries at vt_pos order) of the tile staged in `raw`, built
  // by the value waves, one tile ahead: unit u = 64 (wave - 4) + lane = (eq, co) converts
  // entries 4eq..4eq+3 x channels 8co..8co+7
  auto build_vt_unit = [&](const uint8_t* raw, uint8_t* vtb, int u) {
    const int eq = u & 7;
    const int co = u >> 3;
    uint32_t hv[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 4 * eq + k;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(
          raw + kRawLat + 256 * e + 16 * lat_slot(co >> 2, e) + 4 * (co & 3));
      if (FMT == 1) {
        fp4x8_e4m3_to_f16_pairs(w, raw[kRawScl + 32 * e + (co >> 1)], hv[k]);   // group co/2
      } else {
        const float sc = e8m0_to_f32(raw[kRawScl + 16 * e + (co >> 2)]);        // block co/4
        fp4x8_to_f16_pairs(w, sc, hv[k]);
      }
    }
    uint8_t* dst = vtb + 8 * co * kVtStride + 2 * vt_pos(4 * eq);
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
  };


  const float sc_log2 = p.sm_scale_log2;
  if (scorer_role) {
    // ======================================================== score waves
    const bool active = wave < NHB;                  // score wave of heads 16hb..16hb+15
    // Query operands, per 128-channel chunk kk: the scaled MFMA pairs A lane group gA (one
    // 32-channel block 4kk + gA of an entry) with B lane group 2(gA&1) + (p >= 16), byte
    // p%16 + 16(gA>>1).  So B lane (g, n) carries channels 32(4kk + g/2) + 16(g&1) + [0,16)
    // in bytes 0..15 and the same run of block 4kk + g/2 + 2 in bytes 16..31; it supplies
    // the E8M0 scale of block 4kk + g.  Each block is scaled by 2^X, X = floor(log2
    // max|q|) - 7, and split as hi = fp8(q 2^-X), lo = fp8(q 2^-X - hi): exact for every
    // bf16 value within 2^9 of the block maximum, and within 2^-16 of it below that.
    i32x8 qhi[4], qlo[4];
    int qscp = 0;                                    // byte kk: E8M0 scale of block 4kk + g
    f16x8 qf[4][4];                                  // FMT 1: the query in fp16
    if (FMT == 1) {
      // bf16 -> fp16, to nearest: exact for magnitudes in [2^-14, 65504]
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 v = qraw[kk][j >> 1][j & 1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qf[kk][j][2 * e] = (_Float16)__uint_as_float(v[e] << 16);
            qf[kk][j][2 * e + 1] = (_Float16)__uint_as_float(v[e] & 0xffff0000u);
          }
        }
    }
#pragma unroll
    for (int kk = 0; kk < 4 && FMT == 0; ++kk) {
      float x[2][16];
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const u32x4 v0 = qraw[kk][run][0], v1 = qraw[kk][run][1];
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
      qscp |= (Xs + 127) << (8 * kk);
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const float inv = __uint_as_float((uint32_t)(127 - X[run]) << 23);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float y[4], r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = x[run][4 * d + e] * inv;
          int hh = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          hh = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], hh, true);
          r[0] = y[0] - __builtin_amdgcn_cvt_f32_fp8(hh, 0);
          r[1] = y[1] - __builtin_amdgcn_cvt_f32_fp8(hh, 1);
          r[2] = y[2] - __builtin_amdgcn_cvt_f32_fp8(hh, 2);
          r[3] = y[3] - __builtin_amdgcn_cvt_f32_fp8(hh, 3);
          int ll = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
          ll = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], ll, true);
          qhi[kk][4 * run + d] = hh;
          qlo[kk][4 * run + d] = ll;
        }
      }
    }
    // running state per head n; a finite initial maximum keeps fully masked tiles at
    // 2^(-inf) = 0 instead of -inf - (-inf)
    float m_run = -1.0e30f, l_run = 0.f;
    tile_barrier(s_raw);                             // prologue: raw(0) staged

    for (int i0 = 0; i0 < ntiles2; i0 += kNPre) {
#pragma unroll
      for (int bb = 0; bb < kNPre; ++bb) {           // bb & 1 = i & 1: static buffer parity
        const int i = i0 + bb;
        {
          if (active) {
            // ---- S^T[entries 16mb + 4g + k][head n]: four independent chains
            const uint8_t* raw = s_raw[i & (kRing - 1)];
            f32x4 ah[2], al[2];
            u32x4 ksc[2];                              // the 16 block scales of entry e
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
              ah[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
              al[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
              if (FMT == 0)
                ksc[mb] = *reinterpret_cast<const u32x4*>(raw + kRawScl + 16 * (16 * mb + n));
            }
            // A scale: block 4kk + g = byte g of dword kk, shifted down (op_sel 0); B scale:
            // op_sel = kk picks byte kk of qscp
#define CSA2_QK_CHUNK(kk)                                                                     \
  _Pragma("unroll") for (int mb = 0; mb < 2; ++mb) {                                        \
    const int e = 16 * mb + n;                                                              \
    const u32x4 w4 = *reinterpret_cast<const u32x4*>(                                       \
        raw + kRawLat + 256 * e + 16 * lat_slot(4 * (kk) + g, e));                          \
    const i32x8 ka = {(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3], 0, 0, 0, 0};          \
    const int asc = (int)(ksc[mb][kk] >> (8 * g));                                          \
    ah[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qhi[kk], ah[mb], 4, 0, 0,  \
                                                               asc, kk, qscp);              \
    al[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qlo[kk], al[mb], 4, 0, 0,  \
                                                               asc, kk, qscp);              \
  }
            // FMT 1: the lane dequantizes its 8 codes of step j (dword j of the slot of block
            // 4kk + g, E4M3 group 8kk + 2g + j/2) into fp16; fp16 MFMA; steps alternate
            // between the two accumulators
#define CSA2_QK_E4M3(kk)                                                                      \
  _Pragma("unroll") for (int mb = 0; mb < 2; ++mb) {                                        \
    const int e = 16 * mb + n;                                                              \
    const u32x4 w4 = *reinterpret_cast<const u32x4*>(                                       \
        raw + kRawLat + 256 * e + 16 * lat_slot(4 * (kk) + g, e));                          \
    const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(                                \
        raw + kRawScl + 32 * e + 8 * (kk) + 2 * g);                                         \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                         \
      uint32_t kv[4];                                                                       \
      fp4x8_e4m3_to_f16_pairs(w4[j], (sc2 >> (8 * (j >> 1))) & 0xffu, kv);                  \
      const f16x8 ka = __builtin_bit_cast(f16x8, u32x4{kv[0], kv[1], kv[2], kv[3]});        \
      if (j & 1) al[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[kk][j], al[mb], 0, 0, 0); \
      else ah[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[kk][j], ah[mb], 0, 0, 0);  \
    }                                                                                       \
  }
            if (FMT == 0) {
              CSA2_QK_CHUNK(0)
              CSA2_QK_CHUNK(1)
              CSA2_QK_CHUNK(2)
              CSA2_QK_CHUNK(3)
            } else {
              CSA2_QK_E4M3(0)
              CSA2_QK_E4M3(1)
              CSA2_QK_E4M3(2)
              CSA2_QK_E4M3(3)
            }
#undef CSA2_QK_CHUNK
#undef CSA2_QK_E4M3
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const int chunk = 4 * s2 + g;
              const bf16x8 qr = as_bf16x8(s2 == 0 ? qrope0 : qrope1);
#pragma unroll
              for (int mb = 0; mb < 2; ++mb) {
                const int e = 16 * mb + n;
                const u32x4 rv = *reinterpret_cast<const u32x4*>(
                    raw + kRawRope + 128 * e + 16 * (chunk ^ (e & 7)));
                if (s2 == 0) ah[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rv), qr, ah[mb], 0, 0, 0);
                else al[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rv), qr, al[mb], 0, 0, 0);
              }
            }
            // ---- online softmax; masked slots get -inf (exp2 -> 0)
            const uint32_t tm = s_tmask[i];
            float x[8];
            bool raise_lane = false;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
              const uint32_t bits = tm >> (16 * mb + 4 * g);
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const float v = ((bits >> k) & 1u) ? (ah[mb][k] + al[mb][k]) * sc_log2 : -INFINITY;
                x[4 * mb + k] = v;
                raise_lane |= v > m_run + kRaise;
              }
            }
            if (__ballot(raise_lane)) {              // rare after the first tile
              float tmax = x[0];
#pragma unroll
              for (int k = 1; k < 8; ++k) tmax = fmaxf(tmax, x[k]);
              tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
              tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
              float alpha = 1.f;
              if (tmax > m_run + kRaise) {
                alpha = __builtin_amdgcn_exp2f(m_run - tmax);
                m_run = tmax;
                l_run *= alpha;
              }
              if (g == 0) s_alpha[bb & 1][hb][n] = alpha;
              if (lane == 0) atomicOr(&s_flag[i % 3], 1u << hb);
            }
            f16x8 pb;
            float ps = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float pv = __builtin_amdgcn_exp2f(x[k] - m_run);
              ps += pv;
              pb[k] = (_Float16)pv;
            }
            l_run += ps;
            s_p[bb & 1][hb][lane] = __builtin_bit_cast(u32x4, pb);
          }

          tile_barrier(s_raw);           // P(i), rescale factors, raw(i+1), V^T(i) visible
        }
      }
    }
    // ---- epilogue: publish the softmax denominators
    if (active) {
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      if (g == 0) {
        s_l[hb][n] = l_tot;
        const float lse2 = (l_tot > 0.f) ? m_run + log2f(l_tot) : -INFINITY;
        const int h = h0 + 16 * hb + n;
        if (p.splits == 1) p.lse[(int64_t)t * p.H + h] = lse2 * 0.69314718055994530942f;
        else p.lse_part[((int64_t)t * p.splits + sp) * p.H + h] = lse2;
      }
    }
    __syncthreads();
    return;
  }

  // ========================================================== value waves
  const int rid = wave - 4;                          // 0..7: channels 64rid .. 64rid+63
  // ---- gather by LDS DMA: load unit j of a tile = 1 KB, one 16-byte global load per lane
  // whose data the hardware writes to LDS at (unit base + 16 lane), so the swizzle is applied
  // by choosing what each lane fetches:
  //   j < 8      : codes of entries 4j + l/16; LDS slot l%16 holds chunk lat_slot(l%16, e)
  //   8 <= j < 12: rope of entries 8(j-8) + l/8; slot l%8 holds chunk (l%8) ^ (e%8)
  //   j == 12    : the 16 scale bytes of entry l (lanes >= 32 fill the tile's tail), or
  //                with E4M3 scales the 32 bytes of entry l/2, half l%2
  // Value wave v owns units j = v + 8c; the units past 12 load the zero row into the tail,
  // so that every value wave issues the same number of loads per tile and can wait for a
  // tile with one counter value.  Row indices are read from LDS one tile ahead.
  const uint8_t* u_base[CPW];
  int u_stride[CPW], u_goff[CPW], u_dst[CPW], u_entry[CPW];
  bool u_live[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int j = rid + NV * c;
    const bool codes = j < 8, rope = !codes && j < 12, scl = j == 12;
    const int e = codes ? 4 * j + (lane >> 4)
                        : (rope ? 8 * (j - 8) + (lane >> 3) : (FMT == 1 ? lane >> 1 : lane & 31));
    u_entry[c] = e;
    u_live[c] = codes || rope || (scl && (FMT == 1 || lane < 32));
    u_base[c] = codes ? p.kv_lat : (rope ? reinterpret_cast<const uint8_t*>(p.kv_rope) : p.kv_scl);
    u_stride[c] = codes ? kLatBytes : (rope ? 2 * kRope : (FMT == 1 ? 2 * kScl : kScl));
    u_goff[c] = codes ? 16 * lat_slot(lane & 15, e)
                      : (rope ? 16 * ((lane & 7) ^ (e & 7)) : (FMT == 1 ? 16 * (lane & 1) : 0));
    u_dst[c] = __builtin_amdgcn_readfirstlane(codes ? kRawLat + 1024 * j
                                              : rope ? kRawRope + 1024 * (j - 8)
                                              : scl ? kRawScl : kRawBytes);
  }
  auto rows_of = [&](int tile, int (&rr)[CPW]) {
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      rr[c] = (tile < ntiles && u_live[c]) ? s_rows[tile * kTE + u_entry[c]] : -1;
  };
  auto dma_tile = [&](const int (&rr)[CPW], int slot) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint8_t* src = rr[c] >= 0 ? u_base[c] + (int64_t)rr[c] * u_stride[c] + u_goff[c]
                                      : g_zero_row;
      __builtin_amdgcn_global_load_lds(src, &s_raw[slot][0] + u_dst[c], 16, 0, 0);
    }
  };
  // loads issued after those of the tile awaited: two tiles of CPW loads
  auto wait_ready = [] { __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * CPW)); };
  int rr[CPW];
#pragma unroll
  for (int b = 0; b < kRing - 1; ++b) {
    rows_of(b, rr);
    dma_tile(rr, b);
  }
  rows_of(kRing - 1, rr);                            // rows of the first loop load
  // O^T accumulators: channels 64rid + 16c + 4g + i, head h0 + 16b + n
  f32x4 acc[4][NHB];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int b = 0; b < NHB; ++b) acc[c][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  wait_ready();                                      // raw(0) in LDS
  tile_barrier(s_raw);                               // prologue: raw(0) staged

  // rescale (rare), then O^T += V^T P^T for tile `pt` (parity `par`)
  auto pv_tile = [&](int pt, int par) {
    const uint32_t flag = s_flag[pt % 3];
    if (flag) {
#pragma unroll
      for (int b = 0; b < NHB; ++b) {
        if ((flag >> b) & 1u) {
          const float al = s_alpha[par][b][n];
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c][b] *= al;
        }
      }
    }
    f16x8 pbs[NHB];
#pragma unroll
    for (int b = 0; b < NHB; ++b) pbs[b] = as_f16x8(s_p[par][b][lane]);
    const uint8_t* vt = s_vt[par] + (64 * rid + n) * kVtStride + 16 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f16x8 va = as_f16x8(*reinterpret_cast<const u32x4*>(vt + 16 * c * kVtStride));
#pragma unroll
      for (int b = 0; b < NHB; ++b)
        acc[c][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pbs[b], acc[c][b], 0, 0, 0);
    }
  };

  // Between barriers i-1 and i: PV(i-1), V^T(i) from raw(i), the loads of raw(i+3) into the
  // slot raw(i-1) left, and the wait for raw(i+1).
  for (int i0 = 0; i0 < ntiles2; i0 += kNPre) {
#pragma unroll
    for (int bb = 0; bb < kNPre; ++bb) {             // bb & 1 = i & 1: static buffer parity
      const int i = i0 + bb;
      if (tid == 256) s_flag[(i + 1) % 3] = 0u;      // tile i-2's requests, all read by now
      if (i > 0) pv_tile(i - 1, bb ^ 1);
      build_vt_unit(s_raw[i & (kRing - 1)], s_vt[bb], 64 * rid + lane);
      dma_tile(rr, (i + kRing - 1) & (kRing - 1));
      rows_of(i + kRing, rr);                        // for the next tile's loads
      wait_ready();                                  // raw(i+1) in LDS
      tile_barrier(s_raw);               // P(i), rescale factors, raw(i+1), V^T(i) visible
    }
  }
  pv_tile(ntiles2 - 1, (ntiles2 - 1) & 1);
  wait_vmem_all();                                   // no LDS DMA may outlive the workgroup
  __syncthreads();                                   // denominators published
  // ---- epilogue: normalize and write
#pragma unroll
  for (int b = 0; b < NHB; ++b) {
    const float l_tot = s_l[b][n];
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const int64_t row = (p.splits == 1) ? ((int64_t)t * p.H + h0 + 16 * b + n)
                                        : (((int64_t)t * p.splits + sp) * p.H + h0 + 16 * b + n);
    float* obase = ((p.splits == 1) ? p.o : p.o_part) + row * kLat + 64 * rid + 4 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<f32x4*>(obase + 16 * c) = acc[c][b] * inv;
  }
}

// o = sum_s 2^(lse2_s - lse2) o_s, lse = ln 2 * lse2 with lse2 = log2 sum_s 2^lse2_s.
// Workgroup: 2 heads of one row; the splits' log2-sum-exps go through LDS, and each thread
// (4 channels of one head) loads the partials of up to kMergeUnroll splits at a time, the
// first batch together with the log2-sum-exps.
constexpr int kMergeUnroll = 16;
constexpr int kMergeMaxSplits = 512;
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams p) {
  __shared__ float s_lse[2][kMergeMaxSplits];
  const int hpb = 2;                                   // heads per workgroup
  const int lin = xcd_linear((int)blockIdx.x, (int)gridDim.x);
  const int per_row = p.H / hpb;
  const int t = lin / per_row;
  const int hh = threadIdx.x >> 7;
  const int h = (lin - t * per_row) * hpb + hh;
  const int c = 4 * (threadIdx.x & 127);
  const int S = p.splits;
  // the first kMergeUnroll splits' partials are loaded before the log2-sum-exps are
  // awaited (they do not depend on them), so both round trips overlap
  const float* op = p.o_part + ((int64_t)t * S * p.H + h) * kLat + c;
  f32x4 v0[kMergeUnroll];
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u)                 // (u < S is uniform)
    v0[u] = (u < S) ? *reinterpret_cast<const f32x4*>(op + (int64_t)u * p.H * kLat)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
  const float* lp = p.lse_part + (int64_t)t * S * p.H + (lin - t * per_row) * hpb;
  for (int i = threadIdx.x; i < hpb * S; i += 256) s_lse[i % hpb][i / hpb] = lp[(int64_t)(i / hpb) * p.H + (i % hpb)];
  __syncthreads();
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, s_lse[hh][s]);
  float* o = p.o + ((int64_t)t * p.H + h) * kLat + c;
  if (mx == -INFINITY) {
    *reinterpret_cast<f32x4*>(o) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c == 0) p.lse[(int64_t)t * p.H + h] = -INFINITY;
    return;
  }
  float z = 0.f;
  for (int s = 0; s < S; ++s) z += __builtin_amdgcn_exp2f(s_lse[hh][s] - mx);
  const float lse2 = mx + __log2f(z);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const float wgt = (u < S) ? __builtin_amdgcn_exp2f(s_lse[hh][min(u, S - 1)] - lse2) : 0.f;
    acc += wgt * v0[u];
  }
  for (int s0 = kMergeUnroll; s0 < S; s0 += kMergeUnroll) {
    f32x4 v[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u)
      v[u] = (s0 + u < S) ? *reinterpret_cast<const f32x4*>(op + (int64_t)(s0 + u) * p.H * kLat)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float wgt = (s0 + u < S) ? __builtin_amdgcn_exp2f(s_lse[hh][min(s0 + u, S - 1)] - lse2) : 0.f;
      acc += wgt * v[u];
    }
  }
  *reinterpret_cast<f32x4*>(o) = acc;
  if (c == 0) p.lse[(int64_t)t * p.H + h] = lse2 * 0.69314718055994530942f;
}

template <int FMT>
hipError_t launch_sparse_attn_fmt(const AttnParams& p, hipStream_t s) {
  const unsigned blocks = (unsigned)((int64_t)p.T * p.splits);
  switch (p.H) {
    case 16: CSA2_LAUNCH((sparse_attn_kernel<1, FMT>), dim3(blocks), dim3(768), s, p); break;
    case 32: CSA2_LAUNCH((sparse_attn_kernel<2, FMT>), dim3(blocks), dim3(768), s, p); break;
    case 64: CSA2_LAUNCH((sparse_attn_kernel<4, FMT>), dim3(blocks), dim3(768), s, p); break;
    case 128: CSA2_LAUNCH((sparse_attn_kernel<4, FMT>), dim3(blocks, 2), dim3(768), s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnParams& p, hipStream_t s) {
  if (p.fmt == 1) return launch_sparse_attn_fmt<1>(p, s);
  if (p.fmt == 0) return launch_sparse_attn_fmt<0>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(const MergeParams& p, hipStream_t s) {
  CSA2_LAUNCH(attn_merge_kernel, dim3((unsigned)((int64_t)p.T * p.H / 2)), dim3(256), s, p);
  return hipGetLastError();
}

}  // namespace csa2
