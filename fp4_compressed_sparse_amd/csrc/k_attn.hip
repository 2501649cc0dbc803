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
// score waves and eight value waves, three waves per SIMD.  Entries go in tiles of 64, one
// barrier per tile.
//   gather  : the split's physical rows are resolved once into LDS (by the value waves,
//             while the score waves load and split the query).  Each tile (16 KB codes,
//             8 KB rope, 1 KB scales) goes straight from memory into a ring of four LDS
//             tiles by LDS DMA, 16 bytes per lane, in a column-major image: column s of the
//             codes holds channels 32s..32s+31 of all 64 entries, each entry's 16 bytes at
//             an XOR-swizzled position, so that both the matrix-operand reads of the score
//             waves and the transposing reads of the value waves are bank-conflict free.
//             Value wave v fetches the two code columns that only it reads, so it refills
//             a ring slot as soon as its own reads of that slot are done: three tiles are
//             in flight while one is consumed.
//   QK^T    : score wave hb computes S^T[64 entries x 16 heads 16hb..] over all 576
//             channels.  The latent part runs on the MXFP4 matrix path (v_mfma_scale
//             16x16x128: A = the cached E2M1 codes with their own E8M0 block scales,
//             dequantized inside the MFMA); the query enters as two fp8 (E4M3) parts with
//             per-32-channel E8M0 scales, hi + lo, which reproduce the bf16 query exactly.
//             The rope part is bf16 MFMA.
//   softmax : online, per head, log2 domain, fp32, in the score wave; the running maximum
//             is raised only when a tile exceeds it by more than 2^12 (fp16 P <= 4096).
//             The wave publishes P (fp16) and, when it raised a maximum, the rescale factors.
//   PV      : value wave v accumulates O^T[64 channels 64v.. x all heads] += V^T P^T on
//             fp16 MFMA 16x16x32 with fp32 accumulation.  The V^T operand comes straight
//             from the staged codes: a transposing LDS read (ds_read_b64_tr_b4) gives each
//             lane 16 entries of one channel, converted in registers to fp16 (scale 1, exact)
//             and multiplied by each entry's block scale (fp16, from a per-tile table the
//             value waves build from the staged scale bytes).  fp16 rather than bf16 for P:
//             bf16 rounding of P alone would put the output's relative error near 1.7e-3.
// P, the rescale factors and the scale table are double-buffered by tile parity.  Splits
// write normalized partial outputs plus log2-sum-exp, and a merge kernel combines them.
// Both kernels number their workgroups so that everything of a row runs on one XCD, whose
// L2 then serves the row's shared query and its partial outputs.
#include "csa2_internal.h"
#include "csa2_device.h"

namespace csa2 {

constexpr int kTE = 64;              // entries per tile
constexpr int kMaxPerSplit = 2048;   // idx slots per split (LDS row table size)
constexpr int kNPre = 2;             // loop unroll: the tile parity picks buffers statically
constexpr int kRing = 4;             // raw tiles in LDS: one consumed, three in flight
constexpr float kRaise = 12.f;       // log2 headroom before the running maximum is raised
// raw tile layout in LDS (bytes): 16 code columns [16][64 entries][16 B] (column s holds
// channels 32s..32s+31), 8 rope columns [8][64][16 B] (column r holds rope channels
// 8r..8r+7), then the scale bytes: one unit [64][16 B] of E8M0 scales, or two units of
// E4M3 scales (unit u holds bytes 16u..16u+15 of each entry's 32); entry e of a column
// sits at position ent_pos(e).  Each 1 KB unit is one LDS DMA instruction per wave.
constexpr int kRawLat = 0, kRawRope = 16384, kRawScl = 24576, kRawBytes = 26624;

void attn_plan(int T, int H, int K, int* splits, int* per_split, int cus) {
  const int groups = attn_head_groups(H);
  const int min_s = (K + kMaxPerSplit - 1) / kMaxPerSplit;
  const int max_s = max(1, (K + 2 * kTE - 1) / (2 * kTE));   // >= 2 tiles per split
  cus = max(1, cus);
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

// Position of entry e (0..63) in a column of the staged tile: 16 (e/16) + ((e%16) ^
// 4 (e/16)).  Readers that take 16 entries {16a + 4G + b : a, b in 0..3} (G fixed), and
// readers that take 16 consecutive entries, both hit 16 distinct 16-byte positions of a
// 256-byte bank period.  The map is its own inverse.
__device__ __forceinline__ int ent_pos(int e) { return (e & 48) | ((e & 15) ^ ((e >> 2) & 12)); }

// Barrier for the tile loop: this wave's LDS accesses are complete, no wait on vector
// memory (the raw tiles arrive by LDS DMA, whose completion the loading waves await
// explicitly).  The memory clobber keeps the compiler from moving LDS accesses across it;
// `raw` is passed so that the DMA-filled buffer counts as written by it.
__device__ __forceinline__ void tile_barrier(const void* raw) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : "v"(raw) : "memory");
}

// Workgroup b of n runs on XCD b % 8; return the index of the b-th workgroup when XCD x
// takes the x-th contiguous range of [0, n).
__device__ __forceinline__ int xcd_linear(int b, int n) {
  const int q8 = n >> 3, r8 = n & 7;
  const int x = b & 7, slot = b >> 3;
  return (x < r8) ? x * (q8 + 1) + slot : r8 * (q8 + 1) + (x - r8) * q8 + slot;
}

// Two E4M3 scale bytes (bytes 0 and 1 of w, or 2 and 3 with HI) -> their values as packed
// fp16, by the OCP 8-bit conversion (E4M3 variant: subnormals m 2^-9, S.1111.111 NaN, the
// sign kept), scale 2^0.  Every E4M3 value is exact in fp16.
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, HI);
}

// 8 E2M1 codes times an fp16 scale -> 4 packed f16 pairs.  Exact for an E4M3 scale: at most
// 6 significant bits, magnitudes in [2^-10, 2688].
__device__ __forceinline__ void fp4x8_scaled_f16_pairs(uint32_t w, _Float16 sc, uint32_t out[4]) {
  fp4x8_to_f16_pairs(w, 1.f, out);
  const f16x2 mm = {sc, sc};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    out[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, out[k]) * mm);
}

// E8M0 scale byte -> the fp16 bit pattern of 2^(b - 127): exponents below -24 give 0, above
// 15 give +inf, so that a value the fp16 product cannot hold shows as a non-finite output
// rather than a wrong finite one.
__device__ __forceinline__ uint32_t e8m0_f16_bits(uint32_t b) {
  const int k = (int)b - 127;
  if (k > 15) return 0x7c00u;
  if (k >= -14) return (uint32_t)(k + 15) << 10;
  if (k >= -24) return 1u << (k + 24);
  return 0u;
}

// FMT 0: MXFP4 (E8M0 scale per 32 channels); FMT 1: FP4 with an E4M3 scale per 16 channels
template <int NHB, int FMT>   // NHB: 16-head blocks per workgroup, 1, 2 or 4 (blockIdx.y
__global__ __launch_bounds__(768) void sparse_attn_kernel(AttnParams p) {   // picks 64-head groups)
  constexpr int NV = 8;                              // value waves
  constexpr int kSclBlocks = FMT == 1 ? 32 : 16;     // scale-table rows (channel blocks)

  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kRing][kRawBytes];
  __shared__ __attribute__((aligned(16))) u32x4 s_p[2][NHB][2][64];   // P^T operands
  __shared__ __attribute__((aligned(16))) uint16_t s_sclt[2][kSclBlocks * kTE];   // fp16
  __shared__ float s_alpha[2][NHB][16];              // rescale factors of a raise
  __shared__ float s_l[NHB][16];
  __shared__ uint32_t s_flag[3];                     // per tile mod 3: blocks that raised
  __shared__ int32_t s_rows[kMaxPerSplit];
  __shared__ uint64_t s_tmask[kMaxPerSplit / kTE];

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
  // the loops run whole groups of kNPre tiles (static buffer parity, and no path on which a
  // tile of a group is skipped, so the compiler counts loads in flight exactly); a padding
  // tile has no valid entry
  const int ntiles2 = (ntiles + kNPre - 1) / kNPre * kNPre;
  // Roles: waves 0..3 score (one per SIMD, as waves go to the SIMDs in turn), waves 4..11
  // are value waves (two per SIMD).  Each role runs its own loop; both loops pass the same
  // barriers in the same order.
  const bool scorer_role = wave < 4;

  // ---- the score waves' query loads and conversion, and the value waves' row table.  The
  // query work overlaps the value waves' index loads.  When the sequence's page table fits
  // a raw tile slot (not written before the first loads below), the value waves fetch it
  // together with the indices: one memory round trip instead of two dependent ones.
  const int hb = min(wave, NHB - 1);
  constexpr int kPtPer = 8;                          // page-table entries per value thread
  const bool pt_lds = p.max_pages <= kPtPer * 64 * NV;   // block-uniform; <= 16 KB
  i32x8 qhi[4], qlo[4];
  int qscp = 0;                                      // byte kk: E8M0 scale of block 4kk + g
  f16x8 qf[4][4];                                    // FMT 1: the query in fp16
  u32x4 qrope0, qrope1;
  constexpr int kPer = kMaxPerSplit / (64 * NV);     // slots per value thread
  int jsl[kPer];
  if (scorer_role) {
    const uint16_t* qp = p.q + ((int64_t)t * p.H + h0 + 16 * hb + n) * kDq;
    u32x4 qraw[4][2][2];
    if (FMT == 1) {
      // FMT 1: per 128-channel chunk kk and step j, B lane (g, n) carries query channels
      // 32(4kk + g) + 8j .. +7, the channels A lane (g, n) dequantizes from the 16-byte code
      // slot of block 4kk + g (dword j)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qraw[kk][j >> 1][j & 1] = ld_global_16(qp + 32 * (4 * kk + g) + 8 * j);
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int c0 = 32 * (4 * kk + (g >> 1)) + 16 * (g & 1);
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          qraw[kk][run][0] = ld_global_16(qp + c0 + 64 * run);
          qraw[kk][run][1] = ld_global_16(qp + c0 + 64 * run + 8);
        }
      }
    }
    qrope0 = ld_global_16(qp + kLat + 8 * g);
    qrope1 = ld_global_16(qp + kLat + 32 + 8 * g);
    // Query operands, per 128-channel chunk kk: the scaled MFMA pairs A lane group gA (one
    // 32-channel block 4kk + gA of an entry) with B lane group 2(gA&1) + (p >= 16), byte
    // p%16 + 16(gA>>1).  So B lane (g, n) carries channels 32(4kk + g/2) + 16(g&1) + [0,16)
    // in bytes 0..15 and the same run of block 4kk + g/2 + 2 in bytes 16..31; it supplies
    // the E8M0 scale of block 4kk + g.  Each block is scaled by 2^X, X = floor(log2
    // max|q|) - 7, and split as hi = fp8(q 2^-X), lo = fp8(q 2^-X - hi): exact for every
    // bf16 value within 2^9 of the block maximum, and within 2^-16 of it below that.
    if (FMT == 1) {
      // bf16 -> fp16, to nearest: exact for magnitudes in [2^-14, 65504]
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const u32x4 v = qraw[kk][jj >> 1][jj & 1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            qf[kk][jj][2 * e] = (_Float16)__uint_as_float(v[e] << 16);
            qf[kk][jj][2 * e + 1] = (_Float16)__uint_as_float(v[e] & 0xffff0000u);
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
  } else {
    // ---- value waves: the split's indices (and the page table when it fits)
    const int b = p.seq_id[t];
    const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
    const int32_t* idx = p.idx + (int64_t)t * p.K + k0;
    const int tv = tid - 256;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = tv + 64 * NV * r;
      jsl[r] = (i < nslots) ? idx[i] : -1;
    }
    if (pt_lds) {                                    // all loads in flight at once
      int32_t* s_pt = reinterpret_cast<int32_t*>(&s_raw[kRing - 1][0]);
      int v[kPtPer];
#pragma unroll
      for (int u = 0; u < kPtPer; ++u) v[u] = (tv + 64 * NV * u < p.max_pages) ? pt[tv + 64 * NV * u] : 0;
#pragma unroll
      for (int u = 0; u < kPtPer; ++u)
        if (tv + 64 * NV * u < p.max_pages) s_pt[tv + 64 * NV * u] = v[u];
    }
  }
  if (pt_lds) __syncthreads();                       // page table in LDS
  if (!scorer_role) {
    // ---- value waves: resolve the split's physical rows (-1 = empty slot); one validity
    //      bit per entry of a tile
    const int tv = tid - 256;
    int row[kPer];
    if (pt_lds) {
      const int32_t* s_pt = reinterpret_cast<const int32_t*>(&s_raw[kRing - 1][0]);
#pragma unroll
      for (int r = 0; r < kPer; ++r) row[r] = (jsl[r] >= 0) ? s_pt[jsl[r] >> 6] * kPage + (jsl[r] & 63) : -1;
    } else {
      const int32_t* pt = p.page_table + (int64_t)p.seq_id[t] * p.max_pages;
#pragma unroll
      for (int r = 0; r < kPer; ++r) row[r] = (jsl[r] >= 0) ? pt[jsl[r] >> 6] * kPage + (jsl[r] & 63) : -1;
    }
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = tv + 64 * NV * r;                // tile i / 64 = wave - 4 + 8r
      if (i < ntiles2 * kTE) {
        s_rows[i] = row[r];
        const uint64_t bal = __ballot(row[r] >= 0);
        if (lane == 0) s_tmask[i >> 6] = bal;
      }
    }
    if (tid == 256) s_flag[0] = s_flag[1] = s_flag[2] = 0u;
  }
  __syncthreads();                                   // s_rows ready

  const float sc_log2 = p.sm_scale_log2;
  if (scorer_role) {
    // ======================================================== score waves
    const bool active = wave < NHB;                  // score wave of heads 16hb..16hb+15
    // this lane's entry positions in the staged columns: entry 16mb + n
    int epos[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) epos[mb] = 16 * ent_pos(16 * mb + n);
    // running state per head n; a finite initial maximum keeps fully masked tiles at
    // 2^(-inf) = 0 instead of -inf - (-inf)
    float m_run = -1.0e30f, l_run = 0.f;
    tile_barrier(s_raw);                             // prologue: raw(0) staged

    for (int i0 = 0; i0 < ntiles2; i0 += kNPre) {
#pragma unroll
      for (int bb = 0; bb < kNPre; ++bb) {           // bb & 1 = i & 1: static buffer parity
        const int i = i0 + bb;
        if (active) {
          // ---- S^T[entries 16mb + 4g + k][head n]: four chains, one per entry block; the
          // MFMAs are ordered so that a chain's consecutive MFMAs have three others between
          const uint8_t* raw = s_raw[i & (kRing - 1)];
          f32x4 acc[4];
          u32x4 ksc[4];                              // the 16 block scales of entry e
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (FMT == 0) ksc[mb] = *reinterpret_cast<const u32x4*>(raw + kRawScl + epos[mb]);
          }
          // A scale: block 4kk + g = byte g of dword kk, shifted down (op_sel 0); B scale:
          // op_sel = kk picks byte kk of qscp.  The hi and lo query parts accumulate into
          // the same chain.
#define CSA2_QK_CHUNK(kk)                                                                     \
  {                                                                                         \
    i32x8 ka[4];                                                                            \
    int asc[4];                                                                             \
    _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) {                                      \
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(                                     \
          raw + kRawLat + 1024 * (4 * (kk) + g) + epos[mb]);                                \
      ka[mb] = i32x8{(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3], 0, 0, 0, 0};           \
      asc[mb] = (int)(ksc[mb][kk] >> (8 * g));                                              \
      acc[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[mb], qhi[kk], acc[mb], 4, \
                                                                  0, 0, asc[mb], kk, qscp); \
    }                                                                                       \
    _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                        \
      acc[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[mb], qlo[kk], acc[mb], 4, \
                                                                  0, 0, asc[mb], kk, qscp); \
  }
          // FMT 1: the lane dequantizes its 8 codes of step j (dword j of the slot of block
          // 4kk + g, E4M3 group 8kk + 2g + j/2) into fp16; fp16 MFMA, steps outermost
#define CSA2_QK_E4M3(kk)                                                                      \
  {                                                                                         \
    u32x4 w4[4];                                                                            \
    uint32_t sc2[4];                                                                        \
    _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) {                                      \
      w4[mb] = *reinterpret_cast<const u32x4*>(raw + kRawLat + 1024 * (4 * (kk) + g) + epos[mb]); \
      sc2[mb] = *reinterpret_cast<const uint16_t*>(                                         \
          raw + kRawScl + 1024 * ((kk) >> 1) + epos[mb] + ((8 * (kk) + 2 * g) & 15));       \
    }                                                                                       \
    f16x2 s16[4];                                                                           \
    _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) s16[mb] = e4m3x2_to_f16<false>(sc2[mb]); \
    _Pragma("unroll") for (int jj = 0; jj < 4; ++jj)                                        \
      _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) {                                    \
        uint32_t kv[4];                                                                     \
        fp4x8_scaled_f16_pairs(w4[mb][jj], s16[mb][jj >> 1], kv);                           \
        const f16x8 ka = __builtin_bit_cast(f16x8, u32x4{kv[0], kv[1], kv[2], kv[3]});      \
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[kk][jj], acc[mb], 0, 0, 0); \
      }                                                                                     \
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
            const bf16x8 qr = as_bf16x8(s2 == 0 ? qrope0 : qrope1);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
              const u32x4 rv = *reinterpret_cast<const u32x4*>(
                  raw + kRawRope + 1024 * (4 * s2 + g) + epos[mb]);
              acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rv), qr, acc[mb], 0, 0, 0);
            }
          }
          // ---- online softmax; masked slots get -inf (exp2 -> 0).  A tile whose every slot
          // holds an entry (all but a split's last, mostly) skips the masking.
          const uint64_t tm = s_tmask[i];
          float x[16];
          if (tm == ~0ull) {                         // wave-uniform
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
              for (int k = 0; k < 4; ++k) x[4 * mb + k] = acc[mb][k] * sc_log2;
          } else {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
              const uint32_t bits = (uint32_t)(tm >> (16 * mb + 4 * g));
#pragma unroll
              for (int k = 0; k < 4; ++k)
                x[4 * mb + k] = ((bits >> k) & 1u) ? acc[mb][k] * sc_log2 : -INFINITY;
            }
          }
          float lmax = x[0];                         // this lane's maximum of the tile
#pragma unroll
          for (int k = 1; k < 16; ++k) lmax = fmaxf(lmax, x[k]);
          if (__ballot(lmax > m_run + kRaise)) {     // rare after the first tile
            float tmax = lmax;
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
          float ps = 0.f;
#pragma unroll
          for (int m = 0; m < 2; ++m) {              // P^T operand of PV step m: blocks 2m, 2m+1
            f16x8 pb;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float pv = __builtin_amdgcn_exp2f(x[8 * m + k] - m_run);
              ps += pv;
              pb[k] = (_Float16)pv;
            }
            s_p[bb & 1][hb][m][lane] = __builtin_bit_cast(u32x4, pb);
          }
          l_run += ps;
        }
        tile_barrier(s_raw);             // P(i), rescale factors, scale table(i), raw(i+1)
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
  const int tv = tid - 256;
  // ---- gather by LDS DMA: a load unit is 1 KB, one 16-byte global load per lane whose data
  // the hardware writes to LDS at (unit base + 16 lane).  Lane l fetches entry ent_pos(l)
  // (the column position l holds) in every unit.  Value wave v loads code columns 2v and
  // 2v+1 (the ones only it reads), rope column v, and value waves 0 (and 1, with E4M3
  // scales) the scale unit(s).
  constexpr int kMaxUnits = 4;
  const int nunits = 3 + ((rid == 0 || (FMT == 1 && rid == 1)) ? 1 : 0);
  const int my_e = ent_pos(lane);
  const uint8_t* u_base[kMaxUnits];
  int u_stride[kMaxUnits], u_dst[kMaxUnits];
#pragma unroll
  for (int c = 0; c < kMaxUnits; ++c) {
    if (c < 2) {                                     // code column 2rid + c
      u_base[c] = p.kv_lat + 16 * (2 * rid + c);
      u_stride[c] = p.lat_stride;
      u_dst[c] = kRawLat + 1024 * (2 * rid + c);
    } else if (c == 2) {                             // rope column rid
      u_base[c] = reinterpret_cast<const uint8_t*>(p.kv_rope) + 16 * rid;
      u_stride[c] = p.rope_stride;
      u_dst[c] = kRawRope + 1024 * rid;
    } else {                                         // scale unit rid (0, or 1 for E4M3)
      u_base[c] = p.kv_scl + 16 * rid;
      u_stride[c] = p.scl_stride;
      u_dst[c] = kRawScl + 1024 * rid;
    }
  }
  auto row_of = [&](int tile) { return (tile < ntiles) ? s_rows[tile * kTE + my_e] : -1; };
  // an empty slot loads the zero row; the select is done on the address bits, so that every
  // lane issues the same load instructions (one per unit) whatever the tile's slots hold
  const uint64_t zero_addr = reinterpret_cast<uint64_t>(g_zero_row);
  auto dma_tile = [&](int row, int slot) {
    const uint64_t keep = (uint64_t)0 - (uint64_t)(row >= 0);
    const uint64_t rowu = (uint64_t)(int64_t)max(row, 0);
#pragma unroll
    for (int c = 0; c < kMaxUnits; ++c) {
      if (c < nunits) {
        const uint64_t a = reinterpret_cast<uint64_t>(u_base[c]) + rowu * (uint64_t)u_stride[c];
        const uint8_t* src = reinterpret_cast<const uint8_t*>((a & keep) | (zero_addr & ~keep));
        __builtin_amdgcn_global_load_lds(src, &s_raw[slot][0] + u_dst[c], 16, 0, 0);
      }
    }
  };
  // wait until the tile issued two tiles before the latest (i.e. all but the two latest
  // tiles' loads) has landed
  auto wait_ready = [&] {
    if (nunits == 4) __builtin_amdgcn_s_waitcnt(0x0f70 | 8);
    else __builtin_amdgcn_s_waitcnt(0x0f70 | 6);
  };
  // per-lane offsets of the transposing code reads: lane (G, q) supplies the row of entry
  // E = 16 (q/4) + 4G + q%4, so that nibble q of every lane's result is that entry, the
  // order of the P^T operand (slot 8m + j of lane group G = entry 16(2m + j/4) + 4G + j%4)
  const int tq = lane & 15, tg = lane >> 4;
  const int tr_off = 16 * ent_pos(16 * (tq >> 2) + 4 * tg + (tq & 3));
#pragma unroll
  for (int b = 0; b < kRing - 1; ++b) dma_tile(row_of(b), b);
  int next_row = row_of(kRing - 1);                  // rows of the first loop load
  // O^T accumulators: channels 64rid + 16c + 4g + r, head h0 + 16b + n
  f32x4 acc[4][NHB];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int b = 0; b < NHB; ++b) acc[c][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nunits == 4) __builtin_amdgcn_s_waitcnt(0x0f70 | 8);   // raw(0) in LDS
  else __builtin_amdgcn_s_waitcnt(0x0f70 | 6);
  tile_barrier(s_raw);                               // prologue: raw(0) staged

  // fp16 scale table of tile `tile` (parity par) from its staged scale bytes: row cb holds
  // the scale of channel block cb (32 channels; 16 with E4M3 scales) for entries 0..63
  auto build_sclt = [&](const uint8_t* raw, uint16_t* tb) {
    if (FMT == 0) {
      const int cb = tv >> 5, ep = tv & 31;
      const uint32_t b0 = raw[kRawScl + 16 * ent_pos(2 * ep) + cb];
      const uint32_t b1 = raw[kRawScl + 16 * ent_pos(2 * ep + 1) + cb];
      *reinterpret_cast<uint32_t*>(tb + cb * kTE + 2 * ep) =
          e8m0_f16_bits(b0) | (e8m0_f16_bits(b1) << 16);
    } else {
      const int cb = tv >> 4, eq = tv & 15;
      uint32_t w = 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w |= (uint32_t)raw[kRawScl + 1024 * (cb >> 4) + 16 * ent_pos(4 * eq + k) + (cb & 15)] << (8 * k);
      *reinterpret_cast<u32x2*>(tb + cb * kTE + 4 * eq) =
          u32x2{__builtin_bit_cast(uint32_t, e4m3x2_to_f16<false>(w)),
                __builtin_bit_cast(uint32_t, e4m3x2_to_f16<true>(w))};
    }
  };

  // Period i (between barriers i-1 and i): rescale (rare), then O^T += V^T P^T for tile
  // i-1 (parity par): transposing reads of its codes, its P^T operands and scales; once
  // this wave's reads of raw(i-1) are done, the loads of raw(i+3) into that slot; the
  // conversions and MFMAs; then the scale table of tile i, and the wait for raw(i+1).
  auto pv_tile = [&](int pt, int par, bool refill, int refill_row, int refill_slot) {
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
    const uint8_t* raw = s_raw[pt & (kRing - 1)];
    u32x2 code[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int cg = 4 * rid + c;
      code[c] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr4_b64_v2i32(
          (__attribute__((address_space(3))) i32x2*)(
              const_cast<uint8_t*>(raw) + kRawLat + 1024 * (cg >> 1) + tr_off + 8 * (cg & 1))));
    }
    f16x8 pbs[NHB][2];
#pragma unroll
    for (int b = 0; b < NHB; ++b)
#pragma unroll
      for (int m = 0; m < 2; ++m) pbs[b][m] = as_f16x8(s_p[par][b][m][lane]);
    // scales of the lane's entries, per channel block and PV step: pairs (slot 2k, 2k+1)
    constexpr int NSB = FMT == 1 ? 4 : 2;            // channel blocks of this wave
    u32x2 scl[NSB][2][2];
    const uint16_t* tb = s_sclt[par];
#pragma unroll
    for (int s = 0; s < NSB; ++s) {
      const int cb = (FMT == 1) ? 4 * rid + s : 2 * rid + s;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          scl[s][m][h] = *reinterpret_cast<const u32x2*>(tb + cb * kTE + 32 * m + 16 * h + 4 * tg);
    }
    if (refill) {
      __builtin_amdgcn_s_waitcnt(0xc07f);            // lgkmcnt(0): this wave's reads done
      dma_tile(refill_row, refill_slot);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int s = (FMT == 1) ? c : (c >> 1);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint32_t v4[4];                              // slots (2k, 2k+1), scale 1: exact
        fp4x8_to_f16_pairs(code[c][m], 1.f, v4);
        f16x8 va;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f16x2 w = __builtin_bit_cast(f16x2, v4[k]) *
                          __builtin_bit_cast(f16x2, (uint32_t)scl[s][m][k >> 1][k & 1]);
          va[2 * k] = w[0];
          va[2 * k + 1] = w[1];
        }
#pragma unroll
        for (int b = 0; b < NHB; ++b)
          acc[c][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pbs[b][m], acc[c][b], 0, 0, 0);
      }
    }
  };

  for (int i0 = 0; i0 < ntiles2; i0 += kNPre) {
#pragma unroll
    for (int bb = 0; bb < kNPre; ++bb) {             // bb & 1 = i & 1: static buffer parity
      const int i = i0 + bb;
      if (tid == 256) s_flag[(i + 1) % 3] = 0u;      // tile i-2's requests, all read by now
      const int slot = (i + kRing - 1) & (kRing - 1);   // raw(i-1)'s slot gets raw(i+3)
      if (i > 0) pv_tile(i - 1, bb ^ 1, true, next_row, slot);
      else dma_tile(next_row, slot);
      next_row = row_of(i + kRing);                  // for the next tile's loads
      build_sclt(s_raw[i & (kRing - 1)], s_sclt[bb]);
      wait_ready();                                  // raw(i+1) in LDS
      tile_barrier(s_raw);               // P(i), rescale factors, scale table(i), raw(i+1)
    }
  }
  pv_tile(ntiles2 - 1, (ntiles2 - 1) & 1, false, 0, 0);
  wait_vmem_all();                                   // no LDS DMA may outlive the workgroup
  __syncthreads();                                   // denominators published
  // ---- epilogue: normalize and write
#pragma unroll
  for (int b = 0; b < NHB; ++b) {
    const float l_tot = s_l[b][n];
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const int64_t orow = (p.splits == 1) ? ((int64_t)t * p.H + h0 + 16 * b + n)
                                         : (((int64_t)t * p.splits + sp) * p.H + h0 + 16 * b + n);
    float* obase = ((p.splits == 1) ? p.o : p.o_part) + orow * kLat + 64 * rid + 4 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<f32x4*>(obase + 16 * c) = acc[c][b] * inv;
  }
}

// o = sum_s 2^(lse2_s - lse2) o_s, lse = ln 2 * lse2 with lse2 = log2 sum_s 2^lse2_s.
// Workgroup: HEADS heads of one row, 256 / HEADS threads per head, each thread HEADS / 2
// 4-channel columns (c, c + 128 HEADS / 8 ... ) of its head.  The splits' log2-sum-exps go
// through LDS; each thread loads the partials of up to 32 / HEADS splits for all its columns
// at a time (16 loads in flight), the first batch together with the log2-sum-exps.  Eight
// heads per workgroup when that still makes enough workgroups (the headline merge 8.5 ->
// 5.3 us), else two (4 rows of 16 splits: 4.2 against 6.0 us).
constexpr int kMergeMaxSplits = 512;
template <int HEADS>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams p) {
  constexpr int kMergeHeads = HEADS;
  constexpr int kMergeCols = HEADS / 2;
  constexpr int kMergeUnroll = 32 / HEADS;
  constexpr int kTph = 256 / HEADS;                     // threads per head
  __shared__ float s_lse[kMergeHeads][kMergeMaxSplits];
  const int lin = xcd_linear((int)blockIdx.x, (int)gridDim.x);
  const int per_row = p.H / kMergeHeads;
  const int t = lin / per_row;
  const int hg = lin - t * per_row;
  const int hh = threadIdx.x / kTph;
  const int h = hg * kMergeHeads + hh;
  const int c = 4 * (threadIdx.x % kTph);
  constexpr int kColStride = 4 * kTph;                  // channels between a thread's columns
  const int S = p.splits;
  // the first kMergeUnroll splits' partials are loaded before the log2-sum-exps are
  // awaited (they do not depend on them), so both round trips overlap
  const float* op = p.o_part + ((int64_t)t * S * p.H + h) * kLat + c;
  f32x4 v0[kMergeUnroll][kMergeCols];
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u)                 // (u < S is uniform)
#pragma unroll
    for (int j = 0; j < kMergeCols; ++j)
      v0[u][j] = (u < S) ? *reinterpret_cast<const f32x4*>(op + (int64_t)u * p.H * kLat + kColStride * j)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
  const float* lp = p.lse_part + (int64_t)t * S * p.H + hg * kMergeHeads;
  for (int i = threadIdx.x; i < kMergeHeads * S; i += 256)
    s_lse[i % kMergeHeads][i / kMergeHeads] = lp[(int64_t)(i / kMergeHeads) * p.H + (i % kMergeHeads)];
  __syncthreads();
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, s_lse[hh][s]);
  float* o = p.o + ((int64_t)t * p.H + h) * kLat + c;
  if (mx == -INFINITY) {
#pragma unroll
    for (int j = 0; j < kMergeCols; ++j)
      *reinterpret_cast<f32x4*>(o + kColStride * j) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c == 0) p.lse[(int64_t)t * p.H + h] = -INFINITY;
    return;
  }
  float z = 0.f;
  for (int s = 0; s < S; ++s) z += __builtin_amdgcn_exp2f(s_lse[hh][s] - mx);
  const float lse2 = mx + __log2f(z);
  f32x4 acc[kMergeCols];
#pragma unroll
  for (int j = 0; j < kMergeCols; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const float wgt = (u < S) ? __builtin_amdgcn_exp2f(s_lse[hh][min(u, S - 1)] - lse2) : 0.f;
#pragma unroll
    for (int j = 0; j < kMergeCols; ++j) acc[j] += wgt * v0[u][j];
  }
  for (int s0 = kMergeUnroll; s0 < S; s0 += kMergeUnroll) {
    f32x4 v[kMergeUnroll][kMergeCols];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u)
#pragma unroll
      for (int j = 0; j < kMergeCols; ++j)
        v[u][j] = (s0 + u < S)
                      ? *reinterpret_cast<const f32x4*>(op + (int64_t)(s0 + u) * p.H * kLat + kColStride * j)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float wgt = (s0 + u < S) ? __builtin_amdgcn_exp2f(s_lse[hh][min(s0 + u, S - 1)] - lse2) : 0.f;
#pragma unroll
      for (int j = 0; j < kMergeCols; ++j) acc[j] += wgt * v[u][j];
    }
  }
#pragma unroll
  for (int j = 0; j < kMergeCols; ++j) *reinterpret_cast<f32x4*>(o + kColStride * j) = acc[j];
  if (c == 0) p.lse[(int64_t)t * p.H + h] = lse2 * 0.69314718055994530942f;
}

template <int FMT>
hipError_t launch_sparse_attn_fmt(const AttnParams& p, hipStream_t s) {
  const unsigned blocks = (unsigned)((int64_t)p.T * p.splits);
  switch (p.H) {
    case 16: CSA2_LAUNCH((sparse_attn_kernel<1, FMT>), dim3(blocks), dim3(768), s, p); break;
    case 32: CSA2_LAUNCH((sparse_attn_kernel<2, FMT>), dim3(blocks), dim3(768), s, p); break;
    case 64:
      if (p.split_heads) CSA2_LAUNCH((sparse_attn_kernel<2, FMT>), dim3(blocks, 2), dim3(768), s, p);
      else CSA2_LAUNCH((sparse_attn_kernel<4, FMT>), dim3(blocks), dim3(768), s, p);
      break;
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
  if (p.H % 8) return hipErrorInvalidValue;
  const int64_t wide = (int64_t)p.T * p.H / 8;
  if (wide >= 256) CSA2_LAUNCH(attn_merge_kernel<8>, dim3((unsigned)wide), dim3(256), s, p);
  else CSA2_LAUNCH(attn_merge_kernel<2>, dim3((unsigned)((int64_t)p.T * p.H / 2)), dim3(256), s, p);
  return hipGetLastError();
}

}  // namespace csa2
