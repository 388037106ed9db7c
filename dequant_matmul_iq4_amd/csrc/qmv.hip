// qmv.hip -- T-column quantised matrix-vector product (the verify window's dense
// product, T <= 8 tokens reading the weights once).
//
// Why the matrix cores.  With fp32 activations the plain vector form costs one fp32
// FMA per weight per column plus the index decode: at T = 4 that is more than 4 VALU
// operations per 4.5-bit weight, while streaming the weights at the HBM rate leaves a
// budget of under 3 (256 CUs x 64 lanes x 2.4 GHz against 8 TB/s of 18-byte blocks).
// So the K-reduction runs on the matrix cores instead, exactly:
//
//  * each fp32 activation x is split into three bf16 parts x = hi + mid + lo by
//    truncation (hi keeps the top 8 significand bits, mid the next 8, lo the last 8);
//    the split is exact for |x| >= 2^-100;
//  * codebook levels are integers of at most 7 significant bits, exact in bf16, so
//    every product level * part is exact in fp32;
//  * one v_mfma_f32_16x16x32_bf16 covers one block of 32 weights for 16 weight rows
//    (B operand) against 16 "rows" of A = (part s, token t) pairs, 4s + t;
//  * the block scale d is applied to the 16x16 result with an fp32 FMA per block, the
//    K-slices of the workgroup's waves are summed in a fixed order, and finally the
//    three parts are added (hi + mid) + lo.
//
// Column invariance.  Token t's value never meets another token's: it sits in matrix
// row 4s + (t mod 4) of MFMA group t / 4, the per-block scaling and the reductions run
// the same instruction sequence for every t, and the wave / K-slice split depends on K
// only.  Column t of a T-column call is therefore bitwise the 1-column call on token t
// (the property page 1's verify window relies on: each window token reproduces plain
// greedy decode bit for bit).
//
// Memory.  Weights come in the packed tile layout: per 16-row x 4-block tile each lane
// issues one 128-bit load of indices (coalesced 1 KiB per wave) and one 64-bit load
// of its row's four scales; all loads of a wave's chunk are issued before any decode
// (page 2 found one weight block in flight per warp to be the bottleneck of its
// interleaved matvec).  The index-to-level decode is a byte-indexed table in LDS
// (one byte = two 4-bit indices -> two bf16 levels).
#include "common.hpp"
#include "launch.hpp"

namespace iq4 {

constexpr int kQmvMaxWaves = 8;

__device__ __forceinline__ uint32_t bf16_of_level(int c) {
  return __float_as_uint((float)c) >> 16;  // exact: |c| <= 127
}

// Part s (0 = hi, 1 = mid, 2 = lo) of the exact three-way bf16 split of v.
__device__ __forceinline__ uint32_t split_part(float v, int s) {
  uint32_t u = __float_as_uint(v);
  if (s == 0) return u >> 16;
  float r1 = v - __uint_as_float(u & 0xFFFF0000u);  // exact (Sterbenz)
  uint32_t u1 = __float_as_uint(r1);
  if (s == 1) return u1 >> 16;
  float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);  // exact, <= 8 significant bits
  return __float_as_uint(r2) >> 16;
}

// A fragment of one block for lane (g, row 4s + tt) of token group `grp`: the 8 values
// x[32kb + 4g + j] (low half of VGPR j) and x[32kb + 16 + 4g + j] (high half), part s.
__device__ __forceinline__ u32x4 x_fragment(const float* __restrict__ x, int64_t ldx, int T,
                                            int grp, int s, int tt, int g, int64_t kb) {
  const int t = 4 * grp + tt;
  u32x4 a = {0u, 0u, 0u, 0u};
  if (s < 3 && t < T) {
    const float* p = x + (int64_t)t * ldx + kb * kQK + 4 * g;
    float4 xa = *reinterpret_cast<const float4*>(p);
    float4 xb = *reinterpret_cast<const float4*>(p + 16);
    a[0] = split_part(xa.x, s) | (split_part(xb.x, s) << 16);
    a[1] = split_part(xa.y, s) | (split_part(xb.y, s) << 16);
    a[2] = split_part(xa.z, s) | (split_part(xb.z, s) << 16);
    a[3] = split_part(xa.w, s) | (split_part(xb.w, s) << 16);
  }
  return a;
}

// One workgroup per 16-row tile; its waves split K into runs of whole 4-block quads.
template <bool TWO>
__global__ void __launch_bounds__(512) qmv_kernel(const uint8_t* __restrict__ packed, int kq_n,
                                                  int64_t nibble_bytes, const float* __restrict__ x,
                                                  int64_t ldx, int T, float* __restrict__ y,
                                                  int64_t ldy, int quads_per_wave) {
  __shared__ uint32_t lut[256];
  __shared__ f32x4 red[kQmvMaxWaves][TWO ? 2 : 1][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  for (int i = tid; i < 256; i += blockDim.x)
    lut[i] = bf16_of_level(kCodebook[i & 15]) | (bf16_of_level(kCodebook[i >> 4]) << 16);

  const int64_t rt = blockIdx.x;
  const int g = lane >> 4, c = lane & 15;
  const int s = c >> 2, tt = c & 3;
  const int q0 = wave * quads_per_wave;
  const int q1 = min(q0 + quads_per_wave, kq_n);
  const uint8_t* tiles = packed + rt * kq_n * kTileNibbleBytes + lane * 16;
  const uint8_t* scales = packed + nibble_bytes + rt * kq_n * kTileScaleBytes + c * 8;

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  for (int qc = q0; qc < q1; qc += 4) {
    const int nq = min(4, q1 - qc);
    uint4 nib[4];
    uint2 sc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // every load of the chunk first (tail clamped)
      const int q = qc + min(u, nq - 1);
      nib[u] = *reinterpret_cast<const uint4*>(tiles + (int64_t)q * kTileNibbleBytes);
      sc[u] = *reinterpret_cast<const uint2*>(scales + (int64_t)q * kTileScaleBytes);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u >= nq) break;
      const int64_t kb0 = (int64_t)(qc + u) * kTileBlocks;
      const uint32_t words[4] = {nib[u].x, nib[u].y, nib[u].z, nib[u].w};
      const uint32_t sw[2] = {sc[u].x, sc[u].y};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = words[j];
        u32x4 b;
        b[0] = lut[w & 0xFF];
        b[1] = lut[(w >> 8) & 0xFF];
        b[2] = lut[(w >> 16) & 0xFF];
        b[3] = lut[w >> 24];
        const float d = h2f((uint16_t)(sw[j >> 1] >> (16 * (j & 1))));
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 r0 = mfma_bf16(x_fragment(x, ldx, T, 0, s, tt, g, kb0 + j), b, zero);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc0[i] = __builtin_fmaf(d, r0[i], acc0[i]);
        if (TWO) {
          f32x4 r1 = mfma_bf16(x_fragment(x, ldx, T, 1, s, tt, g, kb0 + j), b, zero);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc1[i] = __builtin_fmaf(d, r1[i], acc1[i]);
        }
      }
    }
  }

  // Lane (g, c) holds D[4g + i][c]: part s = g, token 4 * grp + i, weight row c.
  red[wave][0][lane] = acc0;
  if (TWO) red[wave][TWO ? 1 : 0][lane] = acc1;
  __syncthreads();
  if (tid < T * 16) {
    const int t = tid >> 4, r = tid & 15;
    const int grp = TWO ? (t >> 2) : 0, i = t & 3;
    float part[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      float a = red[0][grp][16 * p + r][i];
      for (int w2 = 1; w2 < nwaves; ++w2) a += red[w2][grp][16 * p + r][i];
      part[p] = a;
    }
    y[(int64_t)t * ldy + rt * kTileRows + r] = (part[0] + part[1]) + part[2];
  }
}

int launch_qmv(const uint8_t* packed, int64_t n, int64_t k, const float* x, int64_t ldx, int T,
               float* y, int64_t ldy, hipStream_t s) {
  const int kq_n = (int)(k / kTileK);
  const int nwaves = kq_n < kQmvMaxWaves ? kq_n : kQmvMaxWaves;
  const int qpw = (kq_n + nwaves - 1) / nwaves;
  const int64_t nibble_bytes = n * (k / kQK) * kNibbleBytes;
  dim3 grid((unsigned)(n / kTileRows)), block(64 * nwaves);
  if (T > 4)
    hipLaunchKernelGGL(qmv_kernel<true>, grid, block, 0, s, packed, kq_n, nibble_bytes, x, ldx, T,
                       y, ldy, qpw);
  else
    hipLaunchKernelGGL(qmv_kernel<false>, grid, block, 0, s, packed, kq_n, nibble_bytes, x, ldx,
                       T, y, ldy, qpw);
  return check_launch("qmv_kernel");
}

}  // namespace iq4
