// format.hip -- the block format on the device: encode (quantise), decode, and the
// one-time rearrangement into the packed tile layout read by the product kernels.
#include "common.hpp"
#include "launch.hpp"

namespace iq4 {

// Codebook midpoints (c_j + c_{j+1}) / 2: a value above the j-th midpoint is nearer
// to level j+1 than to level j.
__constant__ float kMid[15] = {-115.5f, -93.5f, -74.0f, -57.0f, -42.0f, -28.5f, -16.0f, -4.5f,
                               7.0f,    19.0f,  31.5f,  45.5f,  61.0f,  79.0f,  101.0f};

// One thread per block.  d = f16(f32(max|w|) / 127) (IEEE division, round to
// nearest even); index = number of midpoints strictly below w/d, computed as
// w > mid_j * d.  mid_j * d is exact in binary32 (at most 9 x 11 significant bits),
// so the comparison is the exact nearest-level decision with ties to the lower
// index.  d == 0 gives index 8 (the level nearest zero) for every element.
__global__ void __launch_bounds__(256) quantize_kernel(const float* __restrict__ src, int64_t nb,
                                                       uint16_t* __restrict__ dst) {
  int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nb) return;
  const float4* s = reinterpret_cast<const float4*>(src + b * kQK);
  float w[kQK];
#pragma unroll
  for (int i = 0; i < kQK / 4; ++i) {
    float4 v = s[i];
    w[4 * i + 0] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kQK; ++i) amax = fmaxf(amax, fabsf(w[i]));
  __half dh = __float2half_rn(amax / 127.0f);
  float d = __half2float(dh);
  int q[kQK];
#pragma unroll
  for (int i = 0; i < kQK; ++i) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < 15; ++j) c += (w[i] > kMid[j] * d) ? 1 : 0;
    q[i] = (d == 0.0f) ? 8 : c;
  }
  uint16_t* o = dst + b * (kBlockBytes / 2);
  o[0] = __half_as_ushort(dh);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t lo = (uint32_t)q[2 * i] | ((uint32_t)q[2 * i + 16] << 4);
    uint32_t hi = (uint32_t)q[2 * i + 1] | ((uint32_t)q[2 * i + 17] << 4);
    o[1 + i] = (uint16_t)(lo | (hi << 8));
  }
}

// Elements 8p .. 8p+7 of one block are the low (p < 2) or high (p >= 2) nibbles of its
// index bytes 8(p % 2) .. 8(p % 2) + 7 (the four 16-bit words v); they are stored as
// output group i (8 consecutive outputs).
template <bool F16>
__device__ __forceinline__ void decode8(uint16_t dbits, const uint16_t (&v)[4], int p, void* out, int64_t i) {
  uint32_t bytes[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bytes[2 * j] = v[j] & 0xFF;
    bytes[2 * j + 1] = v[j] >> 8;
  }
  uint32_t q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = (p < 2) ? (bytes[j] & 0xF) : (bytes[j] >> 4);
  if (F16) {
    // One binary16 multiply d * c (both exact in binary16) rounds the exact product
    // once to nearest even: the binary16 rounding of the exact fp32 decode, with
    // subnormals and signed zeros kept.
    const uint32_t dd = (uint32_t)dbits | ((uint32_t)dbits << 16);
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t cc = (uint32_t)__half_as_ushort(__int2half_rn(level_of(q[2 * j]))) |
                          ((uint32_t)__half_as_ushort(__int2half_rn(level_of(q[2 * j + 1]))) << 16);
      h[j] = pk_mul_f16(dd, cc);
    }
    reinterpret_cast<uint4*>(out)[i] = make_uint4(h[0], h[1], h[2], h[3]);
  } else {
    const float d = h2f(dbits);
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = d * (float)level_of(q[j]);  // exact
    float4* o = reinterpret_cast<float4*>(out) + 2 * i;
    o[0] = make_float4(w[0], w[1], w[2], w[3]);
    o[1] = make_float4(w[4], w[5], w[6], w[7]);
  }
}

// Any alignment: one thread per 8 consecutive outputs, its block's bytes read directly.
template <bool F16>
__global__ void __launch_bounds__(256) dequant_kernel(const uint16_t* __restrict__ blocks,
                                                      int64_t nb, void* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nb * 4) return;
  const int64_t b = i >> 2;
  const int p = (int)(i & 3);
  const uint16_t* blk = blocks + b * (kBlockBytes / 2);
  uint16_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = blk[1 + 4 * (p & 1) + j];
  decode8<F16>(blk[0], v, p, out, i);
}

// 16-byte-aligned blocks, G groups of 64 per workgroup: the groups' 72 G 16-byte pieces
// come in with coalesced loads, all issued before any is waited for (four groups keep
// about 37 KB of loads in flight per CU), and each thread reads its blocks' bytes back
// from LDS (the direct form issues five 2-byte loads per thread).
constexpr int kStagedBlocks = 64;
constexpr int kStagedChunks = kStagedBlocks * kBlockBytes / 16;  // 72
constexpr int kStagedGroups = 4;

template <bool F16, int G>
__global__ void __launch_bounds__(256) dequant_staged_kernel(const uint4* __restrict__ blocks,
                                                             void* __restrict__ out) {
  constexpr int NC = G * kStagedChunks;
  static_assert(NC <= 3 * 256, "three loads per thread at most");
  __shared__ uint4 st[NC];
  const int tid = threadIdx.x;
  const uint4* src = blocks + (int64_t)blockIdx.x * NC;
  // (separate variables, not an array: an array of them was placed in LDS or scratch)
  const int i0 = tid, i1 = tid + 256, i2 = tid + 512;
  uint4 r0 = {0u, 0u, 0u, 0u}, r1 = {0u, 0u, 0u, 0u}, r2 = {0u, 0u, 0u, 0u};
  if (i0 < NC) r0 = src[i0];
  if (i1 < NC) r1 = src[i1];
  if (i2 < NC) r2 = src[i2];
  if (i0 < NC) st[i0] = r0;
  if (i1 < NC) st[i1] = r1;
  if (i2 < NC) st[i2] = r2;
  __syncthreads();
  const int b = tid >> 2, p = tid & 3;
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    const uint16_t* blk = reinterpret_cast<const uint16_t*>(st + gg * kStagedChunks) + b * (kBlockBytes / 2);
    uint16_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = blk[1 + 4 * (p & 1) + j];
    decode8<F16>(blk[0], v, p, out, ((int64_t)blockIdx.x * G + gg) * 256 + tid);
  }
}

// One thread per packed entry (64 per tile).  Entry l = 16g + j of tile (rt, kq) holds,
// for each of the tile's four blocks of row 16rt + j, the indices of elements
// 8g .. 8g+7 as four bytes, element 8g + 2i in the low and 8g + 2i + 1 in the high
// nibble of byte i (a row-block byte i holds elements i and i + 16 instead); entries
// with g == 0 also write that row's four scales.
__global__ void __launch_bounds__(256) pack_kernel(const uint16_t* __restrict__ blocks, int64_t n,
                                                   int64_t k, uint8_t* __restrict__ packed) {
  const int64_t kq_n = k / kTileK;
  const int64_t ntiles = (n / kTileRows) * kq_n;
  int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t tile = gid >> 6;
  if (tile >= ntiles) return;
  int l = (int)(gid & 63);
  int g = l >> 4, j = l & 15;
  int64_t rt = tile / kq_n, kq = tile % kq_n;
  int64_t row = rt * kTileRows + j;
  const int64_t bpr = k / kQK;
  const int shift = (g >> 1) * 4;  // elements 0..15: low nibbles; 16..31: high nibbles
  uint32_t word[4];
  uint16_t sc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint16_t* blk = blocks + (row * bpr + kq * kTileBlocks + b) * (kBlockBytes / 2);
    sc[b] = blk[0];
    // row-block bytes 8(g & 1) .. 8(g & 1) + 7 carry elements 8g .. 8g+7 (in one nibble half)
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t two = blk[1 + 4 * (g & 1) + i];  // bytes 2i, 2i+1 of that run
      const uint32_t e0 = ((uint32_t)(two & 0xFF) >> shift) & 0xF;
      const uint32_t e1 = ((uint32_t)(two >> 8) >> shift) & 0xF;
      w |= (e0 | (e1 << 4)) << (8 * i);
    }
    word[b] = w;
  }
  uint4* np = reinterpret_cast<uint4*>(packed + tile * kTileNibbleBytes) + l;
  *np = make_uint4(word[0], word[1], word[2], word[3]);
  if (g == 0) {
    uint8_t* sp = packed + (n * bpr) * kNibbleBytes + tile * kTileScaleBytes + 8 * j;
    *reinterpret_cast<uint2*>(sp) =
        make_uint2((uint32_t)sc[0] | ((uint32_t)sc[1] << 16), (uint32_t)sc[2] | ((uint32_t)sc[3] << 16));
  }
}

int launch_quantize(const float* src, int64_t nb, void* blocks, hipStream_t s) {
  if (nb == 0) return 0;
  int64_t grid = (nb + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(256), 0, s, src, nb,
                     static_cast<uint16_t*>(blocks));
  return check_launch("quantize_kernel");
}

int launch_dequant(const void* blocks, int64_t nb, bool f16, void* out, hipStream_t s) {
  if (nb == 0) return 0;
  const uint16_t* b = static_cast<const uint16_t*>(blocks);
  // whole groups of 64 blocks through the staged kernel when the blocks are 16-byte
  // aligned; the rest (or everything, if unaligned) through the direct one
  const int64_t groups = aligned(blocks, 16) ? nb / kStagedBlocks : 0;
  const int64_t wide = groups / kStagedGroups;  // workgroups of kStagedGroups groups
  const uint4* b16 = static_cast<const uint4*>(blocks);
  if (wide > 0) {
    if (f16)
      hipLaunchKernelGGL((dequant_staged_kernel<true, kStagedGroups>), dim3((unsigned)wide), dim3(256), 0, s, b16, out);
    else
      hipLaunchKernelGGL((dequant_staged_kernel<false, kStagedGroups>), dim3((unsigned)wide), dim3(256), 0, s, b16, out);
    if (int e = check_launch("dequant_staged_kernel")) return e;
  }
  if (groups > wide * kStagedGroups) {  // the last groups, one per workgroup
    const int64_t g0 = wide * kStagedGroups;
    const uint4* bg = b16 + g0 * kStagedChunks;
    void* og = static_cast<uint8_t*>(out) + g0 * kStagedBlocks * kQK * (f16 ? 2 : 4);
    if (f16)
      hipLaunchKernelGGL((dequant_staged_kernel<true, 1>), dim3((unsigned)(groups - g0)), dim3(256), 0, s, bg, og);
    else
      hipLaunchKernelGGL((dequant_staged_kernel<false, 1>), dim3((unsigned)(groups - g0)), dim3(256), 0, s, bg, og);
    if (int e = check_launch("dequant_staged_kernel")) return e;
  }
  const int64_t done = groups * kStagedBlocks, rest = nb - done;
  if (rest == 0) return 0;
  const uint16_t* bt = b + done * (kBlockBytes / 2);
  void* ot = static_cast<uint8_t*>(out) + done * kQK * (f16 ? 2 : 4);
  const int64_t grid = (rest * 4 + 255) / 256;
  if (f16)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, bt, rest, ot);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, bt, rest, ot);
  return check_launch("dequant_kernel");
}

int launch_pack(const void* blocks, int64_t n, int64_t k, void* packed, hipStream_t s) {
  int64_t threads = (n / kTileRows) * (k / kTileK) * 64;
  int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const uint16_t*>(blocks), n, k, static_cast<uint8_t*>(packed));
  return check_launch("pack_kernel");
}

}  // namespace iq4
