// xs.hip -- the IQ4_XS super-block format on the device: block decode and the T-column
// matrix-vector product.
//
// Page 2 (the Strata pull request "sm_80 (GA100) tuning") names the format among the
// dense weight types decoded every prompt chunk (its wide-dequant commit message),
// times its matvec on two shapes (the MMVQ-IL harness commit message) and states its
// block dot: the integer sum times the float of the sub-block code minus 32 (the
// MMVQ-IL_PF commit message).  The bytes follow the format's public definition:
//   super-block = 256 weights in 136 bytes, 8-byte aligned;
//   bytes 0-1: d (binary16); bytes 2-3: a 16-bit word whose bits 2i, 2i+1 are the high
//   two bits of sub-block i's 6-bit code ls_i; bytes 4-7: the low four bits of ls_i at
//   bit 4i of the 32-bit word they form; bytes 8 + 16i + m (m < 16): the indices of
//   elements 32i + m (low nibble) and 32i + 16 + m (high nibble);
//   w = d * (ls_i - 32) * c[q], exact in binary32 (at most 11 + 5 + 7 significant bits).
//
// Work unit: a "chunk" is 8 index bytes of one sub-block half, 16 weights: chunk p
// (0..15) of a super-block holds bytes 8 + 8p .. 8 + 8p + 7, i.e. sub-block i = p / 2,
// elements 32i + 8h + j (low nibbles) and 32i + 16 + 8h + j (high nibbles), h = p % 2,
// j = 0..7.  A thread reads its chunk and the super-block's first 8 bytes (d and the
// codes) with two 8-byte loads.
#include "common.hpp"
#include "launch.hpp"

namespace iq4 {

constexpr int kXsQK = 256;
constexpr int kXsBytes = 136;
constexpr int kXsChunks = 16;           // chunks per super-block
constexpr int kXsMaxWaves = 8;          // the matvec's workgroup covers K in <= 8 waves

// d * (ls_i - 32) from the super-block's first 8 bytes (lo = bytes 0-3, hi = bytes 4-7).
__device__ __forceinline__ float xs_subscale(uint32_t lo, uint32_t hi, int i) {
  const uint32_t ls = ((hi >> (4 * i)) & 0xFu) | (((lo >> (16 + 2 * i)) & 0x3u) << 4);
  return h2f((uint16_t)(lo & 0xFFFFu)) * (float)((int)ls - 32);  // exact
}

// Four nibbles (one per byte, 0..15) -> their four codebook levels as int8 bytes: two
// byte permutes from the register-held tables (levels 0-7 and 8-15) and a per-byte
// select on bit 3.
__device__ __forceinline__ uint32_t xs_levels4(uint32_t nib4) {
  const uint32_t sel = nib4 & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(kLevels1, kLevels0, sel);
  const uint32_t hi = __builtin_amdgcn_perm(kLevels3, kLevels2, sel);
  const uint32_t m = ((nib4 >> 3) & 0x01010101u) * 0xFFu;
  return (hi & m) | (lo & ~m);
}

__device__ __forceinline__ float xs_byte_level(uint32_t levels, int j) {
  return (float)((int32_t)(levels << (24 - 8 * j)) >> 24);
}

// The 16 levels of a chunk as floats: a[j] = element 32i + 8h + j, b[j] = 32i + 16 + 8h + j.
__device__ __forceinline__ void xs_chunk_levels(uint2 q, float (&a)[8], float (&b)[8]) {
  const uint32_t la0 = xs_levels4(q.x & 0x0F0F0F0Fu), la1 = xs_levels4(q.y & 0x0F0F0F0Fu);
  const uint32_t lb0 = xs_levels4((q.x >> 4) & 0x0F0F0F0Fu), lb1 = xs_levels4((q.y >> 4) & 0x0F0F0F0Fu);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = xs_byte_level(la0, j);
    a[4 + j] = xs_byte_level(la1, j);
    b[j] = xs_byte_level(lb0, j);
    b[4 + j] = xs_byte_level(lb1, j);
  }
}

// ---------------------------------------------------------------------------------
// Block decode: one thread per chunk, 16 outputs (two runs of 8), binary32 or binary16
// (the binary16 rounding, to nearest even with subnormals, of the exact binary32 value).
template <bool F16>
__global__ void __launch_bounds__(256) xs_dequant_kernel(const uint8_t* __restrict__ sb, int64_t nchunks,
                                                         void* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int64_t s = c >> 4;
  const int p = (int)(c & 15), i = p >> 1, h = p & 1;
  const uint8_t* base = sb + s * kXsBytes;
  const uint2 hdr = *reinterpret_cast<const uint2*>(base);
  const uint2 q = *reinterpret_cast<const uint2*>(base + 8 + 8 * p);
  const float dl = xs_subscale(hdr.x, hdr.y, i);
  float a[8], b[8];
  xs_chunk_levels(q, a, b);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] *= dl;  // exact
    b[j] *= dl;
  }
  const int64_t e = s * kXsQK + 32 * i + 8 * h;  // run a starts here, run b 16 later
  if (F16) {
    // The exact binary32 values are converted one by one (v_cvt_f16_f32, round to
    // nearest even).  The empty asm keeps the compiler from folding the multiply and
    // the conversion into one mixed-precision FMA with a +0 addend, which would turn
    // a -0 product into +0.
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(a[j]), "+v"(b[j]));
    uint32_t ha[4], hb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ha[j] = (uint32_t)__half_as_ushort(__float2half_rn(a[2 * j])) |
              ((uint32_t)__half_as_ushort(__float2half_rn(a[2 * j + 1])) << 16);
      hb[j] = (uint32_t)__half_as_ushort(__float2half_rn(b[2 * j])) |
              ((uint32_t)__half_as_ushort(__float2half_rn(b[2 * j + 1])) << 16);
    }
    uint16_t* o = static_cast<uint16_t*>(out) + e;
    *reinterpret_cast<uint4*>(o) = make_uint4(ha[0], ha[1], ha[2], ha[3]);
    *reinterpret_cast<uint4*>(o + 16) = make_uint4(hb[0], hb[1], hb[2], hb[3]);
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + e);
    o[0] = make_float4(a[0], a[1], a[2], a[3]);
    o[1] = make_float4(a[4], a[5], a[6], a[7]);
    o[4] = make_float4(b[0], b[1], b[2], b[3]);
    o[5] = make_float4(b[4], b[5], b[6], b[7]);
  }
}

// ---------------------------------------------------------------------------------
// T-column matvec Y[t][r] = sum_k W[r][k] X[t][k].
//
// A workgroup owns R consecutive rows and all of K.  Its 64W lanes split K by chunks
// (lane j takes chunks j, j + 64W, ... of every row), so each lane loads the 16 x T
// activations of its chunk once per pass over K and keeps them in registers while it
// streams the R rows' chunks: per lane and row, s_t = sum of the 16 level * x products
// (fixed order), then acc[r][t] += (d (ls - 32)) * s_t.  The R x T partial sums are
// then reduced across the wave (per column: halving exchanges over lane bits 5, 4, ..
// that leave each lane group one row, then plain exchanges over the remaining bits)
// and across the W waves in wave order.  Every column goes through the same operations
// in the same order whatever T is, so column t of a T-column call equals the T = 1
// call bit for bit.
struct XsQmvArgs {
  const uint8_t* W;
  const float* X;
  float* Y;
  int64_t n, ldx, ldy;
  int64_t row_bytes;
  int nchunks;  // chunks per row (k / 16)
};

template <int T, int R>
__global__ void __launch_bounds__(64 * kXsMaxWaves) xs_qmv_kernel(XsQmvArgs a) {
  static_assert((R & (R - 1)) == 0 && R <= 64, "R must be a power of two");
  constexpr int LOG_R = (R >= 64) ? 6 : (R >= 32) ? 5 : (R >= 16) ? 4 : (R >= 8) ? 3 : (R >= 4) ? 2 : (R >= 2) ? 1 : 0;
  __shared__ float red[kXsMaxWaves][R][T];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthr = blockDim.x, nwaves = nthr >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * R;

  float acc[R][T];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[r][t] = 0.0f;

  const uint8_t* rowp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = (row0 + r < a.n) ? row0 + r : a.n - 1;  // tail rows read the last row
    rowp[r] = a.W + row * a.row_bytes;
  }

  for (int c0 = 0; c0 < a.nchunks; c0 += nthr) {  // the same trip count for every lane
    const int c = c0 + tid;
    const bool has = c < a.nchunks;
    const int cc = has ? c : a.nchunks - 1;
    const int s = cc >> 4, p = cc & 15, i = p >> 1, h = p & 1;
    const int64_t hoff = (int64_t)s * kXsBytes;
    // weights first (the long-latency loads), then the activations
    uint2 hdr[R], q[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      hdr[r] = *reinterpret_cast<const uint2*>(rowp[r] + hoff);
      q[r] = *reinterpret_cast<const uint2*>(rowp[r] + hoff + 8 + 8 * p);
    }
    float xa[T][8], xb[T][8];
    const int64_t e = (int64_t)s * kXsQK + 32 * i + 8 * h;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float4* xp = reinterpret_cast<const float4*>(a.X + t * a.ldx + e);
      const float4 v0 = xp[0], v1 = xp[1], v2 = xp[4], v3 = xp[5];
      xa[t][0] = v0.x; xa[t][1] = v0.y; xa[t][2] = v0.z; xa[t][3] = v0.w;
      xa[t][4] = v1.x; xa[t][5] = v1.y; xa[t][6] = v1.z; xa[t][7] = v1.w;
      xb[t][0] = v2.x; xb[t][1] = v2.y; xb[t][2] = v2.z; xb[t][3] = v2.w;
      xb[t][4] = v3.x; xb[t][5] = v3.y; xb[t][6] = v3.z; xb[t][7] = v3.w;
    }
    if (has) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float la[8], lb[8];
        xs_chunk_levels(q[r], la, lb);
        const float dl = xs_subscale(hdr[r].x, hdr[r].y, i);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          float sum = la[0] * xa[t][0];
#pragma unroll
          for (int j = 1; j < 8; ++j) sum = fmaf(la[j], xa[t][j], sum);
#pragma unroll
          for (int j = 0; j < 8; ++j) sum = fmaf(lb[j], xb[t][j], sum);
          acc[r][t] = fmaf(dl, sum, acc[r][t]);
        }
      }
    }
  }

  // wave reduction, column by column
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = acc[r][t];
#pragma unroll
    for (int half = R / 2, mask = 32; half >= 1; half >>= 1, mask >>= 1) {
      const bool up = (lane & mask) != 0;
#pragma unroll
      for (int j = 0; j < half; ++j) {
        const float keep = up ? v[j + half] : v[j];
        const float send = up ? v[j] : v[j + half];
        v[j] = keep + __shfl_xor(send, mask);
      }
    }
#pragma unroll
    for (int mask = 32 >> LOG_R; mask >= 1; mask >>= 1) v[0] += __shfl_xor(v[0], mask);
    if ((lane & ((64 >> LOG_R) - 1)) == 0) red[wave][lane >> (6 - LOG_R)][t] = v[0];
  }
  __syncthreads();
  if (tid < R * T) {
    const int r = tid / T, t = tid % T;
    float sum = red[0][r][t];
    for (int w = 1; w < nwaves; ++w) sum += red[w][r][t];
    if (row0 + r < a.n) a.Y[t * a.ldy + row0 + r] = sum;
  }
}

// ---------------------------------------------------------------------------------

int launch_xs_dequant(const void* sb, int64_t nsb, bool f16, void* out, hipStream_t s) {
  if (nsb == 0) return 0;
  const int64_t nchunks = nsb * kXsChunks;
  const int64_t grid = (nchunks + 255) / 256;
  const uint8_t* p = static_cast<const uint8_t*>(sb);
  if (f16)
    hipLaunchKernelGGL(xs_dequant_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, p, nchunks, out);
  else
    hipLaunchKernelGGL(xs_dequant_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, p, nchunks, out);
  return check_launch("xs_dequant_kernel");
}

// Rows per workgroup: 8 up to T = 4, 4 above (keeps the activations, the partial sums
// and the R rows' loads within 256 registers).
template <int T>
static int launch_xs_qmv_t(const XsQmvArgs& a, int64_t n, int waves, hipStream_t s) {
  constexpr int R = (T <= 4) ? 8 : 4;
  const int64_t grid = (n + R - 1) / R;
  hipLaunchKernelGGL((xs_qmv_kernel<T, R>), dim3((unsigned)grid), dim3(64 * waves), 0, s, a);
  return check_launch("xs_qmv_kernel");
}

int launch_xs_qmv(const void* W, int64_t n, int64_t k, const float* x, int64_t ldx, int T, float* y,
                  int64_t ldy, hipStream_t s) {
  XsQmvArgs a;
  a.W = static_cast<const uint8_t*>(W);
  a.X = x;
  a.Y = y;
  a.n = n;
  a.ldx = ldx;
  a.ldy = ldy;
  a.row_bytes = (k / kXsQK) * kXsBytes;
  a.nchunks = (int)(k / 16);
  // waves per workgroup from K alone (never from T): one chunk per lane where possible
  int waves = (int)((a.nchunks + 63) / 64);
  waves = waves < 1 ? 1 : (waves > kXsMaxWaves ? kXsMaxWaves : waves);
  switch (T) {
    case 1: return launch_xs_qmv_t<1>(a, n, waves, s);
    case 2: return launch_xs_qmv_t<2>(a, n, waves, s);
    case 3: return launch_xs_qmv_t<3>(a, n, waves, s);
    case 4: return launch_xs_qmv_t<4>(a, n, waves, s);
    case 5: return launch_xs_qmv_t<5>(a, n, waves, s);
    case 6: return launch_xs_qmv_t<6>(a, n, waves, s);
    case 7: return launch_xs_qmv_t<7>(a, n, waves, s);
    default: return launch_xs_qmv_t<8>(a, n, waves, s);
  }
}

}  // namespace iq4
