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

template <int N>
struct ColsXs {  // a column count as a type (compile-time pass width)
  static constexpr int value = N;
};

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
// T-column matvec on the matrix cores (K up to 24 super-blocks), the dense matvec's
// scheme on the raw super-blocks: one workgroup per 16 rows, all of K; each of up to NWV
// waves (8, or 4 so that two workgroups share a CU when there are more row tiles than
// CUs) owns a run of WS super-blocks.  A sub-block (32 weights, one scale d (ls - 32))
// is one v_mfma_f32_16x16x32_bf16:
//   B  lane (g, c) needs index bytes 4g .. 4g+3 of row c's sub-block: byte 4g + j holds
//      elements 4g + j (low nibble) and 4g + j + 16 (high), which a byte-indexed level
//      table turns into the bf16 pair at MFMA k = 8g + 2j, 8g + 2j + 1;
//   A  the activations in the same k order: each fp32 x goes in as two bf16 parts, hi =
//      bf16(x) and lo = bf16(x - hi) (x to within 2^-18 |x|), rows 4s + t of the operand
//      (s = 0 hi, 1 lo; t the column within a pass of 4), staged in LDS per wave;
//   the product, exact per term, is scaled by the sub-block scale (exact in fp32) with
//   one FMA per column; the waves' sums are added in wave order, hi parts and lo parts
//   apart, then hi + lo.  A column's arithmetic depends on K only, not on T.
constexpr int kXmWaves = 8;               // waves per workgroup, at most
constexpr int kXmSlot = 9 * 16;          // 8 rows of 16 B + 1 of padding (staging banks)
constexpr int kXmSubStage = 4 * kXmSlot;  // one sub-block's A operand: 576 B
constexpr int kXmMaxWS = 3;              // super-blocks per wave (K <= 24 super-blocks)

template <int WS, int NWV>
struct XmShape {
  static constexpr int kStage = NWV * WS * 8 * kXmSubStage;
  static constexpr int kRed = NWV * 64 * 16;
  static constexpr int kBudget = (NWV == 4 ? 80 : 160) * 1024;  // 4 waves: two workgroups per CU
  // table copies: 64 (each lane its own; the lookup address is one byte permute) where
  // the LDS has room, else 32 or 16
  static constexpr int kLC = (256 * 64 * 4 + kStage + kRed <= kBudget)   ? 64
                             : (256 * 32 * 4 + kStage + kRed <= kBudget) ? 32
                                                                         : 16;
  static constexpr int kLutBytes = 256 * kLC * 4;
  static_assert(kLutBytes + kStage + kRed <= kBudget, "LDS budget");
};

struct XmArgs {
  const uint8_t* W;
  const float* X;
  float* Y;
  int64_t n, ldx, ldy, row_bytes;
  int T, nsb;  // columns; super-blocks per row
  int ws;      // super-blocks per wave (the template's WS)
};

// (4 waves: registers for two workgroups per CU, i.e. two waves per SIMD)
template <int WS, int NWV, int TP>
__global__ void __launch_bounds__(64 * NWV, NWV == 4 ? 2 : 1) xs_qmv_mfma_kernel(XmArgs a) {
  using S = XmShape<WS, NWV>;
  constexpr int LC = S::kLC;
  __shared__ __attribute__((aligned(256))) uint8_t smem[S::kLutBytes + S::kStage + S::kRed];
  // every kernel argument at entry (one scalar wait)
  const uint8_t* const W = a.W;
  const float* const X = a.X;
  float* const Y = a.Y;
  const int64_t n = a.n, ldx = a.ldx, ldy = a.ldy, row_bytes = a.row_bytes;
  const int T_all = a.T, nsb = a.nsb;
  asm volatile("" ::"s"(W), "s"(X), "s"(Y), "s"(n), "s"(ldx), "s"(ldy), "s"(row_bytes), "s"(T_all), "s"(nsb));
  uint8_t* const xs = smem + S::kLutBytes;
  f32x4* const red = reinterpret_cast<f32x4*>(smem + S::kLutBytes + S::kStage);
  typedef __attribute__((address_space(3))) const uint8_t lds_u8;
  lds_u8* const lds = (lds_u8*)(__attribute__((address_space(3))) uint8_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), nwaves = (int)(blockDim.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * kTileRows;
  const int s0 = wave * WS, s1 = min(s0 + WS, nsb);  // this wave's super-blocks
  const int nsub = 8 * (s1 - s0);                     // its sub-blocks (>= 8 for a launched wave)
  uint8_t* const xw = xs + wave * (WS * 8) * kXmSubStage;

  // ---- staging tasks: (column t, sub-block sl, k-group gg) = task t SL + 4 sl + gg ---
  constexpr int SL = 32 * WS;  // tasks per column
  constexpr int NI = 2 * WS;   // 4 SL / 64 task rounds
  float4 xr[NI][2];
  auto load_x = [&](int64_t t0, int T) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int task = lane + 64 * i;
      const int t = task / SL, sl = (task % SL) >> 2, gg = task & 3;
      if (t < T && sl < nsub) {
        const float* p = X + (t0 + t) * ldx + (int64_t)s0 * kXsQK + 32 * sl + 4 * gg;
        xr[i][0] = *reinterpret_cast<const float4*>(p);       // elements 4gg .. 4gg+3
        xr[i][1] = *reinterpret_cast<const float4*>(p + 16);  // elements 4gg+16 .. 4gg+19
      }
    }
  };
  // word j of a k-group slot row pairs elements 4gg + j and 4gg + j + 16 (the index
  // byte order); part s of column t in row 4s + t
  auto store_x = [&](int T) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int task = lane + 64 * i;
      const int t = task / SL, sl = (task % SL) >> 2, gg = task & 3;
      if (t < T && sl < nsub) {
        uint32_t h[4], l[4];
        split_hi_lo(xr[i][0].x, xr[i][1].x, h[0], l[0]);
        split_hi_lo(xr[i][0].y, xr[i][1].y, h[1], l[1]);
        split_hi_lo(xr[i][0].z, xr[i][1].z, h[2], l[2]);
        split_hi_lo(xr[i][0].w, xr[i][1].w, h[3], l[3]);
        uint8_t* dst = xw + (sl * 4 + gg) * kXmSlot + t * 16;
        *reinterpret_cast<uint4*>(dst) = uint4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<uint4*>(dst + 4 * 16) = uint4{l[0], l[1], l[2], l[3]};
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };

  // ---- requests: the first pass's activations, then every weight of the wave ----------
  // (rows past n read row n - 1; their outputs are dropped)
  const uint8_t* const rowp = W + min(r0 + c, n - 1) * row_bytes;
  constexpr int T0 = TP;
  load_x(0, T0);
  // Lane (g, c) loads the index bytes of sub-blocks g and 4 + g of row c (16 bytes
  // each, so a row's 64 bytes per load), and a 4 x 4 transpose across the lane groups
  // (two 32-lane and two 16-lane swaps per set of four) leaves in its register q[u][i]
  // dword g of sub-block i, the lane's B operand.
  typedef uint32_t u32x4a8 __attribute__((ext_vector_type(4), aligned(8)));
  uint2 hdr[WS];
  uint32_t q[WS][8];
#pragma unroll
  for (int u = 0; u < WS; ++u) {
    const int sb = min(s0 + u, s1 - 1);  // idle slots reload a valid super-block
    const uint8_t* p = rowp + (int64_t)sb * kXsBytes;
    hdr[u] = *reinterpret_cast<const uint2*>(p);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4a8 v = *reinterpret_cast<const u32x4a8*>(p + 8 + 16 * (4 * h + g));
#pragma unroll
      for (int j = 0; j < 4; ++j) q[u][4 * h + j] = v[j];
    }
  }
  // register j of lane group g: word j of the group's load -> word g of group j's load
  auto transpose4 = [](uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
    const auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);  // rows: [r0 r0 r2 r2], [r0 r0 r2 r2]
    const auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
    const auto c0 = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto c1 = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    r0 = c0[0];
    r1 = c0[1];
    r2 = c1[0];
    r3 = c1[1];
  };
  // ---- level table: 16-byte chunk qq of LC / 4 per entry, consecutive threads write
  // consecutive chunks (no bank conflicts) --------------------------------------------
  {
    constexpr int PER = LC / 4;
    uint4* dst = reinterpret_cast<uint4*>(smem);
    for (int qq = tid; qq < 256 * PER; qq += 64 * nwaves) {
      const int e = qq / PER;
      const uint32_t v = bf16_of_level(level_of((uint32_t)e & 15u)) | (bf16_of_level(level_of((uint32_t)e >> 4)) << 16);
      dst[qq] = uint4{v, v, v, v};
    }
  }
  const uint32_t lane_copy = (uint32_t)lane * 4u;
  auto lookup = [&](uint32_t w, int b) -> uint32_t {
    uint32_t addr;
    if (LC == 64) {
      addr = __builtin_amdgcn_perm(lane_copy, w, 0x0c0c0004u | ((uint32_t)b << 8));
    } else {
      addr = ((w >> (8 * b)) & 0xFFu) * (LC * 4) + (lane_copy & (LC * 4 - 1));
    }
    return *reinterpret_cast<__attribute__((address_space(3))) const uint32_t*>(lds + addr);
  };
  lds_u8* const arow_p = lds + S::kLutBytes + (wave * (WS * 8) * kXmSubStage + g * kXmSlot + c * 16);

  // NC columns in this pass: accumulator entry i of a lane in k-group g holds row 4g + i
  // (g = 0 hi, 1 lo; column i), so the scale FMAs of columns past NC are skipped
  constexpr int XG = (WS >= 3) ? 2 : 4;  // sub-blocks in flight per step (registers)
  auto multiply = [&](f32x4& acc, auto nc) {
    constexpr int NC = decltype(nc)::value;
    const bool arow = c < 8 && (c & 3) < NC;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < WS; ++u) {
      if (s0 + u >= s1) break;
      __builtin_amdgcn_sched_barrier(0);  // super-block u's work waits for its own weights
      uint32_t qt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) qt[i] = q[u][i];
      transpose4(qt[0], qt[1], qt[2], qt[3]);
      transpose4(qt[4], qt[5], qt[6], qt[7]);
#pragma unroll
      for (int h4 = 0; h4 < 8 / XG; ++h4) {  // sub-blocks XG h4 .. XG h4 + XG - 1
        u32x4 xf[XG], bf[XG];
#pragma unroll
        for (int j = 0; j < XG; ++j) {
          const int i = XG * h4 + j;
          if (arow)
            xf[j] = *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(arow_p + (u * 8 + i) * kXmSubStage);
#pragma unroll
          for (int b = 0; b < 4; ++b) bf[j][b] = lookup(qt[i], b);
        }
        f32x4 prod[XG];
#pragma unroll
        for (int j = 0; j < XG; ++j) prod[j] = mfma_bf16(xf[j], bf[j], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j = 0; j < XG; ++j) {
          const float d = xs_subscale(hdr[u].x, hdr[u].y, XG * h4 + j);
#pragma unroll
          for (int i = 0; i < NC; ++i) acc[i] = __builtin_fmaf(d, prod[j][i], acc[i]);
        }
      }
    }
  };
  // cross-wave sums in wave order, hi and lo apart, then hi + lo
  auto reduce_store = [&](int64_t t0, int T, const f32x4& acc) {
    red[wave * 64 + lane] = acc;
    lds_barrier();
    const int t = tid >> 4, row = tid & 15;
    if (tid < T * kTileRows && r0 + row < n) {
      const float* redf = reinterpret_cast<const float*>(red);
      float pv[2][NWV];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int w2 = 0; w2 < NWV; ++w2) pv[p][w2] = redf[(w2 * 64 + 16 * p + row) * 4 + t];
      float part[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float sum = pv[p][0];
#pragma unroll
        for (int w2 = 1; w2 < NWV; ++w2) sum = (w2 < nwaves) ? sum + pv[p][w2] : sum;
        part[p] = sum;
      }
      Y[(t0 + t) * ldy + r0 + row] = part[0] + part[1];
    }
  };

  // ---- the first pass (up to 4 columns), then passes of 4 -----------------------------
  store_x(T0);    // waits for the activations only
  lds_barrier();  // the table
  f32x4 acc;
  multiply(acc, ColsXs<T0>{});
  reduce_store(0, T0, acc);
  for (int64_t t0 = 4; t0 < T_all; t0 += 4) {
    const int T = (int)min((int64_t)4, (int64_t)T_all - t0);
    lds_barrier();  // every wave is done with red
    load_x(t0, T);
    store_x(T);
    multiply(acc, ColsXs<4>{});
    reduce_store(t0, T, acc);
  }
}

template <int WS, int NWV, int TP>
static int launch_xm_t(const XmArgs& a, int64_t grid, int waves, hipStream_t s) {
  hipLaunchKernelGGL((xs_qmv_mfma_kernel<WS, NWV, TP>), dim3((unsigned)grid), dim3(64 * waves), 0, s, a);
  return check_launch("xs_qmv_mfma_kernel");
}
template <int WS, int NWV>
static int launch_xm(const XmArgs& a, int64_t grid, int waves, hipStream_t s) {
  switch (a.T < 4 ? a.T : 4) {
    case 1: return launch_xm_t<WS, NWV, 1>(a, grid, waves, s);
    case 2: return launch_xm_t<WS, NWV, 2>(a, grid, waves, s);
    case 3: return launch_xm_t<WS, NWV, 3>(a, grid, waves, s);
    default: return launch_xm_t<WS, NWV, 4>(a, grid, waves, s);
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
  const int64_t nsb = k / kXsQK;
  if (nsb <= (int64_t)kXmWaves * kXmMaxWS) {  // the matrix-core form (by the shape alone, never T)
    XmArgs m;
    m.W = static_cast<const uint8_t*>(W);
    m.X = x;
    m.Y = y;
    m.n = n;
    m.ldx = ldx;
    m.ldy = ldy;
    m.row_bytes = nsb * kXsBytes;
    m.T = T;
    m.nsb = (int)nsb;
    const int64_t grid = (n + kTileRows - 1) / kTileRows;
    // more row tiles than CUs and K within 4 waves' reach: 4-wave workgroups, two per
    // CU, so that every tile runs in the first round; else up to 8 waves (shape only)
    const bool four = grid > 256 && nsb <= 4 * kXmMaxWS;
    const int nwv = four ? 4 : kXmWaves;
    m.ws = (int)((nsb + nwv - 1) / nwv);
    const int waves = (int)((nsb + m.ws - 1) / m.ws);
    if (four) {
      switch (m.ws) {
        case 1: return launch_xm<1, 4>(m, grid, waves, s);
        case 2: return launch_xm<2, 4>(m, grid, waves, s);
        default: return launch_xm<3, 4>(m, grid, waves, s);
      }
    }
    switch (m.ws) {
      case 1: return launch_xm<1, kXmWaves>(m, grid, waves, s);
      case 2: return launch_xm<2, kXmWaves>(m, grid, waves, s);
      default: return launch_xm<3, kXmWaves>(m, grid, waves, s);
    }
  }
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
