// gemm.hip -- dequant-fused GEMM on the matrix cores: C = A * W^T with A binary16
// activations (token-major), W IQ4 blocks decoded to binary16 inside the kernel and
// fp32 accumulation (v_mfma_f32_16x16x32_f16, one 32-weight block per instruction).
//
// Three uses of one kernel body:
//   DENSE   the long-prompt projection, one launch per prompt chunk;
//   GATEUP  MoE prefill, first product: rows of A gathered per expert from the routed
//           pairs, gate and up weights side by side, SwiGLU in the epilogue, h stored
//           as binary16 in pair-sorted order;
//   DOWN    MoE prefill, second product: A = h (contiguous per expert), the epilogue
//           scales by the pair's gate weight and writes the pair's row (or adds it
//           atomically into the token's output).
//
// Tiling (workgroup = 4 waves, 128 x 256 outputs):
//   * the 128 x 128 activation tile of one 4-block quad is staged in LDS, already in
//     matrix-core fragment order (a fragment read is one conflict-free 1 KiB
//     ds_read_b128 per wave), double-buffered across quads;
//   * each wave owns 64 weight rows (4 packed row tiles) and decodes them itself,
//     straight from the packed tiles into B fragments: one 128-bit load of indices and
//     one 64-bit load of scales per row tile and quad, a byte-indexed LDS table giving
//     two binary16 levels per byte, and one packed binary16 multiply by the block
//     scale -- the binary16 rounding of the exact decoded weight.  No decoded weight
//     goes through LDS or HBM;
//   * per block a wave issues 8 x 4 MFMAs against 8 A-fragment reads.
//
// Within a fragment the 32 weights of a block are visited in the order
// 0,16,1,17,...,15,31 (low/high nibble of each index byte); the activation tile is
// written to LDS in the same order, so each MFMA still sums one block's products.
#include "common.hpp"
#include "launch.hpp"
#include "gemm.hpp"

namespace iq4 {

constexpr int kBM = 128;                 // rows of A per workgroup
constexpr int kWaveRT = 4;               // packed row tiles (16 rows) per wave
constexpr int kWaves = 4;
constexpr int kBN = kWaves * kWaveRT * kTileRows;  // 256 weight rows per workgroup
constexpr int kMT = kBM / 16;            // 8 fragment rows of A
constexpr int kALdsQuad = kTileBlocks * kMT * 64 * 16;  // 32 KiB per quad

__device__ __forceinline__ uint32_t f16_of_level(int c) {
  return (uint32_t)__half_as_ushort(__int2half_rn(c));  // exact: |c| <= 127
}

// XCD-aware order of the workgroups: hardware deals workgroup b to XCD b mod 8, so
// logical tile L = (b mod 8) * (G / 8) + b / 8 keeps runs of consecutive logical tiles
// (which share weight row tiles) inside one XCD and its L2.
__device__ __forceinline__ int64_t xcd_swizzle(int64_t b, int64_t G) {
  if (G % 8) return b;
  return (b % 8) * (G / 8) + b / 8;
}

template <int MODE>
__global__ void __launch_bounds__(256) qgemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kALdsQuad];
  __shared__ uint32_t lut[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  lut[tid] = f16_of_level(level_of(tid & 15)) | (f16_of_level(level_of(tid >> 4)) << 16);

  // ---- which tile ------------------------------------------------------------------
  int64_t m0, rows;          // first A row (in the launch's row space) and valid rows
  int64_t n0;                // first weight row of the workgroup
  int e = 0;                 // expert (grouped modes)
  int64_t seg0 = 0;          // first sorted pair of the expert (grouped modes)
  const uint8_t* W0 = a.W0;
  const uint8_t* W1 = a.W1;
  if (MODE == kGemmDense) {
    const int64_t G = (int64_t)gridDim.x;
    const int64_t L = xcd_swizzle(blockIdx.x, G);
    const int64_t mt_n = (a.M + kBM - 1) / kBM;
    const int64_t mt = L % mt_n, nt = L / mt_n;
    m0 = mt * kBM;
    rows = min((int64_t)kBM, a.M - m0);
    n0 = nt * kBN;
  } else {
    const int64_t ntl = a.n_tiles_n;
    const int64_t L = xcd_swizzle(blockIdx.x, (int64_t)gridDim.x);
    const int64_t ti = L / ntl, nt = L % ntl;
    if (ti >= *a.num_tiles) return;
    e = a.tiles[2 * ti];
    const int mt = a.tiles[2 * ti + 1];
    seg0 = a.offsets[e];
    const int64_t cnt = a.offsets[e + 1] - seg0;
    m0 = (int64_t)mt * kBM;
    rows = min((int64_t)kBM, cnt - m0);
    // GATEUP: a workgroup covers 128 intermediate columns (each wave 32 gate rows and
    // the same 32 up rows); DOWN: 256 output rows.
    n0 = (MODE == kGemmGateUp) ? nt * (kBN / 2) : nt * kBN;
    W0 += (int64_t)e * a.w_expert_stride;
    if (MODE == kGemmGateUp) W1 += (int64_t)e * a.w_expert_stride;
  }
  const int64_t kq_n = a.K / kTileK;
  const int64_t nib_bytes = a.N * (a.K / kQK) * kNibbleBytes;

  // ---- weight row tiles of this wave -------------------------------------------------
  // DENSE / DOWN: rows n0 + 64w + 16r, r = 0..3 of W0.
  // GATEUP: r = 0,1 -> gate rows n0 + 32w + 16r;  r = 2,3 -> up rows n0 + 32w + 16(r-2).
  const uint8_t* wbase[kWaveRT];
  int64_t wtile0[kWaveRT];
  bool rt_ok[kWaveRT];
#pragma unroll
  for (int r = 0; r < kWaveRT; ++r) {
    int64_t row0;
    if (MODE == kGemmGateUp) {
      row0 = n0 + 32 * wave + 16 * (r & 1);
      wbase[r] = (r < 2) ? W0 : W1;
    } else {
      row0 = n0 + 64 * wave + 16 * r;
      wbase[r] = W0;
    }
    rt_ok[r] = row0 < a.N;
    wtile0[r] = (rt_ok[r] ? row0 / kTileRows : 0) * kq_n;  // tile index of quad 0
  }

  // ---- A staging: 1024 items of (row, block, half) per quad, 4 per thread ----------
  // item = ((row * 4) + block) * 2 + half; reads physical k chunks [8h, 8h+8) and
  // [16 + 8h, 16 + 8h + 8) of the block and writes fragments g = 2h and 2h + 1.
  const uint16_t* arow[4];
  int a_lds_off[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int item = tid + 256 * it;
    const int half = item & 1, blk = (item >> 1) & 3, r = item >> 3;  // r = 0..127
    const uint16_t* p = nullptr;
    if (r < rows) {
      int64_t src_row;
      if (MODE == kGemmDense) {
        src_row = m0 + r;
      } else if (MODE == kGemmGateUp) {
        src_row = a.pairs[seg0 + m0 + r] / a.top_k;  // token of the pair
      } else {
        src_row = seg0 + m0 + r;  // h is stored in pair-sorted order
      }
      p = a.A + src_row * a.lda + blk * kQK + 8 * half;
    }
    arow[it] = p;
    const int mt = r >> 4, rr = r & 15;
    a_lds_off[it] = ((blk * kMT + mt) * 64 + (2 * half) * 16 + rr) * 16;
  }

  uint4 a_reg[4][2];
  auto load_a = [&](int64_t q) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if (arow[it]) {
        const uint4* p = reinterpret_cast<const uint4*>(arow[it] + q * kTileK);
        a_reg[it][0] = p[0];
        a_reg[it][1] = p[2];  // + 16 elements
      } else {
        a_reg[it][0] = make_uint4(0, 0, 0, 0);
        a_reg[it][1] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const uint4 L = a_reg[it][0], H = a_reg[it][1];
      const uint32_t lo[4] = {L.x, L.y, L.z, L.w};
      const uint32_t hi[4] = {H.x, H.y, H.z, H.w};
      uint32_t f[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        f[2 * d] = __builtin_amdgcn_perm(hi[d], lo[d], 0x05040100u);
        f[2 * d + 1] = __builtin_amdgcn_perm(hi[d], lo[d], 0x07060302u);
      }
      uint8_t* dst = &lds_a[buf][a_lds_off[it]];
      *reinterpret_cast<uint4*>(dst) = make_uint4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<uint4*>(dst + 16 * 16) = make_uint4(f[4], f[5], f[6], f[7]);
    }
  };

  uint4 nib[kWaveRT];
  uint2 scl[kWaveRT];
  auto load_b = [&](int64_t q) {
#pragma unroll
    for (int r = 0; r < kWaveRT; ++r) {
      const int64_t tile = wtile0[r] + q;
      nib[r] = *reinterpret_cast<const uint4*>(wbase[r] + tile * kTileNibbleBytes + lane * 16);
      scl[r] = *reinterpret_cast<const uint2*>(wbase[r] + nib_bytes + tile * kTileScaleBytes + c * 8);
    }
  };

  f32x4 acc[kMT][kWaveRT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int r = 0; r < kWaveRT; ++r) acc[i][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();

  for (int64_t q = 0; q < kq_n; ++q) {
    const int buf = (int)(q & 1);
    uint4 cur_nib[kWaveRT];
    uint2 cur_scl[kWaveRT];
#pragma unroll
    for (int r = 0; r < kWaveRT; ++r) {
      cur_nib[r] = nib[r];
      cur_scl[r] = scl[r];
    }
    if (q + 1 < kq_n) {
      load_a(q + 1);
      load_b(q + 1);
    }
#pragma unroll
    for (int j = 0; j < kTileBlocks; ++j) {
      u32x4 bf[kWaveRT];
#pragma unroll
      for (int r = 0; r < kWaveRT; ++r) {
        const uint32_t w = (j == 0) ? cur_nib[r].x : (j == 1) ? cur_nib[r].y : (j == 2) ? cur_nib[r].z : cur_nib[r].w;
        const uint32_t sw = (j < 2) ? cur_scl[r].x : cur_scl[r].y;
        const uint32_t dd = __builtin_amdgcn_perm(sw, sw, (j & 1) ? 0x03020302u : 0x01000100u);
        bf[r][0] = pk_mul_f16(lut[w & 0xFF], dd);
        bf[r][1] = pk_mul_f16(lut[(w >> 8) & 0xFF], dd);
        bf[r][2] = pk_mul_f16(lut[(w >> 16) & 0xFF], dd);
        bf[r][3] = pk_mul_f16(lut[w >> 24], dd);
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const u32x4 af =
            *reinterpret_cast<const u32x4*>(&lds_a[buf][((j * kMT + mt) * 64 + lane) * 16]);
#pragma unroll
        for (int r = 0; r < kWaveRT; ++r) acc[mt][r] = mfma_f16(af, bf[r], acc[mt][r]);
      }
    }
    if (q + 1 < kq_n) store_a(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds D[4g + i][c] of each (mt, r) fragment -------------------
  if (MODE == kGemmDense) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * mt + 4 * g + i;
        if (rr >= rows) continue;
        float* crow = a.C + (m0 + rr) * a.ldc + n0 + 64 * wave + c;
#pragma unroll
        for (int r = 0; r < kWaveRT; ++r)
          if (rt_ok[r]) crow[16 * r] = acc[mt][r][i];
      }
  } else if (MODE == kGemmGateUp) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * mt + 4 * g + i;
        if (rr >= rows) continue;
        uint16_t* hrow = a.H + (seg0 + m0 + rr) * a.ldh + n0 + 32 * wave + c;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (!rt_ok[r]) continue;
          const float gv = acc[mt][r][i], uv = acc[mt][r + 2][i];
          const float h = gv / (1.0f + __expf(-gv)) * uv;
          hrow[16 * r] = __half_as_ushort(__float2half_rn(h));
        }
      }
  } else {  // DOWN
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * mt + 4 * g + i;
        if (rr >= rows) continue;
        const int p = a.pairs[seg0 + m0 + rr];
        const float gw = a.gate_w[p];
        if (a.atomic) {
          float* orow = a.out + (int64_t)(p / a.top_k) * a.ldo + n0 + 64 * wave + c;
#pragma unroll
          for (int r = 0; r < kWaveRT; ++r)
            if (rt_ok[r]) atomicAdd(orow + 16 * r, gw * acc[mt][r][i]);
        } else {
          float* yrow = a.C + (int64_t)p * a.ldc + n0 + 64 * wave + c;
#pragma unroll
          for (int r = 0; r < kWaveRT; ++r)
            if (rt_ok[r]) yrow[16 * r] = gw * acc[mt][r][i];
        }
      }
  }
}

int launch_qgemm_dense(const uint8_t* packed, int64_t n, int64_t k, const uint16_t* x, int64_t m,
                       int64_t ldx, float* y, int64_t ldy, int64_t chunk, hipStream_t s) {
  if (chunk <= 0) chunk = m;
  for (int64_t c0 = 0; c0 < m; c0 += chunk) {
    GemmArgs a{};
    a.A = x + c0 * ldx;
    a.lda = ldx;
    a.W0 = packed;
    a.N = n;
    a.K = k;
    a.M = (m - c0 < chunk) ? (m - c0) : chunk;
    a.C = y + c0 * ldy;
    a.ldc = ldy;
    const int64_t grid = ((a.M + kBM - 1) / kBM) * ((n + kBN - 1) / kBN);
    hipLaunchKernelGGL(qgemm_kernel<kGemmDense>, dim3((unsigned)grid), dim3(256), 0, s, a);
    if (int e = check_launch("qgemm_kernel<dense>")) return e;
  }
  return 0;
}

int launch_qgemm_grouped(int mode, const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  const int64_t grid = max_tiles * a.n_tiles_n;
  if (grid == 0) return 0;
  if (mode == kGemmGateUp)
    hipLaunchKernelGGL(qgemm_kernel<kGemmGateUp>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(qgemm_kernel<kGemmDown>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return check_launch(mode == kGemmGateUp ? "qgemm_kernel<gateup>" : "qgemm_kernel<down>");
}

}  // namespace iq4
