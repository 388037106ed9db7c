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
// Tiling (K walked in 4-block quads; each wave owns 128 x 64 outputs, fp32 accumulators):
//   * the long prompt: 8 waves (two per SIMD), 128 x 256 tiles: 4 column groups of 64
//     weight rows, the two waves of a group multiply blocks 0-1 and 2-3 of each quad and
//     their sums are added once after the loop; a ring of 2 LDS stages filled one quad
//     ahead;
//   * the MoE products: 4 waves, 128 x 256 tiles; the activations in one stage refilled
//     block by block (block j of the next quad once every wave has multiplied block j
//     of this one), the weight tiles in two stages filled one quad ahead; two
//     workgroups share a CU and cover each other's waits;
//   * a stage holds one quad of the workgroup's activations or weight tiles, copied
//     straight from global memory with global_load_lds (no operand passes through VGPRs
//     on its way in):
//       activations  32 KiB: every 16-row x 32-k fragment in matrix-core A order
//                    (lane l = 16g + r holds row r, elements 8g..8g+7), one
//                    dwordx4 copy per fragment, the 32 fragments split over the waves;
//       weights      4.5 KiB per column group: its 4 packed row tiles (1 KiB of
//                    indices + 128 B of scales each) as they are in HBM;
//   * each wave decodes its 64 weight rows into B fragments: a byte-indexed LDS table
//     (replicated, each lane reading its own copy) gives two binary16 levels per index
//     byte, one packed binary16 multiply by the block scale gives the binary16
//     rounding of the exact decoded weight.  No decoded weight goes through LDS or HBM;
//   * per block a wave issues its 16 table reads for the next block and its 8 A-fragment
//     reads, then 8 x 4 MFMAs (the table reads complete under them); the weight
//     fragment is the instruction's first operand and the activation fragment its
//     second (both have the same lane layout), so each accumulator holds its 16 x 16
//     output piece transposed: a lane ends with four consecutive columns of one row.
// The copies are issued from inline assembly so that the compiler, which cannot tell
// the ring stages apart, does not drain every copy in flight before each LDS read; the
// kernel waits for them itself: per quad one s_waitcnt for this wave's copies of the
// quad, then one workgroup barrier (the quad is complete for everyone, and the stage
// filled next is no longer read by anyone).  The block-by-block refill instead waits
// and meets at a barrier after each block, with the wait counts worked out below.
#include <type_traits>

#include "common.hpp"
#include "gemm.hpp"
#include "launch.hpp"

namespace iq4 {

constexpr int kBM = 128;                 // rows of A per workgroup
constexpr int kWaveRT = 4;               // packed row tiles (16 rows) per wave
constexpr int kMT = kBM / 16;            // 8 fragment rows of A
constexpr int kABytes = kTileBlocks * kMT * 1024;                        // 32 KiB
constexpr int kWaveBBytes = kWaveRT * (kTileNibbleBytes + kTileScaleBytes);  // 4.5 KiB

// Shape of a workgroup of NW waves in NW / KS column groups of 64 weight rows; the KS
// waves of a column group split each quad's blocks between them (KS = 2: blocks 0-1 and
// 2-3), their partial sums added once after the loop.  One A quad is shared by all.
// SA, SB: quads of activations and of weights held in LDS.  2 = filled one quad ahead;
// 1 = refilled after each quad (two workgroups share a CU and cover each other's waits).
// PB (one activation stage): the stage is refilled block by block, block j of the next
// quad as soon as every wave has multiplied block j of this one.
template <int NW, int KS, int SA, int SB, bool PB = false>
struct Shape {
  static constexpr int kNC = NW / KS;                                   // column groups
  static constexpr int kBN = kNC * kWaveRT * kTileRows;                 // weight rows per workgroup
  static constexpr int kBStageBytes = kNC * kWaveBBytes;                // one quad of weight tiles
  static constexpr int kAPerWave = kTileBlocks * kMT / NW;              // A fragments each wave copies
  static constexpr int kNibPerWave = kWaveRT / KS;                      // index tiles each wave copies
  static constexpr int kSclPerWave = 2 / KS;                            // scale copies each wave issues
  static constexpr int kBlocksPerWave = kTileBlocks / KS;              // blocks of a quad each wave multiplies
  // replicas of the level table (fewer bank conflicts), as many as the LDS left allows
  static constexpr bool kTwoPerCU = (SA == 1 && NW == 4);  // two workgroups share a CU
  static constexpr int kLutCopies = kTwoPerCU ? (SB == 1 ? 16 : 8) : (kNC == 4) ? 32 : 16;
  static_assert(KS == 1 || KS == 2, "K split");
  static_assert((SA == 1 || SA == 2) && (SB == 1 || SB == 2), "ring depth");
  static_assert(!PB || (KS == 1 && SA == 1 && SB == 2), "block refills: one A stage, two weight stages");
  static_assert(SA * kABytes + SB * kBStageBytes + 256 * 4 * kLutCopies + 1024 <= (kTwoPerCU ? 80 : 160) * 1024,
                "LDS budget");
  static_assert(KS == 1 || (kMT / 2) * kWaveRT * kNC * 64 * 16 <= SA * kABytes,
                "the K-split reduction fits in the activation ring");
};

__device__ __forceinline__ uint32_t f16_of_level(int c) {
  return (uint32_t)__half_as_ushort(__int2half_rn(c));  // exact: |c| <= 127
}

// s_waitcnt vmcnt(n) (gfx9 encoding, other counters left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Global -> LDS copies (saddr form): lane l reads base + voff_l and its bytes land at
// LDS address lds + 16 l (dwordx4) or lds + 4 l (dword).  M0 carries the LDS address
// (written by the compiler); one wait state separates that write from the copy.
__device__ __forceinline__ void copy16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "{m0}"(lds)
               : "memory");
}
__device__ __forceinline__ void copy4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(base), "{m0}"(lds)
               : "memory");
}

// XCD-aware order of the workgroups: hardware deals workgroup b to XCD b mod 8, so
// logical tile L = (b mod 8) * ceil(G / 8) + b / 8 gives each XCD a run of consecutive
// logical tiles (which share activation tiles and weight row tiles) in its own L2.
// G is the number of logical tiles (for the grouped products, known only on the device);
// the grid holds at least 8 * ceil(G / 8) workgroups; -1 = nothing to do.
__device__ __forceinline__ int64_t xcd_swizzle(int64_t b, int64_t G) {
  const int64_t per = (G + 7) / 8;
  const int64_t i = b / 8;
  if (i >= per) return -1;
  const int64_t L = (b % 8) * per + i;
  return (L < G) ? L : -1;
}

// Grouped products: the full tiles' logical range G1 in XCD-contiguous runs as above,
// then the partial tiles (lighter, by descending rows) dealt round-robin over the XCDs,
// so every XCD ends on light work.  The grid holds at least 8 * ceil(G1 / 8) + round8(G - G1)
// workgroups.
__device__ __forceinline__ int64_t xcd_swizzle_grouped(int64_t b, int64_t G1, int64_t G) {
  const int64_t per = (G1 + 7) / 8;
  const int64_t x = b % 8, i = b / 8;
  if (i < per) {
    const int64_t L = x * per + i;
    return (L < G1) ? L : -1;
  }
  const int64_t L = G1 + (i - per) * 8 + x;
  return (L < G) ? L : -1;
}

static inline int64_t round8(int64_t g) { return (g + 7) / 8 * 8; }

// waves per SIMD: NW / 4 per workgroup, times two where two workgroups share a CU
template <int MODE, int NW, int KS, int SA, int SB, bool PB>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu((NW / 4) * (Shape<NW, KS, SA, SB, PB>::kTwoPerCU ? 2 : 1))))
qgemm_kernel(GemmArgs a) {
  using S = Shape<NW, KS, SA, SB, PB>;
  constexpr int kBN = S::kBN, kBStageBytes = S::kBStageBytes, kLutCopies = S::kLutCopies;
  constexpr int kAPerWave = S::kAPerWave, kNC = S::kNC;
  constexpr int kNibPerWave = S::kNibPerWave, kSclPerWave = S::kSclPerWave, kBPW = S::kBlocksPerWave;
  __shared__ __attribute__((aligned(1024))) uint8_t ring_a[SA][kABytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring_b[SB][kBStageBytes];
  __shared__ uint32_t lut[256 * kLutCopies];  // entry e of copy c at e * kLutCopies + c
  __shared__ int32_t tile_pair[kBM];          // DOWN: pair id and gate weight of each row
  __shared__ float tile_gw[kBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = (KS == 1) ? wave : wave % kNC;  // column group (its 64 weight rows)
  const int kp = (KS == 1) ? 0 : wave / kNC;     // which blocks of each quad it multiplies
  const int g = lane >> 4, c = lane & 15;
  if (tid < 256) {
    const uint32_t v = f16_of_level(level_of(tid & 15)) | (f16_of_level(level_of(tid >> 4)) << 16);
#pragma unroll
    for (int cc = 0; cc < kLutCopies; ++cc) lut[tid * kLutCopies + cc] = v;
  }
  const uint32_t* lutc = lut + (lane % kLutCopies);  // this lane's copy

  // ---- which tile ------------------------------------------------------------------
  int64_t m0, rows;          // first A row (in the launch's row space) and valid rows
  int64_t n0;                // first weight row of the workgroup
  int64_t seg0 = 0;          // first sorted pair of the expert (grouped modes)
  const uint8_t* W0 = a.W0;
  const uint8_t* W1 = a.W1;
  if (MODE == kGemmDense) {
    const int64_t mt_n = (a.M + kBM - 1) / kBM;
    const int64_t L = xcd_swizzle(blockIdx.x, mt_n * ((a.N + kBN - 1) / kBN));
    if (L < 0) return;
    const int64_t mt = L % mt_n, nt = L / mt_n;
    m0 = mt * kBM;
    rows = min((int64_t)kBM, a.M - m0);
    n0 = nt * kBN;
  } else {
    const int64_t ntl = a.n_tiles_n;
    const int64_t L = xcd_swizzle_grouped(blockIdx.x, (int64_t)a.num_tiles[1] * ntl, (int64_t)a.num_tiles[0] * ntl);
    if (L < 0) return;
    const int64_t ti = L / ntl, nt = L % ntl;
    const int e = a.tiles[2 * ti];
    const int mt = a.tiles[2 * ti + 1];
    seg0 = a.offsets[e];
    const int64_t cnt = a.offsets[e + 1] - seg0;
    m0 = (int64_t)mt * kBM;
    rows = min((int64_t)kBM, cnt - m0);
    // GATEUP: a workgroup covers 128 intermediate columns (each wave 32 gate rows and
    // the same 32 up rows); DOWN: 256 output rows.
    n0 = (MODE == kGemmGateUp) ? nt * (kBN / 2) : nt * kBN;
    if (a.S0 != nullptr && e == a.shared_e) {  // the shared expert, routed to every token by the caller
      W0 = a.S0;
      W1 = a.S1;
    } else {
      W0 += (int64_t)e * a.w_expert_stride;
      if (MODE == kGemmGateUp) W1 += (int64_t)e * a.w_expert_stride;
    }
  }
  const int kq_n = (int)(a.K / kTileK);
  // fragment rows holding valid rows (a partial last tile of an expert, or of a chunk,
  // multiplies only these; the copies still bring all rows so the wait counts hold)
  const int nfr = __builtin_amdgcn_readfirstlane((int)((rows + 15) / 16));
  const int64_t nib_bytes = a.N * (a.K / kQK) * kNibbleBytes;
  const uint32_t ring_a0 = lds_addr(&ring_a[0][0]), ring_b0 = lds_addr(&ring_b[0][0]);

  // ---- activation rows this lane copies ---------------------------------------------
  // The quad's 32 fragments f = 8 j + mt (block j, fragment row mt) are split evenly over
  // the waves: wave w copies f = w * kAPerWave .. +kAPerWave-1 (one block), lane l = 16g + r
  // bringing row r of the fragment row, elements 8g .. 8g+7.  PB: copies kAB j .. kAB j +
  // kAB-1 of wave w are fragment rows kAB w .. of block j (each block spread over all
  // waves).
  // (rows past the tile's valid rows repeat its last row: read in bounds, never stored)
  const int f0 = wave * kAPerWave;
  constexpr int kAB = kMT / NW;  // PB: this wave's copies per block
  auto a_frag = [&](int i) -> int { return PB ? kMT * (i / kAB) + kAB * wave + i % kAB : f0 + i; };
  // Byte offsets from A (the launcher checks they fit in 32 bits).  PB: the copies of
  // block j are this wave's fragment rows of that block, at block 0's offsets plus the
  // block's 64 bytes (added to the scalar base), so only kAB offsets are kept.
  constexpr int kAOff = PB ? kAB : kAPerWave;
  uint32_t a_off[kAOff];
#pragma unroll
  for (int i = 0; i < kAOff; ++i) {
    const int f = a_frag(i), mt = f % kMT, j = f / kMT;
    const int64_t r = min((int64_t)(16 * mt + c), rows - 1);
    int64_t src_row;
    if (MODE == kGemmDense) src_row = m0 + r;
    else if (MODE == kGemmGateUp) src_row = a.pairs[seg0 + m0 + r] / a.top_k;  // token of the pair
    else src_row = seg0 + m0 + r;                                             // h in sorted order
    a_off[i] = (uint32_t)(2 * (src_row * a.lda + 32 * j + 8 * g));
  }

  // ---- weight row tiles of this wave's column group cg --------------------------------
  // DENSE / DOWN: rows n0 + 64cg + 16r, r = 0..3 of W0.
  // GATEUP: r = 0,1 -> gate rows n0 + 32cg + 16r;  r = 2,3 -> up rows n0 + 32cg + 16(r-2).
  // Row tiles past N are replaced by the last row tile (read in bounds, never stored),
  // so the two tiles of each scale copy are equal or ascending in memory.
  const uint8_t* wbase[kWaveRT];
  int64_t wtile0[kWaveRT];
  bool rt_ok[kWaveRT];
#pragma unroll
  for (int r = 0; r < kWaveRT; ++r) {
    int64_t row0;
    if (MODE == kGemmGateUp) {
      row0 = n0 + 32 * cg + 16 * (r & 1);
      wbase[r] = (r < 2) ? W0 : W1;
    } else {
      row0 = n0 + 64 * cg + 16 * r;
      wbase[r] = W0;
    }
    rt_ok[r] = row0 < a.N;
    wtile0[r] = (min(row0, a.N - kTileRows) / kTileRows) * kq_n;  // tile index of quad 0
  }
  // scale copy i brings row tiles 2i (lanes 0..31) and 2i+1 (lanes 32..63)
  uint32_t s_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    s_off[i] = (uint32_t)(4 * (lane & 31) + (lane >> 5) * (wtile0[2 * i + 1] - wtile0[2 * i]) * kTileScaleBytes);

  // quad q's copies into its stages: this wave's A fragments; its share of its column
  // group's index tiles and scale copies
  auto copy_a = [&](int q) {
    const uint32_t st = ring_a0 + (uint32_t)((q % SA) * kABytes);
#pragma unroll
    for (int i = 0; i < kAPerWave; ++i) {
      if constexpr (PB) copy16(a.A + (int64_t)q * kTileK + 32 * (i / kAB), a_off[i % kAB], st + (uint32_t)(a_frag(i) * 1024));
      else copy16(a.A + (int64_t)q * kTileK, a_off[i], st + (uint32_t)(a_frag(i) * 1024));
    }
  };
  auto copy_a_block = [&](int q, int j) {  // PB: this wave's kAB fragments of block j
#pragma unroll
    for (int k = 0; k < kAB; ++k)
      copy16(a.A + (int64_t)q * kTileK + 32 * j, a_off[k], ring_a0 + (uint32_t)(a_frag(kAB * j + k) * 1024));
  };
  auto copy_b = [&](int q) {
    const uint32_t sb = ring_b0 + (uint32_t)((q % SB) * kBStageBytes + cg * kWaveBBytes);
#pragma unroll
    for (int n = 0; n < kNibPerWave; ++n) {
      const int r = kp * kNibPerWave + n;
      copy16(wbase[r] + (wtile0[r] + q) * kTileNibbleBytes, 16 * lane, sb + r * kTileNibbleBytes);
    }
#pragma unroll
    for (int n = 0; n < kSclPerWave; ++n) {
      const int i = kp * kSclPerWave + n;
      copy4(wbase[2 * i] + nib_bytes + (wtile0[2 * i] + q) * kTileScaleBytes, s_off[i],
            sb + kWaveRT * kTileNibbleBytes + i * 2 * kTileScaleBytes);
    }
  };

  f32x4 acc[kMT][kWaveRT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int r = 0; r < kWaveRT; ++r) acc[i][r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // index word of this wave's block jj (block kp * kBPW + jj of the quad) in a row tile
  auto nib_word = [&](const u32x4& nb, int jj) -> uint32_t {
    if (KS == 1) return (jj == 0) ? nb.x : (jj == 1) ? nb.y : (jj == 2) ? nb.z : nb.w;
    return kp ? (jj ? nb.w : nb.z) : (jj ? nb.y : nb.x);
  };
  // LUT values of one block: 16 independent LDS reads.
  auto lut_reads = [&](const u32x4 (&nib)[kWaveRT], int jj, uint32_t (&lv)[kWaveRT][4]) {
#pragma unroll
    for (int r = 0; r < kWaveRT; ++r) {
      const uint32_t w = nib_word(nib[r], jj);
      lv[r][0] = lutc[(w & 0xFF) * kLutCopies];
      lv[r][1] = lutc[((w >> 8) & 0xFF) * kLutCopies];
      lv[r][2] = lutc[((w >> 16) & 0xFF) * kLutCopies];
      lv[r][3] = lutc[(w >> 24) * kLutCopies];
    }
  };

  // quad 0 (a two-stage ring is filled one quad ahead; a one-stage ring after each quad)
  if (kq_n > 0) {
    copy_b(0);
    copy_a(0);  // (PB: blocks 0, 1, 2, 3 in this order)
    if (PB && kq_n > 1) copy_b(1);
  }
  if (MODE == kGemmDown && tid < rows) {
    // the epilogue's per-row pair id and gate weight, fetched once per tile (after the
    // first copies are in flight) instead of as two dependent loads per stored row
    const int p = a.pairs[seg0 + m0 + tid];
    tile_pair[tid] = p;
    tile_gw[tid] = a.gate_w[p];
  }

  // The main loop, instantiated twice: full tiles multiply all fragment rows with no
  // branch in the unrolled body; a partial tile (an expert's or a chunk's last) skips the
  // fragment rows wholly past its rows (the copies still bring them, so the wait counts
  // hold).
  // PB wait counts: this wave issues kAB activation copies per block and kBC weight
  // copies per quad, in the order  ... blocks 1-3 of quad q, weights of q+1, blocks 0-3
  // of q+1 (each after that block of q is multiplied), weights of q+2 ...
  constexpr int kBC = kNibPerWave + kSclPerWave;
  if constexpr (PB) {
    // weights and block 0 of quad 0: younger are blocks 1-3 and the weights of quad 1
    if (kq_n > 1) wait_vmcnt<3 * kAB + kBC>();
    else wait_vmcnt<3 * kAB>();
    lds_barrier();
  }
  auto main_loop = [&](auto partial_tag) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;
    for (int q = 0; q < kq_n; ++q) {
      if constexpr (!PB) {
        // this wave's copies of quad q are the last it issued: wait for all of them
        wait_vmcnt<0>();
        lds_barrier();  // quad q is in LDS for everyone; quad q-1's stages are free
        if (q + 1 < kq_n) {
          if (SB == 2) copy_b(q + 1);
          if (SA == 2) copy_a(q + 1);
        }
      }

      const uint8_t* st = &ring_a[q % SA][0];
      const uint8_t* sb = &ring_b[q % SB][0] + cg * kWaveBBytes;
      u32x4 nib[kWaveRT];
      u32x2 scl[kWaveRT];
#pragma unroll
      for (int r = 0; r < kWaveRT; ++r) {
        nib[r] = *reinterpret_cast<const u32x4*>(sb + r * kTileNibbleBytes + lane * 16);
        scl[r] = *reinterpret_cast<const u32x2*>(sb + kWaveRT * kTileNibbleBytes + r * kTileScaleBytes + c * 8);
      }
      uint32_t lv[kWaveRT][4];
      lut_reads(nib, 0, lv);
#pragma unroll
      for (int jj = 0; jj < kBPW; ++jj) {
        const int j = kp * kBPW + jj;  // block of the quad
        u32x4 bf[kWaveRT];
#pragma unroll
        for (int r = 0; r < kWaveRT; ++r) {
          const uint32_t sw = (KS == 1) ? ((jj < 2) ? scl[r].x : scl[r].y) : (kp ? scl[r].y : scl[r].x);
          const uint32_t dd = __builtin_amdgcn_perm(sw, sw, (jj & 1) ? 0x03020302u : 0x01000100u);
#pragma unroll
          for (int i = 0; i < 4; ++i) bf[r][i] = pk_mul_f16(lv[r][i], dd);
        }
        if (jj + 1 < kBPW) lut_reads(nib, jj + 1, lv);  // next block's reads under these MFMAs
        const uint8_t* ab = st + j * kMT * 1024 + lane * 16;  // the block's A fragments
        if constexpr (!PARTIAL) {
          // all 8 fragment reads issued before the first MFMA (the scheduler otherwise keeps
          // two in flight and the matrix core waits on each pair)
          u32x4 af[kMT];
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt) af[mt] = *reinterpret_cast<const u32x4*>(ab + mt * 1024);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int r = 0; r < kWaveRT; ++r) acc[mt][r] = mfma_f16(bf[r], af[mt], acc[mt][r]);
        } else {
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt) {
            if (mt >= nfr) break;  // fragment rows wholly past the tile's rows
            const u32x4 af = *reinterpret_cast<const u32x4*>(ab + mt * 1024);
#pragma unroll
            for (int r = 0; r < kWaveRT; ++r) acc[mt][r] = mfma_f16(bf[r], af, acc[mt][r]);
          }
        }
        if constexpr (PB) {
          // block jj + 1 of this quad (jj < 3), or block 0 and the weights of the next,
          // must have landed; once every wave is past block jj, its slot takes block jj
          // of the next quad
          const bool more = q + 1 < kq_n;
          if (jj < 3) {
            if (more) wait_vmcnt<2 * kAB + kBC>();  // younger: 2 blocks' copies, one quad's weights
            else wait_vmcnt<0>();
          } else if (more) {
            wait_vmcnt<2 * kAB>();  // younger: blocks 1-2 of the next quad
          }
          if (jj < 3 || more) lds_barrier();
          if (more) copy_a_block(q + 1, jj);
          if (jj == 3 && q + 2 < kq_n) copy_b(q + 2);
        }
      }
      if (!PB && (SA == 1 || SB == 1) && q + 1 < kq_n) {
        lds_barrier();  // everyone is done reading the one-stage ring(s)
        if (SB == 1) copy_b(q + 1);
        if (SA == 1) copy_a(q + 1);
      }
    }
  };
  if (nfr == kMT) main_loop(std::false_type{});
  else main_loop(std::true_type{});

  if constexpr (KS == 2) {
    // the column group's two partial sums: the kp = 1 wave hands its accumulators to its
    // kp = 0 partner through the (now free) ring, half the fragment rows at a time; the
    // sum is (blocks 0-1) + (blocks 2-3) of every quad, a fixed order
    f32x4* red = reinterpret_cast<f32x4*>(&ring_a[0][0]);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      __syncthreads();  // the ring is free (first half) / the partners have read (second)
      if (kp == 1) {
#pragma unroll
        for (int ml = 0; ml < kMT / 2; ++ml)
#pragma unroll
          for (int r = 0; r < kWaveRT; ++r) red[((ml * kWaveRT + r) * kNC + cg) * 64 + lane] = acc[half * (kMT / 2) + ml][r];
      }
      __syncthreads();
      if (kp == 0) {
#pragma unroll
        for (int ml = 0; ml < kMT / 2; ++ml)
#pragma unroll
          for (int r = 0; r < kWaveRT; ++r) {
            const f32x4 o = red[((ml * kWaveRT + r) * kNC + cg) * 64 + lane];
            f32x4& v = acc[half * (kMT / 2) + ml][r];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = v[i] + o[i];
          }
      }
    }
    if (kp != 0) return;  // the kp = 0 waves store
  }

  // ---- epilogue ------------------------------------------------------------------------
  // The weights are the matrix core's first operand, so every fragment holds its 16 x 16
  // piece of the tile transposed: lane (g, c) has row 16 mt + c and the four consecutive
  // columns 16 r + 4 g .. 16 r + 4 g + 3 of its column group, stored with one vector write.
  if (MODE == kGemmDense) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const int rr = 16 * mt + c;
      if (rr >= rows) continue;
      float* crow = a.C + (m0 + rr) * a.ldc + n0 + 64 * cg + 4 * g;
#pragma unroll
      for (int r = 0; r < kWaveRT; ++r) {
        if (!rt_ok[r]) continue;
        if (a.vec_c) {
          *reinterpret_cast<f32x4*>(crow + 16 * r) = acc[mt][r];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) crow[16 * r + i] = acc[mt][r][i];
        }
      }
    }
  } else if (MODE == kGemmGateUp) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const int rr = 16 * mt + c;
      if (rr >= rows) continue;
      const int64_t o = (seg0 + m0 + rr) * a.ldh + n0 + 32 * cg + 4 * g;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (!rt_ok[r]) continue;
        const f32x4 gv = acc[mt][r], uv = acc[mt][r + 2];
        uint32_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float h = gv[i] / (1.0f + __expf(-gv[i])) * uv[i];
          hb[i] = __half_as_ushort(__float2half_rn(h));
        }
        *reinterpret_cast<u32x2*>(a.H + o + 16 * r) = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
        if (a.G) {  // the intermediates kept (tests): g and u in the same place as h
          *reinterpret_cast<f32x4*>(a.G + o + 16 * r) = gv;
          *reinterpret_cast<f32x4*>(a.U + o + 16 * r) = uv;
        }
      }
    }
  } else {  // DOWN
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const int rr = 16 * mt + c;
      if (rr >= rows) continue;
      const int p = tile_pair[rr];
      const float gw = tile_gw[rr];
      if (a.atomic) {
        float* orow = a.out + (int64_t)(p / a.top_k) * a.ldo + n0 + 64 * cg + 4 * g;
#pragma unroll
        for (int r = 0; r < kWaveRT; ++r)
          if (rt_ok[r])
#pragma unroll
            for (int i = 0; i < 4; ++i) atomicAdd(orow + 16 * r + i, gw * acc[mt][r][i]);
      } else {
        // the row rounded to binary16 (half the bytes of the write and of the combine's
        // read); the product is rounded to binary32 first
        uint16_t* yrow = a.R + (int64_t)p * a.ldc + n0 + 64 * cg + 4 * g;
#pragma unroll
        for (int r = 0; r < kWaveRT; ++r) {
          if (!rt_ok[r]) continue;
          uint32_t hb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = gw * acc[mt][r][i];
            asm volatile("" : "+v"(v));  // no fused multiply-and-convert (it would drop a -0)
            hb[i] = __half_as_ushort(__float2half_rn(v));
          }
          *reinterpret_cast<u32x2*>(yrow + 16 * r) = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
        }
      }
    }
  }
}

// The long prompt: 8 waves (two per SIMD), 128 x 256 tiles, each quad's blocks split
// between the two waves of a column group, two-stage rings; a 512-token chunk stays on
// ~224 CUs.  The MoE products (short K, many small tiles): 4 waves, 128 x 256 tiles,
// one activation stage refilled block by block and two weight stages (77 KiB with an
// 8-copy table), so two workgroups share a CU and one's copy waits, fill and epilogue
// run under the other's MFMAs.
constexpr int kDenseWaves = 8, kDenseKS = 2, kDenseSA = 2, kDenseSB = 2;
constexpr int kGuWaves = 4, kGuKS = 1, kGuSA = 1, kGuSB = 2;
constexpr bool kGuPB = true;
constexpr int kDnWaves = 4, kDnKS = 1, kDnSA = 1, kDnSB = 2;
constexpr bool kDnPB = true;

int launch_qgemm_dense(const uint8_t* packed, int64_t n, int64_t k, const uint16_t* x, int64_t m,
                       int64_t ldx, float* y, int64_t ldy, int64_t chunk, hipStream_t s) {
  constexpr int kBN = Shape<kDenseWaves, kDenseKS, kDenseSA, kDenseSB, false>::kBN;
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
    a.vec_c = (reinterpret_cast<uintptr_t>(y) % 16 == 0) && (ldy % 4 == 0);  // 16-byte row pieces
    const int64_t grid = round8(((a.M + kBM - 1) / kBM) * ((n + kBN - 1) / kBN));
    hipLaunchKernelGGL((qgemm_kernel<kGemmDense, kDenseWaves, kDenseKS, kDenseSA, kDenseSB, false>), dim3((unsigned)grid),
                       dim3(64 * kDenseWaves), 0, s, a);
    if (int e = check_launch("qgemm_kernel<dense>")) return e;
  }
  return 0;
}

template <int MODE, int NW, int KS, int SA, int SB, bool PB>
static int launch_grouped(GemmArgs a, int64_t max_tiles, hipStream_t s) {
  constexpr int kBN = Shape<NW, KS, SA, SB, PB>::kBN;
  // GATEUP: a workgroup covers kBN/2 intermediate columns (gate and up rows side by side)
  a.n_tiles_n = (MODE == kGemmGateUp) ? (a.N + kBN / 2 - 1) / (kBN / 2) : (a.N + kBN - 1) / kBN;
  const int64_t grid = round8(max_tiles * a.n_tiles_n) + 8;  // + the rounding of the full-tile range
  if (grid == 0) return 0;
  hipLaunchKernelGGL((qgemm_kernel<MODE, NW, KS, SA, SB, PB>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a);
  return check_launch(MODE == kGemmGateUp ? "qgemm_kernel<gateup>" : "qgemm_kernel<down>");
}

int launch_qgemm_grouped(int mode, GemmArgs a, int64_t max_tiles, hipStream_t s) {
  if (mode == kGemmGateUp) return launch_grouped<kGemmGateUp, kGuWaves, kGuKS, kGuSA, kGuSB, kGuPB>(a, max_tiles, s);
  return launch_grouped<kGemmDown, kDnWaves, kDnKS, kDnSA, kDnSB, kDnPB>(a, max_tiles, s);
}

}  // namespace iq4
