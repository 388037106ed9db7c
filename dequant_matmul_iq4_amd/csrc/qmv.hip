// qmv.hip -- T-column quantised matrix-vector product (the verify window's dense
// product, T <= 8 tokens reading the weights once).
//
// Why the matrix cores.  With fp32 activations the plain vector form costs one fp32
// FMA per weight per column plus the index decode: at T = 4 that is more than 4 VALU
// operations per 4.5-bit weight, while streaming the weights at the HBM rate leaves a
// budget of under 3 (256 CUs x 64 lanes x 2.4 GHz against 8 TB/s of 18-byte blocks).
// So the K-reduction runs on the matrix cores instead:
//
//  * codebook levels are integers of at most 7 significant bits, exact in bf16;
//  * each fp32 activation x goes in as bf16 parts: the verify-window kernel below uses
//    two (hi = bf16(x), lo = bf16(x - hi): x to within 2^-18 |x|), the grouped MoE
//    decode kernels three (hi, mid, lo by truncation: x exactly, for |x| >= 2^-100);
//    every product level * part is exact in fp32;
//  * one v_mfma_f32_16x16x32_bf16 covers one block of 32 weights for 16 weight rows
//    (B operand) against 16 "rows" of A = (part s, token t) pairs, 4s + t;
//  * the block scale d is applied to the 16x16 result with an fp32 FMA per block, the
//    K-slices of the workgroup's waves are summed in a fixed order, and finally the
//    parts are added.
//
// Column invariance.  Token t's value never meets another token's: it sits in matrix
// row 4s + (t mod 4) of the pass that holds it, the per-block scaling and the
// reductions run the same instruction sequence for every t, and the wave / K-slice
// split depends on K only.  Column t of a T-column call is therefore bitwise the
// 1-column call on token t (the property page 1's verify window relies on: each
// window token reproduces plain greedy decode bit for bit).
//
// Work split.  A workgroup (up to 8 waves) owns RG row tiles (16 rows each) and a slice
// of K of at most 128 blocks; each wave owns a contiguous run of at most 4 quads
// (16 blocks) of the slice and issues every weight load of that run at kernel entry,
// so all of the matrix is in flight from the start (the pages' lesson from their
// interleaved matvec: one block in flight per warp starved it).  The slice's
// activations are staged once in LDS, already split and in fragment order (a wave's
// fragment read is one conflict-free ds_read_b128), up to 4 columns per pass.  A K
// above 4096 is cut into S slices handled by S workgroups, whose partial sums go to
// a caller workspace; the last workgroup to arrive adds them in slice order
// (deterministic).  RG, S and the wave runs depend on the matrix shape only, never
// on T.
//
// Memory.  Weights come in the packed tile layout: per 16-row x 4-block tile each lane
// issues one 128-bit load of indices (coalesced 1 KiB per wave) and one 64-bit load
// of its row's four scales.  The index-to-level decode is a byte-indexed table in LDS
// (one byte = two 4-bit indices of consecutive elements -> two bf16 levels), built from
// register immediates and replicated so that lanes read their own copies.
//
// 8-bit activations.  The same plan, weight stream and table serve the product on
// 8-bit activation codes (quantize_q8_kernel, qmv_q8_kernel at the end of this file):
// a code is exact in bf16, so the matrix core returns each block's integer dot exactly.
#include <mutex>

#include "iq4.h"
#include "common.hpp"
#include "launch.hpp"
#include "qmv.hpp"

namespace iq4 {

constexpr int kWaves = 8;              // waves per workgroup (at most)
constexpr int kMaxWaveQuads = 4;       // quads per wave: all of a wave's weights in registers
constexpr int kSliceQuads = kWaves * kMaxWaveQuads;  // 32 quads = 128 blocks = K 4096
constexpr int kCols = 4;               // columns per pass (rows 4s + t of the A operand)
constexpr int kSplitCols = 8;          // columns of the split-K partials (T <= 8)
constexpr int kDenseRG = 1;            // row tiles per workgroup (dense)
constexpr int kGateUpRG = 1;           // row tiles per matrix (gate + up)
constexpr int kDownRG = 2;             // row tiles per workgroup (down)


// The expert of a grouped workgroup's slot: slot i takes the i-th smallest expert id that
// has routed pairs.  seg0 = its first position in the pair list sorted by (expert, pair
// id), ncols = its pair count; with the ids given, cols = the mask of its pair ids (bit p
// for pair p: the columns in ascending pair order).  e < 0: no such expert.
struct SlotInfo {
  int64_t e, seg0, ncols;
  uint64_t cols;
};

// From the gather's offsets: a ballot over the experts, 64 at a time, in every wave.
__device__ __forceinline__ SlotInfo slot_from_offsets(const QmvArgs& a, int64_t slot, int lane) {
  SlotInfo s{-1, 0, 0, 0};
  int64_t before = 0;
  for (int e0 = 0; e0 < a.n_expert && s.e < 0; e0 += 64) {
    const int ee = e0 + lane;
    const int lo = (ee < a.n_expert) ? a.offsets[ee] : 0;
    const int hi = (ee < a.n_expert) ? a.offsets[ee + 1] : 0;
    const bool act = hi > lo;
    const uint64_t m = __ballot(act);
    const int64_t cnt = __popcll(m);
    if (slot < before + cnt) {
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      const uint64_t hit = __ballot(act && before + __popcll(m & below) == slot);
      const int L = __ffsll((unsigned long long)hit) - 1;
      s.e = e0 + L;
      s.seg0 = __shfl(lo, L);
      s.ncols = __shfl(hi, L) - s.seg0;
    }
    before += cnt;
  }
  return s;
}

// From the routed ids themselves (at most 64 pairs, one per lane, v = this lane's id, -1
// past the pairs), so that no gather has to run first: the wave marks the experts
// present in a bitmap (bm: 32 words of LDS of its own, 1024 experts), counts them per
// word with a prefix sum over lanes, and picks the slot's word and bit.  An id outside
// [0, n_expert) marks nothing.
__device__ __forceinline__ SlotInfo slot_from_ids(int v, int n_expert, int64_t slot, uint32_t* bm,
                                                  int lane) {
  const bool valid = (unsigned)v < (unsigned)n_expert;
  if (lane < 32) bm[lane] = 0u;
  // a wave's LDS accesses execute in order; the fences only keep the compiler from
  // moving them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (valid) atomicOr(bm + (v >> 5), 1u << (v & 31));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint32_t word = (lane < 32) ? bm[lane] : 0u;
  const int cnt = __popc(word);
  int incl = cnt;  // inclusive prefix sum of the per-word counts
#pragma unroll
  for (int d = 1; d < 32; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  const int excl = incl - cnt;
  SlotInfo s{-1, 0, 0, 0};
  const uint64_t hw = __ballot(lane < 32 && excl <= slot && slot < incl);
  if (hw == 0) return s;  // uniform: past the experts present
  const int W = __ffsll((unsigned long long)hw) - 1;
  const uint32_t wd = __shfl(word, W);
  const int r = (int)slot - __shfl(excl, W);
  const bool hb = lane < 32 && ((wd >> lane) & 1u) && __popc(wd & ((1u << lane) - 1u)) == r;
  s.e = W * 32 + (__ffsll((unsigned long long)__ballot(hb)) - 1);
  s.seg0 = __popcll(__ballot(valid && v < s.e));
  s.cols = __ballot(valid && v == s.e);
  s.ncols = __popcll(s.cols);
  return s;
}

// Pair id of column t of the slot (uniform).  The pair list is read through the constant
// address space (it is not written during the call), so the lookup is a scalar load,
// counted apart from the weight loads in flight.
__device__ __forceinline__ int pair_of(const QmvArgs& a, const SlotInfo& s, int64_t t) {
  if (a.ids) {
    uint64_t m = s.cols;
    for (int64_t i = 0; i < t; ++i) m &= m - 1;
    return __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)m) - 1);
  }
  const __attribute__((address_space(4))) int32_t* pairs =
      (const __attribute__((address_space(4))) int32_t*)a.pairs;
  return pairs[__builtin_amdgcn_readfirstlane((int)(s.seg0 + t))];
}

// Column t of the call: where its activations live.
__device__ __forceinline__ const float* column_ptr(const QmvArgs& a, int mode, const SlotInfo& s,
                                                   int64_t t) {
  if (mode == kQmvDense) return a.x + t * a.ldx;
  if (mode == kQmvGateUp) return a.x + (int64_t)(pair_of(a, s, t) / a.top_k) * a.ldx;
  return a.x + (s.seg0 + t) * a.ldx;  // kQmvDown: h rows in pair-sorted order
}

// A-fragment store of the slice in LDS: [block][k-group g][row 4s+t], padding rows
// (s = 3) omitted, 16 bytes each: part s of elements 8g .. 8g+7 of the block (element
// 8g+2i in the low, 8g+2i+1 in the high half of word i, the weights' index order).
constexpr int kFragRows = 12;
// A (block, k-group) slot takes 13 rows of 16 B (12 used): the 16 lanes that stage
// consecutive slots then write 16 distinct groups of 4 banks (a 12-row slot is 48
// banks, which repeats every 4 lanes: 16-way conflicts on every staging store).
constexpr int kFragStride = 13;
static_assert(kFragStride > kFragRows, "a slot holds its rows");
constexpr int kFragBytes = 4 * kFragStride * 16;  // 832 B per block
// The grouped kernel's fragment store puts a column's parts in consecutive rows:
// [block][k-group g][row 4t+s], 16 rows of 16 B per slot (rows 4t+3 unused), so that
// MFMA output lane (g, c) receives column g's three parts in its four entries and adds
// them in-lane.  Staging stores meet bank conflicts (all slots start on the same bank);
// they run once per pass.
constexpr int kGSlot = 16 * 16;           // one (block, k-group) slot: 16 rows of 16 B
constexpr int kGFragBytes = 4 * kGSlot;   // 1 KiB per block

// Exact three-way bf16 split of two values, packed per part: word s holds part s of v0
// in its low and of v1 in its high half.  Part 0 (hi) is the top 16 bits of v; part 1
// (mid) the top 16 bits of r = v - hi; part 2 (lo) is r - mid, which has at most 8
// significant bits: every subtraction is exact, so v = hi + mid + lo.
__device__ __forceinline__ void split_pair(float v0, float v1, uint32_t out[3]) {
  const uint32_t u0 = __float_as_uint(v0), u1 = __float_as_uint(v1);
  const float r0 = v0 - __uint_as_float(u0 & 0xFFFF0000u);  // exact (Sterbenz)
  const float r1 = v1 - __uint_as_float(u1 & 0xFFFF0000u);
  const uint32_t m0 = __float_as_uint(r0), m1 = __float_as_uint(r1);
  const float l0 = r0 - __uint_as_float(m0 & 0xFFFF0000u);  // exact, <= 8 significant bits
  const float l1 = r1 - __uint_as_float(m1 & 0xFFFF0000u);
  out[0] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);  // upper halves of (u0, u1)
  out[1] = __builtin_amdgcn_perm(m1, m0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(__float_as_uint(l1), __float_as_uint(l0), 0x07060302u);
}

// Byte-indexed level table, replicated against bank conflicts: entry e of copy j sits at
// word C e + j and lane l reads copy l mod C.  With C = 32 (32 KiB) only lanes l and l + 32
// share a copy, so a wave's lookups conflict at most two ways.  The grouped gate|up
// matvec, one workgroup per CU, builds the table once for all of its row groups; 8
// copies measured 5 % slower on the MoE decode step.
constexpr int kLutCopies = 32;

// The level table of the grouped kernels: entry e (0..255) holds the bf16 levels of its
// two nibbles (low nibble in the low half), LC copies side by side.  Consecutive
// threads write consecutive 16-byte pieces, so the stores meet no bank conflict.
template <int LC = kLutCopies>
__device__ __forceinline__ void build_pair_table(uint32_t* lut, int tid, int nthreads) {
  constexpr int PER = LC / 4;  // 16-byte pieces per entry
  uint4* dst = reinterpret_cast<uint4*>(lut);
  for (int q = tid; q < 256 * PER; q += nthreads) {
    const int e = q / PER;
    const uint32_t v = bf16_of_level(level_of(e & 15)) | (bf16_of_level(level_of(e >> 4)) << 16);
    dst[q] = uint4{v, v, v, v};
  }
}

template <int N>
struct ColsC {  // a column count as a type (compile-time pass width)
  static constexpr int value = N;
};

// ---------------------------------------------------------------------------------
// Dense verify-window matvec.
//
// Activations.  Each fp32 activation x goes to the matrix core as two bf16 parts,
// hi = bf16_rne(x) and lo = bf16_rne(x - hi), where x - hi is exact in fp32; so
// hi + lo equals x to within 2^-18 |x|, far inside the fp32 paths' tolerance, and
// hi * level and lo * level are exact products.  The parts sit in rows 4s + t of the
// A operand (s = 0 hi, 1 lo; t = the column within a pass of 4), the weight levels
// (exact in bf16) are the B operand; rows 8..15 are never read.
//
// Work split.  One workgroup per row tile (16 rows) and K slice; each wave owns a run
// of WQ quads of the slice.  The code is straight line in the order the data arrive:
// the pass's activations are requested first (L2 hot), then every weight of the wave;
// the level table is built and the activations are split and staged in LDS while the
// weights stream in, and quad u is decoded and multiplied as soon as its own weights
// have landed.
//
// LDS.  The byte-indexed level table (one index byte = two 4-bit indices -> two bf16
// levels) has kDenseLutCopies copies, entry e of copy j at word kDenseLutCopies e + j;
// lane l reads copy l mod kDenseLutCopies, so a wave's 64 lookups are served at the
// full LDS rate.  It sits at LDS offset 0 and is addressed with one byte permute: the
// index byte lands in bits 8..15 of the address, the lane's copy in bits 0..7.  The
// staged activations follow: per wave and block, 4 k-group slots of 8 rows (16 B
// each) plus one row of padding, so the 16 lanes that stage consecutive slots write
// distinct banks.
constexpr int kDenseWaves = 8;  // waves per workgroup (at most)
constexpr int kDenseLutCopies = 64;
constexpr int kDenseLutBytes = 256 * kDenseLutCopies * 4;  // 64 KiB
constexpr int kDenseSlot = 9 * 16;                         // 8 rows + 1 row of padding
constexpr int kDenseBlockStage = 4 * kDenseSlot;           // 576 B per block

// bf16 bit pattern of codebook level q (exact: |level| <= 127)
__device__ __forceinline__ uint32_t bf16_level(uint32_t q) { return bf16_of_level(level_of(q)); }

template <int WQ, int TP>
__global__ void __launch_bounds__(64 * kDenseWaves) qmv_dense_kernel(QmvArgs a) {
  static_assert(TP >= 1 && TP <= kCols, "first pass: 1..4 columns");
  constexpr int XBYTES = kDenseWaves * WQ * 4 * kDenseBlockStage;
  __shared__ __attribute__((aligned(256))) uint8_t smem[kDenseLutBytes + XBYTES + kDenseWaves * 64 * 16];
  __shared__ int s_last;
  // Every kernel argument, loaded at entry.  Left to itself the compiler loads some of
  // them where they are first used, deep in the kernel; while such a scalar load is
  // outstanding each wait for an LDS read must wait for it too.
  const uint8_t* const W0 = a.W0;
  const float* const X = a.x;
  float* const Y = a.y;
  float* const partials = a.partials;
  int* const counters = a.counters;
  const int64_t ldx = a.ldx, ldy = a.ldy, n_rows = a.n, rg_n = a.rg_n, nibble_bytes = a.nibble_bytes;
  const int T_all = a.T, kq_n = a.kq_n, S = a.S, slice_quads = a.slice_quads, wave_quads = a.wave_quads;
  asm volatile("" ::"s"(W0), "s"(X), "s"(Y), "s"(partials), "s"(counters), "s"(ldx), "s"(ldy), "s"(n_rows),
               "s"(rg_n), "s"(nibble_bytes), "s"(T_all), "s"(kq_n), "s"(S), "s"(slice_quads), "s"(wave_quads));

  uint8_t* const xs = smem + kDenseLutBytes;
  f32x4* const red = reinterpret_cast<f32x4*>(smem + kDenseLutBytes + XBYTES);
  typedef __attribute__((address_space(3))) const uint8_t lds_u8;
  lds_u8* const lds = (lds_u8*)(__attribute__((address_space(3))) uint8_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = (int)(blockDim.x >> 6);
  const int c = lane & 15, g = lane >> 4;

  // ---- tile of this workgroup ---------------------------------------------------------
  const int64_t rg = blockIdx.x / S;
  const int slice = (int)(blockIdx.x % S);
  const int64_t ncols = T_all;
  const int kqa = slice * slice_quads;                 // first quad of the slice
  const int nq_slice = min(slice_quads, kq_n - kqa);   // quads in the slice
  const int wq0 = wave * wave_quads;                   // this wave's quads (slice-relative)
  const int wq1 = min(wq0 + wave_quads, nq_slice);
  const int wblk = 4 * (wq1 - wq0);                      // blocks of this wave (0 if idle)
  uint8_t* xw = xs + wave * (4 * WQ) * kDenseBlockStage;  // the wave's own staging region

  // Staging tasks: (column t, block bl, k-group gg) = task (t SLOTS + 4 bl + gg), task =
  // lane + 64 i, fixed at compile time for a full wave; blocks past a short run skipped.
  constexpr int SLOTS = 16 * WQ;
  float4 xr[WQ][2];
  auto load_x = [&](int64_t t0, int T) {
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int task = lane + 64 * i;
      const int t = task / SLOTS, bl = (task % SLOTS) >> 2, gg = task & 3;
      if (t < T && bl < wblk) {
        const float* p = X + (t0 + t) * ldx + ((int64_t)(kqa + wq0) * 4 + bl) * kQK + 8 * gg;
        xr[i][0] = *reinterpret_cast<const float4*>(p);
        xr[i][1] = *reinterpret_cast<const float4*>(p + 4);
      }
    }
  };
  // split and store: part s of column t in row 4s + t.  LDS accesses of one wave execute
  // in order, so the wave's fragment reads see these writes (the fences only keep the
  // compiler from moving them) and a next pass's writes follow this pass's reads.
  auto store_x = [&](int T) {
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int task = lane + 64 * i;
      const int t = task / SLOTS, bl = (task % SLOTS) >> 2, gg = task & 3;
      if (t < T && bl < wblk) {
        uint32_t h[4], l[4];
        split_hi_lo(xr[i][0].x, xr[i][0].y, h[0], l[0]);
        split_hi_lo(xr[i][0].z, xr[i][0].w, h[1], l[1]);
        split_hi_lo(xr[i][1].x, xr[i][1].y, h[2], l[2]);
        split_hi_lo(xr[i][1].z, xr[i][1].w, h[3], l[3]);
        uint8_t* dst = xw + (bl * 4 + gg) * kDenseSlot + t * 16;
        *reinterpret_cast<uint4*>(dst) = uint4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<uint4*>(dst + 4 * 16) = uint4{l[0], l[1], l[2], l[3]};
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };

  uint4 nib[WQ];
  uint2 scl[WQ];
  const uint8_t* tp = W0 + (rg * kq_n + kqa) * kTileNibbleBytes + lane * 16;
  const uint8_t* sp = W0 + nibble_bytes + (rg * kq_n + kqa) * kTileScaleBytes + c * 8;

  // ---- requests: the first pass's activations, then every weight of the wave --------
  constexpr int T0 = TP;  // columns of the first pass, min(T, 4): fixed per instantiation
  load_x(0, T0);
  // (the weights are read once per call: non-temporal loads stream them past the L2, so
  // that they do not evict the activations, which every workgroup reads)
#pragma unroll
  for (int u = 0; u < WQ; ++u) {
    const int q = min(wq0 + u, max(wq1 - 1, 0));  // idle slots reload a valid quad
    nib[u] = load_nt16(tp + (int64_t)q * kTileNibbleBytes);
    scl[u] = load_nt8(sp + (int64_t)q * kTileScaleBytes);
  }
  // ---- level table: 16-byte chunk q (0 .. 4095) holds copies 4(q mod 16) .. +3 of entry
  // q / 16; thread tid writes chunks tid, tid + NT, ... (consecutive lanes, consecutive
  // chunks: no bank conflicts).  With all NT = 64 kDenseWaves threads, a thread's chunks
  // share the low index (tid / 16) mod 16 and a wave's the high index (tid / 256) +
  // (NT / 256) j; a smaller workgroup (short K) takes the general loop.
  if (nwaves == kDenseWaves) {
    constexpr int NT = 64 * kDenseWaves;
    const uint32_t lo = bf16_level((uint32_t)(tid >> 4) & 15u);
    const uint32_t hsel = (uint32_t)__builtin_amdgcn_readfirstlane(tid >> 8);
    uint4* dst = reinterpret_cast<uint4*>(smem) + tid;
#pragma unroll
    for (int j = 0; j < 4096 / NT; ++j) {
      const uint32_t v = lo | (bf16_level(hsel + (uint32_t)(NT / 256) * j) << 16);
      dst[NT * j] = uint4{v, v, v, v};
    }
  } else {
    uint4* dst = reinterpret_cast<uint4*>(smem);
    for (int q = tid; q < 4096; q += 64 * nwaves) {
      const uint32_t e = (uint32_t)q >> 4;
      const uint32_t v = bf16_level(e & 15u) | (bf16_level(e >> 4) << 16);
      dst[q] = uint4{v, v, v, v};
    }
  }
  // A lookup: byte b of index word w -> the lane's copy of entry w.byte[b]
  const uint32_t lane_copy = (uint32_t)lane * 4u;
  auto lookup = [&](uint32_t w, int b) -> uint32_t {
    const uint32_t addr = __builtin_amdgcn_perm(lane_copy, w, 0x0c0c0004u | ((uint32_t)b << 8));
    return *reinterpret_cast<__attribute__((address_space(3))) const uint32_t*>(lds + addr);
  };
  // this lane's A-fragment row in the wave's staging region (block bl at + bl * 4 slots)
  lds_u8* const arow_p = lds + kDenseLutBytes + (wave * (4 * WQ) * kDenseBlockStage + g * kDenseSlot + c * 16);

  // NC (compile time): the pass's columns; accumulator entry i of a lane in k-group g
  // holds row 4g + i (g = 0: hi parts, g = 1: lo parts, column i), so the scale FMAs of
  // columns past NC are skipped.  A-fragment reads are masked to the rows that exist.
  auto multiply = [&](f32x4& acc, auto nc) {
    constexpr int NC = decltype(nc)::value;
    const bool arow = c < 8 && (c & 3) < NC;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < WQ; ++u) {
      if (wq0 + u >= wq1) break;
      __builtin_amdgcn_sched_barrier(0);  // quad u's work waits for quad u's weights only
      u32x4 xf[4], bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bl = 4 * u + j;  // block within this wave's run
        if (arow)
          xf[j] = *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(arow_p + bl * kDenseBlockStage);
        const uint32_t w = (j == 0) ? nib[u].x : (j == 1) ? nib[u].y : (j == 2) ? nib[u].z : nib[u].w;
#pragma unroll
        for (int b = 0; b < 4; ++b) bf[j][b] = lookup(w, b);
      }
      f32x4 prod[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) prod[j] = mfma_bf16(xf[j], bf[j], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t sw = (j < 2) ? scl[u].x : scl[u].y;
        const float d = h2f((uint16_t)(sw >> (16 * (j & 1))));
#pragma unroll
        for (int i = 0; i < NC; ++i) acc[i] = __builtin_fmaf(d, prod[j][i], acc[i]);
      }
    }
  };

  // Cross-wave reduction in wave order, hi parts and lo parts apart, then hi + lo;
  // stores (or split-K partials) for columns t0 .. t0 + T - 1.
  auto reduce_store = [&](int64_t t0, int T, const f32x4& acc) {
    red[wave * 64 + lane] = acc;
    lds_barrier();
    // lane (g, c) held D[4g + i][c]: part g, column i, weight row c
    const int idx = tid;  // T * 16 <= 64 outputs: the first wave
    const int t = idx >> 4, row = idx & 15;
    float v = 0.f;
    if (idx < T * kTileRows) {
      const float* redf = reinterpret_cast<const float*>(red);
      float pv[2][kDenseWaves];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int w2 = 0; w2 < kDenseWaves; ++w2) pv[p][w2] = redf[(w2 * 64 + 16 * p + row) * 4 + t];
      float part[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float sum = pv[p][0];
#pragma unroll
        for (int w2 = 1; w2 < kDenseWaves; ++w2) sum = (w2 < nwaves) ? sum + pv[p][w2] : sum;
        part[p] = sum;
      }
      v = part[0] + part[1];
    }
    const int64_t col = rg * kTileRows + row;  // output row index (weight row)
    const bool ok = idx < T * kTileRows && col < n_rows;
    if (S == 1) {
      if (ok) Y[(t0 + t) * ldy + col] = v;
      return;
    }
    // Split K: partial sums to the workspace; the last of the S workgroups of this row
    // tile adds them in slice order.  The partials are written and read with agent-scope
    // atomic stores / loads, which go to the device coherence point one access at a
    // time, so no cache-wide writeback or invalidate is needed; s_waitcnt(0) makes every
    // store complete before this workgroup's arrival is counted, and the last arriver
    // issues its loads only after seeing the count.
    // Each pass (columns t0 .. t0 + 3) has partial slots and an arrival counter of its
    // own: nothing orders the passes of different workgroups, so a slice that reaches
    // the second pass early must not touch what the first pass's last arriver reads.
    const int pass = (int)(t0 / kCols);
    int* counter = counters + pass * rg_n + rg;
    float* part = partials + (rg * S + slice) * (kSplitCols * kTileRows) + (t0 + t) * kTileRows + row;
    if (idx < T * kTileRows) __hip_atomic_store(part, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    __syncthreads();
    if (s_last) {
      if (ok) {
        const float* p0 = partials + rg * S * (kSplitCols * kTileRows) + (t0 + t) * kTileRows + row;
        float sum = __hip_atomic_load(p0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int sl = 1; sl < S; ++sl)
          sum += __hip_atomic_load(p0 + sl * (kSplitCols * kTileRows), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        Y[(t0 + t) * ldy + col] = sum;
      }
      // leaves the workspace ready for the next call
      if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // the counter and red are reused by a next pass
  };

  // ---- the first pass (up to 4 columns) -------------------------------------------
  store_x(T0);    // waits for the activations only
  lds_barrier();  // the table (LDS only: no wait on the weights in flight)
  f32x4 acc;
  multiply(acc, ColsC<T0>{});
  reduce_store(0, T0, acc);
  // ---- further passes of 4 columns (T > 4): same weights, next columns ---------------
  for (int64_t t0 = kCols; t0 < ncols; t0 += kCols) {
    const int T = (int)min((int64_t)kCols, ncols - t0);
    lds_barrier();  // every wave is done with red
    load_x(t0, T);
    store_x(T);
    multiply(acc, ColsC<kCols>{});
    reduce_store(t0, T, acc);
  }
}

// ---------------------------------------------------------------------------------
// Grouped matvec (MoE decode): one workgroup per (routed expert slot, run of row groups).
// It finds its expert and stages the expert's columns, then walks its row groups,
// loading the next group's weights while the current one is multiplied (two register
// sets).  Each wave adds its three parts in-wave ((hi + mid) + lo, per column) and
// leaves the group's partial sums in LDS without waiting for the other waves; once a
// batch of up to GB groups is done, one barrier, and the workgroup adds the waves'
// partials in wave order and applies the mode's epilogue.  A column's arithmetic is a
// function of K and the plan only (the T-column invariance).
template <int MODE, int RG, int WQ>
__global__ void __launch_bounds__(512) qmv_grouped_kernel(QmvArgs a) {
  constexpr int NMAT = (MODE == kQmvGateUp) ? 2 : 1;
  constexpr int ROWS = RG * kTileRows;
  constexpr int XBYTES = kWaves * WQ * 4 * kGFragBytes;
  // table copies: 64 (every lane its own copy, and the lookup address is one byte
  // permute: index byte in bits 8..15, the lane's copy in bits 0..7) where the LDS has
  // room; 32 for 3 quads per wave, 16 for 4 (a staged K of 4,096)
  constexpr int LC = (WQ <= 2) ? 64 : (WQ == 3) ? 32 : 16;
  // partials of one row group: [wave][matrix][tile][column][row], fp32
  constexpr int SLOT = kWaves * NMAT * RG * kCols * kTileRows;
  constexpr int OTHER = 256 * LC * 4 + XBYTES + 256 + kWaves * 32 * 4;
  constexpr int GB_FIT = (160 * 1024 - OTHER) / (SLOT * 4);
  constexpr int GB = GB_FIT >= 8 ? 8 : (GB_FIT & ~1);  // row groups per batch (even)
  static_assert(GB >= 2, "two row groups' partials fit the LDS");
  // one LDS block: the table at offset 0 (its lookup address then needs no base), the
  // staged columns (+ room for padding-row reads), the partials, the slot bitmaps
  constexpr int XOFF = 256 * LC * 4, POFF = XOFF + XBYTES + 256, BOFF = POFF + GB * SLOT * 4;
  __shared__ __attribute__((aligned(256))) uint8_t smem[BOFF + kWaves * 32 * 4];
  uint32_t* const lut = reinterpret_cast<uint32_t*>(smem);
  uint8_t* const xs = smem + XOFF;
  float* const part = reinterpret_cast<float*>(smem + POFF);
  uint32_t* const bm = reinterpret_cast<uint32_t*>(smem + BOFF);  // slot lookup: a bitmap per wave

  const int tid = threadIdx.x;
  // the wave index as a scalar: per-wave addresses are then computed once, in SGPRs
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), nwaves = (int)(blockDim.x >> 6);
  const int c = lane & 15, g = lane >> 4;

  // Every kernel argument this kernel reads, loaded at entry.  Left to itself the
  // compiler loads some of them where they are first used, and each such load is a
  // scalar round trip on the way to the first weight request.
  {
    const uint8_t *W0 = a.W0, *W1 = a.W1, *S0 = a.S0, *S1 = a.S1;
    const float *X = a.x, *GW = a.gate_w;
    float *Y = a.y, *G = a.G, *U = a.U;
    const int32_t *ids = a.ids, *offsets = a.offsets, *pairs = a.pairs;
    const int64_t wes = a.w_expert_stride, ldx = a.ldx, ldy = a.ldy, n = a.n, nt = a.nt, rg_n = a.rg_n,
                  nib = a.nibble_bytes, rgc = a.rg_chunks;
    const int she = a.shared_e, n_pairs = a.n_pairs, top_k = a.top_k, n_expert = a.n_expert, kq_n = a.kq_n,
              wave_quads = a.wave_quads, rg_per_wg = a.rg_per_wg;
    asm volatile("" ::"s"(W0), "s"(W1), "s"(S0), "s"(S1), "s"(X), "s"(GW), "s"(Y), "s"(G), "s"(U), "s"(ids),
                 "s"(offsets), "s"(pairs), "s"(wes), "s"(ldx), "s"(ldy), "s"(n), "s"(nt), "s"(rg_n), "s"(nib),
                 "s"(rgc), "s"(she), "s"(n_pairs), "s"(top_k), "s"(n_expert), "s"(kq_n), "s"(wave_quads),
                 "s"(rg_per_wg));
  }
  // The routed ids (when given) are requested first and the level table is built while
  // they are in flight: the slot, and with it every weight address, waits for them.
  const int idv = (a.ids != nullptr && lane < a.n_pairs) ? a.ids[lane] : -1;
  build_pair_table<LC>(lut, tid, (int)blockDim.x);
  asm volatile("" ::"v"(idv));  // the ids' wait here, on every path (as in the down kernel)

  // ---- expert slot and row groups of this workgroup ---------------------------------
  // Slot i takes the i-th expert (ascending id) that has pairs, found in every wave from
  // the routed ids (at most 64 pairs) or the gather's offsets; slots past the routed
  // experts exit.
  const int64_t slot = blockIdx.x / a.rg_chunks;
  const int64_t rg0 = (blockIdx.x % a.rg_chunks) * a.rg_per_wg;
  const int64_t rg1 = min(rg0 + (int64_t)a.rg_per_wg, a.rg_n);
  const SlotInfo si = a.ids ? slot_from_ids(idv, a.n_expert, slot, bm + 32 * wave, lane)
                            : slot_from_offsets(a, slot, lane);
  const int64_t e = si.e, seg0 = si.seg0, ncols = si.ncols;
  if (e < 0 || rg0 >= rg1) return;
  const bool sh = a.S0 != nullptr && e == a.shared_e;  // the shared expert, routed to every token by the caller
  const uint8_t* W[2] = {sh ? a.S0 : a.W0 + e * a.w_expert_stride, sh ? a.S1 : a.W1 + e * a.w_expert_stride};
  const int kq_n = a.kq_n;
  const int wq0 = wave * a.wave_quads;  // this wave's quads (a single slice: K <= 4096)
  const int wq1 = min(wq0 + a.wave_quads, kq_n);

  // ---- this wave's activations (blocks [4 wq0, 4 wq1)), staged by the wave itself ----
  const int wblk = 4 * (wq1 - wq0);
  uint8_t* xw = xs + wave * (4 * WQ) * kGFragBytes;
  constexpr int SLOTS = 16 * WQ;  // staging tasks: (t, bl, gg) = task (t SLOTS + 4 bl + gg)
  // the lane's A fragments, read back once per pass and kept in registers for all row
  // groups (up to 2 quads per wave; with more the registers run out and every group
  // reads them from LDS)
  constexpr bool XREG = WQ <= 2;
  u32x4 xf[XREG ? 4 * WQ : 1];
  auto frag = [&](int bl) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(xw + (min(bl, wblk - 1) * 4 + g) * kGSlot + c * 16);
  };
  const uint32_t* lutl = lut + (lane & (LC - 1));  // this lane's table copy
  typedef __attribute__((address_space(3))) const uint8_t lds_u8;
  lds_u8* const lutb = (lds_u8*)(__attribute__((address_space(3))) uint8_t*)lut;
  const uint32_t lane_copy = (uint32_t)lane * 4u;
  // entry `byte b of w` in this lane's copy
  auto lookup = [&](uint32_t w, int b) -> uint32_t {
    if (LC == 64) {
      const uint32_t addr = __builtin_amdgcn_perm(lane_copy, w, 0x0c0c0004u | ((uint32_t)b << 8));
      return *reinterpret_cast<__attribute__((address_space(3))) const uint32_t*>(lutb + addr);
    }
    return lutl[((w >> (8 * b)) & 0xFF) * LC];
  };
  float4 xr[WQ][2];
  auto load_x = [&](int64_t t0, int T) {  // tasks (column t, block, k-group gg), 64 lanes
    const float* col[kCols];
#pragma unroll
    for (int t = 0; t < kCols; ++t) col[t] = column_ptr(a, MODE, si, t0 + min(t, T - 1));
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int task = lane + 64 * i;
      const int t = task / SLOTS, bl = (task % SLOTS) >> 2, gg = task & 3;
      if (t < T && bl < wblk) {
        const float* cp = (t == 0) ? col[0] : (t == 1) ? col[1] : (t == 2) ? col[2] : col[3];
        const float* p = cp + ((int64_t)wq0 * 4 + bl) * kQK + 8 * gg;
        xr[i][0] = *reinterpret_cast<const float4*>(p);
        xr[i][1] = *reinterpret_cast<const float4*>(p + 4);
      }
    }
  };
  auto store_x = [&](int T) {  // split and store in fragment order
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int task = lane + 64 * i;
      const int t = task / SLOTS, bl = (task % SLOTS) >> 2, gg = task & 3;
      if (t < T && bl < wblk) {
        const float4 xa = xr[i][0], xb = xr[i][1];
        uint32_t p0[3], p1[3], p2[3], p3[3];
        split_pair(xa.x, xa.y, p0);
        split_pair(xa.z, xa.w, p1);
        split_pair(xb.x, xb.y, p2);
        split_pair(xb.z, xb.w, p3);
        uint8_t* dst = xw + (bl * 4 + gg) * kGSlot + t * 64;  // rows 4t + s
#pragma unroll
        for (int sp = 0; sp < 3; ++sp)
          *reinterpret_cast<uint4*>(dst + sp * 16) = uint4{p0[sp], p1[sp], p2[sp], p3[sp]};
      }
    }
    // LDS accesses of one wave execute in order: the wave's reads below see these
    // writes; this only keeps the compiler from moving them.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (XREG) {
#pragma unroll
      for (int bl = 0; bl < 4 * WQ; ++bl) xf[bl] = frag(bl);
    }
  };
  // DOWN: each column's pair id and gate weight (scalar loads through the constant
  // address space: the lists are not written during the call)
  const __attribute__((address_space(4))) float* cgate = (const __attribute__((address_space(4))) float*)a.gate_w;
  int32_t pcol[kCols];
  float gwcol[kCols];
  auto load_cols = [&](int64_t t0, int T) {
    if (MODE != kQmvDown) return;
#pragma unroll
    for (int t = 0; t < kCols; ++t) {
      pcol[t] = pair_of(a, si, t0 + min(t, T - 1));
      gwcol[t] = cgate[pcol[t]];
    }
  };

  // ---- weights of one row group (all of this wave's quads) -------------------------
  struct WSet {
    uint4 nib[WQ][NMAT][RG];
    uint2 scl[WQ][NMAT][RG];
  };
  auto load_w = [&](WSet& ws, int64_t rg) {
#pragma unroll
    for (int u = 0; u < WQ; ++u)
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const int64_t rt = min(rg * RG + r, a.nt - 1);  // clamped: rows past n are dropped
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          const uint8_t* tp = W[m] + rt * kq_n * kTileNibbleBytes + lane * 16;
          const uint8_t* sp = W[m] + a.nibble_bytes + rt * kq_n * kTileScaleBytes + c * 8;
          const int q = min(wq0 + u, max(wq1 - 1, 0));  // clamped; unused when past the range
          ws.nib[u][m][r] = load_nt16(tp + (int64_t)q * kTileNibbleBytes);  // read once: streamed
          ws.scl[u][m][r] = load_nt8(sp + (int64_t)q * kTileScaleBytes);
        }
      }
  };
  // the wave's quads, one block at a time; lanes of padding rows (s = 3 or a column
  // >= T) read whatever lies there: an MFMA output row depends on its own A row only.
  // Lane (g, c) gets D[4g + s][c], part s of column g for weight row c: per block it
  // adds the parts, (hi + mid) + lo, and accumulates d times that sum.
  auto multiply = [&](const WSet& ws, float (&acc)[NMAT][RG]) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int r = 0; r < RG; ++r) acc[m][r] = 0.f;
#pragma unroll
    for (int u = 0; u < WQ; ++u) {
      if (wq0 + u >= wq1) break;
      __builtin_amdgcn_sched_barrier(0);  // quad u's work waits for quad u's weights only
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bl = 4 * u + j;
        u32x4 bf[NMAT][RG];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int r = 0; r < RG; ++r) {
            const uint4 nb = ws.nib[u][m][r];
            const uint32_t w = (j == 0) ? nb.x : (j == 1) ? nb.y : (j == 2) ? nb.z : nb.w;
#pragma unroll
            for (int b = 0; b < 4; ++b) bf[m][r][b] = lookup(w, b);
          }
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int r = 0; r < RG; ++r) {
            const f32x4 pr = mfma_bf16(XREG ? xf[bl] : frag(bl), bf[m][r], f32x4{0.f, 0.f, 0.f, 0.f});
            const uint2 sc = ws.scl[u][m][r];
            const uint32_t sw = (j < 2) ? sc.x : sc.y;
            const float d = h2f((uint16_t)(sw >> (16 * (j & 1))));
            acc[m][r] = __builtin_fmaf(d, (pr[0] + pr[1]) + pr[2], acc[m][r]);
          }
      }
    }
  };
  // A group's partials: lane (g, c) holds column g's sum for weight row c.
  auto write_part = [&](int gi, int T, const float (&acc)[NMAT][RG]) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int r = 0; r < RG; ++r)
        if (g < T) part[(((gi * kWaves + wave) * NMAT + m) * RG + r) * (kCols * kTileRows) + g * kTileRows + c] = acc[m][r];
  };
  // A batch's outputs: the waves' partials added in wave order, then the epilogue.
  auto reduce_batch = [&](int64_t b0, int nb, int64_t t0, int T) {
    const int per_group = T * ROWS;
    const int nout = nb * per_group;
    for (int idx0 = 0; idx0 < nout; idx0 += (int)blockDim.x) {  // uniform trip count
      const int idx = idx0 + tid;
      const int gi = idx / per_group, rem = idx % per_group;
      const int t = rem / ROWS, rr = rem % ROWS;
      const int r = rr >> 4, row = rr & 15;
      const int64_t col = (b0 + gi) * ROWS + rr;  // output row index (weight row)
      if (idx < nout && col < a.n) {
        float v[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          float pv[kWaves];  // every slot read at once (absent waves' slots unused)
#pragma unroll
          for (int w2 = 0; w2 < kWaves; ++w2)
            pv[w2] = part[(((gi * kWaves + w2) * NMAT + m) * RG + r) * (kCols * kTileRows) + t * kTileRows + row];
          float sum = pv[0];
#pragma unroll
          for (int w2 = 1; w2 < kWaves; ++w2) sum = (w2 < nwaves) ? sum + pv[w2] : sum;
          v[m] = sum;
        }
        if (MODE == kQmvGateUp) {
          const float gv = v[0], uv = v[NMAT - 1];
          a.y[(seg0 + t0 + t) * a.ldy + col] = gv / (1.0f + expf(-gv)) * uv;  // SwiGLU
          if (a.G) {  // the intermediates kept (tests)
            a.G[(seg0 + t0 + t) * a.ldy + col] = gv;
            a.U[(seg0 + t0 + t) * a.ldy + col] = uv;
          }
        } else {
          const int pc = (t == 0) ? pcol[0] : (t == 1) ? pcol[1] : (t == 2) ? pcol[2] : pcol[3];
          const float gw = (t == 0) ? gwcol[0] : (t == 1) ? gwcol[1] : (t == 2) ? gwcol[2] : gwcol[3];
          a.y[(int64_t)pc * a.ldy + col] = gw * v[0];
        }
      }
    }
  };

  // ---- prologue: the first pass's columns, then the first row group's weights --------
  // (the columns first: loads complete in order, so staging them waits for them alone
  // and runs while the weights are in flight)
  WSet wa, wb;
  const int T0 = (int)min((int64_t)kCols, ncols);
  load_x(0, T0);
  load_cols(0, T0);
  load_w(wa, rg0);
  __syncthreads();  // the table (LDS only: no wait on the loads in flight)
  store_x(T0);

  // Every step requests the next group's weights (in flight during this group's work);
  // the last group requests itself again (an L2 hit).  With the same loads issued on
  // every path the compiler's waits for `cur` count exactly past them: issued under a
  // branch, the waits merged from both paths also waited for the next group's loads,
  // and each group's work waited for the next group's weights.
  auto step = [&](const WSet& cur, WSet& nxt, int64_t rg, int64_t b0, int T) {
    load_w(nxt, min(rg + 1, rg1 - 1));
    float acc[NMAT][RG];
    multiply(cur, acc);
    write_part((int)(rg - b0), T, acc);
  };
  // Passes of up to kCols columns (more than one only past 4 pairs per expert); each
  // walks the row groups in batches of GB.  Batches other than a pass's last hold an
  // even count, so the steps go in pairs and only the last group of the range can be
  // repeated (same weights, same slot, same values).
  for (int64_t t0 = 0; t0 < ncols; t0 += kCols) {
    const int T = (int)min((int64_t)kCols, ncols - t0);
    if (t0 > 0) {  // the wave's own staging region: no barrier needed
      load_x(t0, T);
      load_cols(t0, T);
      load_w(wa, rg0);
      store_x(T);
    }
    for (int64_t b0 = rg0; b0 < rg1; b0 += GB) {
      const int64_t b1 = min(b0 + (int64_t)GB, rg1);
      for (int64_t rg = b0; rg < b1; rg += 2) {
        step(wa, wb, rg, b0, T);
        step(wb, wa, min(rg + 1, b1 - 1), b0, T);
      }
      __syncthreads();  // every wave's partials of the batch
      reduce_batch(b0, (int)(b1 - b0), t0, T);
      if (b1 < rg1 || t0 + kCols < ncols) __syncthreads();  // the slots are written again
    }
  }
}

// Grouped down matvec for a short K (at most 7 quads, e.g. the MoE decode's intermediate
// size): every wave owns whole 16-row tiles, all of K, so a tile's result needs no
// cross-wave reduction and the loop has no barrier.  The workgroup stages its expert's
// activation columns once (all of K, split into the three bf16 parts), every wave
// requests the weights of its first two tiles at entry, and a tile's three parts are
// added across lanes with two shuffles, in the order (hi + mid) + lo.  A column's
// arithmetic never depends on the other columns.
template <int KQ>
__global__ void __launch_bounds__(512) qmv_down_tiles_kernel(QmvArgs a) {
  constexpr int NB = 4 * KQ;  // blocks of K
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * kLutCopies];
  __shared__ __attribute__((aligned(16))) uint8_t xs[NB * kFragBytes + 256];
  __shared__ uint32_t bm[kWaves * 32];  // slot lookup from the ids: a bitmap per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = (int)(blockDim.x >> 6);
  const int c = lane & 15, g = lane >> 4;

  // Every kernel argument, loaded at entry (as in the grouped kernel).
  {
    const uint8_t *W0 = a.W0, *S0 = a.S0;
    const float *X = a.x, *GW = a.gate_w;
    float* Y = a.y;
    const int32_t *ids = a.ids, *offsets = a.offsets, *pairs = a.pairs;
    const int64_t wes = a.w_expert_stride, ldx = a.ldx, ldy = a.ldy, n = a.n, nt = a.nt,
                  nib = a.nibble_bytes, rgc = a.rg_chunks;
    const int she = a.shared_e, n_pairs = a.n_pairs, n_expert = a.n_expert, rg_per_wg = a.rg_per_wg;
    asm volatile("" ::"s"(W0), "s"(S0), "s"(X), "s"(GW), "s"(Y), "s"(ids), "s"(offsets), "s"(pairs),
                 "s"(wes), "s"(ldx), "s"(ldy), "s"(n), "s"(nt), "s"(nib), "s"(rgc), "s"(she), "s"(n_pairs),
                 "s"(n_expert), "s"(rg_per_wg));
  }
  // the routed ids first, the level table while they are in flight
  const int idv = (a.ids != nullptr && lane < a.n_pairs) ? a.ids[lane] : -1;
  build_pair_table(lut, tid, (int)blockDim.x);
  const uint32_t* lutl = lut + (lane & (kLutCopies - 1));
  // the ids' wait here, on every path: left to a later reuse of its register, the
  // compiler's merged wait there also waited for the columns requested after it, and
  // the weight requests went out only once the columns had arrived
  asm volatile("" ::"v"(idv));

  // ---- expert slot (as the grouped kernel) and this workgroup's row tiles ------------
  const int64_t slot = blockIdx.x / a.rg_chunks;
  const int64_t t0 = (blockIdx.x % a.rg_chunks) * a.rg_per_wg;
  const int64_t t1 = min(t0 + (int64_t)a.rg_per_wg, a.nt);
  const SlotInfo si = a.ids ? slot_from_ids(idv, a.n_expert, slot, bm + 32 * wave, lane)
                            : slot_from_offsets(a, slot, lane);
  const int64_t e = si.e, seg0 = si.seg0, ncols = si.ncols;
  if (e < 0 || t0 >= t1) return;  // uniform over the workgroup
  const uint8_t* W = (a.S0 != nullptr && e == a.shared_e) ? a.S0 : a.W0 + e * a.w_expert_stride;  // shared expert

  struct WSet {
    uint4 nib[KQ];
    uint2 scl[KQ];
  };
  auto load_w = [&](WSet& w, int64_t rt) {
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      w.nib[q] = load_nt16(W + (rt * KQ + q) * kTileNibbleBytes + lane * 16);  // read once: streamed
      w.scl[q] = load_nt8(W + a.nibble_bytes + (rt * KQ + q) * kTileScaleBytes + c * 8);
    }
  };
  // The first pass's columns are requested before the weights (loads complete in order,
  // so staging them then waits for them alone): one staging task per thread.
  constexpr int NTASK = kCols * NB * 4;  // (column, block, k-group) staging tasks of a pass
  static_assert(NTASK <= 512, "one staging task per thread");
  const int task_t = tid / (NB * 4), task_bl = (tid >> 2) % NB, task_gg = tid & 3;
  const int T0 = (int)min((int64_t)kCols, ncols);
  float4 x0a = float4{0.f, 0.f, 0.f, 0.f}, x0b = x0a;
  if (tid < NTASK && task_t < T0) {
    const float* p = a.x + (seg0 + task_t) * a.ldx + task_bl * kQK + 8 * task_gg;
    x0a = *reinterpret_cast<const float4*>(p);
    x0b = *reinterpret_cast<const float4*>(p + 4);
  }
  // the wave's first two tiles (a wave without them requests the last tile again, an L2
  // hit, so that every wave issues the same loads and the waits stay exact)
  WSet wa, wb;
  const int64_t r0 = t0 + wave;
  load_w(wa, min(r0, t1 - 1));
  load_w(wb, min(r0 + nwaves, t1 - 1));


  // the pass's columns: h rows seg0 + p0 + t (pair-sorted), their pair ids and gate
  // weights (scalar loads: the lists are not written during the call)
  const __attribute__((address_space(4))) float* cgate = (const __attribute__((address_space(4))) float*)a.gate_w;

  // A pass: the columns p0 .. p0 + 3.  The first pass is its own instantiation, so no
  // branch around a load lies between the entry's requests and the waits for them.
  auto pass = [&](int64_t p0, auto first_tag) {
    constexpr bool FIRST = decltype(first_tag)::value;
    const int T = (int)min((int64_t)kCols, ncols - p0);
    int32_t pc[kCols];
    float gw[kCols];
#pragma unroll
    for (int t = 0; t < kCols; ++t) {
      pc[t] = pair_of(a, si, p0 + min(t, T - 1));
      gw[t] = cgate[pc[t]];
    }
    if (!FIRST) __syncthreads();  // every wave is done with the previous pass's columns
    {
      const int task = tid, t = task_t, bl = task_bl, gg = task_gg;
      if (task < NTASK && t < T) {
        float4 xa = x0a, xb = x0b;  // the first pass's, loaded at entry
        if (!FIRST) {
          const float* p = a.x + (seg0 + p0 + t) * a.ldx + bl * kQK + 8 * gg;
          xa = *reinterpret_cast<const float4*>(p);
          xb = *reinterpret_cast<const float4*>(p + 4);
        }
        uint32_t q0[3], q1[3], q2[3], q3[3];
        split_pair(xa.x, xa.y, q0);
        split_pair(xa.z, xa.w, q1);
        split_pair(xb.x, xb.y, q2);
        split_pair(xb.z, xb.w, q3);
        uint8_t* dst = xs + (bl * 4 + gg) * (kFragStride * 16) + t * 16;
#pragma unroll
        for (int sp = 0; sp < 3; ++sp)
          *reinterpret_cast<uint4*>(dst + sp * 4 * 16) = uint4{q0[sp], q1[sp], q2[sp], q3[sp]};
      }
    }
    __syncthreads();  // the table and the staged columns

    auto tile = [&](const WSet& w, int64_t rt) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        __builtin_amdgcn_sched_barrier(0);  // quad q's work waits for quad q's weights only
        u32x4 xf[4], bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xf[j] = *reinterpret_cast<const u32x4*>(xs + ((4 * q + j) * 4 + g) * (kFragStride * 16) + c * 16);
          const uint32_t wd = (j == 0) ? w.nib[q].x : (j == 1) ? w.nib[q].y : (j == 2) ? w.nib[q].z : w.nib[q].w;
          bf[j][0] = lutl[(wd & 0xFF) * kLutCopies];
          bf[j][1] = lutl[((wd >> 8) & 0xFF) * kLutCopies];
          bf[j][2] = lutl[((wd >> 16) & 0xFF) * kLutCopies];
          bf[j][3] = lutl[(wd >> 24) * kLutCopies];
        }
        f32x4 prod[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) prod[j] = mfma_bf16(xf[j], bf[j], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t sw = (j < 2) ? w.scl[q].x : w.scl[q].y;
          const float d = h2f((uint16_t)(sw >> (16 * (j & 1))));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(d, prod[j][i], acc[i]);
        }
      }
      // lane (g, c) holds D[4g + i][c]: part g of column i, weight row c; lanes of
      // k-group 0 add the parts of lanes c + 16 and c + 32
      float v[kCols];
#pragma unroll
      for (int i = 0; i < kCols; ++i) {
        const float mid = __shfl(acc[i], (lane + 16) & 63);
        const float lo = __shfl(acc[i], (lane + 32) & 63);
        v[i] = (acc[i] + mid) + lo;
      }
      const int64_t col = rt * kTileRows + c;
      if (g == 0 && col < a.n) {
#pragma unroll
        for (int i = 0; i < kCols; ++i)
          if (i < T) a.y[(int64_t)pc[i] * a.ldy + col] = gw[i] * v[i];
      }
    };
    // tiles r0, r0 + nwaves, ...: sets wa / wb alternate, each refilled two tiles ahead
    for (int64_t rt = r0; rt < t1; rt += 2 * nwaves) {
      tile(wa, rt);
      if (rt + 2 * nwaves < t1) load_w(wa, rt + 2 * nwaves);
      if (rt + nwaves < t1) {
        tile(wb, rt + nwaves);
        if (rt + 3 * nwaves < t1) load_w(wb, rt + 3 * nwaves);
      }
    }
  };
  pass(0, std::true_type{});
  for (int64_t p0 = kCols; p0 < ncols; p0 += kCols) {  // a further pass walks the tiles again
    load_w(wa, min(r0, t1 - 1));
    load_w(wb, min(r0 + nwaves, t1 - 1));
    pass(p0, std::false_type{});
  }
}

// Down product and ordered combine in one launch, for a decode call with at most 64
// routed pairs (the ids given): one workgroup per (16-row output tile, token) and one
// wave per slot j of the token.  The wave finds its pair's expert and h row from the
// ids (the h rows are in (expert, pair id) order), stages that row (all of K, three
// bf16 parts in rows 0..2 of the A operand) and multiplies the expert's row tile; lane
// (0, c) then holds the three parts of weight row c and adds them, (hi + mid) + lo.
// The gate-weighted slot rows meet in LDS and the token's outputs are their sum in slot
// order.  Per value this is the arithmetic of the whole-tile down kernel followed by
// the combine (the same products, block order, part order and slot order), so the
// result is bitwise that of the separate launches.
constexpr int kDcSlot = 3 * 16;  // one (block, k-group) slot: the three parts of one column

// (8 waves: registers for two workgroups per CU, four waves per SIMD)
template <int KQ, int NW>
__global__ void __launch_bounds__(64 * NW, NW == 8 ? 4 : 1) qmv_down_combine_kernel(QmvArgs a) {
  constexpr int NB = 4 * KQ;                   // blocks of K
  constexpr int XW = NB * 4 * kDcSlot + 256;   // a wave's staging area (+ room for pad-row reads)
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * kLutCopies];
  __shared__ __attribute__((aligned(16))) uint8_t xs[NW * XW];
  __shared__ float slot_rows[NW * kTileRows];

  // every kernel argument at entry (one scalar wait)
  const uint8_t *const W0 = a.W0, *const S0 = a.S0;
  const float* const X = a.x;
  const float* const GW = a.gate_w;
  float* const Y = a.y;
  const int32_t* const ids = a.ids;
  const int64_t wes = a.w_expert_stride, ldx = a.ldx, ldy = a.ldy, nt = a.nt, nib_bytes = a.nibble_bytes;
  const int she = a.shared_e, n_pairs = a.n_pairs, n_expert = a.n_expert, top_k = a.top_k;
  asm volatile("" ::"s"(W0), "s"(S0), "s"(X), "s"(GW), "s"(Y), "s"(ids), "s"(wes), "s"(ldx), "s"(ldy), "s"(nt),
               "s"(nib_bytes), "s"(she), "s"(n_pairs), "s"(n_expert), "s"(top_k));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t tok = blockIdx.x % (a.n_pairs / top_k), rt = blockIdx.x / (a.n_pairs / top_k);

  // the routed ids (one per lane) first, the level table while they are in flight
  const int idv = (lane < n_pairs) ? ids[lane] : -1;
  build_pair_table(lut, tid, (int)blockDim.x);
  const uint32_t* lutl = lut + (lane & (kLutCopies - 1));
  asm volatile("" ::"v"(idv));

  // this wave's pair: its expert and its h row (the pair's rank in (expert, pair id)
  // order).  A pair whose id is outside [0, n_expert) has no h row: it reads expert 0
  // and row 0 and adds zero.
  const int p = (int)tok * top_k + wave;
  const int e = __builtin_amdgcn_readfirstlane(__shfl(idv, p));
  const bool valid = (unsigned)idv < (unsigned)n_expert;
  const bool e_ok = (unsigned)e < (unsigned)n_expert;
  const int pos = e_ok ? __popcll(__ballot(valid && idv < e)) + __popcll(__ballot(valid && idv == e && lane < p)) : 0;
  const float gw = GW[p];
  const uint8_t* const W = (S0 != nullptr && e == she) ? S0 : W0 + (int64_t)(e_ok ? e : 0) * wes;

  // requests: the h row (tasks (block, k-group), 8 floats each), then the tile's weights
  constexpr int NI = (4 * NB + 63) / 64;
  float4 xr[NI][2];
  const float* const xrow = X + (int64_t)pos * ldx;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int task = min(lane + 64 * i, 4 * NB - 1);  // clamped: every lane issues the same loads
    const float* q = xrow + (task >> 2) * kQK + 8 * (task & 3);
    xr[i][0] = *reinterpret_cast<const float4*>(q);
    xr[i][1] = *reinterpret_cast<const float4*>(q + 4);
  }
  uint4 nib[KQ];
  uint2 scl[KQ];
#pragma unroll
  for (int q = 0; q < KQ; ++q) {
    nib[q] = load_nt16(W + (rt * KQ + q) * kTileNibbleBytes + lane * 16);  // read once: streamed
    scl[q] = load_nt8(W + nib_bytes + (rt * KQ + q) * kTileScaleBytes + c * 8);
  }
  __syncthreads();  // the table (LDS only: no wait on the loads in flight)

  // stage the h row: part s of elements 8gg .. 8gg+7 of block bl in row s of slot
  // (bl, gg) (the wave's own area; its LDS accesses execute in order)
  uint8_t* const xw = xs + wave * XW;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int task = lane + 64 * i;
    if (task < 4 * NB) {
      uint32_t q0[3], q1[3], q2[3], q3[3];
      split_pair(xr[i][0].x, xr[i][0].y, q0);
      split_pair(xr[i][0].z, xr[i][0].w, q1);
      split_pair(xr[i][1].x, xr[i][1].y, q2);
      split_pair(xr[i][1].z, xr[i][1].w, q3);
      uint8_t* dst = xw + task * kDcSlot;
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) *reinterpret_cast<uint4*>(dst + sp * 16) = uint4{q0[sp], q1[sp], q2[sp], q3[sp]};
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // the tile: lane (0, c) receives D[s][c] = part s of the column for weight row c
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f;
#pragma unroll
  for (int q = 0; q < KQ; ++q) {
    __builtin_amdgcn_sched_barrier(0);  // quad q's work waits for quad q's weights only
#pragma unroll
    for (int j2 = 0; j2 < 4; j2 += 2) {  // two blocks at a time (registers)
      u32x4 xf[2], bf[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = j2 + jj;
        xf[jj] = *reinterpret_cast<const u32x4*>(xw + ((4 * q + j) * 4 + g) * kDcSlot + c * 16);
        const uint32_t wd = (j == 0) ? nib[q].x : (j == 1) ? nib[q].y : (j == 2) ? nib[q].z : nib[q].w;
        bf[jj][0] = lutl[(wd & 0xFF) * kLutCopies];
        bf[jj][1] = lutl[((wd >> 8) & 0xFF) * kLutCopies];
        bf[jj][2] = lutl[((wd >> 16) & 0xFF) * kLutCopies];
        bf[jj][3] = lutl[(wd >> 24) * kLutCopies];
      }
      f32x4 prod[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) prod[jj] = mfma_bf16(xf[jj], bf[jj], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = j2 + jj;
        const uint32_t sw = (j < 2) ? scl[q].x : scl[q].y;
        const float d = h2f((uint16_t)(sw >> (16 * (j & 1))));
        acc0 = __builtin_fmaf(d, prod[jj][0], acc0);
        acc1 = __builtin_fmaf(d, prod[jj][1], acc1);
        acc2 = __builtin_fmaf(d, prod[jj][2], acc2);
      }
    }
  }
  if (g == 0) slot_rows[wave * kTileRows + c] = e_ok ? gw * ((acc0 + acc1) + acc2) : 0.f;
  __syncthreads();
  // the token's outputs: its slot rows added in slot order
  if (tid < kTileRows) {
    float sum = slot_rows[tid];
    for (int j = 1; j < top_k; ++j) sum += slot_rows[j * kTileRows + tid];
    Y[tok * ldy + rt * kTileRows + tid] = sum;
  }
}

// Shape-only launch plan (never depends on T): K is cut into slices of at most
// kSliceQuads quads (more than one slice only for K > 4096), each wave of a workgroup
// owns a contiguous run of at most kMaxWaveQuads quads of the slice.
static void qmv_plan(QmvArgs& a, int64_t n, int64_t k, int rg_rows) {
  a.n = n;
  a.nt = n / kTileRows;
  a.kq_n = (int)(k / kTileK);
  a.nibble_bytes = n * (k / kQK) * kNibbleBytes;
  a.rg_n = (a.nt + rg_rows - 1) / rg_rows;
  a.S = (a.kq_n + kSliceQuads - 1) / kSliceQuads;
  a.slice_quads = (a.kq_n + a.S - 1) / a.S;
  a.wave_quads = (a.slice_quads + kWaves - 1) / kWaves;
  a.nwaves = (a.slice_quads + a.wave_quads - 1) / a.wave_quads;
}

// Split-K workspace (both the float and the 8-bit-activation matvec): the arrival
// counters, one per (pass, row group) -- the float call runs up to two passes of 4
// columns, the 8-bit call one pass of 8 and uses the first set -- left at zero by
// each call; then the partial sums [row group][slice][8 columns][16 rows], where pass
// p of the float call owns columns 4p .. 4p + 3.
static inline int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }
static int64_t ws_partials_off(const QmvArgs& a) { return align256(2 * a.rg_n * (int64_t)sizeof(int)); }

int64_t qmv_workspace_bytes(int64_t n, int64_t k) {
  QmvArgs a{};
  qmv_plan(a, n, k, kDenseRG);
  if (a.S == 1) return 0;
  return ws_partials_off(a) + a.rg_n * a.S * kSplitCols * kTileRows * (int64_t)sizeof(float);
}

template <int WQ, int TP>
static int launch_dense_t(const QmvArgs& a, int64_t grid) {
  if (grid == 0) return 0;
  hipLaunchKernelGGL((qmv_dense_kernel<WQ, TP>), dim3((unsigned)grid), dim3(64 * a.nwaves), 0, a.stream, a);
  return check_launch("qmv_dense_kernel");
}

// Instantiation by the first pass's column count.
template <int WQ>
static int launch_dense(const QmvArgs& a, int64_t grid) {
  switch (a.T < kCols ? a.T : kCols) {
    case 1: return launch_dense_t<WQ, 1>(a, grid);
    case 2: return launch_dense_t<WQ, 2>(a, grid);
    case 3: return launch_dense_t<WQ, 3>(a, grid);
    default: return launch_dense_t<WQ, kCols>(a, grid);
  }
}

int launch_qmv(const uint8_t* packed, int64_t n, int64_t k, const float* x, int64_t ldx, int T,
               float* y, int64_t ldy, void* workspace, hipStream_t s) {
  QmvArgs a{};
  a.W0 = packed;
  a.x = x;
  a.ldx = ldx;
  a.T = T;
  a.y = y;
  a.ldy = ldy;
  a.stream = s;
  qmv_plan(a, n, k, kDenseRG);
  a.wave_quads = (a.slice_quads + kDenseWaves - 1) / kDenseWaves;  // this kernel's own wave split
  a.nwaves = (a.slice_quads + a.wave_quads - 1) / a.wave_quads;
  if (a.S > 1) {
    a.counters = static_cast<int*>(workspace);
    a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ws_partials_off(a));
  }
  const int64_t grid = a.rg_n * a.S;
  switch (a.wave_quads) {  // instantiation by quads per wave (the plan gives 1..4)
    case 1: return launch_dense<1>(a, grid);
    case 2: return launch_dense<2>(a, grid);
    case 3: return launch_dense<3>(a, grid);
    default: return launch_dense<kMaxWaveQuads>(a, grid);
  }
}

// ---------------------------------------------------------------------------------
// The matvec without a caller workspace (iq4_qmv_multi_noalloc), for callers that cannot
// allocate: the split-K arrival counters and partial sums of a call live in this
// file-scope device array.  Each GPU holds its own copy until the process ends.  In
// host code the name `scratch` is only a host-side stand-in for the array: kernels get
// the device address that hipGetSymbolAddress returns, looked up once per device (with
// that device current) and kept in g_scratch.  Every call on one GPU shares that GPU's
// copy: calls that overlap in time on one GPU race; calls in one stream order do not
// (each leaves the counters at zero, as a caller workspace is left).
constexpr int64_t kQmvScratchBytes = int64_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kQmvScratchBytes];

__global__ void __launch_bounds__(256) zero_scratch_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch[kMaxDevices];

// The device address of this GPU's scratch; the first call on a device looks it up and
// clears the array with a fill kernel on `s` (a kernel, not a memset, so that a caller
// capturing the call records no memset node).
static int scratch_address(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(IQ4_E_HIP, "iq4_qmv_multi_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(IQ4_E_HIP, "iq4_qmv_multi_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return set_error(IQ4_E_HIP, "iq4_qmv_multi_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(zero_scratch_kernel, dim3(256), dim3(256), 0, s, static_cast<uint4*>(ptr),
                       kQmvScratchBytes / 16);
    if (int rc = check_launch("zero_scratch_kernel")) return rc;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return IQ4_OK;
}

int launch_qmv_noalloc(const uint8_t* packed, int64_t n, int64_t k, const float* x, int64_t ldx, int T,
                       float* y, int64_t ldy, hipStream_t s) {
  const int64_t need = qmv_workspace_bytes(n, k);
  if (need > kQmvScratchBytes)
    return set_error(IQ4_E_WORKSPACE,
                     "iq4_qmv_multi_noalloc: n=%lld k=%lld needs %lld bytes of split-K scratch, above the "
                     "%lld-byte array (use iq4_qmv_multi with a workspace)",
                     (long long)n, (long long)k, (long long)need, (long long)kQmvScratchBytes);
  void* ws = nullptr;
  if (int rc = scratch_address(s, &ws)) return rc;
  return launch_qmv(packed, n, k, x, ldx, T, y, ldy, need > 0 ? ws : nullptr, s);
}

template <int MODE, int RG, int WQ>
static int launch_grouped_mode(const QmvArgs& a, int64_t grid) {
  if (grid == 0) return 0;
  hipLaunchKernelGGL((qmv_grouped_kernel<MODE, RG, WQ>), dim3((unsigned)grid), dim3(64 * a.nwaves), 0, a.stream,
                     a);
  return check_launch("qmv_grouped_kernel");
}

template <int MODE, int RG>
static int launch_grouped_sized(const QmvArgs& a, int64_t grid) {
  switch (a.wave_quads) {
    case 1: return launch_grouped_mode<MODE, RG, 1>(a, grid);
    case 2: return launch_grouped_mode<MODE, RG, 2>(a, grid);
    case 3: return launch_grouped_mode<MODE, RG, 3>(a, grid);
    default: return launch_grouped_mode<MODE, RG, kMaxWaveQuads>(a, grid);
  }
}

// Row groups per workgroup: enough that the grid holds about one workgroup per CU (a
// long walk keeps the next group's weights in flight; measured best against 2 and 4
// workgroups per CU).
static void grouped_split(QmvArgs& a, int64_t slots) {
  const int64_t want = 256;
  int64_t per = (a.rg_n * slots + want - 1) / want;
  if (per < 1) per = 1;
  if (per > a.rg_n) per = a.rg_n;
  a.rg_per_wg = (int)per;
  a.rg_chunks = (a.rg_n + per - 1) / per;
}

constexpr int64_t kMaxDownTilesK = 7 * kTileK;  // 896: two weight sets of 7 quads still fit the registers

template <int KQ>
static int launch_down_tiles(const QmvArgs& a, int64_t grid) {
  if (grid == 0) return 0;
  hipLaunchKernelGGL((qmv_down_tiles_kernel<KQ>), dim3((unsigned)grid), dim3(512), 0, a.stream, a);
  return check_launch("qmv_down_tiles_kernel");
}

int launch_qmv_grouped(int mode, QmvArgs a, int64_t n, int64_t k, int n_expert, int64_t n_pairs) {
  a.n_expert = n_expert;
  const int64_t slots = (n_pairs < n_expert) ? n_pairs : n_expert;  // routed experts at most
  if (mode == kQmvGateUp) {
    qmv_plan(a, n, k, kGateUpRG);
    if (a.S != 1) return set_error(-3, "grouped matvec: K above 4096 is not supported");
    grouped_split(a, slots);
    return launch_grouped_sized<kQmvGateUp, kGateUpRG>(a, slots * a.rg_chunks);
  }
  if (k <= kMaxDownTilesK) {  // whole row tiles per wave (short K)
    qmv_plan(a, n, k, 1);
    const int64_t want = 256;  // workgroups
    int64_t per = (a.nt * slots + want - 1) / want;
    if (per < 1) per = 1;
    a.rg_per_wg = (int)per;
    a.rg_chunks = (a.nt + per - 1) / per;
    const int64_t grid = slots * a.rg_chunks;
    switch (a.kq_n) {
      case 1: return launch_down_tiles<1>(a, grid);
      case 2: return launch_down_tiles<2>(a, grid);
      case 3: return launch_down_tiles<3>(a, grid);
      case 4: return launch_down_tiles<4>(a, grid);
      case 5: return launch_down_tiles<5>(a, grid);
      case 6: return launch_down_tiles<6>(a, grid);
      default: return launch_down_tiles<7>(a, grid);
    }
  }
  qmv_plan(a, n, k, kDownRG);
  if (a.S != 1) return set_error(-3, "grouped matvec: K above 4096 is not supported");
  grouped_split(a, slots);
  return launch_grouped_sized<kQmvDown, kDownRG>(a, slots * a.rg_chunks);
}

template <int KQ, int NW>
static int launch_dc(const QmvArgs& a, int64_t grid) {
  hipLaunchKernelGGL((qmv_down_combine_kernel<KQ, NW>), dim3((unsigned)grid), dim3(64 * a.top_k), 0, a.stream, a);
  return check_launch("qmv_down_combine_kernel");
}
template <int NW>
static int launch_dc_nw(const QmvArgs& a, int64_t grid) {
  switch (a.kq_n) {
    case 1: return launch_dc<1, NW>(a, grid);
    case 2: return launch_dc<2, NW>(a, grid);
    case 3: return launch_dc<3, NW>(a, grid);
    case 4: return launch_dc<4, NW>(a, grid);
    case 5: return launch_dc<5, NW>(a, grid);
    case 6: return launch_dc<6, NW>(a, grid);
    default: return launch_dc<7, NW>(a, grid);
  }
}

bool qmv_down_combine_fits(int64_t k, int top_k, int64_t n_pairs) {
  return k <= kMaxDownTilesK && top_k >= 1 && top_k <= 16 && n_pairs <= kDirectMaxPairs;
}

int launch_qmv_down_combine(QmvArgs a, int64_t n, int64_t k, int n_expert, int64_t n_tok) {
  a.n_expert = n_expert;
  qmv_plan(a, n, k, 1);
  a.n_pairs = (int)(n_tok * a.top_k);
  const int64_t grid = a.nt * n_tok;
  if (grid == 0) return 0;
  return a.top_k <= 8 ? launch_dc_nw<8>(a, grid) : launch_dc_nw<16>(a, grid);
}

// ---------------------------------------------------------------------------------
// 8-bit activations: page 1's decode products read the window's T activation columns
// as q8_1 blocks (verify.hpp member declarations).  Per column and 32-k block:
// d = f32(absmax) / 127, r = 1 / d (IEEE binary32 divisions; r = 0 when d rounds to a
// zero binary16), q = nearest integer of f32(x * r), halves away from zero, clamped to
// +-127; stored: the codes (int8 [T][K]) and d as binary16 ([T][K/32]).

// One lane per 8 consecutive k of one column; the 4 lanes of a block exchange their
// maxima with two xor shuffles (K % 32 == 0, so a block never straddles columns).
__global__ void __launch_bounds__(256) quantize_q8_kernel(const float* __restrict__ x, int64_t T, int64_t K,
                                                          int64_t ldx, int8_t* __restrict__ q,
                                                          uint16_t* __restrict__ d) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = K / 8;
  const bool ok = i < T * per;
  const int64_t t = ok ? i / per : 0, k8 = ok ? (i % per) * 8 : 0;
  float v[8];
  if (ok) {
    const float4 a = *reinterpret_cast<const float4*>(x + t * ldx + k8);
    const float4 b = *reinterpret_cast<const float4*>(x + t * ldx + k8 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.f;
  }
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  const float dd = m / 127.0f;
  const uint16_t h = __half_as_ushort(__float2half_rn(dd));
  const float r = (h != 0) ? 1.0f / dd : 0.0f;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = v[j] * r;
    const float tr = truncf(p);
    float c = tr + ((fabsf(p - tr) >= 0.5f) ? copysignf(1.0f, p) : 0.0f);  // halves away from zero
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    w[j >> 2] |= ((uint32_t)(int)c & 0xFFu) << (8 * (j & 3));
  }
  if (ok) {
    *reinterpret_cast<uint2*>(q + t * K + k8) = uint2{w[0], w[1]};
    if ((i & 3) == 0) d[t * (K / kQK) + k8 / kQK] = h;
  }
}

// T-column matvec on 8-bit activations, T <= 8: the dense kernel's plan, weight stream
// and level table, with A = the codes (one row per token; exact in bf16, |q| <= 127).
// A block's MFMA result is then the exact integer dot sum_i c[q_w,i] * q_i (products of
// at most 14 bits, sums below 2^24), scaled by the exact product of the two binary16
// scales with one fp32 FMA per block.  A column's arithmetic never depends on T.
constexpr int kQ8Rows = 8;                      // tokens per call (A rows 0..7)
constexpr int kQ8Stride = 9;                      // rows per (block, k-group) slot (8 used; see kFragStride)
constexpr int kQ8FragBytes = 4 * kQ8Stride * 16;  // 576 B per block: [k-group g][token][16 B]

template <int WQ, int TP>
__global__ void __launch_bounds__(512) qmv_q8_kernel(QmvArgs a) {
  static_assert(TP >= 1 && TP <= kQ8Rows, "1..8 columns");
  constexpr int XBYTES = kWaves * WQ * 4 * kQ8FragBytes;
  __shared__ uint32_t lut[256 * kLutCopies];
  __shared__ __attribute__((aligned(16))) uint8_t xs[XBYTES];
  __shared__ __attribute__((aligned(16))) uint16_t dxs[kWaves * WQ * 4 * kQ8Rows];  // [block][token]
  __shared__ f32x4 red[kWaves * 64];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = (int)(blockDim.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int T = a.T;  // <= TP

  const int64_t rg = blockIdx.x / a.S;
  const int slice = (int)(blockIdx.x % a.S);
  const int kq_n = a.kq_n;
  const int kqa = slice * a.slice_quads;
  const int nq_slice = min(a.slice_quads, kq_n - kqa);
  const int wq0 = wave * a.wave_quads;
  const int wq1 = min(wq0 + a.wave_quads, nq_slice);
  const int wblk = 4 * (wq1 - wq0);
  uint8_t* xw = xs + wave * (4 * WQ) * kQ8FragBytes;
  uint16_t* dxw = dxs + wave * (4 * WQ) * kQ8Rows;

  // staging tasks (token t, block bl, k-group gg) = task (t SLOTS + 4 bl + gg), task =
  // lane + 64 i: 8 codes each, the gg = 0 task also the block's scale
  constexpr int SLOTS = 16 * WQ;
  constexpr int NT = (TP * SLOTS + 63) / 64;
  uint2 xr[NT];
  uint16_t dr[NT];
  const int64_t kb0 = (int64_t)(kqa + wq0) * 4;  // first block of the wave's run
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int task = lane + 64 * i;
    const int t = task / SLOTS, bl = (task % SLOTS) >> 2, gg = task & 3;
    if (t < T && bl < wblk) {
      xr[i] = *reinterpret_cast<const uint2*>(a.xq + t * a.ldx + (kb0 + bl) * kQK + 8 * gg);
      if (gg == 0) dr[i] = a.xd[t * (a.ldx / kQK) + kb0 + bl];
    }
  }
  uint4 nib[WQ];
  uint2 scl[WQ];
  const uint8_t* tp = a.W0 + (rg * kq_n + kqa) * kTileNibbleBytes + lane * 16;
  const uint8_t* sp = a.W0 + a.nibble_bytes + (rg * kq_n + kqa) * kTileScaleBytes + c * 8;
#pragma unroll
  for (int u = 0; u < WQ; ++u) {
    const int q = min(wq0 + u, max(wq1 - 1, 0));
    nib[u] = load_nt16(tp + (int64_t)q * kTileNibbleBytes);  // read once: streamed
    scl[u] = load_nt8(sp + (int64_t)q * kTileScaleBytes);
  }
  for (int i = tid; i < 512; i += blockDim.x) {
    const int e = i >> 1;
    const uint32_t v = bf16_of_level(level_of(e & 15)) | (bf16_of_level(level_of(e >> 4)) << 16);
    uint4* dst = reinterpret_cast<uint4*>(lut + e * kLutCopies + (i & 1) * 16);
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) dst[w4] = uint4{v, v, v, v};
  }
  const uint32_t* lutl = lut + (lane & (kLutCopies - 1));

  // codes -> bf16 A rows (exact), scales -> LDS
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int task = lane + 64 * i;
    const int t = task / SLOTS, bl = (task % SLOTS) >> 2, gg = task & 3;
    if (t < T && bl < wblk) {
      uint32_t f[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t word = (j < 2) ? xr[i].x : xr[i].y;
        const int s0 = 16 * (j & 1);
        const float lo = (float)(int8_t)((word >> s0) & 0xFFu);
        const float hi = (float)(int8_t)((word >> (s0 + 8)) & 0xFFu);
        f[j] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
      }
      *reinterpret_cast<uint4*>(xw + (bl * 4 + gg) * (kQ8Stride * 16) + t * 16) = uint4{f[0], f[1], f[2], f[3]};
      if (gg == 0) dxw[bl * kQ8Rows + t] = dr[i];
    }
  }
  lds_barrier();  // the table (LDS only: no wait on the weights in flight)

  // lanes of rows >= 8 (and of tokens >= T) read some token's row: their outputs are
  // never used, and an MFMA output row depends on its own A row only
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < WQ; ++u) {
    if (wq0 + u >= wq1) break;
    __builtin_amdgcn_sched_barrier(0);  // quad u's work waits for quad u's weights only
    u32x4 xf[4], bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bl = 4 * u + j;
      xf[j] = *reinterpret_cast<const u32x4*>(xw + (bl * 4 + g) * (kQ8Stride * 16) + (c & 7) * 16);
      const uint32_t w = (j == 0) ? nib[u].x : (j == 1) ? nib[u].y : (j == 2) ? nib[u].z : nib[u].w;
      bf[j][0] = lutl[(w & 0xFF) * kLutCopies];
      bf[j][1] = lutl[((w >> 8) & 0xFF) * kLutCopies];
      bf[j][2] = lutl[((w >> 16) & 0xFF) * kLutCopies];
      bf[j][3] = lutl[(w >> 24) * kLutCopies];
    }
    f32x4 prod[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) prod[j] = mfma_bf16(xf[j], bf[j], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bl = 4 * u + j;
      const uint32_t sw = (j < 2) ? scl[u].x : scl[u].y;
      const float dw = h2f((uint16_t)(sw >> (16 * (j & 1))));
      const uint2 dx4 = *reinterpret_cast<const uint2*>(dxw + bl * kQ8Rows + 4 * (g & 1));
      // below 4 tokens only lanes i < TP of k-group 0 feed an output
#pragma unroll
      for (int i = 0; i < (TP < 4 ? TP : 4); ++i) {
        const uint32_t hw = (i < 2) ? dx4.x : dx4.y;
        const float s = dw * h2f((uint16_t)(hw >> (16 * (i & 1))));  // exact: 11 x 11 bits
        acc[i] = __builtin_fmaf(s, prod[j][i], acc[i]);
      }
    }
  }

  // cross-wave reduction in wave order: lane (g, c) held D[4g + i][c], token 4g + i.
  // Up to 128 outputs: a narrow workgroup (small K) covers them in several rounds.
  red[wave * 64 + lane] = acc;
  lds_barrier();
  const float* redf = reinterpret_cast<const float*>(red);
  const int nout = T * kTileRows;
  auto output = [&](int idx) -> float {
    const int t = idx >> 4, row = idx & 15;
    float pv[kWaves];
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) pv[w2] = redf[(w2 * 64 + 16 * (t >> 2) + row) * 4 + (t & 3)];
    float v = pv[0];
#pragma unroll
    for (int w2 = 1; w2 < kWaves; ++w2) v = (w2 < nwaves) ? v + pv[w2] : v;
    return v;
  };
  if (a.S == 1) {
    for (int idx = tid; idx < nout; idx += (int)blockDim.x) {
      const int64_t col = rg * kTileRows + (idx & 15);
      if (col < a.n) a.y[(idx >> 4) * a.ldy + col] = output(idx);
    }
    return;
  }
  // split K: as the float matvec (agent-scope stores, counter, last arriver adds the
  // slices in order and resets the counter)
  float* part = a.partials + (rg * a.S + slice) * (kQ8Rows * kTileRows);
  for (int idx = tid; idx < nout; idx += (int)blockDim.x)
    __hip_atomic_store(part + idx, output(idx), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(a.counters + rg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.S - 1;
  __syncthreads();
  if (s_last) {
    for (int idx = tid; idx < nout; idx += (int)blockDim.x) {
      const int64_t col = rg * kTileRows + (idx & 15);
      if (col >= a.n) continue;
      const float* p0 = a.partials + rg * a.S * (kQ8Rows * kTileRows) + idx;
      float sum = __hip_atomic_load(p0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int sl = 1; sl < a.S; ++sl)
        sum += __hip_atomic_load(p0 + sl * (kQ8Rows * kTileRows), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.y[(idx >> 4) * a.ldy + col] = sum;
    }
    if (tid == 0) __hip_atomic_store(a.counters + rg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

int launch_quantize_q8(const float* x, int64_t T, int64_t k, int64_t ldx, int8_t* q, uint16_t* d,
                       hipStream_t s) {
  const int64_t n8 = T * (k / 8);
  if (n8 == 0) return 0;
  hipLaunchKernelGGL(quantize_q8_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, T, k, ldx, q, d);
  return check_launch("quantize_q8_kernel");
}

template <int WQ, int TP>
static int launch_q8_t(const QmvArgs& a, int64_t grid) {
  hipLaunchKernelGGL((qmv_q8_kernel<WQ, TP>), dim3((unsigned)grid), dim3(64 * a.nwaves), 0, a.stream, a);
  return check_launch("qmv_q8_kernel");
}

template <int WQ>
static int launch_q8(const QmvArgs& a, int64_t grid) {
  switch (a.T) {
    case 1: return launch_q8_t<WQ, 1>(a, grid);
    case 2: return launch_q8_t<WQ, 2>(a, grid);
    case 3: return launch_q8_t<WQ, 3>(a, grid);
    case 4: return launch_q8_t<WQ, 4>(a, grid);
    default: return launch_q8_t<WQ, kQ8Rows>(a, grid);
  }
}

int launch_qmv_q8(const uint8_t* packed, int64_t n, int64_t k, const int8_t* q, const uint16_t* d, int T,
                  float* y, int64_t ldy, void* workspace, hipStream_t s) {
  QmvArgs a{};
  a.W0 = packed;
  a.xq = q;
  a.xd = d;
  a.ldx = k;
  a.T = T;
  a.y = y;
  a.ldy = ldy;
  a.stream = s;
  qmv_plan(a, n, k, kDenseRG);
  if (a.S > 1) {
    a.counters = static_cast<int*>(workspace);
    a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ws_partials_off(a));
  }
  const int64_t grid = a.rg_n * a.S;
  if (grid == 0) return 0;
  switch (a.wave_quads) {
    case 1: return launch_q8<1>(a, grid);
    case 2: return launch_q8<2>(a, grid);
    case 3: return launch_q8<3>(a, grid);
    default: return launch_q8<kMaxWaveQuads>(a, grid);
  }
}

}  // namespace iq4
