// moe.hip -- the mixture-of-experts path around the products: the gate-weighted
// combine and the orchestration of one MoE layer call.
//
// Prefill (binary16 activations):
//   gather (+ tile list) -> GEMM gate|up (+SwiGLU, h binary16) -> GEMM down (x gate
//   weight, slot rows binary16) -> combine (fp32 sums).
// Decode (fp32 activations, few tokens):
//   gather -> grouped matvec gate|up (+SwiGLU, h fp32) -> grouped matvec down (x gate
//   weight) -> combine; with at most 64 pairs there is no gather launch: each matvec
//   workgroup finds its expert and that expert's pairs from the ids, and the down
//   product and the combine run as one launch (one workgroup per output tile and token).
// The combine adds each token's top_k weighted slot rows in slot order j = 0..k-1, so
// the result does not depend on how pairs were scheduled (page 1's PoolMultiFn:
// per-slot rows (n_tok * k, n_embd), then summed per token).  The atomic variant adds
// the slot rows into the output as they are produced instead.
#include "common.hpp"
#include "gemm.hpp"
#include "launch.hpp"
#include "moe.hpp"
#include "qmv.hpp"

namespace iq4 {

constexpr int kTileM = 128;  // rows per GEMM tile (gemm.hip kBM)
constexpr int kMaxTopK = 16;  // the largest top_k the call accepts

// Four consecutive row elements: fp32 rows (decode) as they are, binary16 rows (prefill)
// widened to fp32 (exact).  Non-temporal: each row is read once.
__device__ __forceinline__ f32x4 load_row4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ f32x4 load_row4(const uint16_t* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return f32x4{h2f((uint16_t)(w.x & 0xFFFFu)), h2f((uint16_t)(w.x >> 16)), h2f((uint16_t)(w.y & 0xFFFFu)),
               h2f((uint16_t)(w.y >> 16))};
}

// out[t][h] = sum_j rows[t * K + j][h], j ascending, in fp32; one thread per 4 outputs,
// K = top_k fixed at compile time.  Every slot row is requested at once, then added in
// slot order.
template <int K, typename RowT>
__global__ void __launch_bounds__(256) combine_kernel(const RowT* __restrict__ rows, int64_t ldr,
                                                      int64_t n_tok, int64_t hidden,
                                                      float* __restrict__ out, int64_t ldo) {
  const int64_t per_tok = hidden / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_tok * per_tok) return;
  const int64_t t = i / per_tok, h = (i % per_tok) * 4;
  const RowT* r = rows + t * K * ldr + h;
  f32x4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = load_row4(r + j * ldr);
  f32x4 acc = v[0];
#pragma unroll
  for (int j = 1; j < K; ++j) {
    acc.x += v[j].x;
    acc.y += v[j].y;
    acc.z += v[j].z;
    acc.w += v[j].w;
  }
  *reinterpret_cast<f32x4*>(out + t * ldo + h) = acc;
}

template <int K, typename RowT>
static int launch_combine_k(const RowT* rows, int64_t n_tok, int64_t hidden, float* out, int64_t ldo,
                            hipStream_t s) {
  const int64_t n4 = n_tok * (hidden / 4);
  // a decode step's few outputs spread over more CUs (64-thread workgroups)
  const int64_t cb = n4 < 65536 ? 64 : 256;
  hipLaunchKernelGGL((combine_kernel<K, RowT>), dim3((unsigned)((n4 + cb - 1) / cb)), dim3((unsigned)cb), 0, s,
                     rows, hidden, n_tok, hidden, out, ldo);
  return check_launch("combine_kernel");
}

template <typename RowT>
static int launch_combine(const RowT* rows, int64_t n_tok, int top_k, int64_t hidden, float* out,
                          int64_t ldo, hipStream_t s) {
  switch (top_k) {
    case 1: return launch_combine_k<1>(rows, n_tok, hidden, out, ldo, s);
    case 2: return launch_combine_k<2>(rows, n_tok, hidden, out, ldo, s);
    case 3: return launch_combine_k<3>(rows, n_tok, hidden, out, ldo, s);
    case 4: return launch_combine_k<4>(rows, n_tok, hidden, out, ldo, s);
    case 5: return launch_combine_k<5>(rows, n_tok, hidden, out, ldo, s);
    case 6: return launch_combine_k<6>(rows, n_tok, hidden, out, ldo, s);
    case 7: return launch_combine_k<7>(rows, n_tok, hidden, out, ldo, s);
    case 8: return launch_combine_k<8>(rows, n_tok, hidden, out, ldo, s);
    case 9: return launch_combine_k<9>(rows, n_tok, hidden, out, ldo, s);
    case 10: return launch_combine_k<10>(rows, n_tok, hidden, out, ldo, s);
    case 11: return launch_combine_k<11>(rows, n_tok, hidden, out, ldo, s);
    case 12: return launch_combine_k<12>(rows, n_tok, hidden, out, ldo, s);
    case 13: return launch_combine_k<13>(rows, n_tok, hidden, out, ldo, s);
    case 14: return launch_combine_k<14>(rows, n_tok, hidden, out, ldo, s);
    case 15: return launch_combine_k<15>(rows, n_tok, hidden, out, ldo, s);
    case 16: return launch_combine_k<16>(rows, n_tok, hidden, out, ldo, s);
    default: return set_error(-1, "combine: top_k must be 1..%d", kMaxTopK);
  }
}

// Zero-fill (a kernel rather than a memset node, so the call stays graph-safe).
__global__ void __launch_bounds__(256) zero_rows_kernel(float* __restrict__ out, int64_t n_tok,
                                                        int64_t hidden, int64_t ldo) {
  const int64_t per_tok = hidden / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_tok * per_tok) return;
  const int64_t t = i / per_tok, h = (i % per_tok) * 4;
  *reinterpret_cast<float4*>(out + t * ldo + h) = make_float4(0.f, 0.f, 0.f, 0.f);
}

static inline int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

// Routing with the shared expert behind: slots 0..k-1 of every token are the routed ones,
// slot k is expert n_expert with gate weight 1, so the combine adds the routed rows in
// slot order and then the shared expert's row (routed sum + shared).
__global__ void __launch_bounds__(256) append_shared_kernel(const int32_t* __restrict__ ids,
                                                             const float* __restrict__ w, int64_t n_tok,
                                                             int top_k, int n_expert,
                                                             int32_t* __restrict__ ids2,
                                                             float* __restrict__ w2) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int k2 = top_k + 1;
  if (i >= n_tok * k2) return;
  const int64_t t = i / k2;
  const int j = (int)(i % k2);
  ids2[i] = (j == top_k) ? n_expert : ids[t * top_k + j];
  w2[i] = (j == top_k) ? 1.0f : w[t * top_k + j];
}

MoeLayout moe_layout(int64_t n_tok, int top_k, int n_expert, int64_t hidden, int64_t inter,
                     bool f16, bool shared, bool keep) {
  MoeLayout L{};
  if (shared) {  // the routed call's sizes with the shared expert as one more expert and slot
    ++top_k;
    ++n_expert;
  }
  const int64_t P = n_tok * top_k;
  int64_t off = 0;
  L.counts = off;    off += align256(4 * (int64_t)n_expert);
  L.offsets = off;   off += align256(4 * ((int64_t)n_expert + 1));
  L.pairs = off;     off += align256(4 * P);
  L.slot_row = off;  off += align256(4 * P);
  L.max_tiles = (P + kTileM - 1) / kTileM + n_expert;
  L.num_tiles = off; off += 256;
  L.tiles = off;     off += align256(8 * L.max_tiles);
  L.h = off;         off += align256(P * inter * (f16 ? 2 : 4));
  L.rows = off;      off += align256(P * hidden * (f16 ? 2 : 4));  // binary16 rows for the prefill
  L.ids2 = off;      off += shared ? align256(4 * P) : 0;
  L.w2 = off;        off += shared ? align256(4 * P) : 0;
  L.g = keep ? off : -1; off += keep ? align256(P * inter * 4) : 0;
  L.u = keep ? off : -1; off += keep ? align256(P * inter * 4) : 0;
  L.total = off;
  return L;
}

int launch_moe(const MoeCall& m, hipStream_t s) {
  const bool shared = m.s_gate != nullptr;
  const MoeLayout L = moe_layout(m.n_tok, m.top_k, m.n_expert, m.hidden, m.inter, m.f16, shared, m.keep);
  float* keep_g = m.keep ? reinterpret_cast<float*>(static_cast<uint8_t*>(m.workspace) + L.g) : nullptr;
  float* keep_u = m.keep ? reinterpret_cast<float*>(static_cast<uint8_t*>(m.workspace) + L.u) : nullptr;
  uint8_t* ws = static_cast<uint8_t*>(m.workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* pairs = reinterpret_cast<int32_t*>(ws + L.pairs);
  int32_t* slot_row = reinterpret_cast<int32_t*>(ws + L.slot_row);
  int32_t* num_tiles = reinterpret_cast<int32_t*>(ws + L.num_tiles);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  float* rows = reinterpret_cast<float*>(ws + L.rows);          // decode: fp32 rows
  uint16_t* rows16 = reinterpret_cast<uint16_t*>(ws + L.rows);  // prefill: binary16 rows
  if (m.n_tok == 0) return 0;
  // the routing the products see: with a shared expert, one more expert and slot
  const int32_t* ids = m.ids;
  const float* w = m.w;
  const int top_k = m.top_k + (shared ? 1 : 0);
  const int n_expert = m.n_expert + (shared ? 1 : 0);
  const int64_t P = m.n_tok * top_k;
  if (shared) {
    int32_t* ids2 = reinterpret_cast<int32_t*>(ws + L.ids2);
    float* w2 = reinterpret_cast<float*>(ws + L.w2);
    hipLaunchKernelGGL(append_shared_kernel, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, s, m.ids, m.w,
                       m.n_tok, m.top_k, m.n_expert, ids2, w2);
    if (int e = check_launch("append_shared_kernel")) return e;
    ids = ids2;
    w = w2;
  }

  // prefill: the gather also writes the grouped GEMM's tile list.  A decode step with
  // few pairs skips it: its matvecs find each expert's pairs from the ids (unless the
  // intermediates are kept: then the gather that indexes them always runs).
  const bool direct = !m.f16 && P <= kDirectMaxPairs && !m.keep;
  if (!direct) {
    if (int e = launch_gather(ids, P, n_expert, counts, offsets, pairs, slot_row, m.f16 ? tiles : nullptr,
                              m.f16 ? num_tiles : nullptr, s))
      return e;
  }

  const int64_t gate_stride = m.inter * (m.hidden / kQK) * kBlockBytes;
  const int64_t down_stride = m.hidden * (m.inter / kQK) * kBlockBytes;
  const bool atomic = m.f16 && m.atomic;
  if (atomic) {
    const int64_t n4 = m.n_tok * (m.hidden / 4);
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, m.out,
                       m.n_tok, m.hidden, m.ldo);
    if (int e = check_launch("zero_rows_kernel")) return e;
  }

  if (m.f16) {
    uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h);
    GemmArgs g{};
    g.A = static_cast<const uint16_t*>(m.x);
    g.lda = m.ldx;
    g.W0 = static_cast<const uint8_t*>(m.w_gate);
    g.W1 = static_cast<const uint8_t*>(m.w_up);
    g.w_expert_stride = gate_stride;
    g.shared_e = m.n_expert;
    g.S0 = static_cast<const uint8_t*>(m.s_gate);
    g.S1 = static_cast<const uint8_t*>(m.s_up);
    g.N = m.inter;
    g.K = m.hidden;
    g.H = h;
    g.ldh = m.inter;
    g.tiles = tiles;
    g.num_tiles = num_tiles;
    g.offsets = offsets;
    g.pairs = pairs;
    g.top_k = top_k;
    g.G = keep_g;
    g.U = keep_u;
    if (int e = launch_qgemm_grouped(kGemmGateUp, g, L.max_tiles, s)) return e;
    GemmArgs d{};
    d.A = h;
    d.lda = m.inter;
    d.W0 = static_cast<const uint8_t*>(m.w_down);
    d.w_expert_stride = down_stride;
    d.shared_e = m.n_expert;
    d.S0 = static_cast<const uint8_t*>(m.s_down);
    d.N = m.hidden;
    d.K = m.inter;
    d.R = rows16;
    d.ldc = m.hidden;
    d.tiles = tiles;
    d.num_tiles = num_tiles;
    d.offsets = offsets;
    d.pairs = pairs;
    d.gate_w = w;
    d.top_k = top_k;
    d.out = m.out;
    d.ldo = m.ldo;
    d.atomic = atomic ? 1 : 0;
    if (int e = launch_qgemm_grouped(kGemmDown, d, L.max_tiles, s)) return e;
  } else {
    float* h = reinterpret_cast<float*>(ws + L.h);
    QmvArgs g{};
    g.W0 = static_cast<const uint8_t*>(m.w_gate);
    g.W1 = static_cast<const uint8_t*>(m.w_up);
    g.w_expert_stride = gate_stride;
    g.shared_e = m.n_expert;
    g.S0 = static_cast<const uint8_t*>(m.s_gate);
    g.S1 = static_cast<const uint8_t*>(m.s_up);
    g.x = static_cast<const float*>(m.x);
    g.ldx = m.ldx;
    g.y = h;
    g.ldy = m.inter;
    g.offsets = offsets;
    g.pairs = pairs;
    g.ids = direct ? ids : nullptr;
    g.n_pairs = (int)P;
    g.top_k = top_k;
    g.G = keep_g;
    g.U = keep_u;
    g.stream = s;
    if (int e = launch_qmv_grouped(kQmvGateUp, g, m.inter, m.hidden, n_expert, P)) return e;
    QmvArgs d{};
    d.W0 = static_cast<const uint8_t*>(m.w_down);
    d.w_expert_stride = down_stride;
    d.shared_e = m.n_expert;
    d.S0 = static_cast<const uint8_t*>(m.s_down);
    d.x = h;
    d.ldx = m.inter;
    d.y = rows;
    d.ldy = m.hidden;
    d.offsets = offsets;
    d.pairs = pairs;
    d.ids = direct ? ids : nullptr;
    d.n_pairs = (int)P;
    d.gate_w = w;
    d.top_k = top_k;
    d.stream = s;
    if (direct && qmv_down_combine_fits(m.inter, top_k, P)) {
      // down product and ordered combine in one launch, straight into the output
      d.y = m.out;
      d.ldy = m.ldo;
      return launch_qmv_down_combine(d, m.hidden, m.inter, n_expert, m.n_tok);
    }
    if (int e = launch_qmv_grouped(kQmvDown, d, m.hidden, m.inter, n_expert, P)) return e;
  }

  if (!atomic) {
    if (int e = m.f16 ? launch_combine(rows16, m.n_tok, top_k, m.hidden, m.out, m.ldo, s)
                      : launch_combine(rows, m.n_tok, top_k, m.hidden, m.out, m.ldo, s))
      return e;
  }
  return 0;
}

}  // namespace iq4
