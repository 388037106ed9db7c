// api.hip -- the extern "C" entry points declared in include/iq4.h: argument
// validation on the host, then the launchers.  Nothing here allocates device memory
// or synchronises a stream.
#include <stdarg.h>
#include <stdio.h>

#include "iq4.h"
#include "common.hpp"
#include "launch.hpp"
#include "qmv.hpp"
#include "gemm.hpp"
#include "moe.hpp"

namespace iq4 {

static thread_local char g_err[512];

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(IQ4_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return IQ4_OK;
}

static inline void clear_error() { g_err[0] = '\0'; }
static inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace iq4

using namespace iq4;

extern "C" {

const char* iq4_last_error(void) { return g_err; }

int iq4_abi_version(void) { return IQ4_ABI_VERSION; }

int iq4_quantize_blocks(const float* src, int64_t n_blocks, void* blocks, void* stream) {
  clear_error();
  if (n_blocks < 0) return set_error(IQ4_E_ARG, "iq4_quantize_blocks: n_blocks < 0");
  if (n_blocks == 0) return IQ4_OK;
  if (!src || !blocks) return set_error(IQ4_E_ARG, "iq4_quantize_blocks: null pointer");
  if (!aligned(src, 16) || !aligned(blocks, 2))
    return set_error(IQ4_E_ALIGN, "iq4_quantize_blocks: src must be 16-byte and blocks 2-byte aligned");
  return launch_quantize(src, n_blocks, blocks, as_stream(stream));
}

int iq4_dequant_blocks(const void* blocks, int64_t n_blocks, int32_t out_dtype, void* out,
                       void* stream) {
  clear_error();
  if (n_blocks < 0) return set_error(IQ4_E_ARG, "iq4_dequant_blocks: n_blocks < 0");
  if (out_dtype != IQ4_F32 && out_dtype != IQ4_F16)
    return set_error(IQ4_E_ARG, "iq4_dequant_blocks: out_dtype must be IQ4_F32 or IQ4_F16");
  if (n_blocks == 0) return IQ4_OK;
  if (!blocks || !out) return set_error(IQ4_E_ARG, "iq4_dequant_blocks: null pointer");
  if (!aligned(blocks, 2) || !aligned(out, 16))
    return set_error(IQ4_E_ALIGN, "iq4_dequant_blocks: blocks must be 2-byte and out 16-byte aligned");
  return launch_dequant(blocks, n_blocks, out_dtype == IQ4_F16, out, as_stream(stream));
}

int64_t iq4_packed_bytes(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || n % kTileRows || k % kTileK) return -1;
  return n * (k / kQK) * kBlockBytes;
}

static int check_matrix(const char* fn, int64_t n, int64_t k) {
  if (n <= 0 || k <= 0) return set_error(IQ4_E_ARG, "%s: n and k must be positive", fn);
  if (n % kTileRows || k % kTileK)
    return set_error(IQ4_E_UNSUPPORTED, "%s: n must be a multiple of 16 and k of 128 (n=%lld k=%lld)",
                     fn, (long long)n, (long long)k);
  if (n > (int64_t)1 << 24 || k > (int64_t)1 << 20)
    return set_error(IQ4_E_UNSUPPORTED, "%s: n or k too large", fn);
  return IQ4_OK;
}

int iq4_pack_weights(const void* blocks, int64_t n, int64_t k, void* packed, void* stream) {
  clear_error();
  if (int e = check_matrix("iq4_pack_weights", n, k)) return e;
  if (!blocks || !packed) return set_error(IQ4_E_ARG, "iq4_pack_weights: null pointer");
  if (!aligned(blocks, 2) || !aligned(packed, 256))
    return set_error(IQ4_E_ALIGN, "iq4_pack_weights: blocks must be 2-byte and packed 256-byte aligned");
  const uint8_t* b = static_cast<const uint8_t*>(blocks);
  const uint8_t* p = static_cast<const uint8_t*>(packed);
  const int64_t bytes = iq4_packed_bytes(n, k);
  if (b < p + bytes && p < b + bytes)
    return set_error(IQ4_E_ARG, "iq4_pack_weights: blocks and packed overlap");
  return launch_pack(blocks, n, k, packed, as_stream(stream));
}

int iq4_qmv_workspace_size(int64_t n, int64_t k, size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(IQ4_E_ARG, "iq4_qmv_workspace_size: null bytes");
  *bytes = 0;
  if (int e = check_matrix("iq4_qmv_workspace_size", n, k)) return e;
  *bytes = (size_t)qmv_workspace_bytes(n, k);
  return IQ4_OK;
}

static int check_qmv(const char* fn, const void* packed, int64_t n, int64_t k, const float* x, int64_t ldx,
                     int32_t T, const float* y, int64_t ldy) {
  if (int e = check_matrix(fn, n, k)) return e;
  if (T < 1 || T > 8) return set_error(IQ4_E_ARG, "%s: T must be in 1..8 (got %d)", fn, T);
  if (ldx < k || ldx % 4) return set_error(IQ4_E_ARG, "%s: ldx must be >= k and a multiple of 4", fn);
  if (ldy < n) return set_error(IQ4_E_ARG, "%s: ldy must be >= n", fn);
  if (!packed || !x || !y) return set_error(IQ4_E_ARG, "%s: null pointer", fn);
  if (!aligned(packed, 256) || !aligned(x, 16) || !aligned(y, 4))
    return set_error(IQ4_E_ALIGN, "%s: packed must be 256-byte, x 16-byte, y 4-byte aligned", fn);
  return IQ4_OK;
}

int iq4_qmv_multi(const void* packed, int64_t n, int64_t k, const float* x, int64_t ldx,
                  int32_t T, float* y, int64_t ldy, void* workspace, size_t ws_bytes,
                  void* stream) {
  clear_error();
  if (int e = check_qmv("iq4_qmv_multi", packed, n, k, x, ldx, T, y, ldy)) return e;
  const int64_t need = qmv_workspace_bytes(n, k);
  if (need > 0) {
    if (!workspace || ws_bytes < (size_t)need)
      return set_error(IQ4_E_WORKSPACE, "iq4_qmv_multi: needs a workspace of %lld bytes", (long long)need);
    if (!aligned(workspace, 256)) return set_error(IQ4_E_ALIGN, "iq4_qmv_multi: workspace must be 256-byte aligned");
  }
  return launch_qmv(static_cast<const uint8_t*>(packed), n, k, x, ldx, T, y, ldy, workspace,
                    as_stream(stream));
}

int iq4_qmv_multi_noalloc(const void* packed, int64_t n, int64_t k, const float* x, int64_t ldx,
                          int32_t T, float* y, int64_t ldy, void* stream) {
  clear_error();
  if (int e = check_qmv("iq4_qmv_multi_noalloc", packed, n, k, x, ldx, T, y, ldy)) return e;
  return launch_qmv_noalloc(static_cast<const uint8_t*>(packed), n, k, x, ldx, T, y, ldy, as_stream(stream));
}

int iq4_quantize_q8_1(const float* x, int64_t T, int64_t k, int64_t ldx, int8_t* q, uint16_t* d,
                      void* stream) {
  clear_error();
  if (T < 0 || k <= 0 || k % kQK || k > (int64_t)1 << 24)
    return set_error(IQ4_E_ARG, "iq4_quantize_q8_1: need T >= 0 and 0 < k <= 2^24, k %% 32 == 0");
  if (ldx < k || ldx % 4) return set_error(IQ4_E_ARG, "iq4_quantize_q8_1: ldx must be >= k and a multiple of 4");
  if (T == 0) return IQ4_OK;
  if (!x || !q || !d) return set_error(IQ4_E_ARG, "iq4_quantize_q8_1: null pointer");
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(d, 2))
    return set_error(IQ4_E_ALIGN, "iq4_quantize_q8_1: x must be 16-byte, q 8-byte, d 2-byte aligned");
  return launch_quantize_q8(x, T, k, ldx, q, d, as_stream(stream));
}

int iq4_qmv_q8(const void* packed, int64_t n, int64_t k, const int8_t* q, const uint16_t* d, int32_t T,
               float* y, int64_t ldy, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (int e = check_matrix("iq4_qmv_q8", n, k)) return e;
  if (T < 1 || T > 8) return set_error(IQ4_E_ARG, "iq4_qmv_q8: T must be in 1..8 (got %d)", T);
  if (ldy < n) return set_error(IQ4_E_ARG, "iq4_qmv_q8: ldy must be >= n");
  if (!packed || !q || !d || !y) return set_error(IQ4_E_ARG, "iq4_qmv_q8: null pointer");
  if (!aligned(packed, 256) || !aligned(q, 8) || !aligned(d, 2) || !aligned(y, 4))
    return set_error(IQ4_E_ALIGN, "iq4_qmv_q8: packed must be 256-byte, q 8-byte, d 2-byte, y 4-byte aligned");
  const int64_t need = qmv_workspace_bytes(n, k);
  if (need > 0) {
    if (!workspace || ws_bytes < (size_t)need)
      return set_error(IQ4_E_WORKSPACE, "iq4_qmv_q8: needs a workspace of %lld bytes", (long long)need);
    if (!aligned(workspace, 256)) return set_error(IQ4_E_ALIGN, "iq4_qmv_q8: workspace must be 256-byte aligned");
  }
  return launch_qmv_q8(static_cast<const uint8_t*>(packed), n, k, q, d, T, y, ldy, workspace, as_stream(stream));
}

int iq4_route_topk(const float* logits, int64_t n_tok, int32_t n_expert, int32_t top_k,
                   int32_t* ids, float* w, void* stream) {
  clear_error();
  if (n_tok < 0 || n_expert < 1 || n_expert > 1024 || top_k < 1 || top_k > 16 || top_k > n_expert)
    return set_error(IQ4_E_ARG, "iq4_route_topk: need n_tok >= 0, 1 <= top_k <= min(n_expert, 16), n_expert <= 1024");
  if (n_tok == 0) return IQ4_OK;
  if (!logits || !ids || !w) return set_error(IQ4_E_ARG, "iq4_route_topk: null pointer");
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(w, 4))
    return set_error(IQ4_E_ALIGN, "iq4_route_topk: pointers must be 4-byte aligned");
  return launch_route_topk(logits, n_tok, n_expert, top_k, ids, w, as_stream(stream));
}

int iq4_moe_gather(const int32_t* ids, int64_t n_pairs, int32_t n_expert, int32_t* counts,
                   int32_t* offsets, int32_t* pairs, int32_t* slot_row, void* stream) {
  clear_error();
  if (n_pairs < 0 || n_pairs > ((int64_t)1 << 24) || n_expert < 1 || n_expert > 1024)
    return set_error(IQ4_E_ARG, "iq4_moe_gather: need 0 <= n_pairs <= 2^24, 1 <= n_expert <= 1024");
  if (!counts || !offsets || (n_pairs > 0 && (!ids || !pairs || !slot_row)))
    return set_error(IQ4_E_ARG, "iq4_moe_gather: null pointer");
  if (!aligned(ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(pairs, 4) ||
      !aligned(slot_row, 4))
    return set_error(IQ4_E_ALIGN, "iq4_moe_gather: pointers must be 4-byte aligned");
  return launch_gather(ids, n_pairs, n_expert, counts, offsets, pairs, slot_row, nullptr, nullptr,
                       as_stream(stream));
}

static int check_moe_sizes(const char* fn, int64_t n_tok, int32_t top_k, int32_t n_expert,
                           int64_t hidden, int64_t inter, int32_t act_dtype) {
  if (n_tok < 0 || n_tok > ((int64_t)1 << 24) / (top_k > 0 ? top_k : 1))
    return set_error(IQ4_E_ARG, "%s: n_tok out of range", fn);
  if (n_expert < 1 || n_expert > 1024 || top_k < 1 || top_k > 16 || top_k > n_expert)
    return set_error(IQ4_E_ARG, "%s: need 1 <= top_k <= min(n_expert, 16), n_expert <= 1024", fn);
  if (act_dtype != IQ4_F32 && act_dtype != IQ4_F16)
    return set_error(IQ4_E_ARG, "%s: act_dtype must be IQ4_F32 or IQ4_F16", fn);
  if (hidden <= 0 || inter <= 0 || hidden % kTileK || inter % kTileK)
    return set_error(IQ4_E_UNSUPPORTED, "%s: hidden and inter must be positive multiples of 128", fn);
  if (act_dtype == IQ4_F32 && (hidden > 4096 || inter > 4096))
    return set_error(IQ4_E_UNSUPPORTED, "%s: the fp32 path supports hidden, inter <= 4096", fn);
  if (hidden > ((int64_t)1 << 16) || inter > ((int64_t)1 << 16))
    return set_error(IQ4_E_UNSUPPORTED, "%s: hidden or inter too large", fn);
  return IQ4_OK;
}

int iq4_moe_workspace_size(int64_t n_tok, int32_t top_k, int32_t n_expert, int64_t hidden,
                           int64_t inter, int32_t act_dtype, size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(IQ4_E_ARG, "iq4_moe_workspace_size: null bytes");
  *bytes = 0;
  if (int e = check_moe_sizes("iq4_moe_workspace_size", n_tok, top_k, n_expert, hidden, inter, act_dtype))
    return e;
  *bytes = (size_t)moe_layout(n_tok, top_k, n_expert, hidden, inter, act_dtype == IQ4_F16).total;
  return IQ4_OK;
}

// The shared-expert call is validated as the routed call with one more expert and slot.
int iq4_moe_shared_workspace_size(int64_t n_tok, int32_t top_k, int32_t n_expert, int64_t hidden,
                                  int64_t inter, int32_t act_dtype, size_t* bytes) {
  clear_error();
  if (!bytes) return set_error(IQ4_E_ARG, "iq4_moe_shared_workspace_size: null bytes");
  *bytes = 0;
  if (top_k < 1 || n_expert < 1) return set_error(IQ4_E_ARG, "iq4_moe_shared_workspace_size: need top_k, n_expert >= 1");
  if (int e = check_moe_sizes("iq4_moe_shared_workspace_size", n_tok, top_k + 1, n_expert + 1, hidden, inter, act_dtype))
    return e;
  *bytes = (size_t)moe_layout(n_tok, top_k, n_expert, hidden, inter, act_dtype == IQ4_F16, true).total;
  return IQ4_OK;
}

static int moe_call(const char* fn, const void* x, int32_t act_dtype, int64_t n_tok, int64_t ldx,
                    const int32_t* ids, const float* w, int32_t top_k, int32_t n_expert, int64_t hidden,
                    int64_t inter, const void* w_gate, const void* w_up, const void* w_down,
                    const void* s_gate, const void* s_up, const void* s_down, float* out, int64_t ldo,
                    void* workspace, size_t ws_bytes, uint32_t flags, void* stream) {
  const bool shared = s_gate || s_up || s_down;
  if (shared && (top_k < 1 || n_expert < 1)) return set_error(IQ4_E_ARG, "%s: need top_k, n_expert >= 1", fn);
  const int sk = shared ? 1 : 0;  // the shared expert counts as one more expert and slot
  if (int e = check_moe_sizes(fn, n_tok, top_k + sk, n_expert + sk, hidden, inter, act_dtype)) return e;
  if (flags & ~(IQ4_MOE_ATOMIC_COMBINE | IQ4_MOE_KEEP_INTERMEDIATE))
    return set_error(IQ4_E_ARG, "%s: unknown flags", fn);
  const bool keep = (flags & IQ4_MOE_KEEP_INTERMEDIATE) != 0;
  if (ldx < hidden || ldo < hidden) return set_error(IQ4_E_ARG, "%s: ldx and ldo must be >= hidden", fn);
  if (n_tok == 0) return IQ4_OK;
  if (!x || !ids || !w || !w_gate || !w_up || !w_down || !out || (shared && !(s_gate && s_up && s_down)))
    return set_error(IQ4_E_ARG, "%s: null pointer", fn);
  const bool f16 = act_dtype == IQ4_F16;
  if (!aligned(x, 16) || ldx % (f16 ? 8 : 4) || !aligned(out, 16) || ldo % 4 || !aligned(ids, 4) ||
      !aligned(w, 4) || !aligned(w_gate, 256) || !aligned(w_up, 256) || !aligned(w_down, 256) ||
      (shared && (!aligned(s_gate, 256) || !aligned(s_up, 256) || !aligned(s_down, 256))))
    return set_error(IQ4_E_ALIGN, "%s: x/out 16-byte aligned with ldx %% %d == 0 and ldo %% 4 == 0, "
                     "weights 256-byte aligned", fn, f16 ? 8 : 4);
  if (n_tok * ldx >= ((int64_t)1 << 31) || n_tok * (top_k + sk) * inter >= ((int64_t)1 << 31))
    return set_error(IQ4_E_UNSUPPORTED, "%s: x and the intermediate rows must span fewer than 2^31 elements", fn);
  const MoeLayout L = moe_layout(n_tok, top_k, n_expert, hidden, inter, f16, shared, keep);
  if (!workspace || ws_bytes < (size_t)L.total)
    return set_error(IQ4_E_WORKSPACE, "%s: needs a workspace of %lld bytes", fn, (long long)L.total);
  if (!aligned(workspace, 256)) return set_error(IQ4_E_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  MoeCall m{};
  m.x = x;
  m.f16 = f16;
  m.n_tok = n_tok;
  m.ldx = ldx;
  m.ids = ids;
  m.w = w;
  m.top_k = top_k;
  m.n_expert = n_expert;
  m.hidden = hidden;
  m.inter = inter;
  m.w_gate = w_gate;
  m.w_up = w_up;
  m.w_down = w_down;
  m.s_gate = shared ? s_gate : nullptr;
  m.s_up = shared ? s_up : nullptr;
  m.s_down = shared ? s_down : nullptr;
  m.out = out;
  m.ldo = ldo;
  m.workspace = workspace;
  m.atomic = (flags & IQ4_MOE_ATOMIC_COMBINE) != 0;
  m.keep = keep;
  return launch_moe(m, as_stream(stream));
}

int iq4_moe_intermediate_layout(int64_t n_tok, int32_t top_k, int32_t n_expert, int64_t hidden,
                                int64_t inter, int32_t act_dtype, int32_t shared, int64_t* layout) {
  clear_error();
  if (!layout) return set_error(IQ4_E_ARG, "iq4_moe_intermediate_layout: null layout");
  const int sk = shared ? 1 : 0;
  if (int e = check_moe_sizes("iq4_moe_intermediate_layout", n_tok, top_k + sk, n_expert + sk, hidden, inter,
                              act_dtype))
    return e;
  const MoeLayout L = moe_layout(n_tok, top_k, n_expert, hidden, inter, act_dtype == IQ4_F16, shared != 0, true);
  layout[IQ4_MOE_LAYOUT_TOTAL] = L.total;
  layout[IQ4_MOE_LAYOUT_COUNTS] = L.counts;
  layout[IQ4_MOE_LAYOUT_OFFSETS] = L.offsets;
  layout[IQ4_MOE_LAYOUT_PAIRS] = L.pairs;
  layout[IQ4_MOE_LAYOUT_SLOT_ROW] = L.slot_row;
  layout[IQ4_MOE_LAYOUT_H] = L.h;
  layout[IQ4_MOE_LAYOUT_ROWS] = L.rows;
  layout[IQ4_MOE_LAYOUT_G] = L.g;
  layout[IQ4_MOE_LAYOUT_U] = L.u;
  return IQ4_OK;
}

int iq4_moe_expert_gemm(const void* x, int32_t act_dtype, int64_t n_tok, int64_t ldx,
                        const int32_t* ids, const float* w, int32_t top_k, int32_t n_expert,
                        int64_t hidden, int64_t inter, const void* w_gate, const void* w_up,
                        const void* w_down, float* out, int64_t ldo, void* workspace,
                        size_t ws_bytes, uint32_t flags, void* stream) {
  clear_error();
  return moe_call("iq4_moe_expert_gemm", x, act_dtype, n_tok, ldx, ids, w, top_k, n_expert, hidden, inter,
                  w_gate, w_up, w_down, nullptr, nullptr, nullptr, out, ldo, workspace, ws_bytes, flags, stream);
}

int iq4_moe_expert_gemm_shared(const void* x, int32_t act_dtype, int64_t n_tok, int64_t ldx,
                               const int32_t* ids, const float* w, int32_t top_k, int32_t n_expert,
                               int64_t hidden, int64_t inter, const void* w_gate, const void* w_up,
                               const void* w_down, const void* s_gate, const void* s_up,
                               const void* s_down, float* out, int64_t ldo, void* workspace,
                               size_t ws_bytes, uint32_t flags, void* stream) {
  clear_error();
  if (!s_gate || !s_up || !s_down) return set_error(IQ4_E_ARG, "iq4_moe_expert_gemm_shared: null shared expert");
  return moe_call("iq4_moe_expert_gemm_shared", x, act_dtype, n_tok, ldx, ids, w, top_k, n_expert, hidden,
                  inter, w_gate, w_up, w_down, s_gate, s_up, s_down, out, ldo, workspace, ws_bytes, flags,
                  stream);
}

int iq4_qgemm(const void* packed, int64_t n, int64_t k, const void* x, int64_t m, int64_t ldx,
              float* y, int64_t ldy, int64_t chunk, void* stream) {
  clear_error();
  if (int e = check_matrix("iq4_qgemm", n, k)) return e;
  if (m < 0 || chunk < 0) return set_error(IQ4_E_ARG, "iq4_qgemm: m and chunk must be >= 0");
  if (ldx < k || ldy < n) return set_error(IQ4_E_ARG, "iq4_qgemm: ldx must be >= k and ldy >= n");
  if (m == 0) return IQ4_OK;
  if (!packed || !x || !y) return set_error(IQ4_E_ARG, "iq4_qgemm: null pointer");
  if (!aligned(packed, 256) || !aligned(x, 16) || ldx % 8 || !aligned(y, 4))
    return set_error(IQ4_E_ALIGN, "iq4_qgemm: packed 256-byte, x 16-byte aligned with ldx %% 8 == 0, y 4-byte");
  if ((chunk > 0 ? (chunk < m ? chunk : m) : m) * ldx >= ((int64_t)1 << 31))
    return set_error(IQ4_E_UNSUPPORTED, "iq4_qgemm: a chunk of x must span fewer than 2^31 elements");
  return launch_qgemm_dense(static_cast<const uint8_t*>(packed), n, k, static_cast<const uint16_t*>(x), m,
                            ldx, y, ldy, chunk, as_stream(stream));
}

// ---- IQ4_XS super-blocks ----------------------------------------------------------

int64_t iq4_xs_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < 1 || k % 256) return -1;
  return n * (k / 256) * 136;
}

int iq4_xs_dequant(const void* sb, int64_t n_superblocks, int32_t out_dtype, void* out, void* stream) {
  clear_error();
  if (n_superblocks < 0) return set_error(IQ4_E_ARG, "iq4_xs_dequant: n_superblocks < 0");
  if (out_dtype != IQ4_F32 && out_dtype != IQ4_F16)
    return set_error(IQ4_E_ARG, "iq4_xs_dequant: out_dtype must be IQ4_F32 or IQ4_F16");
  if (n_superblocks == 0) return IQ4_OK;
  if (!sb || !out) return set_error(IQ4_E_ARG, "iq4_xs_dequant: null pointer");
  if (n_superblocks > ((int64_t)1 << 40))
    return set_error(IQ4_E_UNSUPPORTED, "iq4_xs_dequant: n_superblocks too large");
  if (!aligned(sb, 8) || !aligned(out, 16))
    return set_error(IQ4_E_ALIGN, "iq4_xs_dequant: sb must be 8-byte and out 16-byte aligned");
  return launch_xs_dequant(sb, n_superblocks, out_dtype == IQ4_F16, out, as_stream(stream));
}

int iq4_xs_qmv_multi(const void* w, int64_t n, int64_t k, const float* x, int64_t ldx, int32_t T,
                     float* y, int64_t ldy, void* stream) {
  clear_error();
  if (n < 1 || k < 1) return set_error(IQ4_E_ARG, "iq4_xs_qmv_multi: n and k must be positive");
  if (k % 256 || k > ((int64_t)1 << 20) || n > ((int64_t)1 << 31))
    return set_error(IQ4_E_UNSUPPORTED, "iq4_xs_qmv_multi: k must be a multiple of 256, k <= 2^20, n <= 2^31 "
                     "(n=%lld k=%lld)", (long long)n, (long long)k);
  if (T < 1 || T > 8) return set_error(IQ4_E_ARG, "iq4_xs_qmv_multi: T must be 1..8 (T=%d)", T);
  if (!w || !x || !y) return set_error(IQ4_E_ARG, "iq4_xs_qmv_multi: null pointer");
  if (ldx < k || ldy < n) return set_error(IQ4_E_ARG, "iq4_xs_qmv_multi: ldx < k or ldy < n");
  if (!aligned(w, 8) || !aligned(x, 16) || ldx % 4 || !aligned(y, 4))
    return set_error(IQ4_E_ALIGN, "iq4_xs_qmv_multi: w must be 8-byte, x 16-byte (ldx % 4 == 0) and y 4-byte "
                     "aligned");
  return launch_xs_qmv(w, n, k, x, ldx, T, y, ldy, as_stream(stream));
}

}  // extern "C"
