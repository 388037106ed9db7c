// launch.hpp -- host launchers of the HIP kernels (called by the C ABI in api.hip
// after argument validation).  Each returns 0 or a negative IQ4_E_* status.
#pragma once
#include "common.hpp"

namespace iq4 {

int launch_quantize(const float* src, int64_t nb, void* blocks, hipStream_t s);
int launch_dequant(const void* blocks, int64_t nb, bool f16, void* out, hipStream_t s);
int launch_pack(const void* blocks, int64_t n, int64_t k, void* packed, hipStream_t s);

int launch_qmv(const uint8_t* packed, int64_t n, int64_t k, const float* x, int64_t ldx, int T,
               float* y, int64_t ldy, void* workspace, hipStream_t s);
// as launch_qmv, the split-K scratch from the library's own device array (no workspace)
int launch_qmv_noalloc(const uint8_t* packed, int64_t n, int64_t k, const float* x, int64_t ldx, int T,
                       float* y, int64_t ldy, hipStream_t s);

int launch_route_topk(const float* logits, int64_t n_tok, int n_expert, int top_k, int32_t* ids,
                      float* w, hipStream_t s);
// tiles / num_tiles: the grouped GEMM's tile list, built in the same launch (or null)
int launch_gather(const int32_t* ids, int64_t n_pairs, int n_expert, int32_t* counts,
                  int32_t* offsets, int32_t* pairs, int32_t* slot_row, int32_t* tiles,
                  int32_t* num_tiles, hipStream_t s);

// IQ4_XS super-blocks (xs.hip)
int launch_xs_dequant(const void* sb, int64_t nsb, bool f16, void* out, hipStream_t s);
int launch_xs_qmv(const void* w, int64_t n, int64_t k, const float* x, int64_t ldx, int T, float* y,
                  int64_t ldy, hipStream_t s);

}  // namespace iq4
