// gemm.hpp -- arguments of the dequant-fused GEMM kernel (gemm.hip).
#pragma once
#include "common.hpp"

namespace iq4 {

enum GemmMode { kGemmDense = 0, kGemmGateUp = 1, kGemmDown = 2 };

struct GemmArgs {
  const uint16_t* A;        // binary16 activations, rows of lda elements
  int64_t lda;
  const uint8_t* W0;        // packed weights (DENSE: W; GATEUP: gate bank; DOWN: down bank)
  const uint8_t* W1;        // GATEUP: up bank
  int64_t w_expert_stride;  // bytes between experts' packed matrices
  int shared_e;             // grouped, with S0 set: this expert index takes S0 / S1
  const uint8_t* S0;        // the shared expert's packed matrices (as W0 / W1), or null
  const uint8_t* S1;
  int64_t N, K;             // weight rows and reduction length of one matrix
  int64_t M;                // DENSE: rows of A in this launch
  float* C;                 // DENSE: output [M][ldc]
  int vec_c;                // DENSE: C and ldc allow 16-byte stores of 4 consecutive columns
  uint16_t* R;              // DOWN: per-pair rows w * (Wd h) as binary16 [pairs][ldc]
  int64_t ldc;
  uint16_t* H;              // GATEUP: h = silu(g) * u as binary16 [pairs][ldh] (sorted order)
  int64_t ldh;
  float* G;                 // GATEUP, or null: g and u themselves, fp32 [pairs][ldh] (sorted order)
  float* U;
  const int32_t* tiles;     // grouped: (expert, m tile) pairs
  const int32_t* num_tiles; // grouped: [0] valid entries in `tiles`, [1] of them full tiles (listed first)
  int64_t n_tiles_n;        // grouped: workgroups per m tile along N (set by the launcher)
  const int32_t* offsets;   // grouped: per-expert start in the sorted pair list [E+1]
  const int32_t* pairs;     // grouped: sorted pair ids
  const float* gate_w;      // DOWN: gate weight of each pair (indexed by pair id)
  int top_k;
  float* out;               // DOWN with atomic combine: [n_tok][ldo]
  int64_t ldo;
  int atomic;
};

int launch_qgemm_dense(const uint8_t* packed, int64_t n, int64_t k, const uint16_t* x, int64_t m,
                       int64_t ldx, float* y, int64_t ldy, int64_t chunk, hipStream_t s);
// Sets a.n_tiles_n (workgroups per m tile along N) itself.
int launch_qgemm_grouped(int mode, GemmArgs a, int64_t max_tiles, hipStream_t s);

}  // namespace iq4
