// qmv.hpp -- arguments of the T-column matvec kernel (qmv.hip).
#pragma once
#include "common.hpp"

namespace iq4 {

enum QmvMode { kQmvDense = 0, kQmvGateUp = 1, kQmvDown = 2 };

struct QmvArgs {
  const uint8_t* W0;        // packed weights (DENSE: W; GATEUP: gate bank; DOWN: down bank)
  const uint8_t* W1;        // GATEUP: up bank
  int64_t w_expert_stride;  // bytes between experts' packed matrices
  int shared_e;             // grouped, with S0 set: this expert index takes S0 / S1
  const uint8_t* S0;        // the shared expert's packed matrices (as W0 / W1), or null
  const uint8_t* S1;
  const float* x;           // DENSE: X [T][ldx]; GATEUP: X [n_tok][ldx]; DOWN: h [pairs][ldx]
  const int8_t* xq;         // 8-bit activations: codes [T][K] (ldx = K)
  const uint16_t* xd;       // 8-bit activations: binary16 block scales [T][K/32]
  int64_t ldx;
  int T;                    // DENSE: columns
  float* y;                 // DENSE: Y [T][ldy]; GATEUP: h [pairs][ldy]; DOWN: rows [pairs][ldy]
  int64_t ldy;
  const int32_t* offsets;   // grouped: per-expert start in the sorted pair list [E+1]
  const int32_t* pairs;     // grouped: sorted pair ids
  const int32_t* ids;       // grouped, at most 64 pairs: routed expert per pair id; when
                            // set, each workgroup finds its expert's pairs from these
                            // (offsets and pairs unused: no gather launch)
  int n_pairs;              // grouped: routed pairs (with ids)
  const float* gate_w;      // DOWN: gate weight per pair id
  float* G;                 // GATEUP, or null: g and u themselves, [pairs][ldy] (sorted order)
  float* U;
  int top_k;
  int n_expert;             // grouped: experts in the bank
  float* partials;          // DENSE split K: per-slice partial sums (workspace)
  int* counters;            // DENSE split K: arrival counters per row group (workspace)
  // launch plan (qmv_plan)
  int64_t n, nt, rg_n, nibble_bytes;
  int kq_n, S, slice_quads, wave_quads, nwaves;
  int rg_per_wg;            // grouped: row groups walked by one workgroup
  int64_t rg_chunks;        // grouped: workgroups per expert slot
  hipStream_t stream;
};

// Grouped matvecs find their experts' pairs from the routed ids themselves (no gather
// launch) for at most this many pairs: one id per lane of a wave.
constexpr int kDirectMaxPairs = 64;

int64_t qmv_workspace_bytes(int64_t n, int64_t k);
int launch_quantize_q8(const float* x, int64_t T, int64_t k, int64_t ldx, int8_t* q, uint16_t* d,
                       hipStream_t s);
int launch_qmv_q8(const uint8_t* packed, int64_t n, int64_t k, const int8_t* q, const uint16_t* d, int T,
                  float* y, int64_t ldy, void* workspace, hipStream_t s);
int launch_qmv_grouped(int mode, QmvArgs a, int64_t n, int64_t k, int n_expert, int64_t n_pairs);
// The decode call's down product and ordered combine in one launch (ids given, at most
// kDirectMaxPairs pairs, K at most 896): a.y = the output [n_tok][ldy], a.top_k = pairs
// per token.
bool qmv_down_combine_fits(int64_t k, int top_k, int64_t n_pairs);
int launch_qmv_down_combine(QmvArgs a, int64_t n, int64_t k, int n_expert, int64_t n_tok);

}  // namespace iq4
