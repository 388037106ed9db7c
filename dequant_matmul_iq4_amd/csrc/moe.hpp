// moe.hpp -- workspace layout and arguments of one MoE layer call (moe.hip).
#pragma once
#include "common.hpp"

namespace iq4 {

struct MoeLayout {  // byte offsets into the caller's workspace
  int64_t counts, offsets, pairs, slot_row, num_tiles, tiles, h, rows, ids2, w2;
  int64_t g, u;  // with keep: fp32 gate and up products [pairs][inter], pair-sorted (else -1)
  int64_t total;
  int64_t max_tiles;
};

struct MoeCall {
  const void* x;
  bool f16;
  int64_t n_tok, ldx;
  const int32_t* ids;
  const float* w;
  int top_k, n_expert;
  int64_t hidden, inter;
  const void *w_gate, *w_up, *w_down;
  const void *s_gate, *s_up, *s_down;  // shared expert (gate/up inter x hidden, down
                                       // hidden x inter), or null
  float* out;
  int64_t ldo;
  void* workspace;
  bool atomic;
  bool keep;  // also write the gate and up products (and always run the gather)
};

// shared: the call adds a shared expert (routed as expert n_expert, slot top_k, weight 1)
// keep: the layout of a call with the intermediate products kept (g and u regions after
// everything else)
MoeLayout moe_layout(int64_t n_tok, int top_k, int n_expert, int64_t hidden, int64_t inter, bool f16,
                     bool shared = false, bool keep = false);
int launch_moe(const MoeCall& m, hipStream_t s);

}  // namespace iq4
