// moe.hpp -- workspace layout and arguments of one MoE layer call (moe.hip).
#pragma once
#include "common.hpp"

namespace iq4 {

struct MoeLayout {  // byte offsets into the caller's workspace
  int64_t counts, offsets, pairs, slot_row, num_tiles, tiles, h, rows, total;
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
  float* out;
  int64_t ldo;
  void* workspace;
  bool atomic;
};

MoeLayout moe_layout(int64_t n_tok, int top_k, int n_expert, int64_t hidden, int64_t inter, bool f16);
int launch_moe(const MoeCall& m, hipStream_t s);

}  // namespace iq4
