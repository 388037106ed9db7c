// route.hip -- top-k routing from logits, and the bit-exact token gather of the
// routed pairs (counts, exclusive offsets, pair list grouped by expert, inverse).
#include <climits>

#include "common.hpp"
#include "launch.hpp"

namespace iq4 {

constexpr int kMaxTopK = 16;

// One thread per token: a running top-k by insertion over experts in ascending id
// order.  A logit displaces a kept one only if strictly larger, so equal logits keep
// the lower expert id first.  Gate weights: softmax over the k kept logits in fp32.
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits,
                                                         int64_t n_tok, int n_expert, int top_k,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_tok) return;
  const float* row = logits + t * n_expert;
  float val[kMaxTopK];
  int id[kMaxTopK];
  int kept = 0;
  for (int e = 0; e < n_expert; ++e) {
    const float v = row[e];
    if (kept == top_k && !(v > val[top_k - 1])) continue;
    int pos = kept < top_k ? kept : top_k - 1;
    while (pos > 0 && v > val[pos - 1]) {
      val[pos] = val[pos - 1];
      id[pos] = id[pos - 1];
      --pos;
    }
    val[pos] = v;
    id[pos] = e;
    if (kept < top_k) ++kept;
  }
  const float m = val[0];
  float ex[kMaxTopK];
  float sum = 0.0f;
  for (int j = 0; j < top_k; ++j) {
    ex[j] = expf(val[j] - m);
    sum += ex[j];
  }
  for (int j = 0; j < top_k; ++j) {
    ids[t * top_k + j] = id[j];
    w[t * top_k + j] = ex[j] / sum;
  }
}

// One workgroup per expert e.  Its waves own contiguous segments of the pair list.
// Pass 1 counts, per wave, the pairs routed to e and to experts below e (so the
// workgroup knows offsets[e] without a global scan); pass 2 walks each segment in
// order, ranking matches with a ballot, so pairs of one expert keep ascending order.
//
// With `tiles` given (the grouped GEMM's work list), pass 1 also builds the histogram of
// all experts in LDS, and each workgroup writes its own expert's 128-row tiles into the
// list: every expert's full tiles first (expert-major, an expert's tiles adjacent), then
// the partial last tiles by descending row count (ties: lower expert first), so the
// products run the lighter tiles last.  num_tiles[0] = all tiles, num_tiles[1] = full
// tiles.
constexpr int kGatherThreads = 1024;
constexpr int kGatherMaxExperts = 1024;
constexpr int kTileM = 128;  // rows per grouped-GEMM tile

__global__ void __launch_bounds__(kGatherThreads) gather_kernel(const int32_t* __restrict__ ids,
                                                                int64_t n_pairs, int n_expert,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ pairs,
                                                                int32_t* __restrict__ slot_row,
                                                                int32_t* __restrict__ tiles,
                                                                int32_t* __restrict__ num_tiles) {
  constexpr int kWaves = kGatherThreads / 64;
  __shared__ int eq_cnt[kWaves], lt_cnt[kWaves];
  __shared__ int hist[kGatherMaxExperts];
  const int e = blockIdx.x;
  const bool with_tiles = tiles != nullptr;
  if (with_tiles) {
    for (int i = threadIdx.x; i < n_expert; i += kGatherThreads) hist[i] = 0;
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t seg = ((n_pairs + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int64_t p0 = wave * seg;
  const int64_t p1 = min(p0 + seg, n_pairs);

  // ids are read 32 x 64 at a time (independent loads in flight; out of range -> never
  // equal to, nor below, any expert).  A wave whose segment fits in one batch (up to
  // 32,768 pairs per call) keeps it in registers for pass 2 instead of reading it again.
  constexpr int kBatch = 32;
  const bool one_batch = p1 - p0 <= 64 * kBatch;
  int v[kBatch];
  int eq = 0, lt = 0;
  for (int64_t pb = p0; pb < p1; pb += 64 * kBatch) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t p = pb + 64 * u + lane;
      v[u] = (p < p1) ? ids[p] : INT_MAX;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      eq += (v[u] == e);
      lt += (v[u] < e);
      if (with_tiles && (unsigned)v[u] < (unsigned)n_expert) atomicAdd(&hist[v[u]], 1);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    eq += __shfl_xor(eq, o);
    lt += __shfl_xor(lt, o);
  }
  if (lane == 0) {
    eq_cnt[wave] = eq;
    lt_cnt[wave] = lt;
  }
  __syncthreads();
  int base = 0, total = 0;
  for (int w2 = 0; w2 < kWaves; ++w2) {
    base += lt_cnt[w2];
    total += eq_cnt[w2];
  }
  int run = base;
  for (int w2 = 0; w2 < wave; ++w2) run += eq_cnt[w2];
  if (threadIdx.x == 0) {
    counts[e] = total;
    offsets[e] = base;
    if (e == (int)gridDim.x - 1) offsets[e + 1] = (int32_t)n_pairs;
  }
  if (with_tiles && wave == kWaves - 1) {
    // this expert's tiles (the histogram is complete: the barrier above follows pass 1)
    const int nf = total / kTileM, pr = total % kTileM;
    int full_below = 0, full_all = 0, rank = 0, partial_all = 0;
    for (int e2 = lane; e2 < n_expert; e2 += 64) {
      const int c2 = hist[e2], f2 = c2 / kTileM, p2 = c2 % kTileM;
      full_below += (e2 < e) ? f2 : 0;
      full_all += f2;
      rank += (p2 > pr) || (p2 == pr && e2 < e);
      partial_all += (p2 > 0);
    }
    for (int o = 32; o > 0; o >>= 1) {
      full_below += __shfl_xor(full_below, o);
      full_all += __shfl_xor(full_all, o);
      rank += __shfl_xor(rank, o);
      partial_all += __shfl_xor(partial_all, o);
    }
    for (int i = lane; i < nf; i += 64) {
      tiles[2 * (full_below + i)] = e;
      tiles[2 * (full_below + i) + 1] = i;
    }
    if (lane == 0 && pr > 0) {
      tiles[2 * (full_all + rank)] = e;
      tiles[2 * (full_all + rank) + 1] = nf;
    }
    if (lane == 0 && e == 0) {
      num_tiles[0] = full_all + partial_all;
      num_tiles[1] = full_all;
    }
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t pb = p0; pb < p1; pb += 64 * kBatch) {
    if (!one_batch) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t p = pb + 64 * u + lane;
        v[u] = (p < p1) ? ids[p] : INT_MAX;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {  // in pair order: u, then lane
      const int64_t p = pb + 64 * u + lane;
      const bool hit = v[u] == e;
      const uint64_t mask = __ballot(hit);
      if (hit) {
        const int pos = run + __popcll(mask & below);
        pairs[pos] = (int32_t)p;
        slot_row[p] = pos;
      }
      run += __popcll(mask);
    }
  }
}

int launch_route_topk(const float* logits, int64_t n_tok, int n_expert, int top_k, int32_t* ids,
                      float* w, hipStream_t s) {
  int64_t grid = (n_tok + 255) / 256;
  hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)grid), dim3(256), 0, s, logits, n_tok,
                     n_expert, top_k, ids, w);
  return check_launch("route_topk_kernel");
}

int launch_gather(const int32_t* ids, int64_t n_pairs, int n_expert, int32_t* counts,
                  int32_t* offsets, int32_t* pairs, int32_t* slot_row, int32_t* tiles,
                  int32_t* num_tiles, hipStream_t s) {
  if (n_expert > kGatherMaxExperts) return set_error(-1, "gather: at most %d experts", kGatherMaxExperts);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)n_expert), dim3(kGatherThreads), 0, s, ids,
                     n_pairs, n_expert, counts, offsets, pairs, slot_row, tiles, num_tiles);
  return check_launch("gather_kernel");
}

}  // namespace iq4
