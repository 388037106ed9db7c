// ceilings.hip -- the two reference kernels the benchmark measures beside the library's
// own, to state each kernel's achieved rate against what this GPU sustains in practice:
//   * a plain streaming read of a buffer (16-byte loads, grid-stride), the ceiling of an
//     HBM-bound kernel reading the same number of bytes;
//   * a pure matrix-core loop (v_mfma_f32_16x16x32_f16 on register operands, 8 independent
//     accumulators per wave), the ceiling of an MFMA-bound kernel.
// Built into its own library (libiq4_ceilings.so); the product library does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each thread reads NV 16-byte vectors at a stride of the whole grid; the xor of what it
// read is stored only if it equals a value no buffer of this benchmark produces, so the
// loads stay live and nothing is written.
template <int NV>
__global__ void __launch_bounds__(256) stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x, st = (int64_t)gridDim.x * 256;
  uint4 v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t i = i0 + j * st;
    v[j] = (i < n16) ? p[i] : uint4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  if (acc == 0x9E3779B9u) sink[i0 & 1023] = acc;
}

// iters x 8 independent MFMAs per wave on register operands; the accumulators are stored
// only under a condition that never holds at run time (they stay live).
__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (lane + i));
    b[i] = (_Float16)(0.002f * (lane - i));
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The MFMAs are written as assembly with each accumulator tied to its own registers
  // (the builtin lets the register allocator shuffle the accumulators through copies
  // inside the loop).  The compiler does not see these as matrix instructions, so the
  // wait states around them are explicit: 8 before the loop (vector writes of the
  // operands -> matrix reads), 3 x 8 after it (matrix results -> vector reads); the
  // same accumulator recurs every 8 instructions, far past the result latency.  The
  // waits name every operand, so the compiler cannot move them.
#define IQ4C_WAIT(N)                                                                          \
  asm volatile(N : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]),     \
               "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7]), "+v"(a), "+v"(b))
  IQ4C_WAIT("s_nop 7");
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc[j]) : "v"(a), "v"(b));
  }
  IQ4C_WAIT("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#undef IQ4C_WAIT
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == 12345.678f) sink[threadIdx.x] = s;
}

extern "C" {

// Streaming read of `bytes` (a multiple of 16) at p: grid of `grid` workgroups of 256
// threads, NV = 1, 2, 4 or 8 vectors per thread.  Returns 0 or a hipError_t.
int iq4c_stream_read(const void* p, int64_t bytes, int nv, int grid, void* sink, void* stream) {
  const int64_t n16 = bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (nv) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(grid), dim3(256), 0, s, (const uint4*)p, n16, (uint32_t*)sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(grid), dim3(256), 0, s, (const uint4*)p, n16, (uint32_t*)sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(256), 0, s, (const uint4*)p, n16, (uint32_t*)sink); break;
    default: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(256), 0, s, (const uint4*)p, n16, (uint32_t*)sink); break;
  }
  return (int)hipGetLastError();
}

// `grid` workgroups of 4 waves, each wave iters x 8 MFMAs of 16 x 16 x 32 (16,384 flop).
int iq4c_mfma_loop(int iters, int grid, void* sink, void* stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     (float*)sink);
  return (int)hipGetLastError();
}

}  // extern "C"
