// Measurement aid for bench.py, built into its own library (libra_probe.so),
// not part of the attention library: the throughput of the attention
// kernel's matrix instruction, v_mfma_f32_32x32x16_bf16, with nothing else
// in the loop.  MI355X's sustained clock depends on what the matrix cores
// switch: zero operands let it run at full clock, random bf16 operands hold
// it at the board's power/current limit.  The random figure is the ceiling
// any bf16 MFMA kernel on random data can reach on the part.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each wave keeps 8 A and 8 B operand registers per lane (from src, or
// zero) and cycles through them, so consecutive products see different data;
// 4 independent accumulators keep the matrix pipe full.
template <bool ZERO>
__global__ __launch_bounds__(256) void mfma_loop(const bf16x8 *src, float *sink, int iters) {
  const int l = threadIdx.x & 63;
  bf16x8 A[8], B[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    A[j] = ZERO ? bf16x8{} : src[j * 64 + l];
    B[j] = ZERO ? bf16x8{} : src[512 + j * 64 + l];
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; j += 4) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j], B[(j + 1) & 7], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j + 1], B[(j + 3) & 7], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j + 2], B[(j + 5) & 7], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[j + 3], B[(j + 7) & 7], c3, 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;  // keeps the products live
}

}  // namespace

// zero: 0 = operands from src, 1 = zero operands.  src: 1024 bf16x8 vectors
// (16 KiB, device); sink: grid * 256 floats (device).  Each launch does
// grid * 4 waves * iters * 8 products of 32x32x16 (32768 flops each).
// Returns a hipError_t as int.
extern "C" int ra_probe_mfma_loop(int zero, const void *src, float *sink, int grid, int iters, void *stream) {
  if (grid < 1 || iters < 1 || !sink || (!zero && !src)) return (int)hipErrorInvalidValue;
  if (zero)
    mfma_loop<true><<<grid, 256, 0, (hipStream_t)stream>>>((const bf16x8 *)src, sink, iters);
  else
    mfma_loop<false><<<grid, 256, 0, (hipStream_t)stream>>>((const bf16x8 *)src, sink, iters);
  return (int)hipGetLastError();
}
