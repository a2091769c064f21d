// Calibration loops for the benchmark's "achievable peak" figures (not part of
// the nmsparse ABI; built as libnmcal.so): the 2:4 sparse matrix instruction
// and the dense one with no memory traffic, and a streaming copy. Each call
// enqueues its kernel on the caller's stream, times it with HIP events on that
// stream and returns the rate (it synchronises on its own end event).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16 __attribute__((ext_vector_type(16)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef int i4 __attribute__((ext_vector_type(4)));
typedef int i8v __attribute__((ext_vector_type(8)));
typedef int i16v __attribute__((ext_vector_type(16)));

constexpr int CAL_ACC = 8;   // independent accumulators per wave

// 16-bit: v_smfmac_f32_32x32x32_f16 (65536 dense-equivalent flops per wave
// instruction) or v_mfma_f32_32x32x16_f16 (32768); int8: v_smfmac_i32_32x32x64_i8
// (131072) or v_mfma_i32_32x32x32_i8 (65536).
template <bool SPARSE, bool INT8>
__global__ void __launch_bounds__(256) matrix_loop(float* out, int iters) {
  const int idx = 0x4444;
  float s = 0;
  if constexpr (INT8) {
    i4 a;
    i8v b;
    for (int i = 0; i < 4; i++) a[i] = (int)threadIdx.x * 3 + i;
    for (int i = 0; i < 8; i++) b[i] = i * 5;
    i16v acc[CAL_ACC];
    for (int j = 0; j < CAL_ACC; j++) acc[j] = i16v{};
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int j = 0; j < CAL_ACC; j++) {
        if (SPARSE) acc[j] = __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, acc[j], idx, 0, 0);
        else acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, acc[j], 0, 0, 0);
      }
    }
    for (int j = 0; j < CAL_ACC; j++)
      for (int e = 0; e < 16; e++) s += (float)acc[j][e];
  } else {
    h8 a;
    h16 b;
    for (int i = 0; i < 8; i++) a[i] = (_Float16)(threadIdx.x * 0.001f + i);
    for (int i = 0; i < 16; i++) b[i] = (_Float16)(i * 0.002f);
    f16v acc[CAL_ACC];
    for (int j = 0; j < CAL_ACC; j++) acc[j] = f16v{};
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int j = 0; j < CAL_ACC; j++) {
        if (SPARSE) acc[j] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, acc[j], idx, 0, 0);
        else acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc[j], 0, 0, 0);
      }
    }
    for (int j = 0; j < CAL_ACC; j++)
      for (int e = 0; e < 16; e++) s += acc[j][e];
  }
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) copy_loop(const u4* __restrict__ src, u4* __restrict__ dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

template <typename F>
double timed(hipStream_t s, F launch) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1.0;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return -1.0;
  }
  launch();                                               // warm-up
  float ms = -1.0f;
  bool ok = hipEventRecord(e0, s) == hipSuccess;
  launch();
  ok = ok && hipEventRecord(e1, s) == hipSuccess;
  ok = ok && hipEventSynchronize(e1) == hipSuccess && hipGetLastError() == hipSuccess &&
       hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return ok ? ms : -1.0;
}

}  // namespace

extern "C" {

/* Dense-equivalent TFLOP/s (TOP/s for int8) of the 2:4 sparse matrix
   instruction (sparse != 0) or of the dense one, fp16 (int8 != 0: int8), over
   `blocks` blocks of four waves each running `iters` iterations of eight
   independent instructions. `out` is device memory for blocks * 256 floats.
   Returns a negative value on failure. */
double nmcal_matrix_tflops(int sparse, int int8, float* out, int blocks, int iters, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const double ms = timed(s, [&] {
    if (sparse && int8) hipLaunchKernelGGL((matrix_loop<true, true>), dim3(blocks), dim3(256), 0, s, out, iters);
    else if (sparse) hipLaunchKernelGGL((matrix_loop<true, false>), dim3(blocks), dim3(256), 0, s, out, iters);
    else if (int8) hipLaunchKernelGGL((matrix_loop<false, true>), dim3(blocks), dim3(256), 0, s, out, iters);
    else hipLaunchKernelGGL((matrix_loop<false, false>), dim3(blocks), dim3(256), 0, s, out, iters);
  });
  if (ms <= 0) return -1.0;
  const double per = (sparse ? 65536.0 : 32768.0) * (int8 ? 2.0 : 1.0);
  const double flops = (double)blocks * 4 * iters * CAL_ACC * per;
  return flops / (ms * 1e-3) / 1e12;
}

/* GB/s of a streaming copy of `bytes` (a multiple of 16) from src to dst,
   counting bytes read plus bytes written. Returns a negative value on failure. */
double nmcal_copy_gbs(const void* src, void* dst, size_t bytes, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const size_t n = bytes / 16;
  const double ms = timed(s, [&] {
    hipLaunchKernelGGL(copy_loop, dim3(256 * 16), dim3(256), 0, s, (const u4*)src, (u4*)dst, n);
  });
  if (ms <= 0) return -1.0;
  return 2.0 * (double)bytes / (ms * 1e-3) / 1e9;
}

}  // extern "C"
