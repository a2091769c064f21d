// Device helpers shared by the nmsparse kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Dt { DT_F16 = 0, DT_BF16 = 1, DT_I8 = 2 };

// Magnitude key: unsigned, ordered like |x|. 16-bit floats: bits with the sign
// cleared (+0 and -0 both give 0). int8: |x|.
// Violation counting. Counting kernels stride over their work with at most
// kCheckBlocks blocks (about four per compute unit) and add each block's total
// to the caller's counter with one atomic, none when it is zero: atomics on a
// single address serialize, so one per wave over a large matrix would dominate
// the kernel. Every thread of the block must reach the call.
constexpr int64_t kCheckBlocks = 1024;
__device__ __forceinline__ void block_add_count(int32_t* count, int v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __shared__ int32_t part[16];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t t = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); i++) t += part[i];
    if (t) atomicAdd(count, t);
  }
}

template <int DT> __device__ __forceinline__ uint32_t magkey(uint32_t raw);
template <> __device__ __forceinline__ uint32_t magkey<DT_F16>(uint32_t raw) { return raw & 0x7FFFu; }
template <> __device__ __forceinline__ uint32_t magkey<DT_BF16>(uint32_t raw) { return raw & 0x7FFFu; }
template <> __device__ __forceinline__ uint32_t magkey<DT_I8>(uint32_t raw) {
  int v = (int)(int8_t)(uint8_t)raw;
  return (uint32_t)(v < 0 ? -v : v);
}

// |x| widened exactly to fp64.
template <int DT> __device__ __forceinline__ double absval64(uint32_t raw);
template <> __device__ __forceinline__ double absval64<DT_F16>(uint32_t raw) {
  uint16_t h = (uint16_t)(raw & 0x7FFFu);
  _Float16 f = __builtin_bit_cast(_Float16, h);
  return (double)(float)f;
}
template <> __device__ __forceinline__ double absval64<DT_BF16>(uint32_t raw) {
  uint32_t u = (raw & 0x7FFFu) << 16;
  return (double)__builtin_bit_cast(float, u);
}
template <> __device__ __forceinline__ double absval64<DT_I8>(uint32_t raw) {
  int v = (int)(int8_t)(uint8_t)raw;
  return (double)(v < 0 ? -v : v);
}

// fp32 -> 16-bit float bits, round to nearest even (hardware conversion).
template <int DT> __device__ __forceinline__ uint16_t to_bits16(float x);
template <> __device__ __forceinline__ uint16_t to_bits16<DT_F16>(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <> __device__ __forceinline__ uint16_t to_bits16<DT_BF16>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
template <int DT> __device__ __forceinline__ float from_bits16(uint16_t b);
template <> __device__ __forceinline__ float from_bits16<DT_F16>(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
template <> __device__ __forceinline__ float from_bits16<DT_BF16>(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Top-N selection inside one group of M magnitude keys. Returns a bit mask of
// the kept offsets. Rule: larger magnitude first, equal magnitudes by lower
// offset. Each element gets the composite key (mag << 5 | (31 - j)) + 1, which
// is unique and orders exactly by that rule; the kept set is the N largest
// composite keys (picked one by one, or as the complement of the M - N
// smallest when that is shorter).
template <int M>
__device__ __forceinline__ uint32_t select_topn(const uint32_t (&mag)[M], int N) {
  uint32_t key[M];
#pragma unroll
  for (int j = 0; j < M; j++) key[j] = ((mag[j] << 5) | (uint32_t)(31 - j)) + 1u;
  uint32_t picked = 0;
  const bool pick_kept = N <= M - N;
  const int rounds = pick_kept ? N : M - N;
  for (int s = 0; s < rounds; s++) {
    uint32_t best = pick_kept ? 0u : 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < M; j++) {
      const bool taken = (picked >> j) & 1u;
      if (pick_kept) best = taken ? best : max(best, key[j]);
      else best = taken ? best : min(best, key[j]);
    }
#pragma unroll
    for (int j = 0; j < M; j++) picked |= (key[j] == best) ? (1u << j) : 0u;
  }
  const uint32_t full = (M == 32) ? 0xFFFFFFFFu : ((1u << M) - 1u);
  return pick_kept ? picked : (full & ~picked);
}

// 2 of 4: the kept offsets j0 < j1 under the same rule, without a search. The
// keys (mag << 2) | (3 - j) are unique and order the four exactly by it; with
// a, b the smaller and larger of keys 0 and 1 and c, d those of keys 2 and 3,
// the largest key is max(b, d) and the second largest max(min(b, d), a, c).
// Magnitude keys are below 2^30.
__device__ __forceinline__ void top2of4(const uint32_t (&mag)[4], int& j0, int& j1) {
  const uint32_t k0 = (mag[0] << 2) | 3u, k1 = (mag[1] << 2) | 2u, k2 = (mag[2] << 2) | 1u, k3 = mag[3] << 2;
  const uint32_t a = min(k0, k1), b = max(k0, k1), c = min(k2, k3), d = max(k2, k3);
  const uint32_t t1 = max(b, d) & 3u, t2 = max(max(min(b, d), a), c) & 3u;   // 3 - offset of each
  j0 = 3 - (int)max(t1, t2);
  j1 = 3 - (int)min(t1, t2);
}

}  // namespace nm
