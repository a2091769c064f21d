// Matrix-core kernel templates (included by the per-type instantiation files): D = alpha * op(A) * op(B) + beta * C.
//
//  - A_SPARSE24: A is 2:4 compressed (values + 2-bit offsets). The gfx950
//    sparse matrix instructions (v_smfmac_f32_16x16x64_{f16,bf16},
//    v_smfmac_i32_16x16x128_i8) take the compressed values and the offsets
//    directly: the offsets select which activations (rows of op(B)) meet each
//    kept weight, the mechanism the cuSPARSELt blog describes for Figure 2.
//  - A_DENSE: dense A on the dense MFMA instructions; the same-shape
//    comparator for the sparse speed-up (the blog's dense/sparse table).
//  - A_GATHER: general N:M. Each k-step the block expands its compressed rows
//    into a dense LDS tile (zero fill + scatter of the kept values by their
//    offsets) and runs the dense MFMA on it. Element-wise N:M gives every row
//    its own offsets, so there is no shared gather of B rows to exploit.
//
// Block tile 128 x 128, four waves in a 2 x 2 grid, 64 x 64 per wave, 16 x 16
// instruction tiles. One k-step covers 128 bytes of k per row of op(B): 64
// elements for 16-bit types, 128 for int8. B is staged in LDS column-major
// ([n][k], k contiguous): op_b = T (n x k as stored) copies 16-byte chunks;
// op_b = N (k x n) transposes 4 x 8 (or 4 x 16) register blocks on the way in.
// Global loads for step s+1 are issued before the matrix instructions of
// step s and written to the other LDS buffer afterwards.
//
// Lane layouts used below (checked on gfx950 hardware with one-hot and random
// operands): for the 16x16 instructions lane l covers row/column (l % 16) and
// quarter q = l / 16; the accumulator holds D[4q + r][l % 16], r = 0..3.
//  dense f16/bf16 16x16x32: A and B hold k = 8q .. 8q+7.
//  dense i8 16x16x64:       A and B hold k = 16q .. 16q+15.
//  smfmac 16x16x64 (16-bit): A holds compressed values 8q .. 8q+7 (logical k
//    16q .. 16q+15, four groups), the index word holds their 2-bit offsets as
//    nibbles i0 | i1 << 2, one per group; B holds k = 8q .. 8q+7 and
//    32 + 8q .. 32 + 8q + 7.
//  smfmac 16x16x128 (i8): A holds compressed bytes 16q .. 16q+15 (logical k
//    32q .. 32q+31), 32 index bits; B holds k = 16q .. 16q+15 and
//    64 + 16q .. 64 + 16q + 15.
#pragma once
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "nm_device.h"
#include "nm_internal.h"

namespace nm {

constexpr int NTH = 256;              // four waves
constexpr int KBYTES = 128;           // bytes of k per row of a dense k-step
constexpr int BSTRIDE = KBYTES + 16;  // LDS row stride of B / dense A tiles (bank spread)
constexpr int ASTRIDE_SP = 80;        // LDS row stride of 2:4 compressed A: 64 B values + meta + pad
constexpr int STG_V = 128;            // gather staging: value bytes per row per step (<= 124 used)
constexpr int STG_M = 96;             // gather staging: metadata bytes per row per step

enum AMode { A_SPARSE24 = 0, A_DENSE = 1, A_GATHER = 2 };

struct GemmArgs {
  const uint8_t* a;     // dense A (A_DENSE) or compressed values
  const uint8_t* meta;  // metadata (A_SPARSE24, A_GATHER)
  const uint8_t* b;
  const uint8_t* c;
  uint8_t* d;
  int64_t m, n, k;
  int64_t lda;          // dense A leading dim (elements) or values_ld
  int64_t mld;          // metadata row stride (bytes)
  int64_t ldb;
  int64_t c_rs, c_cs, d_rs, d_cs;   // C/D element (row, col) at row * rs + col * cs (row- or column-major)
  int cd_col;                       // C/D column-major (rs = 1, cs = ld)
  int cd_i8;                        // integer path: C/D are int8 (D saturated) instead of int32
  float alpha, beta;
  int N, M, bits;
  int a_vec, b_vec;     // 16-byte vector loads allowed on A / B rows
  int vshift;           // metadata row of op(A) row r: r >> vshift (0: element-wise; vector-wise N:M shares a row per 2^vshift rows)
  int splits;           // split-k: k ranges (1 = none); with more, each block writes raw partial sums to ws
  uint8_t* ws;          // splits planes of m x n fp32 (int32 for int8) partial sums, in D's storage order
};

// Integer-path epilogue: v = alpha * acc + beta * C exactly in int64, stored as
// int32 (D = v) or, with int8 C/D, saturated to [-128, 127].
__device__ __forceinline__ int64_t int_epilogue(const GemmArgs& A, int64_t acc, int64_t cidx) {
  int64_t v = (int64_t)A.alpha * acc;
  if (A.beta != 0.0f)
    v += (int64_t)A.beta * (A.cd_i8 ? (int64_t)((const int8_t*)A.c)[cidx] : (int64_t)((const int32_t*)A.c)[cidx]);
  return v;
}
__device__ __forceinline__ int32_t sat_i8(int64_t v) { return (int32_t)(v < -128 ? -128 : (v > 127 ? 127 : v)); }
__device__ __forceinline__ void int_store(const GemmArgs& A, int64_t didx, int64_t v) {
  if (A.cd_i8) ((int8_t*)A.d)[didx] = (int8_t)sat_i8(v);
  else ((int32_t*)A.d)[didx] = (int32_t)v;
}

// ---------------------------------------------------------------- operand staging

// One k-step of a "k-major" operand tile (ROWS rows x 128 bytes of k) from a
// source whose rows are k-contiguous (op_b = T, or dense A with op_a = N):
// tile row r is src[(r0 + r) * ld + k0 ...]. ROWS/32 chunks of 16 bytes per thread.
template <int ROWS> struct KChunks { u32x4 v[ROWS / 32]; };

template <int ESZ, int ROWS>
__device__ __forceinline__ void load_kcontig(KChunks<ROWS>& R, const uint8_t* src, int64_t r0, int64_t rows,
                                             int64_t ld, int64_t k0, int64_t k, bool vec) {
  constexpr int EPC = 16 / ESZ;   // elements per chunk
#pragma unroll
  for (int i = 0; i < ROWS / 32; i++) {
    const int id = threadIdx.x + NTH * i;
    const int r = id / 8, part = id % 8;
    const int64_t gr = r0 + r, gk = k0 + part * EPC;
    if (vec && gr < rows && gk + EPC <= k) {
      R.v[i] = *(const u32x4*)(src + (size_t)(gr * ld + gk) * ESZ);
    } else {
      uint8_t tmp[16];
#pragma unroll
      for (int e = 0; e < 16; e++) tmp[e] = 0;
      if (gr < rows) {
        for (int e = 0; e < EPC; e++)
          if (gk + e < k) {
            if (ESZ == 2) ((uint16_t*)tmp)[e] = ((const uint16_t*)src)[gr * ld + gk + e];
            else tmp[e] = src[gr * ld + gk + e];
          }
      }
      R.v[i] = *(u32x4*)tmp;
    }
  }
}

template <int ROWS>
__device__ __forceinline__ void store_kcontig(uint8_t* lds, const KChunks<ROWS>& R) {
#pragma unroll
  for (int i = 0; i < ROWS / 32; i++) {
    const int id = threadIdx.x + NTH * i;
    const int r = id / 8, part = id % 8;
    *(u32x4*)(lds + r * BSTRIDE + part * 16) = R.v[i];
  }
}

// The same tile from a source whose rows run along the tile's rows (op_b = N:
// B stored k x n; dense A with op_a = T). Each (chunk, k-quad) pair is four
// consecutive k rows of one 16-byte column chunk, transposed in registers.
template <int ESZ, int COLS>
__device__ __forceinline__ void load_mncontig(KChunks<COLS>& R, const uint8_t* src, int64_t c0, int64_t cols,
                                              int64_t ld, int64_t k0, int64_t k, bool vec) {
  constexpr int EPC = 16 / ESZ;                 // columns per chunk
  constexpr int CPR = COLS / EPC;               // chunks per k row
#pragma unroll
  for (int j = 0; j < COLS / 128; j++) {
    const int pid = threadIdx.x + NTH * j;
    const int cc = pid % CPR, kq = pid / CPR;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int64_t gk = k0 + kq * 4 + i, gc = c0 + cc * EPC;
      u32x4 val;
      if (vec && gk < k && gc + EPC <= cols) {
        val = *(const u32x4*)(src + (size_t)(gk * ld + gc) * ESZ);
      } else {
        uint8_t tmp[16];
#pragma unroll
        for (int e = 0; e < 16; e++) tmp[e] = 0;
        if (gk < k) {
          for (int e = 0; e < EPC; e++)
            if (gc + e < cols) {
              if (ESZ == 2) ((uint16_t*)tmp)[e] = ((const uint16_t*)src)[gk * ld + gc + e];
              else tmp[e] = src[gk * ld + gc + e];
            }
        }
        val = *(u32x4*)tmp;
      }
      R.v[j * 4 + i] = val;
    }
  }
}

template <int ESZ, int COLS>
__device__ __forceinline__ void store_mncontig(uint8_t* lds, const KChunks<COLS>& R) {
  constexpr int EPC = 16 / ESZ;
  constexpr int CPR = COLS / EPC;
#pragma unroll
  for (int j = 0; j < COLS / 128; j++) {
    const int pid = threadIdx.x + NTH * j;
    const int cc = pid % CPR, kq = pid / CPR;
    const u32x4* v = &R.v[j * 4];
    if (ESZ == 2) {
      // column c of the chunk gets four 16-bit values (k = 4kq .. 4kq+3)
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const uint32_t w0 = v[0][d], w1 = v[1][d], w2 = v[2][d], w3 = v[3][d];
        const u32x2 lo = {(w0 & 0xFFFFu) | (w1 << 16), (w2 & 0xFFFFu) | (w3 << 16)};
        const u32x2 hi = {(w0 >> 16) | (w1 & 0xFFFF0000u), (w2 >> 16) | (w3 & 0xFFFF0000u)};
        const int col = cc * EPC + 2 * d;
        *(u32x2*)(lds + col * BSTRIDE + kq * 8) = lo;
        *(u32x2*)(lds + (col + 1) * BSTRIDE + kq * 8) = hi;
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; d++) {
        const uint32_t w0 = v[0][d], w1 = v[1][d], w2 = v[2][d], w3 = v[3][d];
#pragma unroll
        for (int x = 0; x < 4; x++) {
          const uint32_t val = ((w0 >> (8 * x)) & 0xFFu) | (((w1 >> (8 * x)) & 0xFFu) << 8) |
                               (((w2 >> (8 * x)) & 0xFFu) << 16) | (((w3 >> (8 * x)) & 0xFFu) << 24);
          const int col = cc * EPC + 4 * d + x;
          *(uint32_t*)(lds + col * BSTRIDE + kq * 4) = val;
        }
      }
    }
  }
}

// 2:4 compressed A: per row and k-step 64 bytes of values (ROWS/64 chunks per
// thread) and 8 (16-bit types) or 16 (int8) metadata bytes (thread t loads row t).
template <int ROWS> struct SpChunks { u32x4 v[ROWS / 64]; u32x4 meta; };

template <int ESZ, int ROWS>
__device__ __forceinline__ void load_sp24(SpChunks<ROWS>& R, const GemmArgs& A, int64_t r0, int ks) {
  const int64_t nvals = A.k / 2;                        // compressed elements per row
  constexpr int EPC = 16 / ESZ;
  const int64_t v0 = (int64_t)ks * (64 / ESZ);          // first compressed element of this step
#pragma unroll
  for (int i = 0; i < ROWS / 64; i++) {
    const int id = threadIdx.x + NTH * i;
    const int r = id / 4, part = id % 4;
    const int64_t gr = r0 + r, gv = v0 + part * EPC;
    if (gr < A.m && gv + EPC <= nvals) {
      R.v[i] = *(const u32x4*)(A.a + (size_t)(gr * A.lda + gv) * ESZ);
    } else {
      uint8_t tmp[16];
#pragma unroll
      for (int e = 0; e < 16; e++) tmp[e] = 0;
      if (gr < A.m)
        for (int e = 0; e < EPC; e++)
          if (gv + e < nvals) {
            if (ESZ == 2) ((uint16_t*)tmp)[e] = ((const uint16_t*)A.a)[gr * A.lda + gv + e];
            else tmp[e] = A.a[gr * A.lda + gv + e];
          }
      R.v[i] = *(u32x4*)tmp;
    }
  }
  // Metadata bytes [ks*MB, ks*MB + MB) of the row; the row's zero padding
  // covers a partial last step (its offsets then meet zero values only).
  constexpr int MB = ESZ == 2 ? 8 : 16;
  R.meta = u32x4{0, 0, 0, 0};
  if (threadIdx.x < ROWS) {
    const int64_t gr = r0 + threadIdx.x;
    const int64_t off = (int64_t)ks * MB;
    if (gr < A.m && off + MB <= A.mld) {
      if (MB == 8) {
        const u32x2 t = *(const u32x2*)(A.meta + gr * A.mld + off);
        R.meta = u32x4{t[0], t[1], 0, 0};
      } else {
        R.meta = *(const u32x4*)(A.meta + gr * A.mld + off);
      }
    }
  }
}

template <int ESZ, int ROWS>
__device__ __forceinline__ void store_sp24(uint8_t* lds, const SpChunks<ROWS>& R) {
#pragma unroll
  for (int i = 0; i < ROWS / 64; i++) {
    const int id = threadIdx.x + NTH * i;
    const int r = id / 4, part = id % 4;
    *(u32x4*)(lds + r * ASTRIDE_SP + part * 16) = R.v[i];
  }
  if (threadIdx.x < ROWS) {
    if (ESZ == 2) *(u32x2*)(lds + threadIdx.x * ASTRIDE_SP + 64) = u32x2{R.meta[0], R.meta[1]};
    else *(u32x4*)(lds + threadIdx.x * ASTRIDE_SP + 64) = R.meta;
  }
}

// ---------------------------------------------------------------- general N:M expansion

// Copy the compressed bytes of step ks for the block's rows into LDS staging:
// values (dword aligned: 128*N/M bytes per step) and the dword-aligned window
// of metadata covering the step's offset fields.
template <int ESZ, int ROWS>
__device__ __forceinline__ void stage_gather(uint8_t* stg, const GemmArgs& A, int64_t r0, int ks) {
  const int KL = KBYTES / ESZ;                                // logical k per step
  const int gps = KL / A.M;                                   // groups per step
  const int vbytes = gps * A.N * ESZ;                         // value bytes per row per step
  const int64_t row_vbytes = A.lda * ESZ;                     // padded row: zeros after the last value
  const int64_t bit0 = (int64_t)ks * gps * A.N * A.bits;
  const int64_t w0 = bit0 / 32;
  const int64_t row_mwords = (A.mld) / 4;
  const int nmw = (gps * A.N * A.bits + 31) / 32 + 1;        // words covering the step's fields
  const int vw = vbytes / 4;
  for (int e = threadIdx.x; e < ROWS * (vw + nmw); e += NTH) {
    const int r = e / (vw + nmw), c = e % (vw + nmw);
    const int64_t gr = r0 + r;
    uint32_t val = 0;
    if (c < vw) {
      const int64_t off = (int64_t)ks * vbytes + c * 4;
      if (gr < A.m && off + 4 <= row_vbytes) val = *(const uint32_t*)(A.a + gr * A.lda * ESZ + off);
      *(uint32_t*)(stg + r * STG_V + c * 4) = val;
    } else {
      const int64_t w = w0 + (c - vw);
      if (gr < A.m && w < row_mwords) val = *(const uint32_t*)(A.meta + (gr >> A.vshift) * A.mld + w * 4);
      *(uint32_t*)(stg + ROWS * STG_V + r * STG_M + (c - vw) * 4) = val;
    }
  }
}

// Zero each (row, group) region of the dense A tile and scatter its kept values.
template <int ESZ, int ROWS>
__device__ __forceinline__ void expand_gather(uint8_t* adense, const uint8_t* stg, const GemmArgs& A, int ks) {
  const int KL = KBYTES / ESZ;
  const int gps = KL / A.M;
  const int64_t groups_left = A.k / A.M - (int64_t)ks * gps;
  const int gvalid = (int)(groups_left < gps ? groups_left : gps);
  const int bitoff = (int)(((int64_t)ks * gps * A.N * A.bits) % 32);
  const int gbytes = A.M * ESZ;
  for (int e = threadIdx.x; e < ROWS * gps; e += NTH) {
    const int r = e / gps, g = e % gps;
    uint8_t* dst = adense + r * BSTRIDE + g * gbytes;
    for (int x = 0; x < gbytes; x += 4) *(uint32_t*)(dst + x) = 0u;
    if (g >= gvalid) continue;
    const uint8_t* vrow = stg + r * STG_V;
    const uint32_t* mrow = (const uint32_t*)(stg + ROWS * STG_V + r * STG_M);
    for (int s = 0; s < A.N; s++) {
      const int t = bitoff + (g * A.N + s) * A.bits;
      const uint64_t w = (uint64_t)mrow[t / 32] | ((uint64_t)mrow[t / 32 + 1] << 32);
      const int j = (int)((w >> (t % 32)) & ((1u << A.bits) - 1u));
      if (ESZ == 2) ((uint16_t*)dst)[j] = ((const uint16_t*)vrow)[g * A.N + s];
      else dst[j] = vrow[g * A.N + s];
    }
  }
}

// General N:M with M = 32 and GV value bytes per group (4, 8 or 16): each
// thread owns (row, group) pairs of the block's k-step, loads a pair's kept
// values and the metadata words holding its offsets straight into registers
// one step ahead (indices clamped into the operand: rows past m load row
// m - 1, groups past k the last group), and expands it into the idle dense A
// buffer: zero the group's 32 elements, then write its kept values at their
// offsets.
template <int ESZ, int ROWS, int GV>
struct G32Regs {
  static constexpr int GPS = KBYTES / ESZ / 32;               // groups per row per step
  static constexpr int PAIRS = ROWS * GPS / NTH;
  static constexpr int NV = GV / ESZ;                         // kept values per group
  static constexpr int MW = (31 + 5 * NV + 31) / 32 < 3 ? (31 + 5 * NV + 31) / 32 : 3;
  uint32_t v[PAIRS > 0 ? PAIRS : 1][GV / 4];
  uint32_t m[PAIRS > 0 ? PAIRS : 1][MW];
};

template <int ESZ, int ROWS, int GV>
__device__ __forceinline__ void load_g32(G32Regs<ESZ, ROWS, GV>& R, const GemmArgs& A, int64_t r0, int ks) {
  typedef G32Regs<ESZ, ROWS, GV> G;
  static_assert(G::PAIRS > 0 && (ROWS * G::GPS) % NTH == 0 && (GV == 4 || GV == 8 || GV == 16), "pairs per thread");
  const int64_t groups = A.k >> 5, mwords = A.mld / 4;
#pragma unroll
  for (int i = 0; i < G::PAIRS; i++) {
    const int p = threadIdx.x + i * NTH, r = p / G::GPS, g = p % G::GPS;
    const int64_t row = r0 + r < A.m ? r0 + r : A.m - 1;
    const int64_t gg0 = (int64_t)ks * G::GPS + g;
    const int64_t gg = gg0 < groups ? gg0 : groups - 1;
    const uint8_t* pv = A.a + (row * A.lda + gg * G::NV) * ESZ;
    if constexpr (GV == 16) {
      const u32x4 v = *(const u32x4*)pv;
      R.v[i][0] = v[0]; R.v[i][1] = v[1]; R.v[i][2] = v[2]; R.v[i][3] = v[3];
    } else if constexpr (GV == 8) {
      const u32x2 v = *(const u32x2*)pv;
      R.v[i][0] = v[0]; R.v[i][1] = v[1];
    } else {
      R.v[i][0] = *(const uint32_t*)pv;
    }
    const int64_t w0 = (gg * G::NV * 5) >> 5;                  // the group's bits end inside the row
    const uint32_t* mr = (const uint32_t*)(A.meta + (row >> A.vshift) * A.mld);
#pragma unroll
    for (int x = 0; x < G::MW; x++) R.m[i][x] = mr[w0 + x < mwords ? w0 + x : mwords - 1];
  }
}

template <int ESZ, int ROWS, int GV>
__device__ __forceinline__ void expand_g32(uint8_t* adense, const G32Regs<ESZ, ROWS, GV>& R, const GemmArgs& A,
                                           int ks) {
  typedef G32Regs<ESZ, ROWS, GV> G;
  const int64_t groups = A.k >> 5;
#pragma unroll
  for (int i = 0; i < G::PAIRS; i++) {
    const int p = threadIdx.x + i * NTH, r = p / G::GPS, g = p % G::GPS;
    const int64_t gg = (int64_t)ks * G::GPS + g;
    uint8_t* dst = adense + r * BSTRIDE + g * 32 * ESZ;
#pragma unroll
    for (int x = 0; x < 2 * ESZ; x++) *(u32x4*)(dst + 16 * x) = u32x4{0u, 0u, 0u, 0u};
    if (gg >= groups) continue;                                 // past k: zeros
    const int off = (int)((gg * G::NV * 5) & 31);
    const uint64_t lo = ((uint64_t)R.m[i][1] << 32) | R.m[i][0];
    uint64_t hi = 0;
    if constexpr (G::MW == 3) hi = ((uint64_t)R.m[i][2] << 32) | R.m[i][1];
#pragma unroll
    for (int s = 0; s < G::NV; s++) {
      const int pbit = off + 5 * s;
      uint64_t w;
      if constexpr (G::MW == 3) w = pbit < 32 ? lo >> pbit : hi >> (pbit - 32);
      else w = lo >> pbit;
      const int j = (int)(w & 31u);
      const uint32_t word = R.v[i][(s * ESZ) / 4];
      if constexpr (ESZ == 2) *(uint16_t*)(dst + 2 * j) = (uint16_t)(word >> (16 * (s & 1)));
      else dst[j] = (uint8_t)(word >> (8 * (s & 3)));
    }
  }
}

// ---------------------------------------------------------------- matrix instructions

template <int DT> struct Frag;
template <> struct Frag<DT_F16> { typedef half8_t ab; typedef _Float16 half16_t __attribute__((ext_vector_type(16))); typedef half16_t b2; };
template <> struct Frag<DT_BF16> { typedef bf16x8_t ab; typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16))); typedef bf16x16_t b2; };
template <> struct Frag<DT_I8> { typedef intx4 ab; typedef intx8 b2; };
template <int DT> struct Acc { typedef floatx16 t; };
template <> struct Acc<DT_I8> { typedef intx16 t; };

template <int DT>
__device__ __forceinline__ typename Frag<DT>::b2 concat(const typename Frag<DT>::ab& lo, const typename Frag<DT>::ab& hi) {
  if constexpr (DT == DT_I8) {
    return intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  }
}

// 32x32 sparse instruction: 32 (16-bit) or 64 (int8) logical k.
template <int DT>
__device__ __forceinline__ typename Acc<DT>::t smfmac32(const typename Frag<DT>::ab& a, const typename Frag<DT>::b2& b,
                                                      typename Acc<DT>::t c, int idx) {
  if constexpr (DT == DT_F16) return __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, c, idx, 0, 0);
  else if constexpr (DT == DT_BF16) return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, b, c, idx, 0, 0);
  else return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c, idx, 0, 0);
}

// 32x32 dense instruction: 16 (16-bit) or 32 (int8) k.
template <int DT>
__device__ __forceinline__ typename Acc<DT>::t mfma32(const typename Frag<DT>::ab& a, const typename Frag<DT>::ab& b,
                                                    typename Acc<DT>::t c) {
  if constexpr (DT == DT_F16) return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  else if constexpr (DT == DT_BF16) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Map the hardware block id to a (row tile, column tile). The dispatcher deals
// consecutive block ids round-robin to the eight XCDs, each with its own L2;
// renumbering gives every XCD a contiguous range of logical tiles. Logical ids
// then walk down a band of GROUP row tiles before moving right, so the blocks
// resident on one XCD at the same time cover a compact GROUP x (CUs / GROUP)
// patch and share both A row tiles and B column tiles in that XCD's L2.
constexpr int NUM_XCD = 8;
constexpr int NUM_CU = 256;
__device__ __forceinline__ int64_t xcd_logical_id() {
  const int64_t nb = gridDim.x;
  const int64_t hw = blockIdx.x;
  const int64_t per = nb / NUM_XCD, rem = nb % NUM_XCD;
  const int64_t x = hw % NUM_XCD, local = hw / NUM_XCD;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + local;
}
__device__ __forceinline__ void band_coords(int64_t id, int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  constexpr int GROUP = 8;
  const int64_t per_band = GROUP * tiles_n;
  const int64_t band = id / per_band;
  const int64_t first = band * GROUP;
  const int64_t rows_in_band = (tiles_m - first) < GROUP ? (tiles_m - first) : GROUP;
  const int64_t in = id % per_band;
  tm = first + in % rows_in_band;
  tn = in / rows_in_band;
}
__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  band_coords(xcd_logical_id(), tiles_m, tiles_n, tm, tn);
}
// With split-k the grid is splits x tiles: logical ids run through every tile
// of k range 0, then of range 1, ..., so the blocks one XCD holds at a time
// work on the same k range of neighbouring tiles, as without a split.
__device__ __forceinline__ void split_tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn,
                                                  int& z) {
  const int64_t id = xcd_logical_id(), tiles = tiles_m * tiles_n;
  z = (int)(id / tiles);
  band_coords(id % tiles, tiles_m, tiles_n, tm, tn);
}

// ---------------------------------------------------------------- the tiled kernel

// Block tile BM x BN, four waves in a 2 x 2 grid, (BM/2) x (BN/2) per wave of
// 32 x 32 instruction tiles. Lane l of a 32x32 instruction covers row/column
// l % 32 and half q = l / 32; its accumulator holds D[8(r/4) + 4q + r%4][l % 32].
//  smfmac 32x32x32 (16-bit): A = compressed values 8q..8q+7 of the 16 per row
//   (logical k 16q..16q+15), index = their nibbles (16 bits); B = k 8q..8q+7
//   and 16+8q..16+8q+7.  int8 32x32x64: A = compressed bytes 16q..16q+15,
//   index 32 bits; B = k 16q..16q+15 and 32+16q..32+16q+15.
//  dense 32x32x16 (16-bit) / 32x32x32 (int8): A and B = 16 bytes at 16q.
template <int DT, int AMODE, int BKC, int AKC, int BM, int BN, int GV = 0>
__global__ void __launch_bounds__(NTH) gemm_kernel(GemmArgs A) {
  constexpr int ESZ = DT == DT_I8 ? 1 : 2;
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  constexpr int LDS_A = AMODE == A_SPARSE24 ? BM * ASTRIDE_SP : BM * BSTRIDE;
  constexpr int LDS_B = BN * BSTRIDE;
  constexpr bool SERIAL_GATHER = AMODE == A_GATHER && GV == 0;   // general N:M through LDS staging
  constexpr bool REG_GATHER = AMODE == A_GATHER && GV > 0;       // M = 32 through registers
  __shared__ __attribute__((aligned(16))) uint8_t s_a[SERIAL_GATHER ? 1 : 2][LDS_A];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][LDS_B];
  __shared__ __attribute__((aligned(16))) uint8_t s_stg[SERIAL_GATHER ? BM * (STG_V + STG_M) : 16];

  typedef typename Acc<DT>::t acc_t;
  typedef typename Frag<DT>::ab ab_t;

  const int64_t tiles_m = (A.m + BM - 1) / BM, tiles_n = (A.n + BN - 1) / BN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t r0 = tm * BM, c0 = tn * BN;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const int l32 = lane & 31, q = lane >> 5;

  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

  const int64_t KL = KBYTES / ESZ;                  // logical k per step
  const int ksteps = (int)((A.k + KL - 1) / KL);

  KChunks<BN> rb;
  KChunks<BM> ra;
  SpChunks<BM> rs;
  G32Regs<ESZ, BM, GV == 0 ? 4 : GV> rg;
  auto load_step = [&](int ks) {
    const int64_t k0 = (int64_t)ks * KL;
    if (BKC) load_kcontig<ESZ, BN>(rb, A.b, c0, A.n, A.ldb, k0, A.k, A.b_vec);
    else load_mncontig<ESZ, BN>(rb, A.b, c0, A.n, A.ldb, k0, A.k, A.b_vec);
    if (AMODE == A_DENSE) {
      if (AKC) load_kcontig<ESZ, BM>(ra, A.a, r0, A.m, A.lda, k0, A.k, A.a_vec);
      else load_mncontig<ESZ, BM>(ra, A.a, r0, A.m, A.lda, k0, A.k, A.a_vec);
    }
    if (AMODE == A_SPARSE24) load_sp24<ESZ, BM>(rs, A, r0, ks);
    if constexpr (REG_GATHER) load_g32(rg, A, r0, ks);
  };
  auto store_step = [&](int buf, int ks) {
    if (BKC) store_kcontig<BN>(s_b[buf], rb);
    else store_mncontig<ESZ, BN>(s_b[buf], rb);
    if (AMODE == A_DENSE) {
      if (AKC) store_kcontig<BM>(s_a[buf], ra);
      else store_mncontig<ESZ, BM>(s_a[buf], ra);
    }
    if (AMODE == A_SPARSE24) store_sp24<ESZ, BM>(s_a[buf], rs);
    if constexpr (REG_GATHER) expand_g32(s_a[buf], rg, A, ks);
  };

  auto compute = [&](const uint8_t* la, const uint8_t* lb) {
    if constexpr (AMODE == A_SPARSE24) {
      constexpr int MB = ESZ == 2 ? 8 : 16;           // metadata bytes per row per step
#pragma unroll
      for (int h = 0; h < 2; h++) {
        ab_t av[FM];
        int ai[FM];
#pragma unroll
        for (int fm = 0; fm < FM; fm++) {
          const uint8_t* p = la + (wm0 + fm * 32 + l32) * ASTRIDE_SP;
          av[fm] = *(const ab_t*)(p + 32 * h + 16 * q);
          ai[fm] = ESZ == 2 ? (int)*(const uint16_t*)(p + 64 + h * (MB / 2) + 2 * q)
                            : (int)*(const uint32_t*)(p + 64 + h * (MB / 2) + 4 * q);
        }
#pragma unroll
        for (int fn = 0; fn < FN; fn++) {
          const uint8_t* p = lb + (wn0 + fn * 32 + l32) * BSTRIDE + 64 * h;
          const typename Frag<DT>::b2 bv = concat<DT>(*(const ab_t*)(p + 16 * q), *(const ab_t*)(p + 32 + 16 * q));
#pragma unroll
          for (int fm = 0; fm < FM; fm++) acc[fm][fn] = smfmac32<DT>(av[fm], bv, acc[fm][fn], ai[fm]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        ab_t av[FM];
#pragma unroll
        for (int fm = 0; fm < FM; fm++) av[fm] = *(const ab_t*)(la + (wm0 + fm * 32 + l32) * BSTRIDE + 32 * i + 16 * q);
#pragma unroll
        for (int fn = 0; fn < FN; fn++) {
          const ab_t bv = *(const ab_t*)(lb + (wn0 + fn * 32 + l32) * BSTRIDE + 32 * i + 16 * q);
#pragma unroll
          for (int fm = 0; fm < FM; fm++) acc[fm][fn] = mfma32<DT>(av[fm], bv, acc[fm][fn]);
        }
      }
    }
  };

  if constexpr (SERIAL_GATHER) {
    for (int ks = 0; ks < ksteps; ks++) {
      load_step(ks);
      stage_gather<ESZ, BM>(s_stg, A, r0, ks);
      store_step(0, ks);
      __syncthreads();
      expand_gather<ESZ, BM>(s_a[0], s_stg, A, ks);
      __syncthreads();
      compute(s_a[0], s_b[0]);
      __syncthreads();
    }
  } else {
    // Two-deep prefetch: registers hold step s+1 while step s computes; they
    // go to the idle LDS buffer afterwards and the loads for s+2 start.
    if (ksteps > 0) {
      load_step(0);
      store_step(0, 0);
    }
    if (ksteps > 1) load_step(1);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ks++) {
      const int buf = ks & 1;
      compute(s_a[buf], s_b[buf]);
      if (ks + 1 < ksteps) store_step(buf ^ 1, ks + 1);
      if (ks + 2 < ksteps) load_step(ks + 2);
      __syncthreads();
    }
  }

  // ---- epilogue: D = alpha * acc + beta * C ----
#pragma unroll
  for (int fm = 0; fm < FM; fm++)
#pragma unroll
    for (int fn = 0; fn < FN; fn++) {
      const int64_t col = c0 + wn0 + fn * 32 + l32;
      if (col >= A.n) continue;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t row = r0 + wm0 + fm * 32 + 8 * (r / 4) + 4 * q + (r % 4);
        if (row >= A.m) continue;
        if constexpr (DT == DT_I8) {
          int_store(A, row * A.d_rs + col * A.d_cs, int_epilogue(A, acc[fm][fn][r], row * A.c_rs + col * A.c_cs));
        } else {
          float v = A.alpha * acc[fm][fn][r];
          if (A.beta != 0.0f) v += A.beta * from_bits16<DT>(((const uint16_t*)A.c)[row * A.c_rs + col * A.c_cs]);
          ((uint16_t*)A.d)[row * A.d_rs + col * A.d_cs] = to_bits16<DT>(v);
        }
      }
    }
}

// ---------------------------------------------------------------- LDS-DMA ring kernel (NT)

// For op_b = T (B stored n x k, k contiguous) and operands made of whole tiles:
// global memory is copied straight into LDS (global_load_lds_dwordx4: lane i
// of a wave instruction writes 16 bytes at LDS base + 16 i), into a ring of S
// stages, issued S - 1 k-steps ahead, so no registers stage the copies and
// several steps of loads are in flight while the matrix instructions run.
// Because the DMA fixes where each lane's 16 bytes land, the layouts are
// unpadded and XOR-swizzled instead: each lane fetches the chunk that belongs
// in its slot, slot = chunk ^ swz(row).
//   B and dense A rows: 128 bytes = 8 chunks, swz8(r) = (r1 r2 r3) ^ (r0 << 2)
//     (bits of r), i.e. ((r >> 1) & 7) ^ ((r & 1) << 2).
//   2:4 values rows: 64 bytes = 4 chunks, swz4(r) = r2 << 1 | (r1 ^ r3).
//   metadata rows: MB bytes (8 for 16-bit types, 16 for int8), unswizzled.
// A 16-byte LDS read serves 16 lanes per pass when the LDS presents 64 banks
// (8 lanes with 32): with these swizzles the rows that fall on the same banks
// inside either group always read different slots, so one chunk read by 16
// (or 8) consecutive rows is conflict-free in both cases.

template <int N_>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N_ >= 0 && N_ < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N_ & 0xF) | (0x7 << 4) | (0xF << 8) | ((N_ >> 4) << 14));
}

// Barrier that orders LDS accesses only (the asm clobber keeps the compiler
// from moving memory operations across it; the caller waits for its own DMA).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz8(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
__device__ __forceinline__ int swz4(int r) { return (((r >> 2) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1); }

// Global -> LDS copies (each lane's 16 or 4 bytes land at the wave's LDS base
// + lane * size). They are issued from asm so that the compiler does not track
// them: its own tracking cannot tell the LDS reads of other ring slots apart
// from the copies in flight and would drain every copy before such a read.
// The kernels order the copies themselves (per-wave vmcnt waits, then an LDS
// barrier before a slot is read or refilled). M0 carries the LDS address,
// written with the one wait state a copy needs after it. M0 is a reserved
// register the compiler does not let asm declare clobbered, and it is not
// saved here (two scalar instructions per copy, measured 1-8% on the products):
// this is sound because nothing else in these kernels uses M0, which the build
// checks on the compiled assembly of the 16-bit GEMM unit.
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds_wave_base) {
  const uint32_t l = (uint32_t)(uintptr_t)(lds_ptr_t)lds_wave_base;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(l) : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* g, uint8_t* lds_wave_base) {
  const uint32_t l = (uint32_t)(uintptr_t)(lds_ptr_t)lds_wave_base;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(g), "s"(l) : "memory");
}
// The same from a wave-uniform base (scalar registers) plus a 32-bit per-lane
// byte offset, so that no per-lane 64-bit address is formed (the copy-ring
// kernels run only on operands under 2 GiB).
__device__ __forceinline__ void dma16s(const uint8_t* base, uint32_t off, uint8_t* lds_wave_base) {
  const uint32_t l = (uint32_t)(uintptr_t)(lds_ptr_t)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "s"(l) : "memory");
}
__device__ __forceinline__ void dma4s(const uint8_t* base, uint32_t off, uint8_t* lds_wave_base) {
  const uint32_t l = (uint32_t)(uintptr_t)(lds_ptr_t)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" : : "v"(off), "s"(base), "s"(l) : "memory");
}

// op_b = N (B stored k x n): the B stage keeps the 64 k-rows as stored, rows of
// BN * 2 bytes, with 16-byte slot s of row r holding chunk s ^ (4 * (r & 3)).
// Fragments come from the gfx950 transposing LDS read (ds_read_b64_tr_b16):
// within each 16-lane group, output lane j element t is the (j % 4)-th 16-bit
// value of the 8 bytes addressed by lane 4t + j / 4. With lane s addressing
// k-row base + s / 4 at columns c + 4 (s % 4), lane j receives column c + j at
// k = base .. base + 3, i.e. four consecutive k of its own column, which is
// what the matrix instructions' B operand holds. 16-bit types only.
// LAYOUT bit 0: B stored n x k (k-contiguous rows); bit 1: dense A stored k x m
// (op_a = T), staged and read like B stored k x n; bit 2 (2:4, 16-bit types):
// metadata staged four k-steps at a time (32 bytes per row) in a double-buffered
// slot outside the ring, so that a copy instruction moves 32 contiguous bytes of
// a row instead of 8 (a quarter of the cache-line requests per metadata byte).
template <int DT, int AMODE, int BM, int BN, int S, int WGM, int WGN, int LAYOUT>
__global__ void __launch_bounds__(64 * WGM * WGN) gemm_dma_kernel(GemmArgs A) {
  constexpr int BKC = LAYOUT & 1;
  constexpr bool AT = (LAYOUT & 2) != 0;
  constexpr bool M4 = (LAYOUT & 4) != 0;
  static_assert(!AT || AMODE == A_DENSE, "transposed A is dense only");
  constexpr int NW = WGM * WGN;                          // waves per block
  constexpr int ESZ = DT == DT_I8 ? 1 : 2;
  constexpr int KL = KBYTES / ESZ;
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  constexpr int MB = ESZ == 2 ? 8 : 16;                  // metadata bytes per row per step
  constexpr int MDW = MB / 4;
  constexpr bool SP = AMODE == A_SPARSE24;
  constexpr int A_VAL = SP ? BM * 64 : BM * 128;         // values (2:4) or dense A rows
  static_assert(!M4 || (SP && ESZ == 2), "batched metadata: 2:4 with 16-bit types");
  constexpr int A_META = SP && !M4 ? BM * MB : 0;
  constexpr int B_ST = BN * 128;
  constexpr int STAGE = A_VAL + A_META + B_ST;
  constexpr int MSLOT = M4 ? BM * 4 * MB : 0;            // one metadata slot: 4 k-steps of every row
  static_assert(S * STAGE + 2 * MSLOT <= 160 * 1024, "LDS ring too large");
  // DMA wave instructions per stage (64 lanes x 16 or 4 bytes), split evenly over the waves
  constexpr int TB = BN / 8, TA = SP ? BM / 16 : BM / 8, TMT = SP && !M4 ? BM * MDW / 64 : 0;
  constexpr int NMG = M4 ? BM * 2 / 64 / (WGM * WGN) : 0;  // 16-byte metadata copies per wave and slot fill
  static_assert(!M4 || NMG * 64 * WGM * WGN == BM * 2, "metadata slot split");
  // HALF_META: twice as many waves as metadata instructions; each wave then
  // copies its share with the lower 32 lanes (one instruction, so every wave
  // still issues the same number of copies per stage)
  constexpr bool HALF_META = SP && TMT % NW != 0 && 2 * TMT == NW;
  static_assert(TB % NW == 0 && TA % NW == 0 && (TMT % NW == 0 || HALF_META), "DMA split");
  constexpr int NB = TB / NW, NA = TA / NW, NMT = HALF_META ? 1 : TMT / NW;
  constexpr int L = NB + NA + NMT;                       // per wave per stage (same for every wave)
  constexpr int BSLOTS = BN * ESZ / 16;                  // 16-byte slots per stored k-row (op_b = N)
  // op_b = N: LDS slot of 16-byte chunk c of stored k-row r. A 16-lane
  // transposing read covers 4 rows x 32 bytes (16-bit) or 8 rows x 16 bytes
  // (8-bit); these XORs keep every 32-lane phase of it on distinct banks.
  auto nn_slot_w = [](int r, int c, int W) -> int {        // W: tile width (columns) of the stored k-rows
    if constexpr (ESZ == 2) return c ^ (4 * (r & 3));
    else return c ^ (2 * ((r / (256 / W)) % (W * ESZ / 16 / 2)));
  };
  auto nn_slot = [&](int r, int c) -> int { return nn_slot_w(r, c, BN); };
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * STAGE + 2 * MSLOT];
  uint8_t* const mslots = ring + S * STAGE;

  typedef typename Acc<DT>::t acc_t;
  typedef typename Frag<DT>::ab ab_t;
  typedef typename Frag<DT>::b2 b2_t;

  const int64_t tiles_m = A.m / BM, tiles_n = A.n / BN;
  int64_t tm, tn;
  int z = 0;                                             // k range of this block (split-k)
  split_tile_coords(tiles_m, tiles_n, tm, tn, z);
  const int64_t r0 = tm * BM, c0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: keeps LDS/M0 math scalar
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  const int l32 = lane & 31, q = lane >> 5;
  // k-steps [kb, kb + ksteps) of the A.k / KL; the host keeps splits <= k-steps,
  // so every range holds at least one step
  const int ktotal = (int)(A.k / KL);
  const int kb = (int)((int64_t)z * ktotal / A.splits);
  const int ksteps = (int)((int64_t)(z + 1) * ktotal / A.splits) - kb;

  // ---- DMA: block-uniform bases (advanced per step in scalar registers) and
  // per-lane byte offsets computed once ----
  const size_t bstep = BKC ? (size_t)KBYTES : (size_t)KL * A.ldb * ESZ;
  const uint8_t* bbase = A.b + (size_t)(BKC ? c0 * A.ldb : c0) * ESZ + (size_t)kb * bstep;
  const size_t astep = AT ? (size_t)KL * A.lda * ESZ : (size_t)(SP ? 64 : KBYTES);
  const uint8_t* abase = A.a + (size_t)(AT ? r0 : r0 * A.lda) * ESZ + (size_t)kb * astep;
  constexpr int ASLOTS = BM * ESZ / 16;                  // 16-byte slots per stored k-row of A (AT)
  const uint8_t* mbase = A.meta + (size_t)(r0 * A.mld) + (size_t)kb * MB;
  uint32_t ob[NB], oa[NA], om[NMT > 0 ? NMT : 1];
#pragma unroll
  for (int j = 0; j < NB; j++) {
    if (BKC) {
      const int row = 8 * (wave * NB + j) + lane / 8, slot = lane % 8;
      ob[j] = (uint32_t)(row * A.ldb * ESZ + ((slot ^ swz8(row)) << 4));
    } else {
      const int p = 64 * (wave * NB + j) + lane;         // slot index in the stage
      const int row = p / BSLOTS, slot = p % BSLOTS;
      ob[j] = (uint32_t)(row * A.ldb * ESZ + (nn_slot(row, slot) << 4));
    }
  }
#pragma unroll
  for (int j = 0; j < NA; j++) {
    if (AT) {
      const int p = 64 * (wave * NA + j) + lane;         // slot index in the stage
      const int row = p / ASLOTS, slot = p % ASLOTS;
      oa[j] = (uint32_t)(row * A.lda * ESZ + (nn_slot_w(row, slot, BM) << 4));
    } else if (SP) {
      const int row = 16 * (wave * NA + j) + lane / 4, slot = lane % 4;
      oa[j] = (uint32_t)(row * A.lda * ESZ + ((slot ^ swz4(row)) << 4));
    } else {
      const int row = 8 * (wave * NA + j) + lane / 8, slot = lane % 8;
      oa[j] = (uint32_t)(row * A.lda * ESZ + ((slot ^ swz8(row)) << 4));
    }
  }
  // int8 (16 metadata bytes per row and step): stored dword d of row r holds
  // the row's dword d ^ (2 * bit 4 of r), so that the 32 rows a wave reads at
  // once (rows 16 apart otherwise share banks) fall on 64 distinct banks
  auto meta_dw = [](int row, int d) -> int { return ESZ == 1 ? d ^ (((row >> 4) & 1) << 1) : d; };
#pragma unroll
  for (int j = 0; j < NMT; j++) {                        // 4-byte pieces, MDW per row
    const int p = HALF_META ? 32 * wave + (lane & 31) : 64 * (wave * NMT + j) + lane;
    om[j] = (uint32_t)((p / MDW) * A.mld + meta_dw(p / MDW, p % MDW) * 4);
  }
  // Copies of stage st: the wave's L instructions in the order B, A values,
  // metadata; part `part` of `parts` issues those with index % parts == part,
  // so a refill can be spread over the fragment groups of a step.
  // (slot: st % S, passed in so that the steady loop keeps it in a register)
  auto issue_part_at = [&](int st, int slot, int part, int parts) {
    uint8_t* base = ring + slot * STAGE;
    const uint8_t* bp = bbase + (size_t)st * bstep;
    const uint8_t* ap = abase + (size_t)st * astep;
    const uint8_t* mp = mbase + (size_t)st * MB;
#pragma unroll
    for (int j = 0; j < NB; j++)
      if (j % parts == part) dma16s(bp, ob[j], base + A_VAL + A_META + (wave * NB + j) * 1024);
#pragma unroll
    for (int j = 0; j < NA; j++)
      if ((NB + j) % parts == part) dma16s(ap, oa[j], base + (wave * NA + j) * 1024);
#pragma unroll
    for (int j = 0; j < NMT; j++) {
      if ((NB + NA + j) % parts != part) continue;
      if (HALF_META) {
        if (lane < 32) dma4s(mp, om[j], base + A_VAL + wave * 128);
      } else {
        dma4s(mp, om[j], base + A_VAL + (wave * NMT + j) * 256);
      }
    }
  };
  auto issue = [&](int st) { issue_part_at(st, st % S, 0, 1); };
  // Metadata slot fill: k-steps 4 mg .. 4 mg + 3 of every row (32 bytes) into
  // slot mg % 2; lane p of the fill copies 16-byte chunk p % 2 of row p / 2,
  // stored at chunk (p % 2) ^ bit 3 of the row (two rows 8 apart then read
  // different banks). The launch takes this path only without split-k (the
  // block's metadata then starts on a 16-byte boundary); chunks past the row's
  // padded end are clamped into the row and never read.
  uint32_t omr[NMG > 0 ? NMG : 1], omc[NMG > 0 ? NMG : 1];   // row byte offset, chunk byte offset
#pragma unroll
  for (int j = 0; j < NMG; j++) {
    const int p = 64 * (wave * NMG + j) + lane;
    const int row = p / 2;
    omr[j] = (uint32_t)(row * A.mld);
    omc[j] = (uint32_t)((((p % 2) ^ ((row >> 3) & 1))) * 16);
  }
  auto issue_meta = [&](int mg) {
    uint8_t* base = mslots + (mg % 2) * MSLOT;
#pragma unroll
    for (int j = 0; j < NMG; j++) {
      int64_t o = (int64_t)mg * 32 + omc[j];
      if (o + 16 > A.mld) o = A.mld - 16;
      dma16s(A.meta + (size_t)r0 * A.mld, omr[j] + (uint32_t)o, base + (wave * NMG + j) * 1024);
    }
  };

  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

  auto bchunk = [&](const uint8_t* lb, int row, int c) -> ab_t {
    return *(const ab_t*)(lb + row * 128 + ((c ^ swz8(row)) << 4));
  };
  // Four consecutive k (kbase .. kbase+3) of column `col0 + (lane & 15)` for
  // each lane of a 16-lane group, from a stage of stored k-rows W columns wide:
  // B stored k x n (W = BN) or dense A stored k x m (W = BM).
  typedef short short4_t __attribute__((ext_vector_type(4)));
  auto btr4 = [&](const uint8_t* lb, int kbase, int col0, int W = BN) -> short4_t {
    const int sidx = lane & 15;
    const int row = kbase + sidx / 4;
    const int cbyte = (col0 + 4 * (sidx % 4)) * 2;
    const int off = row * (W * 2) + (nn_slot_w(row, cbyte >> 4, W) << 4) + (cbyte & 15);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(lb + off));
  };
  // int8: eight consecutive k (kbase .. kbase+7) of column `col0 + (lane & 15)`;
  // with lane s addressing k-row kbase + s / 2 at columns col0 + 8 (s % 2), lane
  // j of each 16-lane group receives byte j % 8 of the 8 bytes addressed by
  // lane 2t + j / 8 as its element t (ds_read_b64_tr_b8, measured on gfx950)
  typedef int int2_t __attribute__((ext_vector_type(2)));
  auto btr8 = [&](const uint8_t* lb, int kbase, int col0, int W = BN) -> int2_t {
    const int sidx = lane & 15;
    const int row = kbase + sidx / 2;
    const int cbyte = col0 + 8 * (sidx % 2);
    const int off = row * W + (nn_slot_w(row, cbyte >> 4, W) << 4) + (cbyte & 15);
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) int2_t*)(lb + off));
  };
  // column base of this lane's 16-lane group inside a 32-column fragment
  const int nb16 = lane & 16;

  // ---- fragment groups: a step is G groups; group g's LDS reads are issued
  // before group g-1's matrix instructions. The last group of a step first
  // waits for the next stage, passes the barrier (which frees the slot of the
  // current stage) and reads the next step's first group, so the step
  // boundary does not drain the matrix pipeline. The refill of the freed slot
  // is spread over the next step's groups: a burst of copies would stall the
  // issuing waves on the address unit while their matrix work waits. ----
  constexpr int G = SP ? 2 * FN : 4;
  static_assert(G % 2 == 0, "fragment slots alternate across steps");
  ab_t av[2][FM];
  int iv[2][FM];
  int ivn[FM];                                           // 16-bit types: second half-step's metadata, staged
  int ivo[M4 ? FM : 1][2];                               // batched metadata: the next (odd) step's two words
  b2_t bv[2];
  ab_t bw[2][FN];
  const int qshift = 16 * q;
  // PH: ks % 4 when the caller knows it statically (0 .. 3), else -1
  auto load_group = [&](const uint8_t* st, int g, int ks, auto ph_t) {
    constexpr int PH = decltype(ph_t)::value;
    if constexpr (SP) {
      const uint8_t* la = st;
      const uint8_t* lm = st + A_VAL;
      const uint8_t* lb = st + A_VAL + A_META;
      const int h = g / FN, fn = g % FN;
      if (fn == 0) {
#pragma unroll
        for (int fm = 0; fm < FM; fm++) {
          const int row = wm0 + fm * 32 + l32;
          const int c = 2 * h + q;
          av[h][fm] = *(const ab_t*)(la + row * 64 + ((c ^ swz4(row)) << 4));
          if constexpr (ESZ == 2) {
            // one 8-byte read per row serves both half-steps and both lane
            // halves; the lane's 16 bits are selected at use (shift by 16 q)
            if (h == 0) {
              if constexpr (M4) {
                // steps ks and ks + 1 (ks even) sit in one 16-byte chunk of the
                // row's 32 bytes in slot (ks / 4) % 2: one 16-byte read every
                // other step, whose 16-lane passes (32 rows, two 16-byte
                // chunks apart by bit 3 of the row) fall on distinct banks;
                // the odd step's words wait in registers
                const int k3 = PH >= 0 ? PH : (ks & 3);
                if ((k3 & 1) == 0) {
                  const u32x4 mw = *(const u32x4*)(mslots + ((ks >> 2) & 1) * MSLOT + row * 32 +
                                                   ((((k3 >> 1) ^ (row >> 3)) & 1) << 4));
                  iv[0][fm] = (int)mw[0];
                  ivn[fm] = (int)mw[1];
                  ivo[fm][0] = (int)mw[2];
                  ivo[fm][1] = (int)mw[3];
                } else {
                  iv[0][fm] = ivo[fm][0];
                  ivn[fm] = ivo[fm][1];
                }
              } else {
                typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                const u32x2_t mw = *(const u32x2_t*)(lm + row * MB);
                iv[0][fm] = (int)mw[0];
                ivn[fm] = (int)mw[1];
              }
            } else {
              iv[1][fm] = ivn[fm];
            }
          } else {
            iv[h][fm] = (int)*(const uint32_t*)(lm + row * MB + 4 * meta_dw(row, 2 * h + q));
          }
        }
      }
      if constexpr (BKC) {
        const int row = wn0 + fn * 32 + l32;
        bv[g % 2] = concat<DT>(bchunk(lb, row, 4 * h + q), bchunk(lb, row, 4 * h + 2 + q));
      } else if constexpr (ESZ == 2) {
        // k = 32h + 8q + {0..3, 4..7, 16..19, 20..23}
        const int cb = wn0 + fn * 32 + nb16;
        const int kb = 32 * h + 8 * q;
        const short4_t r0 = btr4(lb, kb, cb), r1 = btr4(lb, kb + 4, cb), r2 = btr4(lb, kb + 16, cb),
                       r3 = btr4(lb, kb + 20, cb);
        typedef short short16_t __attribute__((ext_vector_type(16)));
        const short16_t v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3],
                             r2[0], r2[1], r2[2], r2[3], r3[0], r3[1], r3[2], r3[3]};
        bv[g % 2] = __builtin_bit_cast(b2_t, v);
      } else {
        // int8: k = 64h + 16q + {0..7, 8..15, 32..39, 40..47}
        const int cb = wn0 + fn * 32 + nb16;
        const int kb = 64 * h + 16 * q;
        const int2_t r0 = btr8(lb, kb, cb), r1 = btr8(lb, kb + 8, cb), r2 = btr8(lb, kb + 32, cb),
                     r3 = btr8(lb, kb + 40, cb);
        bv[g % 2] = b2_t{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
      }
    } else {
      const uint8_t* la = st;
      const uint8_t* lb = st + A_VAL;
#pragma unroll
      for (int fm = 0; fm < FM; fm++) {
        if constexpr (!AT) {
          av[g % 2][fm] = bchunk(la, wm0 + fm * 32 + l32, 2 * g + q);
        } else if constexpr (ESZ == 2) {
          // the same k of the lane's row (column of the stored k-rows) as bchunk gives
          const int ca = wm0 + fm * 32 + nb16;
          const short4_t r0 = btr4(la, 16 * g + 8 * q, ca, BM), r1 = btr4(la, 16 * g + 8 * q + 4, ca, BM);
          typedef short short8_t __attribute__((ext_vector_type(8)));
          const short8_t v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
          av[g % 2][fm] = __builtin_bit_cast(ab_t, v);
        } else {
          const int ca = wm0 + fm * 32 + nb16;
          const int2_t r0 = btr8(la, 32 * g + 16 * q, ca, BM), r1 = btr8(la, 32 * g + 16 * q + 8, ca, BM);
          av[g % 2][fm] = ab_t{r0[0], r0[1], r1[0], r1[1]};
        }
      }
#pragma unroll
      for (int fn = 0; fn < FN; fn++) {
        if constexpr (BKC) {
          bw[g % 2][fn] = bchunk(lb, wn0 + fn * 32 + l32, 2 * g + q);
        } else if constexpr (ESZ == 2) {
          // k = 16g + 8q + 0..7
          const int cb = wn0 + fn * 32 + nb16;
          const short4_t r0 = btr4(lb, 16 * g + 8 * q, cb), r1 = btr4(lb, 16 * g + 8 * q + 4, cb);
          typedef short short8_t __attribute__((ext_vector_type(8)));
          const short8_t v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
          bw[g % 2][fn] = __builtin_bit_cast(ab_t, v);
        } else {
          // int8: k = 32g + 16q + 0..15
          const int cb = wn0 + fn * 32 + nb16;
          const int2_t r0 = btr8(lb, 32 * g + 16 * q, cb), r1 = btr8(lb, 32 * g + 16 * q + 8, cb);
          bw[g % 2][fn] = ab_t{r0[0], r0[1], r1[0], r1[1]};
        }
      }
    }
  };
  auto compute_group = [&](int g) {
    if constexpr (SP) {
      const int h = g / FN, fn = g % FN;
#pragma unroll
      for (int fm = 0; fm < FM; fm++)
        acc[fm][fn] = smfmac32<DT>(av[h][fm], bv[g % 2], acc[fm][fn],
                                   ESZ == 2 ? (int)((uint32_t)iv[h][fm] >> qshift) : iv[h][fm]);
    } else {
#pragma unroll
      for (int fn = 0; fn < FN; fn++)
#pragma unroll
        for (int fm = 0; fm < FM; fm++) acc[fm][fn] = mfma32<DT>(av[g % 2][fm], bw[g % 2][fn], acc[fm][fn]);
    }
  };

  // waits until at most n (0 <= n <= S-1) of this wave's issued stages are outstanding
  static_assert(L * (S - 1) <= 63 && S <= 6, "vmcnt range");
  auto wait_stages = [&](int n) {
    if (S > 5 && n >= 5) wait_vmcnt<L * (S > 5 ? 5 : 0)>();
    else if (S > 4 && n == 4) wait_vmcnt<L * (S > 4 ? 4 : 0)>();
    else if (S > 3 && n == 3) wait_vmcnt<L * (S > 3 ? 3 : 0)>();
    else if (n == 2) wait_vmcnt<L * 2>();
    else if (n == 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
  };
  // every slot is filled up front; stage 0 is complete once at most stages
  // 1 .. min(S-1, ksteps-1) are outstanding (the first metadata slot is
  // filled before stage 0)
  if constexpr (M4) issue_meta(0);
#pragma unroll
  for (int st = 0; st < S; st++)
    if (st < ksteps) issue(st);
  wait_stages(min(S - 1, ksteps - 1));
  lds_barrier();
  load_group(ring, 0, 0, std::integral_constant<int, 0>{});
  // One k-step. REFILL (every step but the first and the last S - 1): stage
  // ks + S - 1 goes into the slot freed at the end of step ks - 1, and stage
  // ks + 1 exists; the two kinds of step are separate copies of the body, so
  // the steady loop carries no per-group tests. cur = ks % S is kept in a
  // register rather than recomputed.
  // PH: ks % 4 when known statically (else -1)
  auto kstep = [&](int ks, int cur, auto refill_t, auto ph_t) {
    constexpr bool REFILL = decltype(refill_t)::value;
    constexpr int PH = decltype(ph_t)::value;
    typedef std::integral_constant<int, PH < 0 ? -1 : (PH + 1) & 3> next_ph;
    const int nxt = cur + 1 == S ? 0 : cur + 1;          // (ks + 1) % S
    const int fil = cur == 0 ? S - 1 : cur - 1;          // (ks + S - 1) % S
    const uint8_t* st = ring + cur * STAGE;
    // batched metadata: the slot for k-steps ks + 4 .. ks + 7 is filled at the
    // start of every fourth step (the slot it overwrites was last read at the
    // start of step ks - 1), before that step's ring refill
    const bool meta_fill = M4 && (PH >= 0 ? PH : (ks & 3)) == 0 && ks + 4 < ksteps;
#pragma unroll
    for (int g = 0; g < G; g++) {
      if constexpr (M4) {
        if (g == 0 && meta_fill) issue_meta((ks >> 2) + 1);
      }
      if constexpr (REFILL) issue_part_at(ks + S - 1, fil, g, G);
      if (g + 1 < G) {
        load_group(st, g + 1, ks, ph_t);
      } else if (REFILL || ks + 1 < ksteps) {
        // issued so far: stages up to min(ks+S-1, ksteps-1); stage ks+1 is
        // complete once at most stages ks+2 .. min(ks+S-1, ksteps-1) (and
        // this step's metadata fill, issued after stage ks+1) are outstanding
        if constexpr (M4) {
          static_assert(S == 3, "batched metadata runs with a three-stage ring");
          const bool next_stage = REFILL || ks + 2 < ksteps;
          if (next_stage && meta_fill) wait_vmcnt<L + NMG>();
          else if (next_stage) wait_vmcnt<L>();
          else if (meta_fill) wait_vmcnt<NMG>();
          else wait_vmcnt<0>();
        } else if constexpr (REFILL) {
          wait_stages(S - 2);
        } else {
          wait_stages(min(S - 2, ksteps - ks - 2));
        }
        lds_barrier();                                   // every wave is done reading stage ks
        load_group(ring + nxt * STAGE, 0, ks + 1, next_ph{});
      }
      compute_group(g);
    }
    return nxt;
  };
  typedef std::integral_constant<int, -1> phx;
  int cur = kstep(0, 0, std::false_type{}, std::integral_constant<int, 0>{});
  int ks = 1;
  // steady steps four at a time from ks = 1, so that ks % 4 (which the batched
  // metadata reads and fills depend on) is static in the loop body
  if constexpr (M4) {
    for (; ks + 3 + S - 1 < ksteps; ks += 4) {
      cur = kstep(ks, cur, std::true_type{}, std::integral_constant<int, 1>{});
      cur = kstep(ks + 1, cur, std::true_type{}, std::integral_constant<int, 2>{});
      cur = kstep(ks + 2, cur, std::true_type{}, std::integral_constant<int, 3>{});
      cur = kstep(ks + 3, cur, std::true_type{}, std::integral_constant<int, 0>{});
    }
  }
  for (; ks + S - 1 < ksteps; ks++) cur = kstep(ks, cur, std::true_type{}, phx{});
  for (; ks < ksteps; ks++) cur = kstep(ks, cur, std::false_type{}, phx{});

  // ---- split-k: this block's partial sums go to plane z of the workspace, in
  // D's storage order, raw (alpha, beta and rounding are applied once, by the
  // reduction over the planes) ----
  if (A.splits > 1) {
    typedef typename std::conditional<DT == DT_I8, int32_t, float>::type raw_t;
    typedef typename std::conditional<DT == DT_I8, intx4, floatx4>::type raw4_t;
    raw_t* plane = (raw_t*)A.ws + (size_t)z * (size_t)(A.m * A.n);
#pragma unroll
    for (int fm = 0; fm < FM; fm++)
#pragma unroll
      for (int fn = 0; fn < FN; fn++) {
        const int64_t col = c0 + wn0 + fn * 32 + l32;
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          const int64_t row = r0 + wm0 + fm * 32 + 8 * r4 + 4 * q;
          if (A.cd_col) {
            // four consecutive rows of one column: one 16-byte store
            *(raw4_t*)(plane + col * A.m + row) = raw4_t{(raw_t)acc[fm][fn][4 * r4], (raw_t)acc[fm][fn][4 * r4 + 1],
                                                          (raw_t)acc[fm][fn][4 * r4 + 2], (raw_t)acc[fm][fn][4 * r4 + 3]};
          } else {
#pragma unroll
            for (int t4 = 0; t4 < 4; t4++) plane[(row + t4) * A.n + col] = (raw_t)acc[fm][fn][4 * r4 + t4];
          }
        }
      }
    return;
  }

  // ---- epilogue: D = alpha * acc + beta * C ----
  if constexpr (DT != DT_I8) {
    // column-major 16-bit D with beta = 0: the block tile goes through the
    // (now idle) ring in column-major order, then every 16-byte store covers
    // consecutive rows of one column, so a column of the tile leaves as whole
    // lines instead of one 8-byte piece per lane and line
    constexpr int CP = BM + 8;                               // LDS column pitch (elements)
    if constexpr (BN * CP * 2 <= S * STAGE) {
      if (A.cd_col && A.beta == 0.0f) {
        __syncthreads();                                     // every wave is done reading the ring
        uint16_t* tile = (uint16_t*)ring;
#pragma unroll
        for (int fm = 0; fm < FM; fm++)
#pragma unroll
          for (int fn = 0; fn < FN; fn++)
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
              const int cl = wn0 + fn * 32 + l32, rl = wm0 + fm * 32 + 8 * r4 + 4 * q;
              const uint32_t lo = (uint32_t)to_bits16<DT>(A.alpha * acc[fm][fn][4 * r4]) |
                                  ((uint32_t)to_bits16<DT>(A.alpha * acc[fm][fn][4 * r4 + 1]) << 16);
              const uint32_t hi = (uint32_t)to_bits16<DT>(A.alpha * acc[fm][fn][4 * r4 + 2]) |
                                  ((uint32_t)to_bits16<DT>(A.alpha * acc[fm][fn][4 * r4 + 3]) << 16);
              *(u32x2*)(tile + cl * CP + rl) = u32x2{lo, hi};
            }
        __syncthreads();
        constexpr int PIECES = BM * 2 / 16;                  // 16-byte pieces per tile column
        for (int i = threadIdx.x; i < BN * PIECES; i += 64 * NW) {
          const int c = i / PIECES, pc = i % PIECES;
          const u32x4 v = *(const u32x4*)(tile + c * CP + 8 * pc);
          *(u32x4*)((uint16_t*)A.d + (c0 + c) * A.d_cs + r0 + 8 * pc) = v;
        }
        return;
      }
    }
    // row-major 16-bit D with beta = 0: the same through a row-major image of
    // the tile, so the stores run along rows 16 bytes per lane
    constexpr int RP = BN + 8;                               // LDS row pitch (elements)
    if constexpr (BM * RP * 2 <= S * STAGE) {
      if (!A.cd_col && A.beta == 0.0f) {
        __syncthreads();
        uint16_t* tile = (uint16_t*)ring;
#pragma unroll
        for (int fm = 0; fm < FM; fm++)
#pragma unroll
          for (int fn = 0; fn < FN; fn++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int rl = wm0 + fm * 32 + 8 * (r / 4) + 4 * q + (r % 4), cl = wn0 + fn * 32 + l32;
              tile[rl * RP + cl] = to_bits16<DT>(A.alpha * acc[fm][fn][r]);
            }
        __syncthreads();
        constexpr int PIECES = BN * 2 / 16;                  // 16-byte pieces per tile row
        for (int i = threadIdx.x; i < BM * PIECES; i += 64 * NW) {
          const int rr = i / PIECES, pc = i % PIECES;
          const u32x4 v = *(const u32x4*)(tile + rr * RP + 8 * pc);
          *(u32x4*)((uint16_t*)A.d + (r0 + rr) * A.d_rs + c0 + 8 * pc) = v;
        }
        return;
      }
    }
  }
  {
    // beta != 0 (any D type; 16-bit D with beta = 0 took the path above): the raw 4-byte
    // accumulators go through the ring (when the whole tile does not fit, in
    // rounds: row-major D one fragment column of every wave per round,
    // column-major D one wave column group per round), then each thread step
    // takes four consecutive elements of a D row (column) with one 16-byte LDS
    // read, reads the matching C elements as one vector, applies alpha and beta
    // exactly as the direct path does and stores one vector. In the row-major
    // rounds the C loads of four thread steps are issued before any is waited
    // for (one at a time, each load's latency was paid in full: int8 4096^3
    // with int32 C, 74-77 -> 69-72 us)
    typedef typename std::conditional<DT == DT_I8, int32_t, float>::type raw_t;
    typedef typename std::conditional<DT == DT_I8, intx4, floatx4>::type raw4_t;
    constexpr int P4 = 4;                                    // pitch padding (elements)
    constexpr int LINE = BN + P4, COLP = BM + P4;
    constexpr int RR = BM * LINE * 4 <= S * STAGE ? 1 : WGM; // rounds, row-major image
    constexpr int RC = BN * COLP * 4 <= S * STAGE ? 1 : WGN; // rounds, column-major image
    constexpr bool FIT_R = (BM / RR) * LINE * 4 <= S * STAGE, FIT_C = (BN / RC) * COLP * 4 <= S * STAGE;
    // measured (4096^3 int8, copy-ring kernel): beta != 0 int32 110 -> 85 us, int8 92 -> 77 us; with
    // beta = 0 the integer stores straight from the accumulators are as fast or faster (61 vs 63 us,
    // int8 65 vs 73 us), so only a C operand takes this path
    if constexpr (FIT_R && FIT_C) if (A.beta != 0.0f) {
      raw_t* img = (raw_t*)ring;
      const int wr = wave / WGN, wc = wave % WGN;
      // C of four consecutive elements of one D row (colmajor: one D column) at
      // (row, col): 16 bytes of int32 C, 4 of int8 C, 8 of 16-bit C
      struct C4 { uint32_t w[4]; };
      auto cindex = [&](int64_t row, int64_t col, bool colmajor) -> int64_t {
        return colmajor ? col * A.c_cs + row : row * A.c_rs + col;
      };
      // cd8: int8 C and D (the integer path's runtime flag, decided outside the
      // batched loop below so that its loads are not split by branches)
      auto load_c4t = [&](auto cd8, int64_t cidx, C4& c) {
        if constexpr (DT == DT_I8) {
          if constexpr (decltype(cd8)::value) {
            c.w[0] = *(const uint32_t*)((const int8_t*)A.c + cidx);
          } else {
            const intx4 cv = *(const intx4*)((const int32_t*)A.c + cidx);
            c.w[0] = (uint32_t)cv[0]; c.w[1] = (uint32_t)cv[1]; c.w[2] = (uint32_t)cv[2]; c.w[3] = (uint32_t)cv[3];
          }
        } else {
          const u32x2 cv = *(const u32x2*)((const uint16_t*)A.c + cidx);
          c.w[0] = cv[0]; c.w[1] = cv[1];
        }
      };
      auto finish4c = [&](const raw_t (&a4)[4], const C4& c, int64_t didx) {
        if constexpr (DT == DT_I8) {
          int64_t v[4];
#pragma unroll
          for (int t = 0; t < 4; t++) v[t] = (int64_t)A.alpha * a4[t];
          if (A.cd_i8) {
#pragma unroll
            for (int t = 0; t < 4; t++) v[t] += (int64_t)A.beta * (int64_t)(int8_t)(c.w[0] >> (8 * t));
            uint32_t o = 0;
#pragma unroll
            for (int t = 0; t < 4; t++) o |= ((uint32_t)sat_i8(v[t]) & 0xFFu) << (8 * t);
            *(uint32_t*)((int8_t*)A.d + didx) = o;
          } else {
#pragma unroll
            for (int t = 0; t < 4; t++) v[t] += (int64_t)A.beta * (int64_t)(int32_t)c.w[t];
            *(intx4*)((int32_t*)A.d + didx) = intx4{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
          }
        } else {
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; t++) v[t] = A.alpha * a4[t];
          v[0] += A.beta * from_bits16<DT>((uint16_t)(c.w[0] & 0xFFFFu));
          v[1] += A.beta * from_bits16<DT>((uint16_t)(c.w[0] >> 16));
          v[2] += A.beta * from_bits16<DT>((uint16_t)(c.w[1] & 0xFFFFu));
          v[3] += A.beta * from_bits16<DT>((uint16_t)(c.w[1] >> 16));
          const uint32_t lo = (uint32_t)to_bits16<DT>(v[0]) | ((uint32_t)to_bits16<DT>(v[1]) << 16);
          const uint32_t hi = (uint32_t)to_bits16<DT>(v[2]) | ((uint32_t)to_bits16<DT>(v[3]) << 16);
          *(u32x2*)((uint16_t*)A.d + didx) = u32x2{lo, hi};
        }
      };
      auto finish4 = [&](const raw_t (&a4)[4], int64_t row, int64_t col, bool colmajor) {
        C4 c{{0u, 0u, 0u, 0u}};
        if (DT == DT_I8 && A.cd_i8) load_c4t(std::true_type{}, cindex(row, col, colmajor), c);
        else load_c4t(std::false_type{}, cindex(row, col, colmajor), c);
        finish4c(a4, c, colmajor ? col * A.d_cs + row : row * A.d_rs + col);
      };
      // Row-major image drain, batched: the C loads of U thread steps are
      // issued before any of them is waited for. The image holds W columns of
      // the tile per row (BM rows); image column j maps to tile column colmap(j).
      auto drain_rows_t = [&](auto cd8, int W, int LP, auto colmap) {
        const int qpr = W / 4, steps = BM * qpr / (64 * NW);
        constexpr int U = 4;
#pragma unroll 1
        for (int s0 = 0; s0 < steps; s0 += U) {
          C4 cv[U];
#pragma unroll
          for (int u = 0; u < U; u++) {
            const int i = threadIdx.x + (s0 + u) * 64 * NW;
            cv[u] = C4{{0u, 0u, 0u, 0u}};
            if (s0 + u < steps) load_c4t(cd8, cindex(r0 + i / qpr, c0 + colmap(4 * (i % qpr)), false), cv[u]);
          }
#pragma unroll
          for (int u = 0; u < U; u++) {
            if (s0 + u >= steps) break;
            const int i = threadIdx.x + (s0 + u) * 64 * NW;
            const int rr = i / qpr, j = 4 * (i % qpr);
            const raw4_t w = *(const raw4_t*)(img + rr * LP + j);
            raw_t a4[4];
#pragma unroll
            for (int t = 0; t < 4; t++) a4[t] = w[t];
            finish4c(a4, cv[u], (r0 + rr) * A.d_rs + c0 + colmap(j));
          }
        }
      };
      auto drain_rows = [&](int W, int LP, auto colmap) {
        if (DT == DT_I8 && A.cd_i8) drain_rows_t(std::true_type{}, W, LP, colmap);
        else drain_rows_t(std::false_type{}, W, LP, colmap);
      };
      if (!A.cd_col) {
        constexpr int LINEF = WGN * 32 + P4;               // one 32-column strip per wave column
        if constexpr (RR > 1 && BM * LINEF * 4 <= S * STAGE) {
          // the whole tile does not fit: round f takes every wave's fragment
          // column f (all rows; a 32-column strip per wave column), so each
          // round frees a share of every wave's accumulators
#pragma unroll
          for (int f = 0; f < FN; f++) {
            __syncthreads();
#pragma unroll
            for (int fm = 0; fm < FM; fm++)
#pragma unroll
              for (int r = 0; r < 16; r++) {
                const int rl = wm0 + fm * 32 + 8 * (r / 4) + 4 * q + (r % 4);
                img[rl * LINEF + wc * 32 + l32] = (raw_t)acc[fm][f][r];
              }
            __syncthreads();
            drain_rows(WGN * 32, LINEF, [f](int j) { return (j / 32) * WN + f * 32 + (j % 32); });
          }
        } else {
          constexpr int ROWS = BM / RR, QPR = BN / 4;
#pragma unroll 1
          for (int rd = 0; rd < RR; rd++) {
            __syncthreads();                                 // the ring (or the previous round) is free
            if (RR == 1 || wr == rd) {
#pragma unroll
              for (int fm = 0; fm < FM; fm++)
#pragma unroll
                for (int fn = 0; fn < FN; fn++)
#pragma unroll
                  for (int r = 0; r < 16; r++) {
                    const int rl = wm0 + fm * 32 + 8 * (r / 4) + 4 * q + (r % 4) - rd * ROWS;
                    img[rl * LINE + wn0 + fn * 32 + l32] = (raw_t)acc[fm][fn][r];
                  }
            }
            __syncthreads();
            for (int i = threadIdx.x; i < ROWS * QPR; i += 64 * NW) {
              const int rr = i / QPR, qc = i % QPR;
              const raw4_t w = *(const raw4_t*)(img + rr * LINE + 4 * qc);
              raw_t a4[4];
#pragma unroll
              for (int t = 0; t < 4; t++) a4[t] = w[t];
              finish4(a4, r0 + rd * ROWS + rr, c0 + 4 * qc, false);
            }
          }
        }
      } else {
        constexpr int COLS = BN / RC, QPC = BM / 4;
#pragma unroll 1
        for (int rd = 0; rd < RC; rd++) {
          __syncthreads();
          if (RC == 1 || wc == rd) {
#pragma unroll
            for (int fm = 0; fm < FM; fm++)
#pragma unroll
              for (int fn = 0; fn < FN; fn++)
#pragma unroll
                for (int r4 = 0; r4 < 4; r4++) {
                  const int cl = wn0 + fn * 32 + l32 - rd * COLS, rl = wm0 + fm * 32 + 8 * r4 + 4 * q;
                  *(raw4_t*)(img + cl * COLP + rl) = raw4_t{(raw_t)acc[fm][fn][4 * r4], (raw_t)acc[fm][fn][4 * r4 + 1],
                                                           (raw_t)acc[fm][fn][4 * r4 + 2], (raw_t)acc[fm][fn][4 * r4 + 3]};
                }
          }
          __syncthreads();
          for (int i = threadIdx.x; i < COLS * QPC; i += 64 * NW) {
            const int cc = i / QPC, qr = i % QPC;
            const raw4_t w = *(const raw4_t*)(img + cc * COLP + 4 * qr);
            raw_t a4[4];
#pragma unroll
            for (int t = 0; t < 4; t++) a4[t] = w[t];
            finish4(a4, r0 + 4 * qr, c0 + rd * COLS + cc, true);
          }
        }
      }
      return;
    }
  }
  if (A.cd_col) {
    // column-major C/D: accumulator elements 4(r/4) .. 4(r/4)+3 of a lane are
    // four consecutive rows of one column, i.e. 8 (16-bit), 16 (int32) or 4
    // (int8) contiguous bytes; full tiles and the 16-byte column rule keep
    // them aligned
#pragma unroll
    for (int fm = 0; fm < FM; fm++)
#pragma unroll
      for (int fn = 0; fn < FN; fn++) {
        const int64_t col = c0 + wn0 + fn * 32 + l32;
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          const int64_t row = r0 + wm0 + fm * 32 + 8 * r4 + 4 * q;
          if constexpr (DT == DT_I8) {
            int64_t v[4];
#pragma unroll
            for (int t = 0; t < 4; t++) v[t] = (int64_t)A.alpha * acc[fm][fn][4 * r4 + t];
            if (A.cd_i8) {   // four int8 rows: one dword
              if (A.beta != 0.0f) {
                const uint32_t cv = *(const uint32_t*)((const int8_t*)A.c + col * A.c_cs + row);
#pragma unroll
                for (int t = 0; t < 4; t++) v[t] += (int64_t)A.beta * (int64_t)(int8_t)(cv >> (8 * t));
              }
              uint32_t o = 0;
#pragma unroll
              for (int t = 0; t < 4; t++) o |= ((uint32_t)sat_i8(v[t]) & 0xFFu) << (8 * t);
              *(uint32_t*)((int8_t*)A.d + col * A.d_cs + row) = o;
              continue;
            }
            if (A.beta != 0.0f) {
              const intx4 cv = *(const intx4*)((const int32_t*)A.c + col * A.c_cs + row);
#pragma unroll
              for (int t = 0; t < 4; t++) v[t] += (int64_t)A.beta * cv[t];
            }
            *(intx4*)((int32_t*)A.d + col * A.d_cs + row) = intx4{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
          } else {
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; t++) v[t] = A.alpha * acc[fm][fn][4 * r4 + t];
            if (A.beta != 0.0f) {
              const u32x2 cv = *(const u32x2*)((const uint16_t*)A.c + col * A.c_cs + row);
              v[0] += A.beta * from_bits16<DT>((uint16_t)(cv[0] & 0xFFFFu));
              v[1] += A.beta * from_bits16<DT>((uint16_t)(cv[0] >> 16));
              v[2] += A.beta * from_bits16<DT>((uint16_t)(cv[1] & 0xFFFFu));
              v[3] += A.beta * from_bits16<DT>((uint16_t)(cv[1] >> 16));
            }
            const uint32_t lo = (uint32_t)to_bits16<DT>(v[0]) | ((uint32_t)to_bits16<DT>(v[1]) << 16);
            const uint32_t hi = (uint32_t)to_bits16<DT>(v[2]) | ((uint32_t)to_bits16<DT>(v[3]) << 16);
            *(u32x2*)((uint16_t*)A.d + col * A.d_cs + row) = u32x2{lo, hi};
          }
        }
      }
    return;
  }
#pragma unroll
  for (int fm = 0; fm < FM; fm++)
#pragma unroll
    for (int fn = 0; fn < FN; fn++) {
      const int64_t col = c0 + wn0 + fn * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t row = r0 + wm0 + fm * 32 + 8 * (r / 4) + 4 * q + (r % 4);
        if constexpr (DT == DT_I8) {
          int_store(A, row * A.d_rs + col, int_epilogue(A, acc[fm][fn][r], row * A.c_rs + col));
        } else {
          float v = A.alpha * acc[fm][fn][r];
          if (A.beta != 0.0f) v += A.beta * from_bits16<DT>(((const uint16_t*)A.c)[row * A.c_rs + col]);
          ((uint16_t*)A.d)[row * A.d_rs + col] = to_bits16<DT>(v);
        }
      }
    }
}

// ---------------------------------------------------------------- split-k reduction

// D = alpha * (sum over the planes of the partial sums) + beta * C, four
// consecutive elements of D's storage order per thread: planes added in order
// z = 0, 1, ... in fp32 (exactly in int32 for int8, then alpha and beta in
// int64 as in every integer epilogue), rounded to nearest even once. The
// split-k shapes are whole tiles, so every line (row of row-major D, column of
// column-major D) is a multiple of 128 elements long.
template <int DT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmArgs A) {
  typedef typename std::conditional<DT == DT_I8, intx4, floatx4>::type raw4_t;
  const int64_t len = A.cd_col ? A.m : A.n;             // elements per stored line
  const int64_t quads = A.m * A.n / 4;
  const int64_t qid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (qid >= quads) return;
  const int64_t line = qid / (len / 4), off = (qid % (len / 4)) * 4;
  const int64_t plane = A.m * A.n;
  raw4_t sum = *(const raw4_t*)((const uint8_t*)A.ws + (size_t)(qid * 4) * 4);
  for (int z = 1; z < A.splits; z++) {
    const raw4_t p = *(const raw4_t*)((const uint8_t*)A.ws + (size_t)(z * plane + qid * 4) * 4);
    sum += p;
  }
  const int64_t cld = A.cd_col ? A.c_cs : A.c_rs, dld = A.cd_col ? A.d_cs : A.d_rs;
  const int64_t cidx = line * cld + off, didx = line * dld + off;
  if constexpr (DT == DT_I8) {
    int64_t v[4];
#pragma unroll
    for (int t = 0; t < 4; t++) v[t] = (int64_t)A.alpha * sum[t];
    if (A.beta != 0.0f) {
      if (A.cd_i8) {
        const uint32_t cv = *(const uint32_t*)((const int8_t*)A.c + cidx);
#pragma unroll
        for (int t = 0; t < 4; t++) v[t] += (int64_t)A.beta * (int64_t)(int8_t)(cv >> (8 * t));
      } else {
        const intx4 cv = *(const intx4*)((const int32_t*)A.c + cidx);
#pragma unroll
        for (int t = 0; t < 4; t++) v[t] += (int64_t)A.beta * cv[t];
      }
    }
    if (A.cd_i8) {
      uint32_t o = 0;
#pragma unroll
      for (int t = 0; t < 4; t++) o |= ((uint32_t)sat_i8(v[t]) & 0xFFu) << (8 * t);
      *(uint32_t*)((int8_t*)A.d + didx) = o;
    } else {
      *(intx4*)((int32_t*)A.d + didx) = intx4{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
    }
  } else {
    float v[4];
#pragma unroll
    for (int t = 0; t < 4; t++) v[t] = A.alpha * sum[t];
    if (A.beta != 0.0f) {
      const u32x2 cv = *(const u32x2*)((const uint16_t*)A.c + cidx);
      v[0] += A.beta * from_bits16<DT>((uint16_t)(cv[0] & 0xFFFFu));
      v[1] += A.beta * from_bits16<DT>((uint16_t)(cv[0] >> 16));
      v[2] += A.beta * from_bits16<DT>((uint16_t)(cv[1] & 0xFFFFu));
      v[3] += A.beta * from_bits16<DT>((uint16_t)(cv[1] >> 16));
    }
    const uint32_t lo = (uint32_t)to_bits16<DT>(v[0]) | ((uint32_t)to_bits16<DT>(v[1]) << 16);
    const uint32_t hi = (uint32_t)to_bits16<DT>(v[2]) | ((uint32_t)to_bits16<DT>(v[3]) << 16);
    *(u32x2*)((uint16_t*)A.d + didx) = u32x2{lo, hi};
  }
}

// ---------------------------------------------------------------- tile launch (per element type)

// Block tile: 256 x 256 when that still gives most CUs a tile, 256 x 128 or
// 128 x 128 otherwise. The dense comparator chooses 256 x 128 automatically
// (a ring of four stages fits LDS); its 256 x 256 tile (two stages) is taken
// when an algorithm id asks for it, as the timing-based choice does where it
// is faster (x1 shapes: 3-5%). The general N:M gather path always uses 128 x
// 128 (its staging needs LDS). An algorithm id on the plan pins the choice.
inline int pick_tile(const nm_plan& pl, int amode) {
  if (amode == A_GATHER) return T128;
  if (pl.force_tile == T128 || pl.force_tile == T256x128) return pl.force_tile;   // -1: automatic
  if (pl.force_tile == T256) return T256;
  const int64_t t256 = ((pl.p.m + 255) / 256) * ((pl.p.n + 255) / 256);
  const int64_t t256x128 = ((pl.p.m + 255) / 256) * ((pl.p.n + 127) / 128);
  if (t256 >= 192 && amode != A_DENSE) return T256;
  if (t256x128 >= 192) return T256x128;
  return T128;
}

// Whole tiles, whole k-steps, 16-byte rows and operands addressable with
// 32-bit offsets: the full-tile kernels apply.
inline bool full_tiles(const nm_plan& pl, const GemmArgs& A, int TM, int TN, int amode) {
  const int es = pl.esz_ab;
  const int64_t kl = KBYTES / es;
  if (amode == A_GATHER) return false;
  if (A.m % TM || A.n % TN || A.k % kl || A.k == 0) return false;
  if ((A.ldb * es) % 16 || (A.lda * es) % 16) return false;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t b_rows = pl.p.op_b == NM_OP_N ? A.k : A.n;
  const int64_t a_rows = amode == A_DENSE ? (pl.p.op_a == NM_OP_N ? A.m : A.k) : A.m;
  return b_rows * A.ldb * es < lim && a_rows * A.lda * es < lim && A.m * A.mld < lim;
}

// After a split-k product: the reduction over the partial-sum planes (nothing
// to do without a split).
template <int DT>
hipError_t launch_reduce(const GemmArgs& A, hipStream_t s) {
  if (A.splits <= 1) return launch_status();
  if (!launch_probe().armed) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t quads = A.m * A.n / 4;
  NM_LAUNCH((splitk_reduce_kernel<DT>), dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, A);
  return launch_status();
}

// Stages of the LDS-DMA ring: as many as fit (at most 4), keeping two blocks
// per CU for 128 x 128 tiles; DEEP: one block per CU (grids of at most one
// block per CU), so the ring takes the whole LDS (up to 6 stages): the copies
// are latency-bound and more of them in flight is what helps.
template <int DT, int AMODE, int TM, int TN, bool DEEP = false>
constexpr int dma_stages() {
  constexpr int ES = DT == DT_I8 ? 1 : 2;
  constexpr int STG = (AMODE == A_SPARSE24 ? TM * (64 + (ES == 2 ? 8 : 16)) : TM * 128) + TN * 128;
  constexpr int BUDGET = (TM == 128 && TN == 128 && !DEEP) ? 80 * 1024 : 160 * 1024;
  constexpr int MAXS = DEEP ? 6 : 4;
  return MAXS * STG <= BUDGET ? MAXS : (MAXS - 1) * STG <= BUDGET ? MAXS - 1 : (MAXS - 2) * STG <= BUDGET ? MAXS - 2 : 2;
}

template <int DT, int AMODE, int TM, int TN>
hipError_t launch_tiles_t(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  const int64_t tiles = ((A.m + TM - 1) / TM) * ((A.n + TN - 1) / TN);
  const bool bkc = pl.p.op_b == NM_OP_T;
  const bool akc = pl.p.op_a == NM_OP_N || AMODE != A_DENSE;
  // split-k: only the whole-tile copy-ring kernel of the 2:4 product takes it
  // (spmm_splits decides with the same tile choice and whole-tile test)
  if (A.splits > 1 && (AMODE != A_SPARSE24 || !full_tiles(pl, A, TM, TN, AMODE))) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles * A.splits));
  if constexpr (AMODE != A_GATHER) {
    if (full_tiles(pl, A, TM, TN, AMODE)) {
      // 256-row tiles run eight waves (two per SIMD, 128 x 64 or 64 x 64 each);
      // 128 x 128 tiles run four waves with two blocks per CU.
      constexpr int WGM = TM == 256 ? (TN == 256 ? 2 : 4) : 2;
      constexpr int WGN = TM == 256 ? 4 / (TN == 256 ? 1 : 2) : 2;
      constexpr int S1 = dma_stages<DT, AMODE, TM, TN>();
      constexpr int SD = dma_stages<DT, AMODE, TM, TN, true>();
      // measured: the deep ring lifts the dense 128 x 128 kernel (BERT FC2: 545 ->
      // 700 TFLOP/s) but not the 2:4 one, which stays on the shallow ring
      const bool deep = AMODE == A_DENSE && TM == 128 && TN == 128 && tiles <= NUM_CU;
      if constexpr (AMODE == A_DENSE) {
        // dense A stored k x m (op_a = T): its stored k-rows are staged like
        // those of B stored k x n and read with the transposing LDS reads
        if (!akc) {
          if (bkc && deep)
            NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, SD, WGM, WGN, 3>), grid, dim3(64 * WGM * WGN), 0, s, A);
          else if (bkc)
            NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, S1, WGM, WGN, 3>), grid, dim3(64 * WGM * WGN), 0, s, A);
          else if (deep)
            NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, SD, WGM, WGN, 2>), grid, dim3(64 * WGM * WGN), 0, s, A);
          else
            NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, S1, WGM, WGN, 2>), grid, dim3(64 * WGM * WGN), 0, s, A);
          return launch_status();
        }
      }
      if constexpr (AMODE == A_SPARSE24 && TM == 256 && TN == 256 && DT != DT_I8 && S1 == 3) {
        // 2:4, 16-bit, 256 x 256: metadata staged four k-steps at a time (not
        // with split-k, whose k ranges may start half-way into a 16-byte piece)
        if (A.splits == 1) {
          if (bkc) NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, 3, WGM, WGN, 5>), grid, dim3(64 * WGM * WGN), 0, s, A);
          else NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, 3, WGM, WGN, 4>), grid, dim3(64 * WGM * WGN), 0, s, A);
          return launch_reduce<DT>(A, s);
        }
      }
      if constexpr (AMODE == A_SPARSE24 && TM == 128 && TN == 128 && DT != DT_I8 && S1 == 3) {
        // 2:4, 16-bit, 128 x 128 on four waves: metadata batched as for 256 x
        // 256, 3 x 24 KB of ring + 8 KB of slots, still two blocks per CU.
        // Measured faster than the eight-wave kernel below (which cannot split
        // a metadata fill evenly) also where that one had won: BERT FC2 NN
        // 41-43 -> 33-34 us, PROJ NN 13.4 -> 11-13 us
        if (A.splits == 1) {
          if (bkc) NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, 3, WGM, WGN, 5>), grid, dim3(64 * WGM * WGN), 0, s, A);
          else NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, 3, WGM, WGN, 4>), grid, dim3(64 * WGM * WGN), 0, s, A);
          return launch_reduce<DT>(A, s);
        }
      }
      if constexpr (AMODE == A_SPARSE24 && TM == 128 && TN == 128) {
        // eight waves (2 x 4 of 64 x 32) instead of four: measured faster for B
        // stored k x n when every CU has at most one tile (BERT FC2 NN 41.2 ->
        // 38.4 us, PROJ NN 12.5 -> 11.7 us) and slower for B stored n x k
        // (FC2 NT 37 -> 39.5 us), before the batched metadata above; now int8
        // and split-k only
        if (!bkc && tiles * A.splits <= NUM_CU) {
          NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, S1, 2, 4, 0>), grid, dim3(512), 0, s, A);
          return launch_reduce<DT>(A, s);
        }
      }
      if (bkc && deep)
        NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, SD, WGM, WGN, 1>), grid, dim3(64 * WGM * WGN), 0, s, A);
      else if (bkc)
        NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, S1, WGM, WGN, 1>), grid, dim3(64 * WGM * WGN), 0, s, A);
      else if (deep)
        NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, SD, WGM, WGN, 0>), grid, dim3(64 * WGM * WGN), 0, s, A);
      else
        NM_LAUNCH((gemm_dma_kernel<DT, AMODE, TM, TN, S1, WGM, WGN, 0>), grid, dim3(64 * WGM * WGN), 0, s, A);
      return launch_reduce<DT>(A, s);
    }
  }
  if constexpr (AMODE == A_GATHER) {
    // M = 32 with 4-, 8- or 16-byte groups: expanded from registers, pipelined
    const int gv = (int)(A.N * pl.esz_ab);
    if (A.M == 32 && (gv == 4 || gv == 8 || gv == 16)) {
      if (gv == 4 && bkc) NM_LAUNCH((gemm_kernel<DT, AMODE, 1, 1, TM, TN, 4>), grid, dim3(NTH), 0, s, A);
      else if (gv == 4) NM_LAUNCH((gemm_kernel<DT, AMODE, 0, 1, TM, TN, 4>), grid, dim3(NTH), 0, s, A);
      else if (gv == 8 && bkc) NM_LAUNCH((gemm_kernel<DT, AMODE, 1, 1, TM, TN, 8>), grid, dim3(NTH), 0, s, A);
      else if (gv == 8) NM_LAUNCH((gemm_kernel<DT, AMODE, 0, 1, TM, TN, 8>), grid, dim3(NTH), 0, s, A);
      else if (bkc) NM_LAUNCH((gemm_kernel<DT, AMODE, 1, 1, TM, TN, 16>), grid, dim3(NTH), 0, s, A);
      else NM_LAUNCH((gemm_kernel<DT, AMODE, 0, 1, TM, TN, 16>), grid, dim3(NTH), 0, s, A);
      return launch_status();
    }
  }
  if (bkc && akc) NM_LAUNCH((gemm_kernel<DT, AMODE, 1, 1, TM, TN>), grid, dim3(NTH), 0, s, A);
  else if (!bkc && akc) NM_LAUNCH((gemm_kernel<DT, AMODE, 0, 1, TM, TN>), grid, dim3(NTH), 0, s, A);
  else if (AMODE == A_DENSE && bkc) NM_LAUNCH((gemm_kernel<DT, A_DENSE, 1, 0, TM, TN>), grid, dim3(NTH), 0, s, A);
  else if (AMODE == A_DENSE) NM_LAUNCH((gemm_kernel<DT, A_DENSE, 0, 0, TM, TN>), grid, dim3(NTH), 0, s, A);
  return launch_status();
}

template <int DT>
hipError_t launch_tiles_dt(const nm_plan& pl, int amode, const GemmArgs& A, hipStream_t s) {
  if (amode == A_GATHER) return launch_tiles_t<DT, A_GATHER, 128, 128>(pl, A, s);
  if (amode == A_SPARSE24) {
    switch (pick_tile(pl, A_SPARSE24)) {
      case T256: return launch_tiles_t<DT, A_SPARSE24, 256, 256>(pl, A, s);
      case T256x128: return launch_tiles_t<DT, A_SPARSE24, 256, 128>(pl, A, s);
      default: return launch_tiles_t<DT, A_SPARSE24, 128, 128>(pl, A, s);
    }
  }
  switch (pick_tile(pl, A_DENSE)) {
    case T256: return launch_tiles_t<DT, A_DENSE, 256, 256>(pl, A, s);
    case T256x128: return launch_tiles_t<DT, A_DENSE, 256, 128>(pl, A, s);
    default: return launch_tiles_t<DT, A_DENSE, 128, 128>(pl, A, s);
  }
}

// defined in nm_gemm_f16.hip, nm_gemm_bf16.hip, nm_gemm_i8.hip
hipError_t launch_tiles_f16(const nm_plan& pl, int amode, const GemmArgs& A, hipStream_t s);
hipError_t launch_tiles_bf16(const nm_plan& pl, int amode, const GemmArgs& A, hipStream_t s);
hipError_t launch_tiles_i8(const nm_plan& pl, int amode, const GemmArgs& A, hipStream_t s);

}  // namespace nm
