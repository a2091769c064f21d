// Matrix-core kernels: D = alpha * op(A) * op(B) + beta * C.
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
#include <type_traits>

#include "nm_device.h"
#include "nm_internal.h"

namespace nm {

constexpr int BM = 128, BN = 128, NTH = 256;
constexpr int KBYTES = 128;           // bytes of k per row of a dense k-step
constexpr int BSTRIDE = KBYTES + 16;  // LDS row stride of B / dense A tiles (bank spread)
constexpr int ASTRIDE_SP = 80;        // LDS row stride of 2:4 compressed A: 64 B values + meta + pad
constexpr int LDS_B = BN * BSTRIDE;
constexpr int LDS_A_DENSE = BM * BSTRIDE;
constexpr int LDS_A_SP = BM * ASTRIDE_SP;
constexpr int STG_V = 128;            // gather staging: value bytes per row per step (<= 127 used)
constexpr int STG_M = 96;             // gather staging: metadata bytes per row per step
constexpr int LDS_STG = BM * (STG_V + STG_M);

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
  int64_t ldb, ldc, ldd;
  float alpha, beta;
  int N, M, bits;
  int a_vec, b_vec;     // 16-byte vector loads allowed on A / B rows
};

// ---------------------------------------------------------------- B / dense-A staging

// One k-step of a "k-major" operand tile (BN columns x 128 bytes of k), from a
// source whose rows are k-contiguous (op_b = T, or dense A with op_a = N):
// row r of the tile is src[(r0 + r) * ld + kb0 .. + 128 bytes).
// Four 16-byte chunks per thread.
struct KChunks { u32x4 v[4]; };

template <int ESZ>
__device__ __forceinline__ void load_kcontig(KChunks& R, const uint8_t* src, int64_t r0, int64_t rows, int64_t ld,
                                             int64_t k0, int64_t k, bool vec) {
  constexpr int EPC = 16 / ESZ;   // elements per chunk
#pragma unroll
  for (int i = 0; i < 4; i++) {
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

__device__ __forceinline__ void store_kcontig(uint8_t* lds, const KChunks& R) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int id = threadIdx.x + NTH * i;
    const int r = id / 8, part = id % 8;
    *(u32x4*)(lds + r * BSTRIDE + part * 16) = R.v[i];
  }
}

// Same tile from a source whose rows run along the tile's columns (op_b = N:
// B stored k x n; dense A with op_a = T). Each thread loads four consecutive k
// rows of one 16-byte column chunk and transposes them in registers.
template <int ESZ>
__device__ __forceinline__ void load_mncontig(KChunks& R, const uint8_t* src, int64_t c0, int64_t cols, int64_t ld,
                                              int64_t k0, int64_t k, bool vec) {
  constexpr int EPC = 16 / ESZ;                 // columns per chunk
  constexpr int CPR = BN / EPC;                 // chunks per k row: 16 (16-bit) or 8 (i8)
  const int cc = threadIdx.x % CPR, kq = threadIdx.x / CPR;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t gk = k0 + kq * 4 + i, gc = c0 + cc * EPC;
    if (vec && gk < k && gc + EPC <= cols) {
      R.v[i] = *(const u32x4*)(src + (size_t)(gk * ld + gc) * ESZ);
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
      R.v[i] = *(u32x4*)tmp;
    }
  }
}

template <int ESZ>
__device__ __forceinline__ void store_mncontig(uint8_t* lds, const KChunks& R) {
  constexpr int EPC = 16 / ESZ;
  constexpr int CPR = BN / EPC;
  const int cc = threadIdx.x % CPR, kq = threadIdx.x / CPR;
  if (ESZ == 2) {
    // column c of the chunk gets the four 16-bit values (k = 4kq .. 4kq+3)
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const uint32_t w0 = R.v[0][d], w1 = R.v[1][d], w2 = R.v[2][d], w3 = R.v[3][d];
      const u32x2 lo = {(w0 & 0xFFFFu) | (w1 << 16), (w2 & 0xFFFFu) | (w3 << 16)};
      const u32x2 hi = {(w0 >> 16) | (w1 & 0xFFFF0000u), (w2 >> 16) | (w3 & 0xFFFF0000u)};
      const int col = cc * EPC + 2 * d;
      *(u32x2*)(lds + col * BSTRIDE + kq * 8) = lo;
      *(u32x2*)(lds + (col + 1) * BSTRIDE + kq * 8) = hi;
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const uint32_t w0 = R.v[0][d], w1 = R.v[1][d], w2 = R.v[2][d], w3 = R.v[3][d];
#pragma unroll
      for (int x = 0; x < 4; x++) {
        const uint32_t v = ((w0 >> (8 * x)) & 0xFFu) | (((w1 >> (8 * x)) & 0xFFu) << 8) |
                           (((w2 >> (8 * x)) & 0xFFu) << 16) | (((w3 >> (8 * x)) & 0xFFu) << 24);
        const int col = cc * EPC + 4 * d + x;
        *(uint32_t*)(lds + col * BSTRIDE + kq * 4) = v;
      }
    }
  }
}

// ---------------------------------------------------------------- 2:4 compressed A staging

struct SpChunks { u32x4 v[2]; u32x4 meta; };

// Values: 64 bytes per row per step (2 chunks per thread); metadata: 8 bytes
// (16-bit types, 64 logical k) or 16 bytes (int8, 128 logical k) per row.
template <int ESZ>
__device__ __forceinline__ void load_sp24(SpChunks& R, const GemmArgs& A, int64_t r0, int ks) {
  const int64_t nvals = A.k / 2;                        // compressed elements per row
  constexpr int EPC = 16 / ESZ;
  const int64_t v0 = (int64_t)ks * (64 / ESZ);          // first compressed element of this step
#pragma unroll
  for (int i = 0; i < 2; i++) {
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
  // metadata bytes of this step: [ks * MB, ks * MB + MB) inside the row's
  // (16-byte padded, zero-filled) metadata; past the last group the padding or
  // a zero fill supplies offsets that only meet zero values.
  constexpr int MB = ESZ == 2 ? 8 : 16;
  R.meta = u32x4{0, 0, 0, 0};
  if (threadIdx.x < BM) {
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

template <int ESZ>
__device__ __forceinline__ void store_sp24(uint8_t* lds, const SpChunks& R) {
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int id = threadIdx.x + NTH * i;
    const int r = id / 4, part = id % 4;
    *(u32x4*)(lds + r * ASTRIDE_SP + part * 16) = R.v[i];
  }
  if (threadIdx.x < BM) {
    if (ESZ == 2) *(u32x2*)(lds + threadIdx.x * ASTRIDE_SP + 64) = u32x2{R.meta[0], R.meta[1]};
    else *(u32x4*)(lds + threadIdx.x * ASTRIDE_SP + 64) = R.meta;
  }
}

// ---------------------------------------------------------------- general N:M expansion

// Copy the compressed bytes of step ks for the block's rows into LDS staging:
// values (dword aligned: 128*N/M bytes per step) and the dword-aligned window
// of metadata covering the step's offset fields.
template <int ESZ>
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
  for (int e = threadIdx.x; e < BM * (vw + nmw); e += NTH) {
    const int r = e / (vw + nmw), c = e % (vw + nmw);
    const int64_t gr = r0 + r;
    uint32_t val = 0;
    if (c < vw) {
      const int64_t off = (int64_t)ks * vbytes + c * 4;
      if (gr < A.m && off + 4 <= row_vbytes) val = *(const uint32_t*)(A.a + gr * A.lda * ESZ + off);
      *(uint32_t*)(stg + r * STG_V + c * 4) = val;
    } else {
      const int64_t w = w0 + (c - vw);
      if (gr < A.m && w < row_mwords) val = *(const uint32_t*)(A.meta + gr * A.mld + w * 4);
      *(uint32_t*)(stg + BM * STG_V + r * STG_M + (c - vw) * 4) = val;
    }
  }
}

// Zero each (row, group) region of the dense A tile and scatter its kept values.
template <int ESZ>
__device__ __forceinline__ void expand_gather(uint8_t* adense, const uint8_t* stg, const GemmArgs& A, int ks) {
  const int KL = KBYTES / ESZ;
  const int gps = KL / A.M;
  const int64_t groups_left = A.k / A.M - (int64_t)ks * gps;
  const int gvalid = (int)(groups_left < gps ? groups_left : gps);
  const int bitoff = (int)(((int64_t)ks * gps * A.N * A.bits) % 32);
  const int gbytes = A.M * ESZ;
  for (int e = threadIdx.x; e < BM * gps; e += NTH) {
    const int r = e / gps, g = e % gps;
    uint8_t* dst = adense + r * BSTRIDE + g * gbytes;
    for (int x = 0; x < gbytes; x += 4) *(uint32_t*)(dst + x) = 0u;
    if (g >= gvalid) continue;
    const uint8_t* vrow = stg + r * STG_V;
    const uint32_t* mrow = (const uint32_t*)(stg + BM * STG_V + r * STG_M);
    for (int s = 0; s < A.N; s++) {
      const int t = bitoff + (g * A.N + s) * A.bits;
      const uint64_t w = (uint64_t)mrow[t / 32] | ((uint64_t)mrow[t / 32 + 1] << 32);
      const int j = (int)((w >> (t % 32)) & ((1u << A.bits) - 1u));
      if (ESZ == 2) ((uint16_t*)dst)[j] = ((const uint16_t*)vrow)[g * A.N + s];
      else dst[j] = vrow[g * A.N + s];
    }
  }
}

// ---------------------------------------------------------------- the kernel

template <int DT> struct Frag;
template <> struct Frag<DT_F16> { typedef half8_t ab; typedef _Float16 half16_t __attribute__((ext_vector_type(16))); typedef half16_t b2; typedef floatx4 acc; };
template <> struct Frag<DT_BF16> { typedef bf16x8_t ab; typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16))); typedef bf16x16_t b2; typedef floatx4 acc; };
template <> struct Frag<DT_I8> { typedef intx4 ab; typedef intx8 b2; typedef intx4 acc; };

template <int DT>
__device__ __forceinline__ typename Frag<DT>::b2 concat(const typename Frag<DT>::ab& lo, const typename Frag<DT>::ab& hi) {
  if constexpr (DT == DT_I8) {
    return intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
  }
}

template <int DT>
__device__ __forceinline__ typename Frag<DT>::acc smfmac(const typename Frag<DT>::ab& a, const typename Frag<DT>::b2& b,
                                                       typename Frag<DT>::acc c, int idx) {
  if constexpr (DT == DT_F16) return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, c, idx, 0, 0);
  else if constexpr (DT == DT_BF16) return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, c, idx, 0, 0);
  else return __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c, idx, 0, 0);
}

template <int DT>
__device__ __forceinline__ typename Frag<DT>::acc mfma(const typename Frag<DT>::ab& a, const typename Frag<DT>::ab& b,
                                                     typename Frag<DT>::acc c) {
  if constexpr (DT == DT_F16) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  else if constexpr (DT == DT_BF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Map the linear block id to a (row tile, column tile): consecutive ids walk
// down a band of GROUP row tiles before moving right, so blocks resident at
// the same time share B columns and A rows in L2.
__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  constexpr int GROUP = 8;
  const int64_t id = blockIdx.x;
  const int64_t per_band = GROUP * tiles_n;
  const int64_t band = id / per_band;
  const int64_t first = band * GROUP;
  const int64_t rows_in_band = (tiles_m - first) < GROUP ? (tiles_m - first) : GROUP;
  const int64_t in = id % per_band;
  tm = first + in % rows_in_band;
  tn = in / rows_in_band;
}

template <int DT, int AMODE, int BKC, int AKC>
__global__ void __launch_bounds__(NTH) gemm_kernel(GemmArgs A) {
  constexpr int ESZ = DT == DT_I8 ? 1 : 2;
  constexpr int LDS_A = AMODE == A_SPARSE24 ? LDS_A_SP : LDS_A_DENSE;
  __shared__ __attribute__((aligned(16))) uint8_t s_a[AMODE == A_GATHER ? 1 : 2][LDS_A];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][LDS_B];
  __shared__ __attribute__((aligned(16))) uint8_t s_stg[AMODE == A_GATHER ? LDS_STG : 16];

  typedef typename Frag<DT>::acc acc_t;
  typedef typename Frag<DT>::ab ab_t;

  const int64_t tiles_m = (A.m + BM - 1) / BM, tiles_n = (A.n + BN - 1) / BN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t r0 = tm * BM, c0 = tn * BN;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm0 = (wave >> 1) * 64, wn0 = (wave & 1) * 64;
  const int l16 = lane & 15, q = lane >> 4;

  acc_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = acc_t{0, 0, 0, 0};

  const int64_t KL = KBYTES / ESZ;                  // logical k per step
  const int ksteps = (int)((A.k + KL - 1) / KL);

  KChunks rb, ra;
  SpChunks rs;
  auto load_step = [&](int ks) {
    const int64_t k0 = (int64_t)ks * KL;
    if (BKC) load_kcontig<ESZ>(rb, A.b, c0, A.n, A.ldb, k0, A.k, A.b_vec);
    else load_mncontig<ESZ>(rb, A.b, c0, A.n, A.ldb, k0, A.k, A.b_vec);
    if (AMODE == A_DENSE) {
      if (AKC) load_kcontig<ESZ>(ra, A.a, r0, A.m, A.lda, k0, A.k, A.a_vec);
      else load_mncontig<ESZ>(ra, A.a, r0, A.m, A.lda, k0, A.k, A.a_vec);
    }
    if (AMODE == A_SPARSE24) load_sp24<ESZ>(rs, A, r0, ks);
  };
  auto store_step = [&](int buf) {
    if (BKC) store_kcontig(s_b[buf], rb);
    else store_mncontig<ESZ>(s_b[buf], rb);
    if (AMODE == A_DENSE) {
      if (AKC) store_kcontig(s_a[buf], ra);
      else store_mncontig<ESZ>(s_a[buf], ra);
    }
    if (AMODE == A_SPARSE24) store_sp24<ESZ>(s_a[buf], rs);
  };

  auto compute = [&](int buf) {
    const uint8_t* la = s_a[buf];
    const uint8_t* lb = s_b[buf];
    if constexpr (AMODE == A_SPARSE24) {
      ab_t av[4];
      int ai[4];
#pragma unroll
      for (int fm = 0; fm < 4; fm++) {
        const uint8_t* p = la + (wm0 + fm * 16 + l16) * ASTRIDE_SP;
        av[fm] = *(const ab_t*)(p + q * 16);
        ai[fm] = ESZ == 2 ? (int)*(const uint16_t*)(p + 64 + 2 * q) : (int)*(const uint32_t*)(p + 64 + 4 * q);
      }
#pragma unroll
      for (int fn = 0; fn < 4; fn++) {
        const uint8_t* p = lb + (wn0 + fn * 16 + l16) * BSTRIDE;
        const typename Frag<DT>::b2 bv = concat<DT>(*(const ab_t*)(p + q * 16), *(const ab_t*)(p + 64 + q * 16));
#pragma unroll
        for (int fm = 0; fm < 4; fm++) acc[fm][fn] = smfmac<DT>(av[fm], bv, acc[fm][fn], ai[fm]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; h++) {
        ab_t av[4];
#pragma unroll
        for (int fm = 0; fm < 4; fm++) av[fm] = *(const ab_t*)(la + (wm0 + fm * 16 + l16) * BSTRIDE + h * 64 + q * 16);
#pragma unroll
        for (int fn = 0; fn < 4; fn++) {
          const ab_t bv = *(const ab_t*)(lb + (wn0 + fn * 16 + l16) * BSTRIDE + h * 64 + q * 16);
#pragma unroll
          for (int fm = 0; fm < 4; fm++) acc[fm][fn] = mfma<DT>(av[fm], bv, acc[fm][fn]);
        }
      }
    }
  };

  if constexpr (AMODE == A_GATHER) {
    for (int ks = 0; ks < ksteps; ks++) {
      load_step(ks);
      stage_gather<ESZ>(s_stg, A, r0, ks);
      store_step(0);
      __syncthreads();
      expand_gather<ESZ>(s_a[0], s_stg, A, ks);
      __syncthreads();
      compute(0);
      __syncthreads();
    }
  } else {
    if (ksteps > 0) {
      load_step(0);
      store_step(0);
      __syncthreads();
    }
    for (int ks = 0; ks < ksteps; ks++) {
      const int buf = ks & 1;
      const bool more = ks + 1 < ksteps;
      if (more) load_step(ks + 1);
      compute(buf);
      if (more) store_step(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: D = alpha * acc + beta * C ----
#pragma unroll
  for (int fm = 0; fm < 4; fm++)
#pragma unroll
    for (int fn = 0; fn < 4; fn++) {
      const int64_t col = c0 + wn0 + fn * 16 + l16;
      if (col >= A.n) continue;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int64_t row = r0 + wm0 + fm * 16 + q * 4 + r;
        if (row >= A.m) continue;
        if constexpr (DT == DT_I8) {
          int64_t v = (int64_t)A.alpha * acc[fm][fn][r];
          if (A.beta != 0.0f) v += (int64_t)A.beta * ((const int32_t*)A.c)[row * A.ldc + col];
          ((int32_t*)A.d)[row * A.ldd + col] = (int32_t)v;
        } else {
          float v = A.alpha * acc[fm][fn][r];
          if (A.beta != 0.0f) v += A.beta * from_bits16<DT>(((const uint16_t*)A.c)[row * A.ldc + col]);
          ((uint16_t*)A.d)[row * A.ldd + col] = to_bits16<DT>(v);
        }
      }
    }
}

// ---------------------------------------------------------------- skinny (small n)

// Small n (GEMV and up to 16 columns): the compressed rows stream from HBM
// once; op(B) is staged in LDS in chunks of k as fp32 [k][16]; each wave owns
// rows, its lanes walk the groups, decode each kept offset and accumulate
// value * B[g*M + offset][0 .. n) (the metadata selects the activation rows).
// DENSE_A = true streams a dense A instead (the small-n comparator).
constexpr int SK_KC = 512;           // k per LDS chunk
constexpr int SK_NMAX = 16;
constexpr int SK_ROWS_PER_WAVE = 4;

template <int DT, bool DENSE_A>
__global__ void __launch_bounds__(NTH) skinny_kernel(GemmArgs A, int b_op_t, int a_op_t) {
  constexpr int ESZ = DT == DT_I8 ? 1 : 2;
  constexpr int FDT = DT == DT_I8 ? DT_F16 : DT;          // 16-bit decode type (unused for int8)
  typedef typename std::conditional<DT == DT_I8, int32_t, float>::type acc_t;   // int8: exact int32
  __shared__ acc_t s_b[SK_KC][SK_NMAX + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row_base = ((int64_t)blockIdx.x * 4 + wave) * SK_ROWS_PER_WAVE;
  const int n = (int)A.n;
  acc_t acc[SK_ROWS_PER_WAVE][SK_NMAX];
#pragma unroll
  for (int r = 0; r < SK_ROWS_PER_WAVE; r++)
#pragma unroll
    for (int c = 0; c < SK_NMAX; c++) acc[r][c] = 0;

  auto elem = [&](const uint8_t* p, int64_t idx) -> acc_t {
    if constexpr (ESZ == 2) return from_bits16<FDT>(((const uint16_t*)p)[idx]);
    else return (acc_t)(int8_t)p[idx];
  };

  for (int64_t kc = 0; kc < A.k; kc += SK_KC) {
    const int kn = (int)((A.k - kc) < SK_KC ? (A.k - kc) : SK_KC);
    __syncthreads();
    for (int e = threadIdx.x; e < kn * n; e += NTH) {
      const int kk = b_op_t ? e % kn : e / n, c = b_op_t ? e / kn : e % n;
      s_b[kk][c] = elem(A.b, b_op_t ? (int64_t)c * A.ldb + kc + kk : (kc + kk) * A.ldb + c);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < SK_ROWS_PER_WAVE; r++) {
      const int64_t row = row_base + r;
      if (row >= A.m) continue;
      if constexpr (DENSE_A) {
        for (int kk = lane; kk < kn; kk += 64) {
          const acc_t v = elem(A.a, a_op_t ? (kc + kk) * A.lda + row : row * A.lda + kc + kk);
#pragma unroll
          for (int c = 0; c < SK_NMAX; c++)
            if (c < n) acc[r][c] += v * s_b[kk][c];
        }
      } else {
        const int gps = kn / A.M;
        const int64_t g0 = kc / A.M;
        const uint8_t* mrow = A.meta + row * A.mld;
        for (int g = lane; g < gps; g += 64) {
          for (int s = 0; s < A.N; s++) {
            const int64_t slot = (g0 + g) * A.N + s;
            const int64_t t = slot * A.bits;
            uint32_t w = mrow[t / 8];
            if ((t % 8) + A.bits > 8) w |= (uint32_t)mrow[t / 8 + 1] << 8;   // field spans two bytes
            const int j = (int)((w >> (t % 8)) & ((1u << A.bits) - 1u));
            const acc_t v = elem(A.a, row * A.lda + slot);
            const int kk = g * A.M + j;
#pragma unroll
            for (int c = 0; c < SK_NMAX; c++)
              if (c < n) acc[r][c] += v * s_b[kk][c];
          }
        }
      }
    }
  }
  // reduce across the wave and write
#pragma unroll
  for (int r = 0; r < SK_ROWS_PER_WAVE; r++) {
    const int64_t row = row_base + r;
#pragma unroll
    for (int c = 0; c < SK_NMAX; c++) {
      if (c >= n) continue;
      acc_t v = acc[r][c];
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0 && row < A.m) {
        if constexpr (DT == DT_I8) {
          int64_t iv = (int64_t)A.alpha * v;
          if (A.beta != 0.0f) iv += (int64_t)A.beta * ((const int32_t*)A.c)[row * A.ldc + c];
          ((int32_t*)A.d)[row * A.ldd + c] = (int32_t)iv;
        } else {
          float o = A.alpha * v;
          if (A.beta != 0.0f) o += A.beta * from_bits16<DT>(((const uint16_t*)A.c)[row * A.ldc + c]);
          ((uint16_t*)A.d)[row * A.ldd + c] = to_bits16<DT>(o);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- launchers

static GemmArgs make_gemm_args(const nm_plan& pl, float alpha, const void* a, const void* meta, const void* b,
                               float beta, const void* c, void* d, bool dense_a) {
  GemmArgs A{};
  A.a = (const uint8_t*)a; A.meta = (const uint8_t*)meta; A.b = (const uint8_t*)b;
  A.c = (const uint8_t*)c; A.d = (uint8_t*)d;
  A.m = pl.p.m; A.n = pl.p.n; A.k = pl.p.k;
  A.lda = dense_a ? pl.p.lda : pl.vld;
  A.mld = pl.mld;
  A.ldb = pl.p.ldb; A.ldc = pl.p.ldc; A.ldd = pl.p.ldd;
  A.alpha = alpha; A.beta = beta;
  A.N = pl.p.nm_n; A.M = pl.p.nm_m; A.bits = pl.bits;
  A.a_vec = (A.lda * pl.esz_ab) % 16 == 0;
  A.b_vec = (A.ldb * pl.esz_ab) % 16 == 0;
  return A;
}

template <int DT, int AMODE>
static hipError_t launch_tiles(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  const int64_t tiles = ((A.m + BM - 1) / BM) * ((A.n + BN - 1) / BN);
  const dim3 grid((unsigned)tiles);
  const bool bkc = pl.p.op_b == NM_OP_T;
  const bool akc = pl.p.op_a == NM_OP_N || AMODE != A_DENSE;
  if (bkc && akc) hipLaunchKernelGGL((gemm_kernel<DT, AMODE, 1, 1>), grid, dim3(NTH), 0, s, A);
  else if (!bkc && akc) hipLaunchKernelGGL((gemm_kernel<DT, AMODE, 0, 1>), grid, dim3(NTH), 0, s, A);
  else if (AMODE == A_DENSE && bkc) hipLaunchKernelGGL((gemm_kernel<DT, A_DENSE, 1, 0>), grid, dim3(NTH), 0, s, A);
  else if (AMODE == A_DENSE) hipLaunchKernelGGL((gemm_kernel<DT, A_DENSE, 0, 0>), grid, dim3(NTH), 0, s, A);
  return hipGetLastError();
}

template <int AMODE>
static hipError_t launch_tiles_dt(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  switch (pl.p.type_ab) {
    case NM_F16: return launch_tiles<DT_F16, AMODE>(pl, A, s);
    case NM_BF16: return launch_tiles<DT_BF16, AMODE>(pl, A, s);
    default: return launch_tiles<DT_I8, AMODE>(pl, A, s);
  }
}

template <bool DENSE_A>
static hipError_t launch_skinny_dt(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  const dim3 grid((unsigned)((A.m + 4 * SK_ROWS_PER_WAVE - 1) / (4 * SK_ROWS_PER_WAVE)));
  const int bt = pl.p.op_b == NM_OP_T, at = pl.p.op_a == NM_OP_T;
  switch (pl.p.type_ab) {
    case NM_F16: hipLaunchKernelGGL((skinny_kernel<DT_F16, DENSE_A>), grid, dim3(NTH), 0, s, A, bt, at); break;
    case NM_BF16: hipLaunchKernelGGL((skinny_kernel<DT_BF16, DENSE_A>), grid, dim3(NTH), 0, s, A, bt, at); break;
    default: hipLaunchKernelGGL((skinny_kernel<DT_I8, DENSE_A>), grid, dim3(NTH), 0, s, A, bt, at); break;
  }
  return hipGetLastError();
}

hipError_t launch_spmm_smfmac(const nm_plan& pl, float alpha, const void* vals, const void* meta, const void* b,
                              float beta, const void* c, void* d, hipStream_t s) {
  return launch_tiles_dt<A_SPARSE24>(pl, make_gemm_args(pl, alpha, vals, meta, b, beta, c, d, false), s);
}

hipError_t launch_spmm_gather(const nm_plan& pl, float alpha, const void* vals, const void* meta, const void* b,
                              float beta, const void* c, void* d, hipStream_t s) {
  return launch_tiles_dt<A_GATHER>(pl, make_gemm_args(pl, alpha, vals, meta, b, beta, c, d, false), s);
}

hipError_t launch_spmm_skinny(const nm_plan& pl, float alpha, const void* vals, const void* meta, const void* b,
                              float beta, const void* c, void* d, hipStream_t s) {
  return launch_skinny_dt<false>(pl, make_gemm_args(pl, alpha, vals, meta, b, beta, c, d, false), s);
}

hipError_t launch_dense_gemm(const nm_plan& pl, float alpha, const void* a, const void* b, float beta, const void* c,
                             void* d, hipStream_t s) {
  const GemmArgs A = make_gemm_args(pl, alpha, a, a, b, beta, c, d, true);
  if (pl.p.n <= SK_NMAX) return launch_skinny_dt<true>(pl, A, s);
  return launch_tiles_dt<A_DENSE>(pl, A, s);
}

}  // namespace nm
