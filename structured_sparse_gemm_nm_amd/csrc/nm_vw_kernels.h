// Vector-wise N:M product on the dense matrix instructions (included by the
// per-type instantiation files): D = alpha * A * B + beta * C with A in the
// vector-wise compressed form (V consecutive rows share their kept offsets)
// and B stored k x n.
//
// Why a gather works here (apex PR "[sparse] update support for arbitrary N:M
// settings sparse", extension 2: vector-wise N:M for nmSPARSE, to reach a
// higher speed-up): the rows of a V-row block multiply the same kept rows of
// B, so for every 16-row fragment of the block the kept k form a dense
// product of width k N / M on which the dense matrix instructions run with
// no wasted work. Element-wise N:M has no such shared gather.
//
// Block tile 256 x 128, eight waves, each 32 rows (two 16-row fragments) x
// all 128 columns. Per k-step (128 k for 16-bit types, 256 for int8) the copy
// ring stages in LDS: the k-step's rows of B as stored (dense: together the
// block's 16 fragments need nearly all of them), the fragments' compressed
// values (k N / M per row) and the raw metadata words covering the step. A
// lane then finds the B row of its k slot from the metadata and reads its B
// operand with the gfx950 transposing LDS read, whose 16-lane groups take one
// address per lane: lane s of a group addresses gathered row t = s / 4 (s / 2
// for int8) at columns c + 4 (s % 4) (c + 8 (s % 2)), and lane j receives
// column c + j at the group's four (eight) gathered k, the B operand layout of
// the 16 x 16 instructions. Matrix instructions: v_mfma_f32_16x16x16_{f16,
// bf16} and v_mfma_i32_16x16x32_i8 (lane l covers row / column l % 16 and
// quarter q = l / 16, holding k 4q .. 4q+3 (8q .. 8q+7 for int8); the
// accumulator holds D[4q + r][l % 16]).
#pragma once
#include "nm_gemm_kernels.h"

namespace nm {

constexpr int VW_BM = 256, VW_BN = 128, VW_WAVES = 8;

template <int DT> struct VwFrag;
template <> struct VwFrag<DT_F16> { typedef _Float16 ab __attribute__((ext_vector_type(4))); typedef floatx4 acc; };
template <> struct VwFrag<DT_BF16> { typedef short ab __attribute__((ext_vector_type(4))); typedef floatx4 acc; };
template <> struct VwFrag<DT_I8> { typedef long ab; typedef intx4 acc; };

template <int DT>
__device__ __forceinline__ typename VwFrag<DT>::acc vw_mfma(typename VwFrag<DT>::ab a, typename VwFrag<DT>::ab b,
                                                            typename VwFrag<DT>::acc c) {
  if constexpr (DT == DT_F16) return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  else if constexpr (DT == DT_BF16) return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
}

// KP: kept k per row and k-step (k-step x N / M); S: ring stages.
template <int DT, int KP, int S>
__global__ void __launch_bounds__(64 * VW_WAVES) vw_gemm_kernel(GemmArgs A) {
  constexpr int ESZ = DT == DT_I8 ? 1 : 2;
  constexpr int BM = VW_BM, BN = VW_BN;
  constexpr int KS = 256 / ESZ;                           // logical k per step (256 bytes of a B column)
  constexpr int CH = DT == DT_I8 ? 32 : 16;               // k per matrix instruction
  static_assert(KP % CH == 0 && KP <= KS / 2, "kept k per step");
  constexpr int FR = BM / 16;                             // 16-row fragments per block
  constexpr int FPW = FR / VW_WAVES;                      // fragments per wave
  constexpr int FN = BN / 16;                             // 16-column fragments
  constexpr int B_ROW = BN * ESZ;                         // bytes per staged B row
  constexpr int BSLOTS = B_ROW / 16;
  constexpr int B_ST = KS * B_ROW;                        // 32 KB
  constexpr int A_ROW = KP * ESZ;                         // compressed bytes per row and step
  constexpr int CPR = A_ROW / 16;                         // 16-byte chunks per A row (2, 4 or 8)
  constexpr int A_ST = BM * A_ROW;
  constexpr int RAWW = 32;                                // metadata words staged per fragment
  constexpr int M_ST = FR * RAWW * 4;
  constexpr int STAGE = B_ST + A_ST + M_ST;
  static_assert(S * STAGE <= 160 * 1024, "LDS ring");
  constexpr int NB = B_ST / 1024 / VW_WAVES;              // 16-byte copies per wave and stage
  constexpr int NA = A_ST / 1024 / VW_WAVES;
  static_assert(NB * 1024 * VW_WAVES == B_ST && NA * 1024 * VW_WAVES == A_ST && NA >= 1, "copy split");
  constexpr int L = NB + NA + 1;                          // + one 4-byte copy of metadata words
  static_assert(L * (S - 1) <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * STAGE];

  typedef typename VwFrag<DT>::ab ab_t;
  typedef typename VwFrag<DT>::acc acc_t;

  const int64_t tiles_m = A.m / BM, tiles_n = A.n / BN;
  int64_t tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t r0 = tm * BM, c0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q = lane >> 4, l16 = lane & 15;
  const int ksteps = (int)(A.k / KS);
  const int b = A.bits, Mm = A.M, lnN = __builtin_ctz(A.N), mmask = A.M - 1;

  auto bswz = [](int r, int c) -> int {                   // LDS slot of 16-byte chunk c of staged B row r
    if constexpr (ESZ == 2) return c ^ (4 * (r & 3));
    else return c ^ (2 * ((r >> 1) & 3));
  };
  auto aswz = [](int r) -> int { return (r / (16 / CPR)) % CPR; };

  // ---- per-lane copy offsets ----
  uint32_t ob[NB], oa[NA];
#pragma unroll
  for (int j = 0; j < NB; j++) {
    const int p = 64 * (wave * NB + j) + lane;
    const int row = p / BSLOTS, slot = p % BSLOTS;
    ob[j] = (uint32_t)(row * A.ldb * ESZ + (bswz(row, slot) << 4));
  }
#pragma unroll
  for (int j = 0; j < NA; j++) {
    const int p = 64 * (wave * NA + j) + lane;
    const int row = p / CPR, slot = p % CPR;
    oa[j] = (uint32_t)(row * A.lda * ESZ + ((slot ^ aswz(row)) << 4));
  }
  // metadata words: lane p of the block stages word p % 32 of fragment p / 32's window
  const int mp = 64 * wave + lane;
  const int mfrag = mp / RAWW, mword = mp % RAWW;
  const int64_t mrow = (r0 + 16 * mfrag) >> A.vshift;
  const int64_t mwords = A.mld / 4;
  const uint8_t* bbase = A.b + (size_t)c0 * ESZ;
  const size_t bstep = (size_t)KS * A.ldb * ESZ;
  const uint8_t* abase = A.a + (size_t)r0 * A.lda * ESZ;
  const uint32_t* mbase = (const uint32_t*)(A.meta + mrow * A.mld);

  auto issue = [&](int st) {
    uint8_t* base = ring + (st % S) * STAGE;
    const uint8_t* bp = bbase + (size_t)st * bstep;
    const uint8_t* ap = abase + (size_t)st * A_ROW;
#pragma unroll
    for (int j = 0; j < NB; j++) dma16s(bp, ob[j], base + (wave * NB + j) * 1024);
#pragma unroll
    for (int j = 0; j < NA; j++) dma16s(ap, oa[j], base + B_ST + (wave * NA + j) * 1024);
    // words from the one holding the step's first field; clamped into the row
    const int64_t w0 = ((int64_t)st * KP * b) >> 5;
    const int64_t w = w0 + mword < mwords ? w0 + mword : mwords - 1;
    dma4((const uint8_t*)(mbase + w), base + B_ST + A_ST + wave * 256);   // (per-lane row: not a scalar base)
  };

  acc_t acc[FPW][FN];
#pragma unroll
  for (int f = 0; f < FPW; f++)
#pragma unroll
    for (int n = 0; n < FN; n++)
#pragma unroll
      for (int r = 0; r < 4; r++) acc[f][n][r] = 0;

  auto wait_stages = [&](int n) {
    if (S > 2 && n >= 2) wait_vmcnt<L * (S > 2 ? 2 : 0)>();
    else if (n == 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
  };

  auto compute = [&](int st) {
    const uint8_t* base = ring + (st % S) * STAGE;
    const uint8_t* lb = base;
    const uint8_t* la = base + B_ST;
    const uint32_t* lm = (const uint32_t*)(base + B_ST + A_ST);
    const int pbase = (int)(((int64_t)st * KP * b) & 31);   // bit of the step's first field in word 0
#pragma unroll
    for (int ch = 0; ch < KP / CH; ch++) {
#pragma unroll
      for (int f = 0; f < FPW; f++) {
        const int fr = wave * FPW + f;
        const int arow = 16 * fr + l16;
        // A operand: kept values CH*ch + (CH/4) q .. + CH/4 - 1 of row arow
        const int abyte = (CH * ch + (CH / 4) * q) * ESZ;
        const ab_t av = *(const ab_t*)(la + arow * A_ROW + (((abyte >> 4) ^ aswz(arow)) << 4) + (abyte & 15));
        // this lane's gathered k slot and its staged B row
        const int kk = CH * ch + (CH / 4) * q + (ESZ == 2 ? (l16 >> 2) : (l16 >> 1));
        const int p = pbase + kk * b;
        const uint64_t wv = (uint64_t)lm[fr * RAWW + (p >> 5)] | ((uint64_t)lm[fr * RAWW + (p >> 5) + 1] << 32);
        const int srow = ((kk >> lnN) * Mm) + (int)((wv >> (p & 31)) & (uint64_t)mmask);
#pragma unroll
        for (int n = 0; n < FN; n++) {
          ab_t bv;
          if constexpr (ESZ == 2) {
            const int cbyte = (16 * n + 4 * (l16 & 3)) * 2;
            const int off = srow * B_ROW + (bswz(srow, cbyte >> 4) << 4) + (cbyte & 15);
            typedef short short4_t __attribute__((ext_vector_type(4)));
            const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4_t*)(lb + off));
            bv = __builtin_bit_cast(ab_t, v);
          } else {
            const int cbyte = 16 * n + 8 * (l16 & 1);
            const int off = srow * B_ROW + (bswz(srow, cbyte >> 4) << 4) + (cbyte & 15);
            typedef int int2_t __attribute__((ext_vector_type(2)));
            const int2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) int2_t*)(lb + off));
            bv = __builtin_bit_cast(ab_t, v);
          }
          acc[f][n] = vw_mfma<DT>(av, bv, acc[f][n]);
        }
      }
    }
  };

#pragma unroll
  for (int st = 0; st < S - 1; st++)
    if (st < ksteps) issue(st);
  // steps that refill the ring and the last S - 1 that do not, as separate
  // loop bodies (no per-step tests in the steady loop)
  auto vstep = [&](int ks, auto refill_t) {
    if constexpr (decltype(refill_t)::value) {
      issue(ks + S - 1);                                  // the slot freed at the end of step ks - 1
      wait_stages(S - 1);                                 // stage ks has landed (this wave's copies)
    } else {
      wait_stages(min(S - 1, ksteps - 1 - ks));
    }
    lds_barrier();                                        // ... and every wave's
    compute(ks);
    lds_barrier();                                        // every wave is done reading slot ks % S
  };
  int ks = 0;
  for (; ks + S - 1 < ksteps; ks++) vstep(ks, std::true_type{});
  for (; ks < ksteps; ks++) vstep(ks, std::false_type{});

  // ---- epilogue: D = alpha * acc + beta * C, accumulator element r of lane l
  // is D[4q + r][l % 16] of its 16 x 16 tile ----
#pragma unroll
  for (int f = 0; f < FPW; f++)
#pragma unroll
    for (int n = 0; n < FN; n++) {
      const int64_t col = c0 + 16 * n + l16;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int64_t row = r0 + 16 * (wave * FPW + f) + 4 * q + r;
        if constexpr (DT == DT_I8) {
          int_store(A, row * A.d_rs + col * A.d_cs, int_epilogue(A, acc[f][n][r], row * A.c_rs + col * A.c_cs));
        } else {
          float v = A.alpha * acc[f][n][r];
          if (A.beta != 0.0f) v += A.beta * from_bits16<DT>(((const uint16_t*)A.c)[row * A.c_rs + col * A.c_cs]);
          ((uint16_t*)A.d)[row * A.d_rs + col * A.d_cs] = to_bits16<DT>(v);
        }
      }
    }
}

// Kept k per step for this plan, or 0 when the vector-wise matrix-core kernel
// does not take it.
inline int vw_kp(const nm_plan& pl) {
  const int es = pl.esz_ab;
  const int ks = 256 / es;
  const int N = pl.p.nm_n, M = pl.p.nm_m;
  if ((N & (N - 1)) != 0) return 0;
  const int kp = ks * N / M;
  if (es == 2 && (kp == 16 || kp == 32 || kp == 64)) return kp;
  if (es == 1 && (kp == 32 || kp == 64 || kp == 128)) return kp;
  return 0;
}

template <int DT>
hipError_t launch_vw_dt(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  const dim3 grid((unsigned)((A.m / VW_BM) * (A.n / VW_BN)));
  const dim3 block(64 * VW_WAVES);
  constexpr int ES = DT == DT_I8 ? 1 : 2;
  switch (vw_kp(pl) * ES) {                               // kept bytes per row and step: 32, 64 or 128
    case 32: NM_LAUNCH((vw_gemm_kernel<DT, 32 / ES, 3>), grid, block, 0, s, A); break;
    case 64: NM_LAUNCH((vw_gemm_kernel<DT, 64 / ES, 3>), grid, block, 0, s, A); break;
    case 128: NM_LAUNCH((vw_gemm_kernel<DT, 128 / ES, 2>), grid, block, 0, s, A); break;
    default: return hipErrorInvalidValue;
  }
  return launch_status();
}

// defined in nm_gemm_f16.hip, nm_gemm_bf16.hip, nm_gemm_i8.hip
hipError_t launch_vw_f16(const nm_plan& pl, const GemmArgs& A, hipStream_t s);
hipError_t launch_vw_bf16(const nm_plan& pl, const GemmArgs& A, hipStream_t s);
hipError_t launch_vw_i8(const nm_plan& pl, const GemmArgs& A, hipStream_t s);

}  // namespace nm
