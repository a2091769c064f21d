// The general small-n kernel (any N:M, any layout) and the top-level product
// launchers. The tiled matrix-core kernels live in nm_gemm_kernels.h and the
// streamed small-n kernels in nm_skinny_kernels.h, each instantiated per
// element type in nm_gemm_{f16,bf16,i8}.hip and nm_skinny_{f16,bf16,i8}.hip.
#include "nm_gemm_kernels.h"
#include "nm_skinny_kernels.h"
#include "nm_vw_kernels.h"

namespace nm {

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
        const uint8_t* mrow = A.meta + (row >> A.vshift) * A.mld;
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
          int_store(A, row * A.d_rs + c * A.d_cs, int_epilogue(A, v, row * A.c_rs + c * A.c_cs));
        } else {
          float o = A.alpha * v;
          if (A.beta != 0.0f) o += A.beta * from_bits16<DT>(((const uint16_t*)A.c)[row * A.c_rs + c * A.c_cs]);
          ((uint16_t*)A.d)[row * A.d_rs + c * A.d_cs] = to_bits16<DT>(o);
        }
      }
    }
  }
}

static GemmArgs make_gemm_args(const nm_plan& pl, float alpha, const void* a, const void* meta, const void* b,
                               float beta, const void* c, void* d, bool dense_a) {
  GemmArgs A{};
  A.a = (const uint8_t*)a; A.meta = (const uint8_t*)meta; A.b = (const uint8_t*)b;
  A.c = (const uint8_t*)c; A.d = (uint8_t*)d;
  A.m = pl.p.m; A.n = pl.p.n; A.k = pl.p.k;
  A.lda = dense_a ? pl.p.lda : pl.vld;
  A.mld = pl.mld;
  A.ldb = pl.p.ldb;
  const bool col = pl.p.order_cd == NM_COL_MAJOR;
  A.c_rs = col ? 1 : pl.p.ldc; A.c_cs = col ? pl.p.ldc : 1;
  A.d_rs = col ? 1 : pl.p.ldd; A.d_cs = col ? pl.p.ldd : 1;
  A.cd_col = col;
  A.cd_i8 = pl.p.type_cd == NM_I8;
  A.alpha = alpha; A.beta = beta;
  A.N = pl.p.nm_n; A.M = pl.p.nm_m; A.bits = pl.bits;
  A.a_vec = (A.lda * pl.esz_ab) % 16 == 0;
  A.b_vec = (A.ldb * pl.esz_ab) % 16 == 0;
  A.vshift = pl.vshift;
  A.splits = 1;
  A.ws = nullptr;
  return A;
}

int spmm_splits(const nm_plan& pl) {
  if (pl.split_k <= 1 || pl.kernel != K_SMFMAC_24 || pl.p.m == 0 || pl.p.n == 0) return 1;
  const GemmArgs A = make_gemm_args(pl, 1.0f, nullptr, nullptr, nullptr, 0.0f, nullptr, nullptr, false);
  int tm = 128, tn = 128;
  switch (pick_tile(pl, A_SPARSE24)) {
    case T256: tm = 256; tn = 256; break;
    case T256x128: tm = 256; tn = 128; break;
    default: break;
  }
  if (!full_tiles(pl, A, tm, tn, A_SPARSE24)) return 1;
  const int64_t ksteps = pl.p.k / (KBYTES / pl.esz_ab);
  const int64_t sp = pl.split_k < ksteps ? pl.split_k : ksteps;
  return (int)(sp > 1 ? sp : 1);
}

size_t spmm_workspace_bytes(const nm_plan& pl) {
  const int sp = spmm_splits(pl);
  return sp > 1 ? (size_t)sp * (size_t)pl.p.m * (size_t)pl.p.n * 4u : 0u;
}

static hipError_t launch_tiles_any(const nm_plan& pl, int amode, const GemmArgs& A, hipStream_t s) {
  switch (pl.p.type_ab) {
    case NM_F16: return launch_tiles_f16(pl, amode, A, s);
    case NM_BF16: return launch_tiles_bf16(pl, amode, A, s);
    default: return launch_tiles_i8(pl, amode, A, s);
  }
}

// The streamed small-n kernel needs each group's kept values to be one
// naturally aligned load (N * esize a power of two <= 16 bytes) and its
// offsets inside a 3-dword window (N * b <= 64); for the dense comparator,
// op_a = N, 16-byte aligned rows and k a whole number of 16-byte chunks. Its
// row, k and group indices are 32-bit: m and k below 2^30.
static bool skinny2_ok(const nm_plan& pl, bool dense_a) {
  if (pl.p.m >= ((int64_t)1 << 30) || pl.p.k >= ((int64_t)1 << 30)) return false;
  if (dense_a)
    return pl.p.op_a == NM_OP_N && (pl.p.lda * pl.esz_ab) % 16 == 0 && (pl.p.k * pl.esz_ab) % 16 == 0;
  const int vb = pl.p.nm_n * pl.esz_ab;
  return (vb == 1 || vb == 2 || vb == 4 || vb == 8 || vb == 16) && pl.p.nm_n * pl.bits <= 64;
}

template <bool DENSE_A>
static hipError_t launch_skinny_dt(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  if (skinny2_ok(pl, DENSE_A)) {
    switch (pl.p.type_ab) {
      case NM_F16: return launch_skinny2_f16(pl, A, s, DENSE_A);
      case NM_BF16: return launch_skinny2_bf16(pl, A, s, DENSE_A);
      default: return launch_skinny2_i8(pl, A, s, DENSE_A);
    }
  }
  const dim3 grid((unsigned)((A.m + 4 * SK_ROWS_PER_WAVE - 1) / (4 * SK_ROWS_PER_WAVE)));
  const int bt = pl.p.op_b == NM_OP_T, at = pl.p.op_a == NM_OP_T;
  switch (pl.p.type_ab) {
    case NM_F16: NM_LAUNCH((skinny_kernel<DT_F16, DENSE_A>), grid, dim3(NTH), 0, s, A, bt, at); break;
    case NM_BF16: NM_LAUNCH((skinny_kernel<DT_BF16, DENSE_A>), grid, dim3(NTH), 0, s, A, bt, at); break;
    default: NM_LAUNCH((skinny_kernel<DT_I8, DENSE_A>), grid, dim3(NTH), 0, s, A, bt, at); break;
  }
  return launch_status();
}

hipError_t launch_spmm_smfmac(const nm_plan& pl, float alpha, const void* vals, const void* meta, const void* b,
                              float beta, const void* c, void* d, void* ws, hipStream_t s) {
  GemmArgs A = make_gemm_args(pl, alpha, vals, meta, b, beta, c, d, false);
  A.splits = spmm_splits(pl);
  A.ws = (uint8_t*)ws;
  return launch_tiles_any(pl, A_SPARSE24, A, s);
}

// The vector-wise matrix-core kernel: blocks of 16 rows share their offsets
// (vrows a multiple of 16), B stored k x n, whole 256 x 128 tiles and k-steps,
// N a power of two with k-step x N / M kept k per step in its instantiated set,
// 16-byte rows, operands addressable with 32-bit offsets.
bool vw_mfma_ok(const nm_plan& pl) {
  const nm_problem_t& p = pl.p;
  if (pl.vrows < 16 || pl.vrows % 16 || p.op_a != NM_OP_N || p.op_b != NM_OP_N || vw_kp(pl) == 0) return false;
  const int64_t ks = 256 / pl.esz_ab;
  if (p.m % VW_BM || p.n % VW_BN || p.k % ks || p.k == 0 || (p.ldb * pl.esz_ab) % 16) return false;
  const int64_t lim = (int64_t)1 << 31;
  return p.k * p.ldb * pl.esz_ab < lim && p.m * pl.vld * pl.esz_ab < lim && (p.m / pl.vrows) * pl.mld < lim;
}

hipError_t launch_spmm_vw(const nm_plan& pl, float alpha, const void* vals, const void* meta, const void* b,
                          float beta, const void* c, void* d, hipStream_t s) {
  const GemmArgs A = make_gemm_args(pl, alpha, vals, meta, b, beta, c, d, false);
  if (!vw_mfma_ok(pl)) return hipErrorInvalidValue;
  switch (pl.p.type_ab) {
    case NM_F16: return launch_vw_f16(pl, A, s);
    case NM_BF16: return launch_vw_bf16(pl, A, s);
    default: return launch_vw_i8(pl, A, s);
  }
}

hipError_t launch_spmm_gather(const nm_plan& pl, float alpha, const void* vals, const void* meta, const void* b,
                              float beta, const void* c, void* d, hipStream_t s) {
  return launch_tiles_any(pl, A_GATHER, make_gemm_args(pl, alpha, vals, meta, b, beta, c, d, false), s);
}

hipError_t launch_spmm_skinny(const nm_plan& pl, float alpha, const void* vals, const void* meta, const void* b,
                              float beta, const void* c, void* d, hipStream_t s) {
  return launch_skinny_dt<false>(pl, make_gemm_args(pl, alpha, vals, meta, b, beta, c, d, false), s);
}

hipError_t launch_dense_gemm(const nm_plan& pl, float alpha, const void* a, const void* b, float beta, const void* c,
                             void* d, hipStream_t s) {
  const GemmArgs A = make_gemm_args(pl, alpha, a, a, b, beta, c, d, true);
  if (pl.p.n <= SK_NMAX) return launch_skinny_dt<true>(pl, A, s);
  return launch_tiles_any(pl, A_DENSE, A, s);
}

}  // namespace nm
