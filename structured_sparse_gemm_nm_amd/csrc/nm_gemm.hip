// Small-n kernels (GEMV and up to 16 columns) and the top-level product
// launchers. The tiled matrix-core kernels live in nm_gemm_kernels.h and are
// instantiated per element type in nm_gemm_{f16,bf16,i8}.hip.
#include "nm_gemm_kernels.h"

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

// ---------------------------------------------------------------- small n, streamed

// Small-n product built for bandwidth: op(B) is staged once per block in LDS
// in its own element type, [k][NP] (NP = n rounded up to 1, 2, 4, 8 or 16);
// each wave owns 4 rows and keeps all four in flight; a lane takes whole
// groups: one vector load brings the group's N kept values, a 3-dword window
// of the row's metadata brings their offsets, and each kept value meets the
// B row its offset selects. DENSE_A streams a dense row instead (16-byte
// chunks per lane, op_a = N). Partial sums are combined across the wave with
// butterfly shuffles. Requirements (checked by the launcher): N * ESZ a power
// of two up to 16 bytes, N * b <= 64, and k small enough that... any k works:
// B is staged in chunks of KC rows.
constexpr int SK2_RW = 4;   // rows per wave

template <int ESZ>
__device__ __forceinline__ void load_group_vals(const uint8_t* p, int nbytes, uint32_t (&w)[4]) {
  w[0] = w[1] = w[2] = w[3] = 0;
  switch (nbytes) {
    case 16: { const u32x4 v = *(const u32x4*)p; w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3]; break; }
    case 8: { const u32x2 v = *(const u32x2*)p; w[0] = v[0]; w[1] = v[1]; break; }
    case 4: w[0] = *(const uint32_t*)p; break;
    case 2: w[0] = *(const uint16_t*)p; break;
    default: w[0] = *(const uint8_t*)p; break;
  }
}

template <int DT, int NP, bool DENSE_A>
__global__ void __launch_bounds__(NTH) skinny2_kernel(GemmArgs A, int b_op_t) {
  constexpr int ESZ = DT == DT_I8 ? 1 : 2;
  constexpr int FDT = DT == DT_I8 ? DT_F16 : DT;
  constexpr int KC = (64 * 1024) / (NP * ESZ);           // k rows of B per LDS chunk
  typedef typename std::conditional<DT == DT_I8, int32_t, float>::type acc_t;
  __shared__ __attribute__((aligned(16))) uint8_t s_b[KC * NP * ESZ];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = (int)A.n;
  const int64_t groups = (A.m + 4 * SK2_RW - 1) / (4 * SK2_RW);     // row groups of 4 waves x SK2_RW rows
  const bool one_chunk = A.k <= KC;                               // then B is staged once per block
  // contiguous k x NP block (op_b = N, ld = n = NP): 16-byte staging copies
  const bool b_flat = !b_op_t && n == NP && A.ldb == NP && ((A.k * NP * ESZ) % 16 == 0);
  auto bval = [&](int kk, int c) -> acc_t {          // staged B element
    if constexpr (ESZ == 2) return from_bits16<FDT>(((const uint16_t*)s_b)[kk * NP + c]);
    else return (acc_t)(int8_t)s_b[kk * NP + c];
  };
  auto elem = [&](uint32_t raw) -> acc_t {
    if constexpr (ESZ == 2) return from_bits16<FDT>((uint16_t)raw);
    else return (acc_t)(int8_t)(uint8_t)raw;
  };
  const int M = A.M, N = A.N, b = A.bits;
  const int vbytes = N * ESZ;
  const int64_t mwords = A.mld / 4;

  for (int64_t grp = blockIdx.x; grp < groups; grp += (one_chunk ? gridDim.x : groups)) {
  const int64_t row0 = (grp * 4 + wave) * SK2_RW;
  acc_t acc[SK2_RW][NP];
#pragma unroll
  for (int r = 0; r < SK2_RW; r++)
#pragma unroll
    for (int c = 0; c < NP; c++) acc[r][c] = 0;
  for (int64_t kc = 0; kc < A.k; kc += KC) {
    const int kn = (int)((A.k - kc) < KC ? (A.k - kc) : KC);
    const bool stage = !(one_chunk && grp != blockIdx.x);         // staged already on this block's first group
    if (stage) __syncthreads();
    if (stage && b_flat) {
      const int nbytes = kn * NP * ESZ;
      const uint8_t* src = A.b + (size_t)kc * NP * ESZ;
      for (int e = threadIdx.x * 16; e < nbytes; e += NTH * 16) *(u32x4*)(s_b + e) = *(const u32x4*)(src + e);
    }
    for (int e = threadIdx.x; stage && !b_flat && e < kn * NP; e += NTH) {
      const int kk = b_op_t ? e % kn : e / NP, c = b_op_t ? e / kn : e % NP;
      uint32_t raw = 0;
      if (c < n) {
        const int64_t gi = b_op_t ? (int64_t)c * A.ldb + kc + kk : (kc + kk) * A.ldb + c;
        raw = ESZ == 2 ? (uint32_t)((const uint16_t*)A.b)[gi] : (uint32_t)A.b[gi];
      }
      if (ESZ == 2) ((uint16_t*)s_b)[kk * NP + c] = (uint16_t)raw;
      else s_b[kk * NP + c] = (uint8_t)raw;
    }
    if (stage) __syncthreads();
    if constexpr (DENSE_A) {
      constexpr int EPC = 16 / ESZ;
      for (int kk0 = lane * EPC; kk0 < kn; kk0 += 64 * EPC) {
        uint32_t w[SK2_RW][4];
#pragma unroll
        for (int r = 0; r < SK2_RW; r++) {
          const int64_t row = row0 + r;
          w[r][0] = w[r][1] = w[r][2] = w[r][3] = 0;
          if (row < A.m) {
            const uint8_t* p = A.a + (size_t)(row * A.lda + kc + kk0) * ESZ;
            if (kk0 + EPC <= kn && A.a_vec) {
              const u32x4 v = *(const u32x4*)p;
              w[r][0] = v[0]; w[r][1] = v[1]; w[r][2] = v[2]; w[r][3] = v[3];
            } else {
              for (int e = 0; e < EPC && kk0 + e < kn; e++) {
                const uint32_t x = ESZ == 2 ? (uint32_t)((const uint16_t*)p)[e] : (uint32_t)p[e];
                w[r][(e * ESZ) / 4] |= x << (8 * ((e * ESZ) % 4));
              }
            }
          }
        }
#pragma unroll
        for (int e = 0; e < EPC; e++) {
          if (kk0 + e >= kn) break;
          acc_t bv[NP];
#pragma unroll
          for (int c = 0; c < NP; c++) bv[c] = bval(kk0 + e, c);
#pragma unroll
          for (int r = 0; r < SK2_RW; r++) {
            const uint32_t raw = (w[r][(e * ESZ) / 4] >> (8 * ((e * ESZ) % 4))) & (ESZ == 2 ? 0xFFFFu : 0xFFu);
            const acc_t av = elem(raw);
#pragma unroll
            for (int c = 0; c < NP; c++) acc[r][c] += av * bv[c];
          }
        }
      }
    } else {
      const int gps = kn / M;
      const int64_t g0 = kc / M;
      for (int g = lane; g < gps; g += 64) {
        uint32_t vw[SK2_RW][4];
        uint32_t mw[SK2_RW][3];
        const int64_t t0 = (g0 + g) * N * b;                // first metadata bit of the group
        const int64_t w0 = t0 >> 5;
#pragma unroll
        for (int r = 0; r < SK2_RW; r++) {
          const int64_t row = row0 + r;
          if (row < A.m) {
            load_group_vals<ESZ>(A.a + (size_t)(row * A.lda + (g0 + g) * N) * ESZ, vbytes, vw[r]);
            const uint32_t* mr = (const uint32_t*)(A.meta + row * A.mld);
#pragma unroll
            for (int x = 0; x < 3; x++) mw[r][x] = (w0 + x < mwords) ? mr[w0 + x] : 0u;
          } else {
            vw[r][0] = vw[r][1] = vw[r][2] = vw[r][3] = 0;
            mw[r][0] = mw[r][1] = mw[r][2] = 0;
          }
        }
        const int off = (int)(t0 & 31);
        for (int s = 0; s < N; s++) {
          const int pbit = off + s * b;
#pragma unroll
          for (int r = 0; r < SK2_RW; r++) {
            const uint64_t win = pbit < 32 ? (((uint64_t)mw[r][1] << 32) | mw[r][0]) >> pbit
                                           : (((uint64_t)mw[r][2] << 32) | mw[r][1]) >> (pbit - 32);
            const int j = (int)(win & ((1u << b) - 1u));
            const uint32_t raw = (vw[r][(s * ESZ) / 4] >> (8 * ((s * ESZ) % 4))) & (ESZ == 2 ? 0xFFFFu : 0xFFu);
            const acc_t av = elem(raw);
            const int kk = g * M + j;
#pragma unroll
            for (int c = 0; c < NP; c++) acc[r][c] += av * bval(kk, c);
          }
        }
      }
    }
  }
  // combine across the wave; every lane ends with the sums, lane c writes column c
#pragma unroll
  for (int r = 0; r < SK2_RW; r++)
#pragma unroll
    for (int c = 0; c < NP; c++)
      for (int o = 32; o > 0; o >>= 1) acc[r][c] += __shfl_xor(acc[r][c], o);
#pragma unroll
  for (int r = 0; r < SK2_RW; r++) {
    const int64_t row = row0 + r;
    if (row >= A.m) continue;
#pragma unroll
    for (int c = 0; c < NP; c++) {
      if (lane != c || c >= n) continue;
      if constexpr (DT == DT_I8) {
        int64_t iv = (int64_t)A.alpha * acc[r][c];
        if (A.beta != 0.0f) iv += (int64_t)A.beta * ((const int32_t*)A.c)[row * A.ldc + c];
        ((int32_t*)A.d)[row * A.ldd + c] = (int32_t)iv;
      } else {
        float o = A.alpha * acc[r][c];
        if (A.beta != 0.0f) o += A.beta * from_bits16<DT>(((const uint16_t*)A.c)[row * A.ldc + c]);
        ((uint16_t*)A.d)[row * A.ldd + c] = to_bits16<DT>(o);
      }
    }
  }
  }  // row groups
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

static hipError_t launch_tiles_any(const nm_plan& pl, int amode, const GemmArgs& A, hipStream_t s) {
  switch (pl.p.type_ab) {
    case NM_F16: return launch_tiles_f16(pl, amode, A, s);
    case NM_BF16: return launch_tiles_bf16(pl, amode, A, s);
    default: return launch_tiles_i8(pl, amode, A, s);
  }
}

template <int DT, bool DENSE_A>
static hipError_t launch_skinny2_np(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  // one block per row group, at most 512 blocks (two per CU) when all of k fits
  // one LDS chunk (each block then stages B once and walks several groups)
  const int64_t groups = (A.m + 4 * SK2_RW - 1) / (4 * SK2_RW);
  const int np = A.n <= 1 ? 1 : A.n <= 2 ? 2 : A.n <= 4 ? 4 : A.n <= 8 ? 8 : 16;
  const int64_t kc = (64 * 1024) / (np * pl.esz_ab);
  const int64_t blocks = A.k <= kc ? (groups < 512 ? groups : 512) : groups;
  const dim3 grid((unsigned)blocks);
  const int bt = pl.p.op_b == NM_OP_T;
  const int64_t n = A.n;
  if (n <= 1) NM_LAUNCH((skinny2_kernel<DT, 1, DENSE_A>), grid, dim3(NTH), 0, s, A, bt);
  else if (n <= 2) NM_LAUNCH((skinny2_kernel<DT, 2, DENSE_A>), grid, dim3(NTH), 0, s, A, bt);
  else if (n <= 4) NM_LAUNCH((skinny2_kernel<DT, 4, DENSE_A>), grid, dim3(NTH), 0, s, A, bt);
  else if (n <= 8) NM_LAUNCH((skinny2_kernel<DT, 8, DENSE_A>), grid, dim3(NTH), 0, s, A, bt);
  else NM_LAUNCH((skinny2_kernel<DT, 16, DENSE_A>), grid, dim3(NTH), 0, s, A, bt);
  return launch_status();
}

// The streamed small-n kernel needs each group's kept values to be one
// naturally aligned load (N * esize a power of two <= 16 bytes), its offsets
// inside a 3-dword window (N * b <= 64), and, for the dense comparator,
// op_a = N.
static bool skinny2_ok(const nm_plan& pl, bool dense_a) {
  if (dense_a) return pl.p.op_a == NM_OP_N;
  const int vb = pl.p.nm_n * pl.esz_ab;
  return (vb == 1 || vb == 2 || vb == 4 || vb == 8 || vb == 16) && pl.p.nm_n * pl.bits <= 64;
}

template <bool DENSE_A>
static hipError_t launch_skinny_dt(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  if (skinny2_ok(pl, DENSE_A) && !pl.old_skinny) {
    switch (pl.p.type_ab) {
      case NM_F16: return launch_skinny2_np<DT_F16, DENSE_A>(pl, A, s);
      case NM_BF16: return launch_skinny2_np<DT_BF16, DENSE_A>(pl, A, s);
      default: return launch_skinny2_np<DT_I8, DENSE_A>(pl, A, s);
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
                              float beta, const void* c, void* d, hipStream_t s) {
  return launch_tiles_any(pl, A_SPARSE24, make_gemm_args(pl, alpha, vals, meta, b, beta, c, d, false), s);
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
