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

// Small-n product built for latency and bandwidth. A block of SK2_WAVES waves
// takes SK2_WAVES rows, one per wave; a lane takes whole groups (one vector
// load brings a group's N kept values, a 3-dword window of the row's bit
// stream its offsets; DENSE_A takes 16-byte chunks of a dense row instead).
// op(B) is staged in LDS once per block (when k fits one chunk) as records of
// RB bytes: the n values of one k in B's own type, zero-padded to NP columns
// and to at least 4 bytes. Records are laid out so a wave's reads never share
// a bank: within each window of 64 groups of MG consecutive k (MG = M, or the
// elements of a 16-byte chunk for DENSE_A), the record of k = 64 MG w + MG g
// + j sits at 64 MG w + 64 j + g, so lane g reads record 64 j + g whatever its
// offset j. The first A loads of a row are issued before the staging barrier
// and the next iteration's loads before the current one's arithmetic, so
// the memory latencies overlap. Partial sums are combined across the wave with
// butterfly shuffles. Requirements (checked by the launcher): N * ESZ a power
// of two up to 16 bytes and N * b <= 64; DENSE_A needs op_a = N.
constexpr int SK2_WAVES = 16;
constexpr int SK2_DEPTH = 4;         // iterations of A loads in flight per lane (2 for the int8 dense rows)
constexpr int SK2_LDS = 64 * 1024;   // bytes of staged B per chunk

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

template <int DT, int NP>
struct SkinnyRec {
  static constexpr int ESZ = DT == DT_I8 ? 1 : 2;
  static constexpr int RB = NP * ESZ;                       // bytes per staged k
  static constexpr int KC = SK2_LDS / RB;                   // k per chunk (a multiple of every window)
};

template <int DT, int NP, bool DENSE_A, int RW>
__global__ void __launch_bounds__(64 * SK2_WAVES) skinny2_kernel(GemmArgs A, int b_op_t) {
  constexpr int ESZ = SkinnyRec<DT, NP>::ESZ;
  constexpr int RB = SkinnyRec<DT, NP>::RB;
  constexpr int KC = SkinnyRec<DT, NP>::KC;
  constexpr int FDT = DT == DT_I8 ? DT_F16 : DT;
  constexpr int EPC = 16 / ESZ;                             // DENSE_A: elements per 16-byte chunk
  constexpr int DEPTH = RW > 1 || (DENSE_A && ESZ == 1) ? 2 : SK2_DEPTH;
  typedef typename std::conditional<DT == DT_I8, int32_t, float>::type acc_t;
  extern __shared__ __attribute__((aligned(16))) uint8_t s_b[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = (int)A.n;
  const int M = DENSE_A ? EPC : A.M, N = A.N, b = A.bits;
  const int W = 64 * M;                                     // k per window
  const int64_t row_groups = (A.m + SK2_WAVES * RW - 1) / (SK2_WAVES * RW);
  const bool one_chunk = A.k <= KC;
  const int vbytes = N * ESZ;
  const int64_t mwords = A.mld / 4;

  auto elem = [&](uint32_t raw) __attribute__((always_inline)) -> acc_t {
    if constexpr (ESZ == 2) return from_bits16<FDT>((uint16_t)raw);
    else return (acc_t)(int8_t)(uint8_t)raw;
  };
  // the NP staged values of record r
  auto brec = [&](int r, acc_t (&bv)[NP]) __attribute__((always_inline)) {
    const uint8_t* p = s_b + r * RB;
    uint32_t w[RB < 4 ? 1 : RB / 4];
    if constexpr (RB == 1) w[0] = *p;
    else if constexpr (RB == 2) w[0] = *(const uint16_t*)p;
    else if constexpr (RB == 4) w[0] = *(const uint32_t*)p;
    else if constexpr (RB == 8) { const u32x2 v = *(const u32x2*)p; w[0] = v[0]; w[1] = v[1]; }
    else {
#pragma unroll
      for (int q = 0; q < RB / 16; q++) {
        const u32x4 v = *(const u32x4*)(p + 16 * q);
        w[4 * q] = v[0]; w[4 * q + 1] = v[1]; w[4 * q + 2] = v[2]; w[4 * q + 3] = v[3];
      }
    }
#pragma unroll
    for (int c = 0; c < NP; c++) bv[c] = elem(w[(c * ESZ) / 4] >> (8 * ((c * ESZ) % 4)));
  };
  // A data of one iteration of one lane: up to 16 value bytes, 3 metadata words
  struct Piece { uint32_t v[4]; uint32_t m[3]; };
  auto load_piece = [&](int64_t row, int64_t kc, int kn, int it, Piece& pc) __attribute__((always_inline)) {
    pc.v[0] = pc.v[1] = pc.v[2] = pc.v[3] = 0;
    pc.m[0] = pc.m[1] = pc.m[2] = 0;
    if (row >= A.m) return;
    const int g = it * 64 + lane;
    if constexpr (DENSE_A) {
      const int kk0 = g * EPC;
      if (kk0 >= kn) return;
      const uint8_t* p = A.a + (size_t)(row * A.lda + kc + kk0) * ESZ;
      if (kk0 + EPC <= kn && A.a_vec) {
        const u32x4 v = *(const u32x4*)p;
        pc.v[0] = v[0]; pc.v[1] = v[1]; pc.v[2] = v[2]; pc.v[3] = v[3];
      } else {
#pragma unroll
        for (int wi = 0; wi < 4; wi++) {
          uint32_t word = 0;
          for (int t = 0; t < 4 / ESZ; t++) {
            const int e = wi * (4 / ESZ) + t;
            if (kk0 + e >= kn) break;
            const uint32_t x = ESZ == 2 ? (uint32_t)((const uint16_t*)p)[e] : (uint32_t)p[e];
            word |= x << (8 * ESZ * t);
          }
          pc.v[wi] = word;
        }
      }
    } else {
      if (g >= kn / M) return;
      const int64_t gg = kc / M + g;
      load_group_vals<ESZ>(A.a + (size_t)(row * A.lda + gg * N) * ESZ, vbytes, pc.v);
      const int64_t w0 = (gg * N * b) >> 5;
      const uint32_t* mr = (const uint32_t*)(A.meta + row * A.mld);
#pragma unroll
      for (int x = 0; x < 3; x++) pc.m[x] = (w0 + x < mwords) ? mr[w0 + x] : 0u;
    }
  };
  auto use_piece = [&](int64_t kc, int kn, int it, const Piece& pc, acc_t (&acc)[NP]) __attribute__((always_inline)) {
    const int g = it * 64 + lane;
    const int rbase = it * W + lane;                        // record of offset 0 of this lane's group
    if constexpr (DENSE_A) {
      const int kk0 = g * EPC;
#pragma unroll
      for (int wi = 0; wi < 4; wi++) {                      // value word, then its elements
        const uint32_t word = pc.v[wi];
        for (int t = 0; t < 4 / ESZ; t++) {
          const int e = wi * (4 / ESZ) + t;
          if (kk0 + e >= kn) break;
          acc_t bv[NP];
          brec(rbase + 64 * e, bv);
          const acc_t av = elem(word >> (8 * ESZ * t));
#pragma unroll
          for (int c = 0; c < NP; c++) acc[c] += av * bv[c];
        }
      }
    } else {
      if (g >= kn / M) return;
      const int off = (int)(((kc / M + g) * N * b) & 31);
      const uint64_t lo = ((uint64_t)pc.m[1] << 32) | pc.m[0], hi = ((uint64_t)pc.m[2] << 32) | pc.m[1];
#pragma unroll
      for (int wi = 0; wi < 4; wi++) {                      // N * ESZ <= 16: value word, then its slots
        const uint32_t word = pc.v[wi];
        for (int t = 0; t < 4 / ESZ; t++) {
          const int s = wi * (4 / ESZ) + t;
          if (s >= N) break;
          const int pbit = off + s * b;
          const uint64_t win = pbit < 32 ? lo >> pbit : hi >> (pbit - 32);
          const int j = (int)(win & ((1u << b) - 1u));
          acc_t bv[NP];
          brec(rbase + 64 * j, bv);
          const acc_t av = elem(word >> (8 * ESZ * t));
#pragma unroll
          for (int c = 0; c < NP; c++) acc[c] += av * bv[c];
        }
      }
    }
  };

  for (int64_t grp = blockIdx.x; grp < row_groups; grp += (one_chunk ? gridDim.x : row_groups)) {
    const int64_t row0 = (grp * SK2_WAVES + wave) * RW;    // this wave's RW rows
    acc_t acc[RW][NP];
#pragma unroll
    for (int rr = 0; rr < RW; rr++)
#pragma unroll
      for (int c = 0; c < NP; c++) acc[rr][c] = 0;
    for (int64_t kc = 0; kc < A.k; kc += KC) {
      const int kn = (int)((A.k - kc) < KC ? (A.k - kc) : KC);
      const int units = DENSE_A ? (kn + EPC - 1) / EPC : kn / M;   // groups (chunks) of this k chunk
      const int nit = (units + 63) / 64;
      // DEPTH iterations in flight per lane; the first ones while B is staged
      Piece pc[RW][DEPTH];
#pragma unroll
      for (int u = 0; u < DEPTH; u++)
#pragma unroll
        for (int rr = 0; rr < RW; rr++) load_piece(row0 + rr, kc, kn, u, pc[rr][u]);
      const bool stage = !(one_chunk && grp != blockIdx.x);
      if (stage) {
        __syncthreads();                                    // previous chunk's readers are done
        for (int kk = threadIdx.x; kk < kn; kk += 64 * SK2_WAVES) {
          uint32_t w[RB < 4 ? 1 : RB / 4];
#pragma unroll
          for (int q = 0; q < (RB < 4 ? 1 : RB / 4); q++) w[q] = 0;
#pragma unroll
          for (int c = 0; c < NP; c++) {
            if (c >= n) break;
            const int64_t gi = b_op_t ? (int64_t)c * A.ldb + kc + kk : (kc + kk) * A.ldb + c;
            const uint32_t raw = ESZ == 2 ? (uint32_t)((const uint16_t*)A.b)[gi] : (uint32_t)A.b[gi];
            w[(c * ESZ) / 4] |= raw << (8 * ((c * ESZ) % 4));
          }
          const int win = kk / W, in = kk % W;
          const int r = win * W + (in % M) * 64 + in / M;
          uint8_t* d = s_b + r * RB;
          if constexpr (RB == 1) *d = (uint8_t)w[0];
          else if constexpr (RB == 2) *(uint16_t*)d = (uint16_t)w[0];
          else {
#pragma unroll
            for (int q = 0; q < RB / 4; q++) ((uint32_t*)d)[q] = w[q];
          }
        }
        __syncthreads();
      }
      for (int it0 = 0; it0 < nit; it0 += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; u++) {
#pragma unroll
          for (int rr = 0; rr < RW; rr++) {
            if (it0 + u < nit) use_piece(kc, kn, it0 + u, pc[rr][u], acc[rr]);
            load_piece(row0 + rr, kc, kn, it0 + u + DEPTH, pc[rr][u]);   // empty beyond the chunk
          }
        }
      }
    }
    // combine across the wave; lane c writes column c
#pragma unroll
    for (int rr = 0; rr < RW; rr++) {
      const int64_t row = row0 + rr;
#pragma unroll
      for (int c = 0; c < NP; c++)
        for (int o = 32; o > 0; o >>= 1) acc[rr][c] += __shfl_xor(acc[rr][c], o);
      if (row < A.m) {
#pragma unroll
        for (int c = 0; c < NP; c++) {
          if (lane != c || c >= n) continue;
          if constexpr (DT == DT_I8) {
            int64_t iv = (int64_t)A.alpha * acc[rr][c];
            if (A.beta != 0.0f) iv += (int64_t)A.beta * ((const int32_t*)A.c)[row * A.ldc + c];
            ((int32_t*)A.d)[row * A.ldd + c] = (int32_t)iv;
          } else {
            float o = A.alpha * acc[rr][c];
            if (A.beta != 0.0f) o += A.beta * from_bits16<DT>(((const uint16_t*)A.c)[row * A.ldc + c]);
            ((uint16_t*)A.d)[row * A.ldd + c] = to_bits16<DT>(o);
          }
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

template <int DT, bool DENSE_A, int NP, int RW>
static hipError_t launch_skinny2_rw(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  // one block per SK2_WAVES * RW rows; when all of k fits one LDS chunk the
  // grid is capped at two blocks per CU and each block stages B once and
  // walks several row groups
  constexpr int KC = SkinnyRec<DT, NP>::KC;
  const int64_t groups = (A.m + SK2_WAVES * RW - 1) / (SK2_WAVES * RW);
  const int64_t blocks = A.k <= KC ? (groups < 512 ? groups : 512) : groups;
  // records are placed within whole windows of 64 groups (64 M, or 64 chunks
  // of 16 bytes for a dense A), so the staged chunk is rounded up to a window;
  // KC is a multiple of every window, so this stays within SK2_LDS
  const int64_t win = 64 * (DENSE_A ? (int64_t)(16 / SkinnyRec<DT, NP>::ESZ) : (int64_t)A.M);
  const int64_t kn = A.k < KC ? A.k : KC;
  const int64_t kr = kn > 0 ? (kn + win - 1) / win * win : win;
  const size_t lds = (size_t)kr * SkinnyRec<DT, NP>::RB;
  NM_LAUNCH((skinny2_kernel<DT, NP, DENSE_A, RW>), dim3((unsigned)blocks), dim3(64 * SK2_WAVES), lds, s, A,
            (int)(pl.p.op_b == NM_OP_T));
  return launch_status();
}

// Tall problems (m >= 16384 rows) give each wave several rows, so that the
// staged B serves more rows per block (16-bit types; the int8 variants would
// spill).
template <int DT, bool DENSE_A, int NP>
static hipError_t launch_skinny2_t(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  constexpr int RW_TALL = DT == DT_I8 ? 1 : NP <= 2 ? 4 : NP <= 8 ? 2 : 1;
  if (A.m >= 16384 && RW_TALL > 1) return launch_skinny2_rw<DT, DENSE_A, NP, RW_TALL>(pl, A, s);
  return launch_skinny2_rw<DT, DENSE_A, NP, 1>(pl, A, s);
}

template <int DT, bool DENSE_A>
static hipError_t launch_skinny2_np(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  const int64_t n = A.n;
  if (n <= 1) return launch_skinny2_t<DT, DENSE_A, 1>(pl, A, s);
  if (n <= 2) return launch_skinny2_t<DT, DENSE_A, 2>(pl, A, s);
  if (n <= 4) return launch_skinny2_t<DT, DENSE_A, 4>(pl, A, s);
  if (n <= 8) return launch_skinny2_t<DT, DENSE_A, 8>(pl, A, s);
  return launch_skinny2_t<DT, DENSE_A, 16>(pl, A, s);
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
