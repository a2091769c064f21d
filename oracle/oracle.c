/*
 * Oracle for the N:M structured-sparse GEMM path — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct CPU reference. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it. It shares no code,
 * tables or headers with the GPU library; nothing in the product path calls it.
 *
 * Sources for what is computed (titles of the web pages the method is taken from):
 *  - "[sparse] update support for arbitrary N:M settings sparse" (NVIDIA apex
 *    pull request 1631), extension 1, the mn_1d_greedy mask calculator:
 *    magnitude top-N per group of M consecutive elements along the last dim;
 *    extension 2, vector-wise N:M for nmSPARSE, with its vector score (the
 *    absolute value of the sum of the vector's elements).
 *  - "backpropagation for sparse semi-structured" (pytorch issue 126420), the
 *    maintainer reply: 4x4 tiles that are 2:4 sparse in both directions, so the
 *    same weight serves the forward (W x) and backward (W^T dy) products.
 *  - "Exploiting Ampere structured sparsity with cuSPARSELt" (NVIDIA blog):
 *    Figure 2 text (2:4 pattern, compression to half size plus index metadata
 *    that selects the matching activations); the operation
 *    D = alpha*op(A)*op(B) + beta*C; the prune-check snippet (non-zero result
 *    means the matrix does not conform); the type list (fp16/bf16 with fp32
 *    accumulation, int8 with int32 accumulation).
 *
 * Readings where the pages are silent (listed again in the design notes):
 *  - ties in the top-N go to the lower index inside the group;
 *  - the tile mask is the first, in a fixed enumeration order, of the 90
 *    4x4 patterns with two kept per row and per column that maximises the
 *    kept sum of |w|, the sum taken in fp64 in a fixed order;
 *  - the compressed layout (values, b-bit indices, zero padding to 16 bytes)
 *    is this library's own definition: b = ceil(log2 M).
 *
 * Floating point: every product and sum is fp64, no fused multiply-add
 * (build with -ffp-contract=off).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

enum { OR_F16 = 0, OR_BF16 = 1, OR_I8 = 2 };

/* ---------- element decoding (IEEE-754 binary16 and bfloat16 definitions) ---------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double or_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp((double)(f + 1024), e - 25);             /* (1 + f/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32 (8 exponent bits, bias 127, 7 fraction bits). */
double or_bf16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xFF;
  int f = b & 0x7F;
  double v;
  if (e == 0) v = ldexp((double)f, -133);                /* f * 2^-126 * 2^-7 */
  else if (e == 255) v = f ? NAN : INFINITY;
  else v = ldexp((double)(f + 128), e - 134);             /* (1 + f/128) * 2^(e-127) */
  return sign ? -v : v;
}

static size_t esize(int dt) { return dt == OR_I8 ? 1 : 2; }

static double elem_f64(const void* p, int dt, size_t i) {
  if (dt == OR_F16) return or_f16_to_f64(((const uint16_t*)p)[i]);
  if (dt == OR_BF16) return or_bf16_to_f64(((const uint16_t*)p)[i]);
  return (double)((const int8_t*)p)[i];
}

void or_decode(const void* src, int dt, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; i++) dst[i] = elem_f64(src, dt, (size_t)i);
}

/* Magnitude key: an unsigned integer that orders elements by |x|.  For the
 * 16-bit float formats, clearing the sign bit leaves a bit pattern whose
 * unsigned order equals the order of |x| (both +0 and -0 give 0). For int8 the
 * key is |x| itself. */
static uint32_t mag_key(const void* p, int dt, size_t i) {
  if (dt == OR_I8) { int v = ((const int8_t*)p)[i]; return (uint32_t)(v < 0 ? -v : v); }
  return ((const uint16_t*)p)[i] & 0x7FFFu;
}

static int is_nonzero(const void* p, int dt, size_t i) {
  if (dt == OR_I8) return ((const int8_t*)p)[i] != 0;
  return (((const uint16_t*)p)[i] & 0x7FFFu) != 0;      /* -0.0 counts as zero */
}

static void copy_elem(void* dst, size_t di, const void* src, size_t si, int dt) {
  size_t es = esize(dt);
  memcpy((char*)dst + di * es, (const char*)src + si * es, es);
}

static void zero_elem(void* dst, size_t di, int dt) {
  memset((char*)dst + di * esize(dt), 0, esize(dt));
}

/* ---------- 1-D N:M selection (apex mn_1d_greedy: top-N of |w| in each group of M) ---------- */

/* Order the M positions of one group by decreasing magnitude with a stable
 * insertion sort (equal keys keep their original, lower-index-first order),
 * then keep the first N. keep[j] = 1 for kept offsets j in [0, M). */
static void select_group(const void* row, int dt, int64_t g, int N, int M, uint8_t* keep) {
  int order[32];
  uint32_t key[32];
  for (int j = 0; j < M; j++) { order[j] = j; key[j] = mag_key(row, dt, (size_t)(g * M + j)); }
  for (int a = 1; a < M; a++) {
    int o = order[a];
    int b = a - 1;
    while (b >= 0 && key[order[b]] < key[o]) { order[b + 1] = order[b]; b--; }
    order[b + 1] = o;
  }
  memset(keep, 0, (size_t)M);
  for (int s = 0; s < N; s++) keep[order[s]] = 1;
}

/* a: logical op(A), rows x cols, contiguous row-major. Groups run along cols.
 * out: same shape (may alias a); keep: one byte per element (1 = kept). */
void or_prune_1d(const void* a, int dt, int64_t rows, int64_t cols, int N, int M,
                 void* out, uint8_t* keep) {
  uint8_t k[32];
  for (int64_t r = 0; r < rows; r++) {
    const void* row = (const char*)a + (size_t)(r * cols) * esize(dt);
    for (int64_t g = 0; g < cols / M; g++) {
      select_group(row, dt, g, N, M, k);
      for (int j = 0; j < M; j++) {
        size_t idx = (size_t)(r * cols + g * M + j);
        if (keep) keep[idx] = k[j];
        if (k[j]) { if (out != a) copy_elem(out, idx, a, idx, dt); }
        else zero_elem(out, idx, dt);
      }
    }
  }
}

/* ---------- transposable 2:4 mask on 4x4 tiles ---------- */

/* The six ways of keeping two of four positions, in increasing order. */
static const int PAIR[6][2] = {{0, 1}, {0, 2}, {0, 3}, {1, 2}, {1, 3}, {2, 3}};

/* All choices (p0, p1, p2, p3) of one pair per tile row, p0 outermost, in
 * lexicographic order, kept when every column is also chosen exactly twice.
 * Returns the number written (90). */
int or_tile_patterns(int* pat /* [90][4] */) {
  int n = 0;
  for (int p0 = 0; p0 < 6; p0++)
    for (int p1 = 0; p1 < 6; p1++)
      for (int p2 = 0; p2 < 6; p2++)
        for (int p3 = 0; p3 < 6; p3++) {
          int p[4] = {p0, p1, p2, p3};
          int col[4] = {0, 0, 0, 0};
          for (int r = 0; r < 4; r++) { col[PAIR[p[r]][0]]++; col[PAIR[p[r]][1]]++; }
          if (col[0] == 2 && col[1] == 2 && col[2] == 2 && col[3] == 2) {
            if (pat) for (int r = 0; r < 4; r++) pat[n * 4 + r] = p[r];
            n++;
          }
        }
  return n;
}

/* a: stored matrix rows x cols (both multiples of 4), contiguous row-major.
 * For each tile the score of a pattern is ((s0 + s1) + s2) + s3 with
 * s_r = |w[r][a_r]| + |w[r][b_r]| in fp64; the first strictly-greatest
 * pattern in enumeration order wins. */
void or_prune_tile(const void* a, int dt, int64_t rows, int64_t cols, void* out, uint8_t* keep) {
  int pat[90 * 4];
  int np = or_tile_patterns(pat);
  for (int64_t ti = 0; ti < rows / 4; ti++)
    for (int64_t tj = 0; tj < cols / 4; tj++) {
      double w[4][4];
      for (int r = 0; r < 4; r++)
        for (int c = 0; c < 4; c++) w[r][c] = fabs(elem_f64(a, dt, (size_t)((ti * 4 + r) * cols + tj * 4 + c)));
      int best = 0;
      double best_score = -1.0;
      for (int q = 0; q < np; q++) {
        double s[4];
        for (int r = 0; r < 4; r++) s[r] = w[r][PAIR[pat[q * 4 + r]][0]] + w[r][PAIR[pat[q * 4 + r]][1]];
        double score = ((s[0] + s[1]) + s[2]) + s[3];
        if (score > best_score) { best_score = score; best = q; }
      }
      for (int r = 0; r < 4; r++)
        for (int c = 0; c < 4; c++) {
          size_t idx = (size_t)((ti * 4 + r) * cols + tj * 4 + c);
          int kept = (c == PAIR[pat[best * 4 + r]][0]) || (c == PAIR[pat[best * 4 + r]][1]);
          if (keep) keep[idx] = (uint8_t)kept;
          if (kept) { if (out != a) copy_elem(out, idx, a, idx, dt); }
          else zero_elem(out, idx, dt);
        }
    }
}

/* ---------- conformance checks (the blog's prune-check: non-zero = does not conform) ---------- */

/* Number of groups of M along cols that hold more than N non-zeros. */
int64_t or_check_1d(const void* a, int dt, int64_t rows, int64_t cols, int N, int M) {
  int64_t bad = 0;
  for (int64_t r = 0; r < rows; r++)
    for (int64_t g = 0; g < cols / M; g++) {
      int nz = 0;
      for (int j = 0; j < M; j++) nz += is_nonzero(a, dt, (size_t)(r * cols + g * M + j));
      if (nz > N) bad++;
    }
  return bad;
}

/* Number of tile rows plus tile columns (over all 4x4 tiles) with more than two non-zeros. */
int64_t or_check_tile(const void* a, int dt, int64_t rows, int64_t cols) {
  int64_t bad = 0;
  for (int64_t ti = 0; ti < rows / 4; ti++)
    for (int64_t tj = 0; tj < cols / 4; tj++)
      for (int x = 0; x < 4; x++) {
        int nr = 0, nc = 0;
        for (int y = 0; y < 4; y++) {
          nr += is_nonzero(a, dt, (size_t)((ti * 4 + x) * cols + tj * 4 + y));
          nc += is_nonzero(a, dt, (size_t)((ti * 4 + y) * cols + tj * 4 + x));
        }
        bad += (nr > 2) + (nc > 2);
      }
  return bad;
}

/* ---------- compressed form: kept values plus b-bit in-group indices ---------- */

int or_meta_bits(int M) { int b = 0; while ((1 << b) < M) b++; return b; }

static void put_bit(uint8_t* row, int64_t t, int v) {
  if (v) row[t / 8] |= (uint8_t)(1u << (t % 8));
}
static int get_bit(const uint8_t* row, int64_t t) { return (row[t / 8] >> (t % 8)) & 1; }

/* a: logical op(A) rows x cols contiguous. vals: rows x vals_ld elements; meta:
 * rows x meta_ld bytes. Both buffers are fully written (padding = 0).
 * For kept offsets i_0 < ... < i_{N-1} of group g:
 *   vals[r][g*N + s] = a[r][g*M + i_s]
 *   bits [(g*N + s)*b, (g*N + s + 1)*b) of row r's little-endian bit stream = i_s */
void or_compress(const void* a, int dt, int64_t rows, int64_t cols, int N, int M,
                 void* vals, int64_t vals_ld, uint8_t* meta, int64_t meta_ld) {
  int b = or_meta_bits(M);
  uint8_t keep[32];
  memset(vals, 0, (size_t)(rows * vals_ld) * esize(dt));
  memset(meta, 0, (size_t)(rows * meta_ld));
  for (int64_t r = 0; r < rows; r++) {
    const void* row = (const char*)a + (size_t)(r * cols) * esize(dt);
    uint8_t* mrow = meta + r * meta_ld;
    for (int64_t g = 0; g < cols / M; g++) {
      select_group(row, dt, g, N, M, keep);
      int s = 0;
      for (int j = 0; j < M; j++) {
        if (!keep[j]) continue;
        copy_elem(vals, (size_t)(r * vals_ld + g * N + s), row, (size_t)(g * M + j), dt);
        int64_t t0 = (g * N + s) * (int64_t)b;
        for (int q = 0; q < b; q++) put_bit(mrow, t0 + q, (j >> q) & 1);
        s++;
      }
    }
  }
}

/* Inverse: scatter the kept values to their indices, +0 elsewhere. */
void or_decompress(const void* vals, int64_t vals_ld, const uint8_t* meta, int64_t meta_ld,
                   int dt, int64_t rows, int64_t cols, int N, int M, void* out) {
  int b = or_meta_bits(M);
  memset(out, 0, (size_t)(rows * cols) * esize(dt));
  for (int64_t r = 0; r < rows; r++) {
    const uint8_t* mrow = meta + r * meta_ld;
    for (int64_t g = 0; g < cols / M; g++)
      for (int s = 0; s < N; s++) {
        int64_t t0 = (g * N + s) * (int64_t)b;
        int j = 0;
        for (int q = 0; q < b; q++) j |= get_bit(mrow, t0 + q) << q;
        copy_elem(out, (size_t)(r * cols + g * M + j), vals, (size_t)(r * vals_ld + g * N + s), dt);
      }
  }
}

/* ---------- vector-wise N:M: V consecutive rows share one kept-offset set ---------- */

/* The apex pull request (extension 2) extends the mask calculators to
 * vector-wise (VW) and block-wise N:M for nmSPARSE. Its vector-wise routine
 * scores a vector by the absolute value of the SUM of its elements (signed
 * values added first, abs taken last), unlike the block-wise routine, which
 * sums absolute values; the VW reading here keeps that score. A vector is V
 * consecutive rows of op(A) at one column; within every group of M columns the
 * N vectors of largest score are kept for all V rows, ties to the lower
 * in-group offset. The score is accumulated in fp64 in increasing row order;
 * scores are compared through the bit pattern of the (non-negative) fp64
 * value as an unsigned integer, which orders them numerically with NaN above
 * +Inf. */
static double vw_score(const void* a, int dt, int64_t cols, int64_t r0, int V, int64_t c) {
  double s = 0.0;
  for (int v = 0; v < V; v++) s += elem_f64(a, dt, (size_t)((r0 + v) * cols + c));
  return fabs(s);
}

static uint64_t score_key(double x) {
  uint64_t u;
  memcpy(&u, &x, sizeof u);
  return u & 0x7FFFFFFFFFFFFFFFull;
}

/* keep[j] = 1 for the N offsets kept in group g of the V-row block starting at r0. */
static void select_vw_group(const void* a, int dt, int64_t cols, int64_t r0, int V, int64_t g, int N, int M,
                            uint8_t* keep) {
  int order[32];
  uint64_t key[32];
  for (int j = 0; j < M; j++) { order[j] = j; key[j] = score_key(vw_score(a, dt, cols, r0, V, g * M + j)); }
  for (int x = 1; x < M; x++) {                 /* stable insertion sort, descending */
    int o = order[x];
    int y = x - 1;
    while (y >= 0 && key[order[y]] < key[o]) { order[y + 1] = order[y]; y--; }
    order[y + 1] = o;
  }
  memset(keep, 0, (size_t)M);
  for (int s = 0; s < N; s++) keep[order[s]] = 1;
}

/* a: logical op(A), rows x cols (rows a multiple of V). out / keep as or_prune_1d. */
void or_prune_vw(const void* a, int dt, int64_t rows, int64_t cols, int V, int N, int M, void* out, uint8_t* keep) {
  uint8_t k[32];
  for (int64_t b = 0; b < rows / V; b++)
    for (int64_t g = 0; g < cols / M; g++) {
      select_vw_group(a, dt, cols, b * V, V, g, N, M, k);
      for (int v = 0; v < V; v++)
        for (int j = 0; j < M; j++) {
          size_t idx = (size_t)((b * V + v) * cols + g * M + j);
          if (keep) keep[idx] = k[j];
          if (k[j]) { if (out != a) copy_elem(out, idx, a, idx, dt); }
          else zero_elem(out, idx, dt);
        }
    }
}

/* Groups of V-row blocks whose rows hold non-zeros at more than N offsets
 * (the union over the block's rows), i.e. blocks that do not conform. */
int64_t or_check_vw(const void* a, int dt, int64_t rows, int64_t cols, int V, int N, int M) {
  int64_t bad = 0;
  for (int64_t b = 0; b < rows / V; b++)
    for (int64_t g = 0; g < cols / M; g++) {
      int used = 0;
      for (int j = 0; j < M; j++) {
        int any = 0;
        for (int v = 0; v < V; v++) any |= is_nonzero(a, dt, (size_t)((b * V + v) * cols + g * M + j));
        used += any;
      }
      if (used > N) bad++;
    }
  return bad;
}

/* VW compressed form: values exactly as the element-wise layout (row r keeps
 * its own values, in increasing offset order, at the offsets its block
 * selected); metadata has one row per block of V rows, with the element-wise
 * bit-stream layout: field (g*N + s) of block row b holds the s-th kept offset
 * of group g. All padding is zero. */
void or_compress_vw(const void* a, int dt, int64_t rows, int64_t cols, int V, int N, int M,
                    void* vals, int64_t vals_ld, uint8_t* meta, int64_t meta_ld) {
  int b = or_meta_bits(M);
  uint8_t keep[32];
  memset(vals, 0, (size_t)(rows * vals_ld) * esize(dt));
  memset(meta, 0, (size_t)((rows / V) * meta_ld));
  for (int64_t blk = 0; blk < rows / V; blk++) {
    uint8_t* mrow = meta + blk * meta_ld;
    for (int64_t g = 0; g < cols / M; g++) {
      select_vw_group(a, dt, cols, blk * V, V, g, N, M, keep);
      int s = 0;
      for (int j = 0; j < M; j++) {
        if (!keep[j]) continue;
        for (int v = 0; v < V; v++) {
          int64_t r = blk * V + v;
          copy_elem(vals, (size_t)(r * vals_ld + g * N + s), a, (size_t)(r * cols + g * M + j), dt);
        }
        int64_t t0 = (g * N + s) * (int64_t)b;
        for (int q = 0; q < b; q++) put_bit(mrow, t0 + q, (j >> q) & 1);
        s++;
      }
    }
  }
}

void or_decompress_vw(const void* vals, int64_t vals_ld, const uint8_t* meta, int64_t meta_ld, int dt,
                      int64_t rows, int64_t cols, int V, int N, int M, void* out) {
  int b = or_meta_bits(M);
  memset(out, 0, (size_t)(rows * cols) * esize(dt));
  for (int64_t r = 0; r < rows; r++) {
    const uint8_t* mrow = meta + (r / V) * meta_ld;
    for (int64_t g = 0; g < cols / M; g++)
      for (int s = 0; s < N; s++) {
        int64_t t0 = (g * N + s) * (int64_t)b;
        int j = 0;
        for (int q = 0; q < b; q++) j |= get_bit(mrow, t0 + q) << q;
        copy_elem(out, (size_t)(r * cols + g * M + j), vals, (size_t)(r * vals_ld + g * N + s), dt);
      }
  }
}

/* ---------- the product D = alpha * op(A) * op(B) + beta * C ---------- */

/* Dense triple loop in fp64, k ascending for every output. A: m x k, B: k x n,
 * C, D: m x n, all contiguous row-major (op() already applied by the caller).
 * C may be NULL when beta == 0. */
void or_gemm_f64(const double* A, const double* B, const double* C, double* D,
                 int64_t m, int64_t n, int64_t k, double alpha, double beta) {
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; i++) {
    double* acc = (double*)calloc((size_t)n, sizeof(double));
    for (int64_t kk = 0; kk < k; kk++) {
      double a = A[i * k + kk];
      const double* brow = B + kk * n;
      for (int64_t j = 0; j < n; j++) acc[j] += a * brow[j];
    }
    for (int64_t j = 0; j < n; j++)
      D[i * n + j] = alpha * acc[j] + (beta != 0.0 ? beta * C[i * n + j] : 0.0);
    free(acc);
  }
}

/* The same product at chosen output points (i[p], j[p]); B given transposed
 * (Bt: n x k) so one output is a dot product of two contiguous rows. */
void or_gemm_f64_points(const double* A, const double* Bt, const double* Cpts, double* Dpts,
                        int64_t k, const int64_t* pi, const int64_t* pj, int64_t npts,
                        double alpha, double beta) {
  #pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < npts; p++) {
    double acc = 0.0;
    const double* a = A + pi[p] * k;
    const double* b = Bt + pj[p] * k;
    for (int64_t kk = 0; kk < k; kk++) acc += a[kk] * b[kk];
    Dpts[p] = alpha * acc + (beta != 0.0 ? beta * Cpts[p] : 0.0);
  }
}

/* Integer product for the int8 path: exact in int64 (every partial sum of
 * int8 products stays far below 2^63). alpha and beta are integers. */
void or_gemm_i64(const int8_t* A, const int8_t* B, const int32_t* C, int64_t* D,
                 int64_t m, int64_t n, int64_t k, int64_t alpha, int64_t beta) {
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; i++) {
    int64_t* acc = (int64_t*)calloc((size_t)n, sizeof(int64_t));
    for (int64_t kk = 0; kk < k; kk++) {
      int64_t a = A[i * k + kk];
      if (a == 0) continue;                      /* exact: skipping a zero term changes nothing */
      const int8_t* brow = B + kk * n;
      for (int64_t j = 0; j < n; j++) acc[j] += a * (int64_t)brow[j];
    }
    for (int64_t j = 0; j < n; j++) D[i * n + j] = alpha * acc[j] + (C ? beta * (int64_t)C[i * n + j] : 0);
    free(acc);
  }
}

/* "Sparse loop": the same fp64 product read straight from the compressed form,
 * summing only the kept entries of each row in increasing k. A self-check for
 * the dense loop and for the layout (metadata must point at the right B rows). */
void or_spmm_compressed_f64(const void* vals, int64_t vals_ld, const uint8_t* meta, int64_t meta_ld,
                            int dt, int64_t m, int64_t k, int N, int M,
                            const double* B, int64_t n, const double* C, double* D,
                            double alpha, double beta) {
  int b = or_meta_bits(M);
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; i++) {
    double* acc = (double*)calloc((size_t)n, sizeof(double));
    const uint8_t* mrow = meta + i * meta_ld;
    for (int64_t g = 0; g < k / M; g++)
      for (int s = 0; s < N; s++) {
        int64_t t0 = (g * N + s) * (int64_t)b;
        int j = 0;
        for (int q = 0; q < b; q++) j |= get_bit(mrow, t0 + q) << q;
        double a = elem_f64(vals, dt, (size_t)(i * vals_ld + g * N + s));
        const double* brow = B + (g * M + j) * n;
        for (int64_t c = 0; c < n; c++) acc[c] += a * brow[c];
      }
    for (int64_t c = 0; c < n; c++) D[i * n + c] = alpha * acc[c] + (beta != 0.0 ? beta * C[i * n + c] : 0.0);
    free(acc);
  }
}

/* The sparse loop for the vector-wise form: row i reads metadata row i / V. */
void or_spmm_compressed_vw_f64(const void* vals, int64_t vals_ld, const uint8_t* meta, int64_t meta_ld,
                               int dt, int64_t m, int64_t k, int V, int N, int M,
                               const double* B, int64_t n, double* D) {
  int b = or_meta_bits(M);
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; i++) {
    double* acc = (double*)calloc((size_t)n, sizeof(double));
    const uint8_t* mrow = meta + (i / V) * meta_ld;
    for (int64_t g = 0; g < k / M; g++)
      for (int s = 0; s < N; s++) {
        int64_t t0 = (g * N + s) * (int64_t)b;
        int j = 0;
        for (int q = 0; q < b; q++) j |= get_bit(mrow, t0 + q) << q;
        double a = elem_f64(vals, dt, (size_t)(i * vals_ld + g * N + s));
        const double* brow = B + (g * M + j) * n;
        for (int64_t c = 0; c < n; c++) acc[c] += a * brow[c];
      }
    for (int64_t c = 0; c < n; c++) D[i * n + c] = acc[c];
    free(acc);
  }
}

/* Number of threads the OpenMP loops above use (reported with CPU timings). */
#ifdef _OPENMP
#include <omp.h>
int or_threads(void) { return omp_get_max_threads(); }
#else
int or_threads(void) { return 1; }
#endif
