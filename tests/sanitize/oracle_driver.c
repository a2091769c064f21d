/* Exercise of every oracle routine for the AddressSanitizer / UndefinedBehavior
 * build, on small seeded inputs (finite, tie-heavy and NaN-holding), with the
 * round trips checked: prune then check is conforming, decompress(compress(A))
 * equals prune(A), the sparse loop equals the dense loop. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void or_prune_1d(const void*, int, int64_t, int64_t, int, int, void*, uint8_t*);
void or_prune_tile(const void*, int, int64_t, int64_t, void*, uint8_t*);
int or_tile_patterns(int*);
int64_t or_check_1d(const void*, int, int64_t, int64_t, int, int);
int64_t or_check_tile(const void*, int, int64_t, int64_t);
int or_meta_bits(int);
void or_compress(const void*, int, int64_t, int64_t, int, int, void*, int64_t, uint8_t*, int64_t);
void or_decompress(const void*, int64_t, const uint8_t*, int64_t, int, int64_t, int64_t, int, int, void*);
void or_prune_vw(const void*, int, int64_t, int64_t, int, int, int, void*, uint8_t*);
int64_t or_check_vw(const void*, int, int64_t, int64_t, int, int, int);
void or_compress_vw(const void*, int, int64_t, int64_t, int, int, int, void*, int64_t, uint8_t*, int64_t);
void or_decompress_vw(const void*, int64_t, const uint8_t*, int64_t, int, int64_t, int64_t, int, int, int, void*);
void or_decode(const void*, int, int64_t, double*);
void or_gemm_f64(const double*, const double*, const double*, double*, int64_t, int64_t, int64_t, double, double);
void or_spmm_compressed_f64(const void*, int64_t, const uint8_t*, int64_t, int, int64_t, int64_t, int, int,
                            const double*, int64_t, const double*, double*, double, double);
void or_gemm_i64(const int8_t*, const int8_t*, const int32_t*, int64_t*, int64_t, int64_t, int64_t, int64_t, int64_t);

static int failures = 0;
static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }

static void fill(void* a, int dt, size_t n, int mode) {
  for (size_t i = 0; i < n; i++) {
    if (dt == 2) { ((int8_t*)a)[i] = (int8_t)((int)(next() % 7) - 3); continue; }
    uint16_t v;
    if (mode == 0) v = (uint16_t)(next() & 0xFBFF);                     /* finite fp16 / bf16 patterns */
    else { static const uint16_t t[6] = {0, 0x8000, 0x3800, 0xB800, 0x3C00, 0x4000}; v = t[next() % 6]; }
    if (dt == 1 && mode == 0) v = (uint16_t)((v & 0x807F) | ((next() % 60 + 100) << 7));  /* bf16 exponents */
    if (mode == 2 && next() % 17 == 0) v = dt == 0 ? 0x7E00 : 0x7FC0;    /* a few NaN */
    ((uint16_t*)a)[i] = v;
  }
}

int main(void) {
  const int64_t rows = 64, cols = 128, n = 24;
  const int nm[5][2] = {{2, 4}, {1, 4}, {3, 8}, {4, 32}, {8, 32}};
  int pat[90 * 4];
  if (or_tile_patterns(pat) != 90) failures++;
  for (int dt = 0; dt < 3; dt++)
    for (int mode = 0; mode < 3; mode++) {
      const size_t es = dt == 2 ? 1 : 2;
      void* a = malloc(rows * cols * es);
      void* p = malloc(rows * cols * es);
      void* back = malloc(rows * cols * es);
      uint8_t* keep = malloc(rows * cols);
      fill(a, dt, rows * cols, mode);
      or_prune_tile(a, dt, rows, cols, p, keep);
      if (mode != 2 && or_check_tile(p, dt, rows, cols) != 0) failures++;
      for (int c = 0; c < 5; c++) {
        const int N = nm[c][0], M = nm[c][1], b = or_meta_bits(M);
        const int64_t vld = (cols * N / M + 15) / 16 * 16, mld = ((cols / M) * N * b + 127) / 128 * 16;
        void* vals = malloc(rows * vld * es);
        uint8_t* meta = malloc(rows * mld);
        or_prune_1d(a, dt, rows, cols, N, M, p, keep);
        if (or_check_1d(p, dt, rows, cols, N, M) != 0) failures++;
        or_compress(a, dt, rows, cols, N, M, vals, vld, meta, mld);
        or_decompress(vals, vld, meta, mld, dt, rows, cols, N, M, back);
        if (memcmp(back, p, rows * cols * es)) failures++;
        for (int V = 2; V <= 32; V *= 4) {
          or_prune_vw(a, dt, rows, cols, V, N, M, p, keep);
          if (or_check_vw(p, dt, rows, cols, V, N, M) != 0) failures++;
          or_compress_vw(a, dt, rows, cols, V, N, M, vals, vld, meta, mld);
          or_decompress_vw(vals, vld, meta, mld, dt, rows, cols, V, N, M, back);
          if (memcmp(back, p, rows * cols * es)) failures++;
        }
        if (dt != 2 && mode == 0) {
          double* A = malloc(rows * cols * sizeof(double));
          double* B = malloc(cols * n * sizeof(double));
          double* D1 = malloc(rows * n * sizeof(double));
          double* D2 = malloc(rows * n * sizeof(double));
          or_prune_1d(a, dt, rows, cols, N, M, p, keep);
          or_compress(a, dt, rows, cols, N, M, vals, vld, meta, mld);
          or_decode(p, dt, rows * cols, A);
          for (int64_t i = 0; i < cols * n; i++) B[i] = (double)((int)(next() % 9) - 4) * 0.25;
          or_gemm_f64(A, B, NULL, D1, rows, n, cols, 1.0, 0.0);
          or_spmm_compressed_f64(vals, vld, meta, mld, dt, rows, cols, N, M, B, n, NULL, D2, 1.0, 0.0);
          for (int64_t i = 0; i < rows * n; i++) if (D1[i] != D2[i] && !(isnan(D1[i]) && isnan(D2[i]))) { failures++; break; }
          free(A); free(B); free(D1); free(D2);
        }
        free(vals); free(meta);
      }
      if (dt == 2) {
        int8_t* B = malloc(cols * n);
        int32_t* C = malloc(rows * n * sizeof(int32_t));
        int64_t* D = malloc(rows * n * sizeof(int64_t));
        fill(B, 2, cols * n, 0);
        for (int64_t i = 0; i < rows * n; i++) C[i] = (int32_t)(next() % 2001) - 1000;
        or_gemm_i64((const int8_t*)a, B, C, D, rows, n, cols, 2, -1);
        free(B); free(C); free(D);
      }
      free(a); free(p); free(back); free(keep);
    }
  printf("oracle driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
