// Prune, prune check, compress and decompress kernels (HBM-bound).
//
// What they compute:
//  - 1-D N:M selection: keep the N largest |x| in every group of M along k of
//    op(A), ties to the lower offset (apex PR "[sparse] update support for
//    arbitrary N:M settings sparse", extension 1, greedy per-group top-N).
//  - Transposable 2:4 on 4x4 tiles: two kept per tile row and per tile column,
//    chosen to maximise the kept |x| (pytorch issue 126420 "backpropagation for
//    sparse semi-structured", maintainer reply).
//  - Prune check: count of non-conforming groups (cuSPARSELt blog, the
//    prune-check snippet, whose non-zero flag means "does not conform").
//  - Compress / decompress: kept values plus b-bit in-group offsets (cuSPARSELt
//    blog, Figure 2 text), in the layout documented in include/nmsparse.h.
//
// Design: a block owns a tile of 64 logical rows x 256 logical k of op(A).
// The tile is copied between HBM and LDS in the *stored* orientation with
// 16-byte row-contiguous accesses (so op_a = T costs the same as op_a = N);
// threads then work group by group out of LDS, and results (pruned tile, keep
// mask, values, metadata bytes) are staged in LDS and written back row-
// contiguously. Every tile writes the row padding of the compressed buffers
// when it holds the row's last group.
#include "nm_internal.h"
#include "nm_device.h"

namespace nm {

constexpr int TILE_K = 256;   // logical k per tile
constexpr int TPB = 256;      // threads per block

struct TileArgs {
  const uint8_t* a;     // stored dense input (prune, compress)
  uint8_t* out;         // stored dense output (prune, decompress)
  uint32_t* mask;       // optional keep mask (prune)
  uint8_t* vals;        // compressed values (out for compress, in for decompress)
  uint8_t* meta;        // metadata bytes
  int64_t m, k;         // logical op(A) dims
  int64_t lda;          // stored leading dimension (elements)
  int64_t mask_ld;      // words per stored row of the mask
  int64_t vld, mld;     // compressed strides (elements, bytes)
  int N, op_t, bits, vec_ok;
};

enum TileOp { T_PRUNE = 0, T_COMPRESS = 1, T_DECOMPRESS = 2 };

// Copy a stored sub-block [sr0, sr0+SR) x [sc0, sc0+SC) between HBM and LDS
// (LDS row stride SC elements). Out-of-matrix elements read as 0 and are not
// written back.
template <int ESZ, int SR, int SC>
__device__ __forceinline__ void tile_in(uint8_t* lds, const uint8_t* g, int64_t sr0, int64_t sc0,
                                        int64_t rows, int64_t cols, int64_t ld, bool vec_ok) {
  constexpr int CH = 16 / ESZ;
  constexpr int CPR = SC / CH;
  for (int c = threadIdx.x; c < SR * CPR; c += TPB) {
    const int r = c / CPR, cc = (c % CPR) * CH;
    const int64_t gr = sr0 + r, gc = sc0 + cc;
    uint8_t* dst = lds + (size_t)(r * SC + cc) * ESZ;
    if (vec_ok && gr < rows && gc + CH <= cols) {
      *(u32x4*)dst = __builtin_nontemporal_load((const u32x4*)(g + (size_t)(gr * ld + gc) * ESZ));
    } else {
      for (int e = 0; e < CH; e++) {
        const bool in = gr < rows && gc + e < cols;
        if (ESZ == 2) ((uint16_t*)dst)[e] = in ? ((const uint16_t*)g)[gr * ld + gc + e] : (uint16_t)0;
        else dst[e] = in ? g[gr * ld + gc + e] : (uint8_t)0;
      }
    }
  }
}

template <int ESZ, int SR, int SC>
__device__ __forceinline__ void tile_out(uint8_t* g, const uint8_t* lds, int64_t sr0, int64_t sc0,
                                         int64_t rows, int64_t cols, int64_t ld, bool vec_ok) {
  constexpr int CH = 16 / ESZ;
  constexpr int CPR = SC / CH;
  for (int c = threadIdx.x; c < SR * CPR; c += TPB) {
    const int r = c / CPR, cc = (c % CPR) * CH;
    const int64_t gr = sr0 + r, gc = sc0 + cc;
    if (gr >= rows) continue;
    const uint8_t* src = lds + (size_t)(r * SC + cc) * ESZ;
    if (vec_ok && gc + CH <= cols) {
      __builtin_nontemporal_store(*(const u32x4*)src, (u32x4*)(g + (size_t)(gr * ld + gc) * ESZ));
    } else {
      for (int e = 0; e < CH && gc + e < cols; e++) {
        if (ESZ == 2) ((uint16_t*)g)[gr * ld + gc + e] = ((const uint16_t*)src)[e];
        else g[gr * ld + gc + e] = src[e];
      }
    }
  }
}

template <int ESZ>
__device__ __forceinline__ uint32_t lds_elem(const uint8_t* lds, int idx) {
  return ESZ == 2 ? (uint32_t)((const uint16_t*)lds)[idx] : (uint32_t)lds[idx];
}
template <int ESZ>
__device__ __forceinline__ void lds_set(uint8_t* lds, int idx, uint32_t v) {
  if (ESZ == 2) ((uint16_t*)lds)[idx] = (uint16_t)v;
  else lds[idx] = (uint8_t)v;
}

// Largest metadata bytes per tile row over all (N, M) supported: (TILE_K / M) * N * b / 8 with N = M - 1:
// M=4: 64*3*2/8 = 48, M=8: 32*7*3/8 = 84, M=16: 16*15*4/8 = 120, M=32: 8*31*5/8 = 155.
constexpr int META_ROW_BYTES = 160;                     // rounded up to a whole number of words

// Rows per tile: 16 when groups run along stored rows (op N: each stored row
// of the tile is 256 contiguous elements), 64 when they run down stored
// columns (op T: each stored row of the tile is then 64 contiguous elements).
// Small tiles keep many blocks in flight on BERT-sized weights.
template <int OPT> struct TileRows { static constexpr int value = OPT ? 64 : 16; };

template <int DT, int ESZ, int M, int OP, int OPT>
__global__ void __launch_bounds__(TPB) tile_kernel(TileArgs A) {
  constexpr int TR = TileRows<OPT>::value;
  constexpr int LDS_DENSE = TR * TILE_K * ESZ;
  constexpr int LDS_VALS = TR * TILE_K * ESZ;           // N <= M - 1 < M: values never exceed the dense tile
  constexpr int LDS_META = TR * META_ROW_BYTES;
  constexpr int LDS_MASK = TR * TILE_K / 8;
  __shared__ __attribute__((aligned(16))) uint8_t s_dense[LDS_DENSE];
  __shared__ __attribute__((aligned(16))) uint8_t s_vals[OP == T_PRUNE ? 16 : LDS_VALS];
  __shared__ __attribute__((aligned(16))) uint32_t s_meta[OP == T_PRUNE ? 4 : LDS_META / 4];
  __shared__ __attribute__((aligned(16))) uint32_t s_mask[OP == T_PRUNE ? LDS_MASK / 4 : 4];

  constexpr int GPR = TILE_K / M;           // groups per tile row
  constexpr int VROW = GPR * (M - 1) * ESZ; // LDS bytes reserved per row of values (>= GPR * N * ESZ)
  const int N = A.N, b = A.bits;
  const int64_t i0 = (int64_t)blockIdx.y * TR;
  const int64_t k0 = (int64_t)blockIdx.x * TILE_K;
  const int64_t srows = OPT ? A.k : A.m, scols = OPT ? A.m : A.k;   // stored dims
  const int64_t sr0 = OPT ? k0 : i0, sc0 = OPT ? i0 : k0;
  const int rows_here = (int)min((int64_t)TR, A.m - i0);
  const int groups_here = (int)(min((int64_t)TILE_K, A.k - k0) / M);
  const int vals_per_row = groups_here * N;                          // elements
  const int meta_bits_row = groups_here * N * b;
  const int meta_bytes_row = (meta_bits_row + 7) / 8;
  const int meta_words_row = META_ROW_BYTES / 4;
  const bool last_k_tile = k0 + TILE_K >= A.k;
  // Value bytes of this tile inside a compressed row: a whole number of dwords,
  // since (256 / M) * N * esize is a multiple of 8; the last tile of a row runs
  // on to the row's 16-byte padded end (vld * esize).
  const int64_t vbyte0 = (k0 / M) * N * ESZ;
  const int64_t mbase = (k0 / M) * N * b / 8;          // first metadata byte (byte aligned)
  const int64_t vrow_bytes = A.vld * ESZ;

  // ---- stage inputs ----
  if (OP == T_PRUNE || OP == T_COMPRESS) {
    if (OPT) tile_in<ESZ, TILE_K, TR>(s_dense, A.a, sr0, sc0, srows, scols, A.lda, A.vec_ok);
    else tile_in<ESZ, TR, TILE_K>(s_dense, A.a, sr0, sc0, srows, scols, A.lda, A.vec_ok);
  }
  if (OP == T_PRUNE) {
    for (int w = threadIdx.x; w < LDS_MASK / 4; w += TPB) s_mask[w] = 0;
  }
  if (OP == T_COMPRESS) {
    for (int w = threadIdx.x; w < LDS_META / 4; w += TPB) s_meta[w] = 0;
  }
  if (OP == T_DECOMPRESS) {
    for (int w = threadIdx.x; w < LDS_DENSE / 16; w += TPB) ((u32x4*)s_dense)[w] = u32x4{0, 0, 0, 0};
    const int vwords = (vals_per_row * ESZ + 3) / 4;      // dwords covering this tile's values in a row
    for (int e = threadIdx.x; e < TR * vwords; e += TPB) {
      const int r = e / vwords, c = e % vwords;
      if (r < rows_here) {
        const uint32_t v = *(const uint32_t*)(A.vals + (i0 + r) * vrow_bytes + vbyte0 + 4 * c);
        *(uint32_t*)(s_vals + r * VROW + 4 * c) = v;
      }
    }
    for (int e = threadIdx.x; e < TR * meta_bytes_row; e += TPB) {
      const int r = e / meta_bytes_row, c = e % meta_bytes_row;
      if (r < rows_here) ((uint8_t*)s_meta)[r * META_ROW_BYTES + c] = A.meta[(i0 + r) * A.mld + mbase + c];
    }
  }
  __syncthreads();

  // ---- per-group work out of LDS ----
  for (int it = threadIdx.x; it < TR * GPR; it += TPB) {
    int i, g;
    if (OPT) { i = it % TR; g = it / TR; }
    else { i = it / GPR; g = it % GPR; }
    if (i >= rows_here || g >= groups_here) continue;
    // element (i, g*M + j) of the logical tile lives at this LDS index:
    auto at = [&](int j) { return OPT ? (g * M + j) * TR + i : i * TILE_K + g * M + j; };
    if (OP == T_DECOMPRESS) {
      const uint8_t* mrow = (const uint8_t*)s_meta + i * META_ROW_BYTES;
      for (int s = 0; s < N; s++) {
        const int t0 = (g * N + s) * b;
        uint32_t w = (uint32_t)mrow[t0 / 8] | ((uint32_t)mrow[t0 / 8 + 1] << 8);
        const int j = (int)((w >> (t0 % 8)) & ((1u << b) - 1u));
        lds_set<ESZ>(s_dense, at(j), lds_elem<ESZ>(s_vals + i * VROW, g * N + s));
      }
      continue;
    }
    uint32_t mag[M];
#pragma unroll
    for (int j = 0; j < M; j++) mag[j] = magkey<DT>(lds_elem<ESZ>(s_dense, at(j)));
    const uint32_t keep = select_topn<M>(mag, N);
    if (OP == T_PRUNE) {
#pragma unroll
      for (int j = 0; j < M; j++)
        if (!((keep >> j) & 1u)) lds_set<ESZ>(s_dense, at(j), 0u);
      if (A.mask) {
        if (!OPT) {
          // bits (i, g*M .. g*M+M-1) of the stored tile; M divides 32
          const int bit = g * M;
          atomicOr(&s_mask[i * (TILE_K / 32) + bit / 32], keep << (bit % 32));
        } else {
#pragma unroll
          for (int j = 0; j < M; j++)
            if ((keep >> j) & 1u) atomicOr(&s_mask[(g * M + j) * (TR / 32) + i / 32], 1u << (i % 32));
        }
      }
    } else {  // T_COMPRESS
      int s = 0;
      uint8_t* vrow = s_vals + i * VROW;
      uint32_t* mrow = s_meta + i * meta_words_row;
#pragma unroll
      for (int j = 0; j < M; j++) {
        if (!((keep >> j) & 1u)) continue;
        lds_set<ESZ>(vrow, g * N + s, lds_elem<ESZ>(s_dense, at(j)));
        const int t0 = (g * N + s) * b;
        atomicOr(&mrow[t0 / 32], (uint32_t)j << (t0 % 32));
        if ((t0 % 32) + b > 32) atomicOr(&mrow[t0 / 32 + 1], (uint32_t)j >> (32 - t0 % 32));
        s++;
      }
    }
  }
  __syncthreads();

  // ---- write back ----
  if (OP == T_PRUNE || OP == T_DECOMPRESS) {
    if (OPT) tile_out<ESZ, TILE_K, TR>(A.out, s_dense, sr0, sc0, srows, scols, A.lda, A.vec_ok);
    else tile_out<ESZ, TR, TILE_K>(A.out, s_dense, sr0, sc0, srows, scols, A.lda, A.vec_ok);
  }
  if (OP == T_PRUNE && A.mask) {
    constexpr int WPR = OPT ? TR / 32 : TILE_K / 32;
    constexpr int SR = OPT ? TILE_K : TR;
    for (int e = threadIdx.x; e < SR * WPR; e += TPB) {
      const int r = e / WPR, w = e % WPR;
      const int64_t gr = sr0 + r, gw = sc0 / 32 + w;
      if (gr < srows && gw < A.mask_ld) A.mask[gr * A.mask_ld + gw] = s_mask[e];
    }
  }
  if (OP == T_COMPRESS) {
    // values: this tile's dwords, plus the zero padding of the row after its last group
    const int vbytes = vals_per_row * ESZ;
    const int64_t vend = last_k_tile ? vrow_bytes : vbyte0 + vbytes;
    const int vwords = (int)((vend - vbyte0) / 4);
    for (int e = threadIdx.x; e < rows_here * vwords; e += TPB) {
      const int r = e / vwords, c = e % vwords;
      uint32_t v = 0;
      if (4 * c < vbytes) {
        v = *(const uint32_t*)(s_vals + r * VROW + 4 * c);
        if (4 * c + 4 > vbytes) v &= 0xFFFFFFFFu >> (8 * (4 * c + 4 - vbytes));   // bytes past the values are padding
      }
      *(uint32_t*)(A.vals + (i0 + r) * vrow_bytes + vbyte0 + 4 * c) = v;
    }
    const int64_t mend = last_k_tile ? A.mld : mbase + meta_bytes_row;
    const int mcount = (int)(mend - mbase);
    for (int e = threadIdx.x; e < rows_here * mcount; e += TPB) {
      const int r = e / mcount, c = e % mcount;
      const uint8_t v = c < meta_bytes_row ? ((const uint8_t*)s_meta)[r * META_ROW_BYTES + c] : (uint8_t)0;
      A.meta[(i0 + r) * A.mld + mbase + c] = v;
    }
  }
}

// ------------------------------------------------------------------ 4x4 tiles

// Pair p keeps columns PA[p] and PB[p] of a tile row.
__device__ constexpr int PA[6] = {0, 0, 0, 1, 1, 2};
__device__ constexpr int PB[6] = {1, 2, 3, 2, 3, 3};

// Number of (p0, p1, p2, p3) choices with every column chosen twice; p3 is
// forced by the first three rows (the two columns still at one).
constexpr int count_tile_patterns() {
  constexpr int pa[6] = {0, 0, 0, 1, 1, 2}, pb[6] = {1, 2, 3, 2, 3, 3};
  int n = 0;
  for (int p0 = 0; p0 < 6; p0++)
    for (int p1 = 0; p1 < 6; p1++)
      for (int p2 = 0; p2 < 6; p2++) {
        int c[4] = {0, 0, 0, 0};
        c[pa[p0]]++; c[pb[p0]]++; c[pa[p1]]++; c[pb[p1]]++; c[pa[p2]]++; c[pb[p2]]++;
        int ones = 0, bad = 0;
        for (int x = 0; x < 4; x++) { ones += c[x] == 1; bad += (c[x] == 0 || c[x] > 2); }
        n += (!bad && ones == 2);
      }
  return n;
}
static_assert(count_tile_patterns() == 90, "4x4 tiles with two per row and column: 90 patterns");

// Row masks (4 bits per tile row, row 0 lowest) of the first pattern in the
// scan order: the winner when no candidate's score compares greater than the
// start value, which happens only when every candidate keeps a NaN.
constexpr uint32_t first_tile_pattern() {
  constexpr int pa[6] = {0, 0, 0, 1, 1, 2}, pb[6] = {1, 2, 3, 2, 3, 3};
  for (int p0 = 0; p0 < 6; p0++)
    for (int p1 = 0; p1 < 6; p1++)
      for (int p2 = 0; p2 < 6; p2++)
        for (int p3 = 0; p3 < 6; p3++) {
          const int p[4] = {p0, p1, p2, p3};
          int c[4] = {0, 0, 0, 0};
          uint32_t bits = 0;
          for (int r = 0; r < 4; r++) {
            c[pa[p[r]]]++; c[pb[p[r]]]++;
            bits |= ((1u << pa[p[r]]) | (1u << pb[p[r]])) << (4 * r);
          }
          if (c[0] == 2 && c[1] == 2 && c[2] == 2 && c[3] == 2) return bits;
        }
  return 0;
}
constexpr uint32_t kFirstTilePattern = first_tile_pattern();   // folded here, not evaluated per tile
static_assert(kFirstTilePattern == 0xCC33u, "first pattern keeps (0,1), (0,1), (2,3), (2,3)");

template <int DT, int ESZ>
__device__ __forceinline__ uint32_t load_raw(const uint8_t* p, int64_t idx) {
  return ESZ == 2 ? (uint32_t)((const uint16_t*)p)[idx] : (uint32_t)p[idx];
}

// One row of a 4x4 tile, element by element (four elements from idx on): the
// ragged last tiles of a row and rows that are not 16-byte aligned.
template <int ESZ>
__device__ __forceinline__ void load_row4(const uint8_t* p, int64_t idx, uint32_t (&v)[4]) {
#pragma unroll
  for (int c = 0; c < 4; c++) v[c] = load_raw<0, ESZ>(p, idx + c);
}
template <int ESZ>
__device__ __forceinline__ void store_row4(uint8_t* p, int64_t idx, const uint32_t (&v)[4]) {
#pragma unroll
  for (int c = 0; c < 4; c++) {
    if (ESZ == 2) ((uint16_t*)p)[idx + c] = (uint16_t)v[c];
    else p[idx + c] = (uint8_t)v[c];
  }
}

// Row-pair decomposition of the 90 patterns. After tile rows 0 and 1 keep
// pairs p0 and p1, rows 2 and 3 must keep what each column still needs: a
// need vector with entries in {0, 1, 2} summing to 4 (19 such vectors). Each
// (p0, p1) leads to one need state, and each state has 1, 2 or 6 completions
// (p2, p3). In order of increasing p2 the completions of a state, and in
// lexicographic order the (p0, p1), enumerate the 90 patterns in the scan's
// order.
struct TilePairTables {
  int nstates;
  int state_of[36];       // (p0 * 6 + p1) -> need state
  int ncomp[19];
  int comp_p2[19][6], comp_p3[19][6];
};
constexpr TilePairTables make_pair_tables() {
  constexpr int pa[6] = {0, 0, 0, 1, 1, 2}, pb[6] = {1, 2, 3, 2, 3, 3};
  TilePairTables t{};
  int need[19][4] = {};
  for (int p0 = 0; p0 < 6; p0++)
    for (int p1 = 0; p1 < 6; p1++) {
      int nd[4] = {2, 2, 2, 2};
      nd[pa[p0]]--; nd[pb[p0]]--; nd[pa[p1]]--; nd[pb[p1]]--;
      int st = -1;
      for (int x = 0; x < t.nstates; x++)
        if (need[x][0] == nd[0] && need[x][1] == nd[1] && need[x][2] == nd[2] && need[x][3] == nd[3]) st = x;
      if (st < 0) {
        st = t.nstates++;
        for (int c = 0; c < 4; c++) need[st][c] = nd[c];
        t.ncomp[st] = 0;
        for (int p2 = 0; p2 < 6; p2++) {
          int rest[4] = {nd[0], nd[1], nd[2], nd[3]};
          rest[pa[p2]]--; rest[pb[p2]]--;
          bool ok = true;
          for (int c = 0; c < 4; c++) ok = ok && rest[c] >= 0 && rest[c] <= 1;
          if (!ok) continue;
          for (int p3 = 0; p3 < 6; p3++)
            if (rest[pa[p3]] == 1 && rest[pb[p3]] == 1) {
              t.comp_p2[st][t.ncomp[st]] = p2;
              t.comp_p3[st][t.ncomp[st]] = p3;
              t.ncomp[st]++;
            }
        }
      }
      t.state_of[p0 * 6 + p1] = st;
    }
  return t;
}
constexpr TilePairTables kPairTab = make_pair_tables();
constexpr int count_pair_patterns() {
  int n = 0;
  for (int i = 0; i < 36; i++) n += kPairTab.ncomp[kPairTab.state_of[i]];
  return n;
}
static_assert(kPairTab.nstates == 19 && count_pair_patterns() == 90, "19 need states, 90 patterns");

// Tie ranks. With column offsets o = (4, 2, 1, 0), pair p of a row gets
// f(p) = o[PA[p]] + o[PB[p]] = 6 - p, and a candidate gets the rank
// 49 f(p0) + 7 f(p1) + f(p2) (p3 follows from the other three): base-7 digits in
// 1..6, so increasing rank is decreasing (p0, p1, p2) in lexicographic order,
// the scan's order reversed. Ranks lie in [57, 342]; the table gives each used
// rank's pattern as four row masks (row 0 lowest).
struct TilePatternTable {
  uint16_t pat[343];
};
constexpr TilePatternTable make_pattern_table() {
  constexpr int pa[6] = {0, 0, 0, 1, 1, 2}, pb[6] = {1, 2, 3, 2, 3, 3};
  TilePatternTable t{};
  for (int i = 0; i < 36; i++) {
    const int st = kPairTab.state_of[i], p0 = i / 6, p1 = i % 6;
    const int m0 = (1 << pa[p0]) | (1 << pb[p0]), m1 = (1 << pa[p1]) | (1 << pb[p1]);
    for (int c = 0; c < kPairTab.ncomp[st]; c++) {
      const int p2 = kPairTab.comp_p2[st][c], p3 = kPairTab.comp_p3[st][c];
      t.pat[49 * (6 - p0) + 7 * (6 - p1) + (6 - p2)] =
          (uint16_t)(m0 | m1 << 4 | ((1 << pa[p2]) | (1 << pb[p2])) << 8 | ((1 << pa[p3]) | (1 << pb[p3])) << 12);
    }
  }
  return t;
}
__constant__ TilePatternTable kTilePatterns = make_pattern_table();
static_assert(make_pattern_table().pat[49 * 6 + 7 * 6 + 1] == kFirstTilePattern,
              "the highest rank (p0 = p1 = 0, p2 = 5) is the scan's first pattern");
constexpr int kRowWeight[4] = {49, 7, 1, 0};
constexpr int kColOffset[4] = {4, 2, 1, 0};

// The key of a candidate is its score plus its rank in units uu. When every
// score is a multiple of 512 uu and every key lies below 2^53 uu (fp64) or 2^31
// (int32), all sums are exact, the largest key has the largest score, and among
// equal scores it has the highest rank: the scan's first maximum. Adding
// kRowWeight[r] * kColOffset[c] * uu to element (r, c) puts the rank into the
// row-pair sums t[r][p], so a key is a plain sum of four row terms and its
// maximum is taken in stages: per need state over rows 2 and 3, then per p0
// over p1, then over p0.
__device__ __forceinline__ double kmax(double x, double y) { return fmax(x, y); }
__device__ __forceinline__ int32_t kmax(int32_t x, int32_t y) { return x > y ? x : y; }

template <typename K, int ST, int C>
__device__ __forceinline__ void best_completion(const K (&s2)[6], const K (&s3)[6], K& b) {
  if constexpr (C < kPairTab.ncomp[ST]) {
    const K v = s2[kPairTab.comp_p2[ST][C]] + s3[kPairTab.comp_p3[ST][C]];
    if constexpr (C == 0) b = v;
    else b = kmax(b, v);
    best_completion<K, ST, C + 1>(s2, s3, b);
  }
}
template <typename K, int ST>
__device__ __forceinline__ void best_completions(const K (&s2)[6], const K (&s3)[6], K (&b)[19]) {
  best_completion<K, ST, 0>(s2, s3, b[ST]);
  if constexpr (ST + 1 < 19) best_completions<K, ST + 1>(s2, s3, b);
}
template <typename K, int P0, int P1>
__device__ __forceinline__ void best_row1(const K (&s1)[6], const K (&b)[19], K& m) {
  const K v = s1[P1] + b[kPairTab.state_of[P0 * 6 + P1]];
  if constexpr (P1 == 0) m = v;
  else m = kmax(m, v);
  if constexpr (P1 + 1 < 6) best_row1<K, P0, P1 + 1>(s1, b, m);
}
template <typename K, int P0>
__device__ __forceinline__ void best_key(const K (&s0)[6], const K (&s1)[6], const K (&b)[19], K& key) {
  K m;
  best_row1<K, P0, 0>(s1, b, m);
  const K v = s0[P0] + m;
  if constexpr (P0 == 0) key = v;
  else key = kmax(key, v);
  if constexpr (P0 + 1 < 6) best_key<K, P0 + 1>(s0, s1, b, key);
}
// The largest key over all 90 candidates, from the row-pair terms.
template <typename K>
__device__ __forceinline__ K max_key(const K (&t)[4][6]) {
  K b[19], key;
  best_completions<K, 0>(t[2], t[3], b);
  best_key<K, 0>(t[0], t[1], b, key);
  return key;
}

// The fixed-order scan of all 90 candidates, for tiles whose keys could round
// (a NaN or Inf, or bf16 magnitudes spread over more than 32 binades). Kept out
// of line: it is rare, and its registers would otherwise bound the occupancy of
// the common path.
struct TileRaw {
  uint32_t v[16];
};
template <int DT>
__device__ __attribute__((noinline)) uint32_t scan_tile(TileRaw raw) {
  double s[4][6];
#pragma unroll
  for (int r = 0; r < 4; r++)
#pragma unroll
    for (int p = 0; p < 6; p++) s[r][p] = absval64<DT>(raw.v[4 * r + PA[p]]) + absval64<DT>(raw.v[4 * r + PB[p]]);
  constexpr auto bits = [](int p) { return (1u << PA[p]) | (1u << PB[p]); };
  uint32_t bmask = kFirstTilePattern;
  // scan candidates in order (p0 outermost); replace only on a strictly larger
  // score. The winner is kept as its four row masks packed in one constant (one
  // select per candidate), and the best score as a running maximum (the same
  // value the strict replacement keeps; a NaN score changes neither). It starts
  // at the first pattern, which stays when every candidate keeps a NaN.
  double best = -1.0;
#pragma unroll
  for (int p0 = 0; p0 < 6; p0++)
#pragma unroll
    for (int p1 = 0; p1 < 6; p1++)
#pragma unroll
      for (int p2 = 0; p2 < 6; p2++) {
        int c[4] = {0, 0, 0, 0};
        c[PA[p0]]++; c[PB[p0]]++; c[PA[p1]]++; c[PB[p1]]++; c[PA[p2]]++; c[PB[p2]]++;
        int ones = 0, bad = 0, lo = -1, hi = -1;
#pragma unroll
        for (int x = 0; x < 4; x++) {
          ones += c[x] == 1; bad += (c[x] == 0 || c[x] > 2);
          if (c[x] == 1) { if (lo < 0) lo = x; else hi = x; }
        }
        if (bad || ones != 2) continue;
        int p3 = 0;
#pragma unroll
        for (int p = 0; p < 6; p++) if (PA[p] == lo && PB[p] == hi) p3 = p;
        const double score = ((s[0][p0] + s[1][p1]) + s[2][p2]) + s[3][p3];
        const uint32_t cand = bits(p0) | bits(p1) << 4 | bits(p2) << 8 | bits(p3) << 12;
        bmask = score > best ? cand : bmask;
        best = fmax(best, score);
      }
  return bmask;
}

// The transposable pattern of one 4x4 tile (raw element bits, row-major; for
// 16-bit types also the tile's eight 32-bit words, row r in words 2r, 2r + 1):
// its four row masks, row 0 lowest.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
template <int DT>
__device__ __forceinline__ uint32_t select_tile(const uint32_t (&raw)[4][4], const uint32_t (&wd)[8]) {
  if constexpr (DT == DT_I8) {
    // magnitudes are integers up to 128, u = 1: int32 keys 512 s + rank, below 2^20
    int32_t w[4][4], t[4][6];
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const int32_t v = (int32_t)(int8_t)(uint8_t)raw[r][c];
        w[r][c] = ((v < 0 ? -v : v) << 9) + kRowWeight[r] * kColOffset[c];
      }
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
      for (int p = 0; p < 6; p++) t[r][p] = w[r][PA[p]] + w[r][PB[p]];
    return kTilePatterns.pat[max_key<int32_t>(t) & 511];
  } else {
    // The unit u that every magnitude is a multiple of, and the key unit
    // uu = u / 512: fp16 u = 2^-24 (scores below 2^19); bf16 u = the unit of
    // the smallest non-zero exponent field E (at least 1), 2^(E - 134), with
    // scores below 2^(Emax - 123). Keys are exact for every finite fp16 tile
    // and for bf16 tiles with Emax - E <= 32; others (a NaN or Inf, or bf16
    // magnitudes spread further) take the scan of all 90 in the fixed order.
    double w[4][4];
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
      for (int c = 0; c < 4; c++) {
        if constexpr (DT == DT_F16)
          w[r][c] = (double)fabsf((float)__builtin_bit_cast(_Float16, (uint16_t)raw[r][c]));
        else
          w[r][c] = absval64<DT>(raw[r][c]);
      }
    bool exact;
    int uexp = -33;                                          // log2 uu
    if constexpr (DT == DT_F16) {
      // no NaN or Inf: the sum of all sixteen finite magnitudes is finite
      double total = 0.0;
#pragma unroll
      for (int r = 0; r < 4; r++) total += (w[r][0] + w[r][1]) + (w[r][2] + w[r][3]);
      exact = total < __builtin_huge_val();
    } else {
      // largest magnitude, and smallest non-zero one minus 1 (0xFFFF when all are zero)
      u16x2 mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const u16x2 m = __builtin_bit_cast(u16x2, wd[i] & 0x7FFF7FFFu);
        mx = __builtin_elementwise_max(mx, m);
        mn = __builtin_elementwise_min(mn, m - (u16x2){1, 1});
      }
      const int emax = (int)((mx[0] > mx[1] ? mx[0] : mx[1]) >> 7);
      const uint32_t mn1 = mn[0] < mn[1] ? mn[0] : mn[1];
      const int emin = mn1 == 0xFFFFu ? 1 : (int)((mn1 + 1u) >> 7);
      const int e1 = emin > 1 ? emin : 1;
      exact = emax != 0xFF && emax - e1 <= 32;
      uexp = e1 - 143;
    }
    uint32_t bmask;
    if (exact) {
      const double uu = __longlong_as_double((long long)(1023 + uexp) << 52);
      double t[4][6];
#pragma unroll
      for (int r = 0; r < 4; r++) {
#pragma unroll
        for (int c = 0; c < 4; c++)
          if (kRowWeight[r] * kColOffset[c] != 0) w[r][c] = fma((double)(kRowWeight[r] * kColOffset[c]), uu, w[r][c]);
#pragma unroll
        for (int p = 0; p < 6; p++) t[r][p] = w[r][PA[p]] + w[r][PB[p]];
      }
      const double x = max_key<double>(t) * __longlong_as_double((long long)(1023 - uexp) << 52);   // key / uu
      const double hi = floor(x * (1.0 / 512.0));
      bmask = kTilePatterns.pat[(int)fma(hi, -512.0, x)];
    } else {
      bmask = scan_tile<DT>(TileRaw{{raw[0][0], raw[0][1], raw[0][2], raw[0][3], raw[1][0], raw[1][1], raw[1][2], raw[1][3],
                                     raw[2][0], raw[2][1], raw[2][2], raw[2][3], raw[3][0], raw[3][1], raw[3][2], raw[3][3]}});
    }
    return bmask;
  }
}

// Each thread takes TPT horizontally adjacent tiles, one 16-byte word per tile
// row (one load, one store per row when rows are 16-byte aligned); lanes run
// along tile columns so each row access is contiguous across the wave. Blocks
// stride down the tile rows, loading the next tile row while selecting the
// current one.
template <int ESZ>
__device__ __forceinline__ void load_tile_rows(const uint8_t* a, int64_t ti, int64_t ld, int64_t tj0,
                                               int64_t ntiles, bool full, u32x4 (&pk)[4]) {
  constexpr int TPT = 16 / (4 * ESZ);
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int64_t idx = (ti * 4 + r) * ld + tj0 * 4;
    if (full) {
      pk[r] = *(const u32x4*)(a + idx * ESZ);
    } else {
      uint32_t v[TPT][4];
#pragma unroll
      for (int t = 0; t < TPT; t++) {
        if (tj0 + t < ntiles) load_row4<ESZ>(a, idx + 4 * t, v[t]);
        else v[t][0] = v[t][1] = v[t][2] = v[t][3] = 0u;
      }
#pragma unroll
      for (int d = 0; d < 4; d++) {
        uint32_t word = 0;
#pragma unroll
        for (int x = 0; x < 4 / ESZ; x++) {
          const int e = d * (4 / ESZ) + x;
          word |= v[e / 4][e % 4] << (8 * ESZ * x);
        }
        pk[r][d] = word;
      }
    }
  }
}

template <int DT, int ESZ>
__global__ void __launch_bounds__(TPB) tile4_prune_kernel(const uint8_t* a, uint8_t* out, uint32_t* mask,
                                                          int64_t rows, int64_t cols, int64_t ld,
                                                          int64_t mask_ld, int vec) {
  constexpr int TPT = 16 / (4 * ESZ);
  const int64_t ntiles = cols / 4, ntr = rows / 4;
  const int64_t tj0 = ((int64_t)blockIdx.x * TPB + threadIdx.x) * TPT;
  const bool full = vec && tj0 + TPT <= ntiles;
  const bool any = tj0 < ntiles;
  u32x4 pk[4];
  int64_t ti = blockIdx.y;
  if (any && ti < ntr) load_tile_rows<ESZ>(a, ti, ld, tj0, ntiles, full, pk);
  for (; ti < ntr; ti += gridDim.y) {
    u32x4 nx[4];
    const int64_t tn = ti + gridDim.y;
    if (any && tn < ntr) load_tile_rows<ESZ>(a, tn, ld, tj0, ntiles, full, nx);
    uint32_t rowbits[4] = {0u, 0u, 0u, 0u};   // TPT * 4 bits per row, tile t at bit 4 t
#pragma unroll
    for (int t = 0; t < TPT; t++) {
      uint32_t raw[4][4];
#pragma unroll
      for (int r = 0; r < 4; r++)
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const int e = 4 * t + c;
          const uint32_t word = pk[r][e * ESZ / 4];
          raw[r][c] = ESZ == 2 ? (word >> (16 * (e & 1))) & 0xFFFFu : (word >> (8 * (e & 3))) & 0xFFu;
        }
      uint32_t wd[8];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        wd[2 * r] = pk[r][(2 * t) & 3];
        wd[2 * r + 1] = pk[r][(2 * t + 1) & 3];
      }
      const uint32_t bm = tj0 + t < ntiles ? select_tile<DT>(raw, wd) : 0u;   // no bits past the last tile
#pragma unroll
      for (int r = 0; r < 4; r++) rowbits[r] |= ((bm >> (4 * r)) & 15u) << (4 * t);
      __builtin_amdgcn_sched_barrier(0);   // one tile's selection at a time: bounds live registers
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
      // keep mask of the row's 4 TPT elements, element e at bits [8 ESZ e, 8 ESZ (e + 1))
      u32x4 wv;
#pragma unroll
      for (int d = 0; d < 4; d++) {
        uint32_t m = 0;
#pragma unroll
        for (int x = 0; x < 4 / ESZ; x++) {
          const int e = d * (4 / ESZ) + x;
          m |= ((rowbits[r] >> e) & 1u) ? (ESZ == 2 ? 0xFFFFu : 0xFFu) << (8 * ESZ * x) : 0u;
        }
        wv[d] = pk[r][d] & m;
      }
      const int64_t idx = (ti * 4 + r) * ld + tj0 * 4;
      if (full) {
        *(u32x4*)(out + idx * ESZ) = wv;
      } else {
#pragma unroll
        for (int t = 0; t < TPT; t++) {
          if (tj0 + t >= ntiles) continue;
          uint32_t v[4];
#pragma unroll
          for (int c = 0; c < 4; c++) {
            const int e = 4 * t + c;
            v[c] = ESZ == 2 ? (wv[e / 2] >> (16 * (e & 1))) & 0xFFFFu : (wv[e / 4] >> (8 * (e & 3))) & 0xFFu;
          }
          store_row4<ESZ>(out, idx + 4 * t, v);
        }
      }
    }
    if (mask) {
      // 8 consecutive tiles share a 32-bit mask word per row: OR the 8 / TPT lanes holding them.
      const int sub = (int)(tj0 % 8);
#pragma unroll
      for (int r = 0; r < 4; r++) {
        uint32_t v = rowbits[r] << (4 * sub);
#pragma unroll
        for (int off = 1; off < 8 / TPT; off <<= 1) v |= __shfl_xor(v, off);
        if (any && sub == 0) mask[(ti * 4 + r) * mask_ld + tj0 / 8] = v;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; r++) pk[r] = nx[r];
  }
}

// ------------------------------------------------------------------ checks

template <int DT, int ESZ>
__global__ void __launch_bounds__(TPB) check1d_kernel(const uint8_t* a, int64_t m, int64_t k, int64_t lda,
                                                      int N, int M, int op_t, int vec_ok, int32_t* count) {
  const int64_t groups = k / M;
  int bad = 0;
  for (int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x; t < m * groups; t += (int64_t)gridDim.x * TPB) {
    int64_t i, g;
    if (op_t) { i = t % m; g = t / m; }        // lanes along stored columns
    else { i = t / groups; g = t % groups; }   // lanes along a stored row
    int nz = 0;
    const int gbytes = M * ESZ;
    if (!op_t && vec_ok && gbytes >= 4) {
      // the group is M * esize contiguous, naturally aligned bytes: whole-dword loads
      const uint8_t* p = a + (size_t)(i * lda + g * M) * ESZ;
      for (int x = 0; x < gbytes; x += 16) {
        uint32_t w[4] = {0, 0, 0, 0};
        const int nb = gbytes - x < 16 ? gbytes - x : 16;
        if (nb == 16) { const u32x4 v = *(const u32x4*)(p + x); w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3]; }
        else if (nb == 8) { const u32x2 v = *(const u32x2*)(p + x); w[0] = v[0]; w[1] = v[1]; }
        else w[0] = *(const uint32_t*)(p + x);
#pragma unroll
        for (int d = 0; d < 4; d++) {
          if (ESZ == 2) nz += ((w[d] & 0x7FFFu) != 0u) + (((w[d] >> 16) & 0x7FFFu) != 0u);
          else nz += ((w[d] & 0xFFu) != 0u) + ((w[d] & 0xFF00u) != 0u) + ((w[d] & 0xFF0000u) != 0u) + ((w[d] & 0xFF000000u) != 0u);
        }
      }
    } else {
      for (int j = 0; j < M; j++) {
        const int64_t idx = op_t ? (g * M + j) * lda + i : i * lda + g * M + j;
        nz += magkey<DT>(load_raw<DT, ESZ>(a, idx)) != 0u;
      }
    }
    bad += nz > N;
  }
  block_add_count(count, bad);
}

template <int DT, int ESZ>
__global__ void __launch_bounds__(TPB) check_tile_kernel(const uint8_t* a, int64_t rows, int64_t cols, int64_t ld,
                                                         int vec, int32_t* count) {
  // the tile prune's geometry: TPT adjacent tiles per thread, 16-byte rows when aligned
  constexpr int TPT = 16 / (4 * ESZ);
  const int64_t ntiles = cols / 4;
  const int64_t tj0 = ((int64_t)blockIdx.x * TPB + threadIdx.x) * TPT;
  const bool full = vec && tj0 + TPT <= ntiles;
  int bad = 0;
  for (int64_t ti = blockIdx.y; tj0 < ntiles && ti < rows / 4; ti += gridDim.y) {
    u32x4 pk[4];
    load_tile_rows<ESZ>(a, ti, ld, tj0, ntiles, full, pk);
#pragma unroll
    for (int t = 0; t < TPT; t++) {
      uint32_t nzm = 0;   // bit r*4+c set when element (r, c) of tile t is non-zero
#pragma unroll
      for (int r = 0; r < 4; r++)
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const int e = 4 * t + c;
          const uint32_t word = pk[r][e * ESZ / 4];
          const uint32_t raw = ESZ == 2 ? (word >> (16 * (e & 1))) & 0xFFFFu : (word >> (8 * (e & 3))) & 0xFFu;
          nzm |= (magkey<DT>(raw) != 0u ? 1u : 0u) << (r * 4 + c);
        }
#pragma unroll
      for (int x = 0; x < 4; x++) {
        bad += __builtin_popcount((nzm >> (4 * x)) & 0xFu) > 2;
        bad += __builtin_popcount(nzm & (0x1111u << x)) > 2;
      }
    }
  }
  block_add_count(count, bad);
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v) { *p = v; }

// ------------------------------------------------------------------ launchers

static TileArgs make_args(const nm_plan& pl) {
  TileArgs A{};
  A.m = pl.p.m; A.k = pl.p.k; A.lda = pl.p.lda;
  A.N = pl.p.nm_n; A.op_t = pl.p.op_a == NM_OP_T; A.bits = pl.bits;
  A.vld = pl.vld; A.mld = pl.mld;
  A.mask_ld = (pl.a_cols + 31) / 32;
  A.vec_ok = (pl.p.lda * pl.esz_ab) % 16 == 0;
  return A;
}

template <int OP, int DT, int ESZ, int OPT>
static hipError_t dispatch_tile_mo(const nm_plan& pl, const TileArgs& A, hipStream_t s) {
  constexpr int TR = TileRows<OPT>::value;
  const dim3 grid((unsigned)((pl.p.k + TILE_K - 1) / TILE_K), (unsigned)((pl.p.m + TR - 1) / TR));
  switch (pl.p.nm_m) {
    case 4: hipLaunchKernelGGL((tile_kernel<DT, ESZ, 4, OP, OPT>), grid, dim3(TPB), 0, s, A); break;
    case 8: hipLaunchKernelGGL((tile_kernel<DT, ESZ, 8, OP, OPT>), grid, dim3(TPB), 0, s, A); break;
    case 16: hipLaunchKernelGGL((tile_kernel<DT, ESZ, 16, OP, OPT>), grid, dim3(TPB), 0, s, A); break;
    case 32: hipLaunchKernelGGL((tile_kernel<DT, ESZ, 32, OP, OPT>), grid, dim3(TPB), 0, s, A); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int OP, int DT, int ESZ>
static hipError_t dispatch_tile_m(const nm_plan& pl, const TileArgs& A, hipStream_t s) {
  if (A.op_t) return dispatch_tile_mo<OP, DT, ESZ, 1>(pl, A, s);
  return dispatch_tile_mo<OP, DT, ESZ, 0>(pl, A, s);
}

template <int OP>
static hipError_t dispatch_tile(const nm_plan& pl, const TileArgs& A, hipStream_t s) {
  if (pl.p.m == 0 || pl.p.k == 0) return hipSuccess;
  switch (pl.p.type_ab) {
    case NM_F16: return dispatch_tile_m<OP, DT_F16, 2>(pl, A, s);
    case NM_BF16: return dispatch_tile_m<OP, DT_BF16, 2>(pl, A, s);
    default: return dispatch_tile_m<OP, DT_I8, 1>(pl, A, s);
  }
}

hipError_t launch_prune_1d(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s) {
  if (row_path_ok(pl) && !pl.tile_elemwise) return launch_row_prune(pl, a, out, mask, s);
  TileArgs A = make_args(pl);
  A.a = (const uint8_t*)a; A.out = (uint8_t*)out; A.mask = mask;
  return dispatch_tile<T_PRUNE>(pl, A, s);
}

hipError_t launch_compress(const nm_plan& pl, const void* a, void* vals, void* meta, hipStream_t s) {
  if (row_path_ok(pl) && !pl.tile_elemwise) return launch_row_compress(pl, a, vals, meta, s);
  if (colT_path_ok(pl) && !pl.tile_elemwise) return launch_colT_compress(pl, a, vals, meta, s);
  TileArgs A = make_args(pl);
  A.a = (const uint8_t*)a; A.vals = (uint8_t*)vals; A.meta = (uint8_t*)meta;
  // k == 0 gives zero-length compressed rows: nothing to write.
  return dispatch_tile<T_COMPRESS>(pl, A, s);
}

hipError_t launch_decompress(const nm_plan& pl, const void* vals, const void* meta, void* out, hipStream_t s) {
  if (row_path_ok(pl) && !pl.tile_elemwise) return launch_row_decompress(pl, vals, meta, out, s);
  if (colT_path_ok(pl) && !pl.tile_elemwise) return launch_colT_decompress(pl, vals, meta, out, s);
  TileArgs A = make_args(pl);
  A.vals = (uint8_t*)vals; A.meta = (uint8_t*)meta; A.out = (uint8_t*)out;
  return dispatch_tile<T_DECOMPRESS>(pl, A, s);
}

// X (the stored shape of A, lda) keeps the elements whose keep-mask bit is set
// and gets +0 elsewhere: one thread per mask word (32 consecutive elements of
// a stored row).
template <int ESZ>
__global__ void __launch_bounds__(TPB) mask_apply_kernel(const uint32_t* mask, uint8_t* x, int64_t rows, int64_t cols,
                                                         int64_t ld, int64_t mask_ld) {
  const int64_t wid = (int64_t)blockIdx.x * TPB + threadIdx.x;
  if (wid >= rows * mask_ld) return;
  const int64_t r = wid / mask_ld, w = wid % mask_ld;
  const uint32_t bits = mask[r * mask_ld + w];
  const int64_t c0 = w * 32;
  const int n = cols - c0 < 32 ? (int)(cols - c0) : 32;
  for (int e = 0; e < n; e++)
    if (!((bits >> e) & 1u)) {
      if (ESZ == 2) ((uint16_t*)x)[r * ld + c0 + e] = 0;
      else x[r * ld + c0 + e] = 0;
    }
}

hipError_t launch_mask_apply(const nm_plan& pl, const uint32_t* mask, void* x, hipStream_t s) {
  const int64_t rows = pl.a_rows, cols = pl.a_cols;
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t mld = (cols + 31) / 32;
  const dim3 grid((unsigned)((rows * mld + TPB - 1) / TPB));
  if (pl.esz_ab == 2)
    hipLaunchKernelGGL((mask_apply_kernel<2>), grid, dim3(TPB), 0, s, mask, (uint8_t*)x, rows, cols, pl.p.lda, mld);
  else
    hipLaunchKernelGGL((mask_apply_kernel<1>), grid, dim3(TPB), 0, s, mask, (uint8_t*)x, rows, cols, pl.p.lda, mld);
  return hipGetLastError();
}

// Every row starts on a 16-byte boundary.
static bool rows_aligned16(const nm_plan& pl, const void* p) {
  return ((uintptr_t)p % 16) == 0 && (pl.p.lda * pl.esz_ab) % 16 == 0;
}

hipError_t launch_prune_tile(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s) {
  const int64_t rows = pl.a_rows, cols = pl.a_cols;
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t tpt = 16 / (4 * pl.esz_ab);   // tiles per thread
  // about 1024 blocks (four resident per compute unit), each striding down the tile rows
  const int64_t gx = (cols / 4 + tpt * TPB - 1) / (tpt * TPB);
  const int64_t gy = std::min<int64_t>(rows / 4, std::max<int64_t>(1, 1024 / gx));
  const dim3 grid((unsigned)gx, (unsigned)gy);
  const int64_t mld = (cols + 31) / 32;
  const uint8_t* ap = (const uint8_t*)a;
  uint8_t* op = (uint8_t*)out;
  const int vec = rows_aligned16(pl, a) && rows_aligned16(pl, out);
  switch (pl.p.type_ab) {
    case NM_F16: hipLaunchKernelGGL((tile4_prune_kernel<DT_F16, 2>), grid, dim3(TPB), 0, s, ap, op, mask, rows, cols, pl.p.lda, mld, vec); break;
    case NM_BF16: hipLaunchKernelGGL((tile4_prune_kernel<DT_BF16, 2>), grid, dim3(TPB), 0, s, ap, op, mask, rows, cols, pl.p.lda, mld, vec); break;
    default: hipLaunchKernelGGL((tile4_prune_kernel<DT_I8, 1>), grid, dim3(TPB), 0, s, ap, op, mask, rows, cols, pl.p.lda, mld, vec); break;
  }
  return hipGetLastError();
}

hipError_t launch_check(const nm_plan& pl, const void* a, int mode, int32_t* count, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(1), 0, s, count, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint8_t* ap = (const uint8_t*)a;
  if (mode == NM_PRUNE_TILE4X4) {
    const int64_t rows = pl.a_rows, cols = pl.a_cols;
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t tpt = 16 / (4 * pl.esz_ab);
    const int64_t gx = (cols / 4 + tpt * TPB - 1) / (tpt * TPB);
    const dim3 grid((unsigned)gx, (unsigned)std::min<int64_t>(rows / 4, std::max<int64_t>(1, kCheckBlocks / gx)));
    const int vec = rows_aligned16(pl, a);
    switch (pl.p.type_ab) {
      case NM_F16: hipLaunchKernelGGL((check_tile_kernel<DT_F16, 2>), grid, dim3(TPB), 0, s, ap, rows, cols, pl.p.lda, vec, count); break;
      case NM_BF16: hipLaunchKernelGGL((check_tile_kernel<DT_BF16, 2>), grid, dim3(TPB), 0, s, ap, rows, cols, pl.p.lda, vec, count); break;
      default: hipLaunchKernelGGL((check_tile_kernel<DT_I8, 1>), grid, dim3(TPB), 0, s, ap, rows, cols, pl.p.lda, vec, count); break;
    }
    return hipGetLastError();
  }
  const int64_t total = pl.p.m * (pl.p.k / pl.p.nm_m);
  if (total == 0) return hipSuccess;
  if (check_row_ok(pl) && !pl.tile_elemwise) return launch_check_row(pl, a, count, s);
  const dim3 grid((unsigned)std::min<int64_t>((total + TPB - 1) / TPB, kCheckBlocks));
  const int opt = pl.p.op_a == NM_OP_T;
  const int vec = (pl.p.lda * pl.esz_ab) % 16 == 0;
  switch (pl.p.type_ab) {
    case NM_F16: hipLaunchKernelGGL((check1d_kernel<DT_F16, 2>), grid, dim3(TPB), 0, s, ap, pl.p.m, pl.p.k, pl.p.lda, pl.p.nm_n, pl.p.nm_m, opt, vec, count); break;
    case NM_BF16: hipLaunchKernelGGL((check1d_kernel<DT_BF16, 2>), grid, dim3(TPB), 0, s, ap, pl.p.m, pl.p.k, pl.p.lda, pl.p.nm_n, pl.p.nm_m, opt, vec, count); break;
    default: hipLaunchKernelGGL((check1d_kernel<DT_I8, 1>), grid, dim3(TPB), 0, s, ap, pl.p.m, pl.p.k, pl.p.lda, pl.p.nm_n, pl.p.nm_m, opt, vec, count); break;
  }
  return hipGetLastError();
}

}  // namespace nm
