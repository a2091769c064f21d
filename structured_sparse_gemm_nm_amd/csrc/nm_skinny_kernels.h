// Small-n product (GEMV and up to 16 columns), streamed: templates included by
// the per-type instantiation files nm_skinny_{f16,bf16,i8}.hip.
//
// D = alpha * A * op(B) + beta * C with A given as compressed N:M rows
// (values plus the b-bit offsets of each kept value), or as a dense row-major
// A for the small-n dense comparator (DENSE_A).
//
// A block of SK2_WAVES waves takes SK2_WAVES * RW rows, RW per wave; a lane
// takes whole groups of M (one naturally aligned vector load brings a group's
// NV kept values, a window of the row's bit stream their offsets; DENSE_A takes
// 16-byte chunks of a dense row instead). op(B) is staged in LDS as records of
// RB bytes: the n values of one k in B's own type, zero-padded to NP columns.
// Records are laid out so a wave's reads never share a bank: within each
// window of 64 groups of MG consecutive k (MG = M, or the elements of a 16-byte
// chunk for DENSE_A), the record of k = 64 MG w + MG g + j sits at
// 64 MG w + 64 j + g, so lane g reads record 64 j + g whatever its offset j;
// the staging writes record by record (consecutive lanes, consecutive
// records). Records past the end of k are zero, so the arithmetic needs no
// bounds tests. Blocks are persistent (one per CU) and walk row groups; each
// block's work is one sequence of (row group, k chunk, iteration) along which
// A is loaded DEPTH steps ahead of use, across chunk and group ends. Partial
// sums are combined across the wave with butterfly shuffles.
#pragma once
#include "nm_gemm_kernels.h"

namespace nm {

constexpr int SK2_WAVES = 16;
constexpr int SK2_LDS = 128 * 1024;  // bytes of staged B per chunk (one block per CU: registers allow no more)

template <int DT, int NP>
struct SkinnyRec {
  static constexpr int ESZ = DT == DT_I8 ? 1 : 2;
  static constexpr int RB = NP * ESZ;                       // bytes per staged k
  static constexpr int KC = SK2_LDS / RB;                   // k per chunk (a multiple of every window)
};

// NV: kept values per group (the N of N:M, NV * ESZ a power of two up to 16
// bytes), 0 for DENSE_A.
template <int DT, int NP, bool DENSE_A, int RW, int NV>
__global__ void __launch_bounds__(64 * SK2_WAVES) skinny2_kernel(GemmArgs A, int b_op_t) {
  constexpr int ESZ = SkinnyRec<DT, NP>::ESZ;
  constexpr int RB = SkinnyRec<DT, NP>::RB;
  constexpr int KC = SkinnyRec<DT, NP>::KC;
  constexpr int FDT = DT == DT_I8 ? DT_F16 : DT;
  constexpr int EPC = 16 / ESZ;                             // DENSE_A: elements per 16-byte chunk
  constexpr int VB = DENSE_A ? 16 : NV * ESZ;               // value bytes per lane and iteration
  constexpr int PV = VB < 4 ? 1 : VB / 4;                   // value words per piece
  constexpr int ELS = DENSE_A ? EPC : NV;                   // elements per piece
  constexpr int EPW = 4 / ESZ;                              // elements per value word
  constexpr int TPW = ELS < EPW ? ELS : EPW;                // elements used per word
  constexpr bool BIG = ELS * NP >= 256;                     // too many products to unroll the words
  // offset bits of a group start at bit 0..31 of the first word and span at most 5 NV bits
  constexpr int MW = DENSE_A ? 0 : (31 + 5 * NV + 31) / 32 < 3 ? (31 + 5 * NV + 31) / 32 : 3;
  // iterations of A loads in flight per lane: about 8 pieces per wave across
  // its RW rows, fewer for wide groups (registers)
  constexpr int DEPTH = ELS >= 16 ? 2 : ELS == 8 ? (RW > 1 ? 2 : 4) : (8 / RW > 2 ? 8 / RW : 2);
  static_assert(DENSE_A ? NV == 0 : (VB == 1 || VB == 2 || VB == 4 || VB == 8 || VB == 16), "group width");
  typedef typename std::conditional<DT == DT_I8, int32_t, float>::type acc_t;
  extern __shared__ __attribute__((aligned(16))) uint8_t s_b[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = (int)A.n;
  const int M = DENSE_A ? EPC : A.M, b = A.bits;
  const int W = 64 * M;                                     // k per window
  const int lm = __builtin_ctz(M), lw = lm + 6;             // M and W are powers of two
  // B rows can be copied whole: op N, n equal to the record width, rows aligned to it
  const bool b_rowvec = RB <= 16 && !b_op_t && n == NP && ((A.ldb * ESZ) % RB) == 0;
  // the host launches this kernel only for m, k < 2^30, so row, k and group
  // indices are 32-bit; byte offsets are formed in 64 bits
  const int mm = (int)A.m;
  const int row_groups = (mm + SK2_WAVES * RW - 1) / (SK2_WAVES * RW);
  const bool one_chunk = A.k <= KC;
  const int mwords = (int)(A.mld / 4);

  auto elem = [&](uint32_t raw) __attribute__((always_inline)) -> acc_t {
    if constexpr (ESZ == 2) return from_bits16<FDT>((uint16_t)raw);
    else return (acc_t)(int8_t)(uint8_t)raw;
  };
  const uint8_t* s_cur = s_b;                               // the staged chunk being read
  // the NP staged values of record r
  auto brec = [&](int r, acc_t (&bv)[NP]) __attribute__((always_inline)) {
    const uint8_t* p = s_cur + r * RB;
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
  // A data of one iteration of one lane: its value bytes and offset words
  struct Piece { uint32_t v[PV]; uint32_t m[MW > 0 ? MW : 1]; };
  // Loads are unconditional (indices clamped into the operand) so that none
  // sits behind a branch: rows past m load row m - 1 and are never written;
  // groups past the chunk load its last group and are zeroed at use.
  auto load_piece = [&](int row, int kc, int kn, int it, Piece& pc) __attribute__((always_inline)) {
    row = row < mm ? row : mm - 1;
    const int g = it * 64 + lane;
    if constexpr (DENSE_A) {                                // k is a whole number of 16-byte chunks
      const int kk0 = g * EPC < kn - EPC ? g * EPC : kn - EPC;
      const u32x4 v = *(const u32x4*)(A.a + ((size_t)row * (size_t)A.lda + (size_t)(kc + kk0)) * ESZ);
      pc.v[0] = v[0]; pc.v[1] = v[1]; pc.v[2] = v[2]; pc.v[3] = v[3];
    } else {
      const int units = kn >> lm;
      const int gg = (kc >> lm) + (g < units ? g : units - 1);
      const uint8_t* p = A.a + ((size_t)row * (size_t)A.lda + (size_t)gg * NV) * ESZ;
      if constexpr (VB == 16) { const u32x4 v = *(const u32x4*)p; pc.v[0] = v[0]; pc.v[1] = v[1]; pc.v[2] = v[2]; pc.v[3] = v[3]; }
      else if constexpr (VB == 8) { const u32x2 v = *(const u32x2*)p; pc.v[0] = v[0]; pc.v[1] = v[1]; }
      else if constexpr (VB == 4) pc.v[0] = *(const uint32_t*)p;
      else if constexpr (VB == 2) pc.v[0] = *(const uint16_t*)p;
      else pc.v[0] = *p;
      // the group's bits end inside the row's stream, so clamping the word
      // index only ever replaces words that are not used
      const int w0 = (int)(((int64_t)gg * NV * b) >> 5);
      const uint32_t* mr = (const uint32_t*)(A.meta + (size_t)(row >> A.vshift) * (size_t)A.mld);
#pragma unroll
      for (int x = 0; x < MW; x++) pc.m[x] = mr[w0 + x < mwords ? w0 + x : mwords - 1];
    }
  };
  auto use_piece = [&](int kc, int kn, int it, const Piece& pc, acc_t (&acc)[NP]) __attribute__((always_inline)) {
    const int g = it * 64 + lane;
    const int rbase = it * W + lane;                        // record of offset 0 of this lane's group
    const bool valid = DENSE_A ? g * EPC < kn : g < (kn >> lm);
    uint64_t lo = 0, hi = 0;
    int off = 0;
    if constexpr (!DENSE_A) {
      off = (int)((((int64_t)(kc >> lm) + g) * NV * b) & 31);
      lo = ((uint64_t)pc.m[1] << 32) | pc.m[0];
      if constexpr (MW == 3) hi = ((uint64_t)pc.m[2] << 32) | pc.m[1];
    }
    // value word by word; lanes past the chunk use zero values, and their
    // offsets (whatever they are) select records past k, which are zero
    constexpr int WUNROLL = BIG ? 1 : PV;
#pragma unroll WUNROLL
    for (int wi = 0; wi < PV; wi++) {
      uint32_t word = pc.v[0];
#pragma unroll
      for (int q = 1; q < PV; q++)
        if (wi == q) word = pc.v[q];                        // a select when this loop is not unrolled
      word = valid ? word : 0u;
#pragma unroll
      for (int t = 0; t < TPW; t++) {
        const int e = wi * EPW + t;
        int j = e;
        if constexpr (!DENSE_A) {
          const int pbit = off + e * b;
          uint64_t win;
          if constexpr (MW == 3) win = pbit < 32 ? lo >> pbit : hi >> (pbit - 32);
          else win = lo >> pbit;
          j = (int)(win & ((1u << b) - 1u));
        }
        acc_t bv[NP];
        brec(rbase + 64 * j, bv);
        const acc_t av = elem(word >> (8 * ESZ * t));
#pragma unroll
        for (int c = 0; c < NP; c++) acc[c] += av * bv[c];
      }
    }
  };
  // stage B rows kc .. kc + kn - 1 into LDS, and zeros up to the window end.
  // One record per thread and step, consecutive records on consecutive lanes
  // (so the LDS writes never share a bank); record r holds k = win W + j M + o.
  // Each thread issues the loads of SB records (indices clamped into B, past-k
  // records zeroed after the loads) before it writes any of them.
  auto rec_k = [&](int r) __attribute__((always_inline)) -> int {
    const int win = r >> lw, rem = r & (W - 1);
    return (win << lw) + ((rem & 63) << lm) + (rem >> 6);
  };
  auto put_rec = [&](uint8_t* base, int r, const uint32_t* w) __attribute__((always_inline)) {
    uint8_t* d = base + r * RB;
    if constexpr (RB == 1) *d = (uint8_t)w[0];
    else if constexpr (RB == 2) *(uint16_t*)d = (uint16_t)w[0];
    else if constexpr (RB == 4) *(uint32_t*)d = w[0];
    else if constexpr (RB == 8) *(u32x2*)d = u32x2{w[0], w[1]};
    else {
#pragma unroll
      for (int q = 0; q < RB / 16; q++) *(u32x4*)(d + 16 * q) = u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
    }
  };
  auto stage_chunk = [&](int64_t kc, int kn) {
    const int kn_r = (kn + W - 1) & ~(W - 1);               // whole windows (KC is a multiple of W)
    constexpr int RWD = RB < 4 ? 1 : RB / 4;                // words per record
    constexpr int NT = 64 * SK2_WAVES;
    if (b_rowvec) {                                         // a record is one row of B
      constexpr int SB = 32 / RWD < 8 ? 32 / RWD : 8;
      for (int r0 = threadIdx.x; r0 < kn_r; r0 += NT * SB) {
        uint32_t w[SB][RWD];
#pragma unroll
        for (int q = 0; q < SB; q++) {
          const int kk = rec_k(r0 + q * NT);
          const uint8_t* g = A.b + ((kc + (kk < kn ? kk : kn - 1)) * A.ldb) * ESZ;
          if constexpr (RB == 1) w[q][0] = *g;
          else if constexpr (RB == 2) w[q][0] = *(const uint16_t*)g;
          else if constexpr (RB == 4) w[q][0] = *(const uint32_t*)g;
          else if constexpr (RB == 8) { const u32x2 v = *(const u32x2*)g; w[q][0] = v[0]; w[q][1] = v[1]; }
          else { const u32x4 v = *(const u32x4*)g; w[q][0] = v[0]; w[q][1] = v[1]; w[q][2] = v[2]; w[q][3] = v[3]; }
        }
#pragma unroll
        for (int q = 0; q < SB; q++) {
          const int r = r0 + q * NT;
          if (r >= kn_r) break;
          const bool in = rec_k(r) < kn;
#pragma unroll
          for (int x = 0; x < RWD; x++) w[q][x] = in ? w[q][x] : 0u;
          put_rec(s_b, r, w[q]);
        }
      }
    } else {                                                // column by column (op T, or n < NP)
      constexpr int SB = 32 / NP < 8 ? (32 / NP > 0 ? 32 / NP : 1) : 8;
      for (int r0 = threadIdx.x; r0 < kn_r; r0 += NT * SB) {
        uint32_t raw[SB][NP];
#pragma unroll
        for (int q = 0; q < SB; q++) {
          const int kk = rec_k(r0 + q * NT);
          const int64_t kq = kc + (kk < kn ? kk : kn - 1);
#pragma unroll
          for (int c = 0; c < NP; c++) {
            const int cq = c < n ? c : n - 1;
            const int64_t gi = b_op_t ? (int64_t)cq * A.ldb + kq : kq * A.ldb + cq;
            raw[q][c] = ESZ == 2 ? (uint32_t)((const uint16_t*)A.b)[gi] : (uint32_t)A.b[gi];
          }
        }
#pragma unroll
        for (int q = 0; q < SB; q++) {
          const int r = r0 + q * NT;
          if (r >= kn_r) break;
          const bool in = rec_k(r) < kn;
          uint32_t w[RWD];
#pragma unroll
          for (int x = 0; x < RWD; x++) w[x] = 0;
#pragma unroll
          for (int c = 0; c < NP; c++)
            if (in && c < n) w[(c * ESZ) / 4] |= raw[q][c] << (8 * ((c * ESZ) % 4));
          put_rec(s_b, r, w);
        }
      }
    }
  };
  // Double-buffered staging (B rows copied whole into 16-byte records; for
  // narrower records the registers it takes cost more than it saves): the
  // block reads one half of the LDS while the next chunk's rows, loaded into
  // registers at the start of the current chunk, are written into the other
  // half at its last iteration.
  constexpr bool DB_OK = RB == 16;
  constexpr int RWDB = RB < 4 ? 1 : RB / 4;                 // words per record
  constexpr int RPT = DB_OK ? (KC / 2) / (64 * SK2_WAVES) : 1;   // records per thread in half a chunk
  const bool db = DB_OK && !one_chunk && b_rowvec;
  uint32_t sreg[RPT][RWDB];
  auto db_issue = [&](int64_t kc, int kn) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < RPT; q++) {
      const int kk = rec_k(threadIdx.x + q * 64 * SK2_WAVES);
      const uint8_t* g = A.b + ((kc + (kk < kn ? kk : kn - 1)) * A.ldb) * ESZ;
      if constexpr (RB == 4) sreg[q][0] = *(const uint32_t*)g;
      else if constexpr (RB == 8) { const u32x2 v = *(const u32x2*)g; sreg[q][0] = v[0]; sreg[q][1] = v[1]; }
      else if constexpr (RB == 16) {
        const u32x4 v = *(const u32x4*)g;
        sreg[q][0] = v[0]; sreg[q][1] = v[1]; sreg[q][2] = v[2]; sreg[q][3] = v[3];
      }
    }
  };
  auto db_put = [&](uint8_t* base, int kn) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < RPT; q++) {
      const int r = threadIdx.x + q * 64 * SK2_WAVES;
      const bool in = rec_k(r) < kn;
#pragma unroll
      for (int x = 0; x < RWDB; x++) sreg[q][x] = in ? sreg[q][x] : 0u;
      put_rec(base, r, sreg[q]);
    }
  };
  // combine this wave's sums of row group grp, write them, clear them
  auto flush = [&](int grp, acc_t (&acc)[RW][NP]) __attribute__((always_inline)) {
    const int64_t row0 = ((int64_t)grp * SK2_WAVES + wave) * RW;
#pragma unroll
    for (int rr = 0; rr < RW; rr++) {
      const int64_t row = row0 + rr;
#pragma unroll
      for (int c = 0; c < NP; c++)
        for (int o = 32; o > 0; o >>= 1) acc[rr][c] += __shfl_xor(acc[rr][c], o);
      if (row < A.m) {                                      // lane c writes column c
#pragma unroll
        for (int c = 0; c < NP; c++) {
          if (lane != c || c >= n) continue;
          if constexpr (DT == DT_I8) {
            int_store(A, row * A.d_rs + c * A.d_cs, int_epilogue(A, acc[rr][c], row * A.c_rs + c * A.c_cs));
          } else {
            float o = A.alpha * acc[rr][c];
            if (A.beta != 0.0f) o += A.beta * from_bits16<DT>(((const uint16_t*)A.c)[row * A.c_rs + c * A.c_cs]);
            ((uint16_t*)A.d)[row * A.d_rs + c * A.d_cs] = to_bits16<DT>(o);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < NP; c++) acc[rr][c] = 0;
    }
  };

  acc_t acc[RW][NP];
#pragma unroll
  for (int rr = 0; rr < RW; rr++)
#pragma unroll
    for (int c = 0; c < NP; c++) acc[rr][c] = 0;
  const int gstride = gridDim.x;                            // blocks walk row groups blockIdx.x + j gridDim.x
  const int kcs = db ? KC / 2 : KC;                         // k per chunk (a multiple of every window)
  const int nchunks = (int)((A.k + kcs - 1) / kcs);
  if (nchunks == 0) {                                       // k = 0: D = beta C
    for (int grp = blockIdx.x; grp < row_groups; grp += gstride) flush(grp, acc);
    return;
  }
  const int kn_last = (int)(A.k - (int64_t)(nchunks - 1) * kcs);
  const int nit_full = kcs / W;
  const int nit_last = DENSE_A ? ((kn_last + EPC - 1) / EPC + 63) / 64 : (kn_last / M + 63) / 64;
  struct Cur { int grp, c, it; };
  auto advance = [&](Cur& q) __attribute__((always_inline)) {
    if (++q.it == (q.c == nchunks - 1 ? nit_last : nit_full)) {
      q.it = 0;
      if (++q.c == nchunks) { q.c = 0; q.grp += gstride; }
    }
  };
  Cur ld{(int)blockIdx.x, 0, 0}, us = ld;
  Piece pc[RW][DEPTH];
#pragma unroll
  for (int u = 0; u < DEPTH; u++) {
    const int row0 = (ld.grp * SK2_WAVES + wave) * RW;
#pragma unroll
    for (int rr = 0; rr < RW; rr++)
      load_piece(row0 + rr, ld.c * kcs, ld.c == nchunks - 1 ? kn_last : kcs, ld.it, pc[rr][u]);
    advance(ld);
  }
  bool staged = false;
  const int half = (KC / 2) * RB;                           // bytes of one LDS half (double-buffered)
  int begun = 0;                                            // chunks begun (double-buffered)
  bool pend = false;                                        // the next chunk is in registers
  int pend_kn = 0;
  if (db) {                                                 // chunk 0 into half 0
    db_issue(0, nchunks == 1 ? kn_last : kcs);
    db_put(s_b, nchunks == 1 ? kn_last : kcs);
  }
  while (us.grp < row_groups) {
#pragma unroll
    for (int u = 0; u < DEPTH; u++) {
      if (us.grp >= row_groups) break;
      const int kc = us.c * kcs;
      const int kn = us.c == nchunks - 1 ? kn_last : kcs;
      if (us.it == 0) {
        if (us.c == 0 && us.grp != blockIdx.x) flush(us.grp - gstride, acc);
        if (db) {
          // this chunk is in its half; every wave is done with the previous
          // chunk, so the other half is free
          __syncthreads();
          s_cur = s_b + (begun & 1) * half;
          begun++;
          const int nc = us.c + 1 == nchunks ? 0 : us.c + 1;
          pend = (nc == 0 ? us.grp + gstride : us.grp) < row_groups;
          if (pend) {
            pend_kn = nc == nchunks - 1 ? kn_last : kcs;
            db_issue((int64_t)nc * kcs, pend_kn);
          }
        } else if (!(one_chunk && staged)) {
          __syncthreads();                                  // the previous chunk's readers are done
          stage_chunk(kc, kn);
          __syncthreads();
          staged = true;
        }
      }
      const int lrow0 = (ld.grp * SK2_WAVES + wave) * RW;
      const int lkc = ld.c * kcs;
      const int lkn = ld.c == nchunks - 1 ? kn_last : kcs;
#pragma unroll
      for (int rr = 0; rr < RW; rr++) {
        use_piece(kc, kn, us.it, pc[rr][u], acc[rr]);
        load_piece(lrow0 + rr, lkc, lkn, ld.it, pc[rr][u]);   // rows past m load nothing
      }
      if (pend && us.it == (us.c == nchunks - 1 ? nit_last : nit_full) - 1) {
        db_put(s_b + (begun & 1) * half, pend_kn);          // the next chunk, into the free half
        pend = false;
      }
      advance(ld);
      advance(us);
    }
  }
  flush(us.grp - gstride, acc);
}

template <int DT, bool DENSE_A, int NP, int RW, int NV>
static hipError_t launch_skinny2_rw(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  // row groups of SK2_WAVES * RW rows; persistent blocks, as many as fit the
  // CUs at once, each walking every gridDim-th group; when all of k fits one
  // LDS chunk a block stages B once
  constexpr int KC = SkinnyRec<DT, NP>::KC;
  // records are placed within whole windows of 64 groups (64 M, or 64 chunks
  // of 16 bytes for a dense A), so the staged chunk is rounded up to a window;
  // KC is a multiple of every window, so this stays within SK2_LDS
  const int64_t win = 64 * (DENSE_A ? (int64_t)(16 / SkinnyRec<DT, NP>::ESZ) : (int64_t)A.M);
  const int64_t kn = A.k < KC ? A.k : KC;
  const int64_t kr = kn > 0 ? (kn + win - 1) / win * win : win;
  const size_t lds = (size_t)kr * SkinnyRec<DT, NP>::RB;
  static thread_local size_t occ_lds = ~(size_t)0;
  static thread_local int occ_blocks = 1;
  if (occ_lds != lds) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, skinny2_kernel<DT, NP, DENSE_A, RW, NV>,
                                                     64 * SK2_WAVES, lds) != hipSuccess || nb < 1) nb = 1;
    occ_lds = lds;
    occ_blocks = nb;
  }
  const int64_t groups = (A.m + SK2_WAVES * RW - 1) / (SK2_WAVES * RW);
  const int64_t cap = (int64_t)NUM_CU * occ_blocks;
  const int64_t blocks = groups < cap ? groups : cap;
  NM_LAUNCH((skinny2_kernel<DT, NP, DENSE_A, RW, NV>), dim3((unsigned)blocks), dim3(64 * SK2_WAVES), lds, s, A, (int)(pl.p.op_b == NM_OP_T));
  return launch_status();
}

// Tall problems (m >= 16384 rows) give each wave several rows, so that the
// staged B serves more rows per block; how many depends on the registers a
// row takes (elements per lane and iteration, columns).
template <int DT, bool DENSE_A, int NP, int NV>
static hipError_t launch_skinny2_t(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  constexpr int ELS = DENSE_A ? 16 / SkinnyRec<DT, NP>::ESZ : NV;
  constexpr int RW_TALL = ELS >= 16 ? 1 : ELS == 8 ? (NP <= 2 ? 2 : 1) : NP <= 2 ? 4 : NP <= 8 ? 2 : 1;
  if (A.m >= 16384 && RW_TALL > 1) return launch_skinny2_rw<DT, DENSE_A, NP, RW_TALL, NV>(pl, A, s);
  return launch_skinny2_rw<DT, DENSE_A, NP, 1, NV>(pl, A, s);
}

template <int DT, bool DENSE_A, int NV>
static hipError_t launch_skinny2_np(const nm_plan& pl, const GemmArgs& A, hipStream_t s) {
  const int64_t n = A.n;
  if (n <= 1) return launch_skinny2_t<DT, DENSE_A, 1, NV>(pl, A, s);
  if (n <= 2) return launch_skinny2_t<DT, DENSE_A, 2, NV>(pl, A, s);
  if (n <= 4) return launch_skinny2_t<DT, DENSE_A, 4, NV>(pl, A, s);
  if (n <= 8) return launch_skinny2_t<DT, DENSE_A, 8, NV>(pl, A, s);
  return launch_skinny2_t<DT, DENSE_A, 16, NV>(pl, A, s);
}

// Entry for one element type: the dense comparator (op_a = N, rows 16-byte
// aligned, k a multiple of 16 bytes), or compressed A with N * esize in
// {1, 2, 4, 8, 16} bytes (other N return hipErrorInvalidValue; the caller
// checks first).
template <int DT>
static hipError_t launch_skinny2_dt(const nm_plan& pl, const GemmArgs& A, hipStream_t s, bool dense_a) {
  if (dense_a) return launch_skinny2_np<DT, true, 0>(pl, A, s);
  switch (A.N) {
    case 1: return launch_skinny2_np<DT, false, 1>(pl, A, s);
    case 2: return launch_skinny2_np<DT, false, 2>(pl, A, s);
    case 4: return launch_skinny2_np<DT, false, 4>(pl, A, s);
    case 8: return launch_skinny2_np<DT, false, 8>(pl, A, s);
    default:
      if constexpr (DT == DT_I8) {
        if (A.N == 16) return launch_skinny2_np<DT, false, 16>(pl, A, s);
      }
      return hipErrorInvalidValue;
  }
}

hipError_t launch_skinny2_f16(const nm_plan& pl, const GemmArgs& A, hipStream_t s, bool dense_a);
hipError_t launch_skinny2_bf16(const nm_plan& pl, const GemmArgs& A, hipStream_t s, bool dense_a);
hipError_t launch_skinny2_i8(const nm_plan& pl, const GemmArgs& A, hipStream_t s, bool dense_a);

}  // namespace nm
