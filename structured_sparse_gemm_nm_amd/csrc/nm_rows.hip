// Register-path prune, compress and decompress for groups that run along
// stored rows (op_a = N) with 16-byte row starts.
//
// What they compute is the same as the tile kernels in nm_prune.hip (per-group
// top-N by magnitude, ties to the lower offset, after the apex N:M greedy
// calculator; kept values plus b-bit offsets after the cuSPARSELt blog's
// compressed form, in the layout of include/nmsparse.h).
//
// Design: a group of M elements is M * esize contiguous bytes of a stored row,
// so a lane can take whole groups straight from HBM into registers. A lane's
// unit is one 16-byte chunk (16 / (M * esize) groups) or, for 32- and 64-byte
// groups, one group. A wave owns a segment of 64 consecutive units of one row:
// loads are 16-byte vector loads spread over the whole wave, kept values go out
// as one aligned store per lane, and the segment's metadata (64 units' fields,
// a whole number of qwords) is assembled dword by dword from the neighbouring
// lanes' fields with cross-lane reads, then stored coalesced. No LDS is
// allocated and no block barrier is needed. With 16-byte units the dense
// matrices (prune and compress input, prune and decompress output) are
// streamed with non-temporal accesses so they do not displace the compressed
// operand and activations the following product reads from the caches (with
// ordinary stores the first BERT-sized product after them ran up to 30%
// slower); values and metadata use ordinary stores for that reason.
#include "nm_internal.h"
#include "nm_device.h"

namespace nm {

struct RowArgs {
  const uint8_t* a;     // stored dense input (prune, compress)
  uint8_t* out;         // stored dense output (prune, decompress)
  uint32_t* mask;       // optional keep mask (prune)
  uint8_t* vals;        // compressed values
  uint8_t* meta;        // metadata bytes
  int64_t m, k, lda;    // rows, row length, row stride (elements)
  int64_t mask_ld;      // mask words per row
  int64_t vld, mld;     // compressed strides (elements, bytes)
  int64_t units;        // units per row
  int64_t segs;         // segments (64 units) per row
};

template <int ESZ, int N, int M>
struct RowGeom {
  static constexpr int GB = M * ESZ;                   // bytes per group
  static constexpr int UB = GB > 16 ? GB : 16;         // bytes per unit
  static constexpr int GU = UB / GB;                   // groups per unit
  static constexpr int EPU = UB / ESZ;                 // elements per unit
  static constexpr int DW = UB / 4;                    // dwords per unit
  static constexpr int GD = GB / 4;                    // dwords per group
  static constexpr int B = M == 4 ? 2 : M == 8 ? 3 : M == 16 ? 4 : 5;   // offset bits
  static constexpr int VB = GU * N * ESZ;              // value bytes per unit
  static constexpr int FB = GU * N * B;                // metadata bits per unit
  static constexpr int SPW = UB >= 64 ? 1 : 64 / UB;   // segments per wave (64 bytes per lane in flight)
  static_assert(GB % 4 == 0, "groups are whole dwords");
  static_assert(VB % 4 == 0 && 16 % VB == 0, "a unit's values are one aligned 4-, 8- or 16-byte store");
  static_assert(FB < 64, "a unit's offsets fit one qword");
};

template <int ESZ>
__device__ __forceinline__ uint32_t elem_of(const uint32_t* d, int e) {   // e compile-time after unrolling
  return ESZ == 2 ? (d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu : (d[e >> 2] >> (8 * (e & 3))) & 0xFFu;
}

// Element j (run-time) of a group whose GD dwords start at d: select the dword,
// then shift.
template <int ESZ, int GD>
__device__ __forceinline__ uint32_t pick_elem(const uint32_t* d, int j) {
  const int byte = j * ESZ;
  uint32_t w = d[0];
#pragma unroll
  for (int t = 1; t < GD; t++) w = (byte >> 2) == t ? d[t] : w;
  return (w >> (8 * (byte & 3))) & (ESZ == 2 ? 0xFFFFu : 0xFFu);
}

// Non-temporal only for 16-byte units: then one wave instruction covers 1 KB
// of contiguous row. Wider units (32- and 64-byte groups) leave gaps between a
// lane's 16-byte pieces in each instruction, and non-temporal accesses there
// are not merged into whole lines: measured on a 32768 x 32768 4:32 weight,
// 12% more bytes fetched and 1.6x (prune) to 2.2x (decompress) more written.
template <int ESZ, int DW>
__device__ __forceinline__ void load_unit(uint32_t (&d)[DW], const uint8_t* p, int valid_dw) {
  if (valid_dw == DW) {
#pragma unroll
    for (int c = 0; c < DW / 4; c++) {
      const u32x4 v = DW == 4 ? __builtin_nontemporal_load((const u32x4*)(p + 16 * c)) : *(const u32x4*)(p + 16 * c);
      d[4 * c] = v[0]; d[4 * c + 1] = v[1]; d[4 * c + 2] = v[2]; d[4 * c + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int t = 0; t < DW; t++) d[t] = t < valid_dw ? ((const uint32_t*)p)[t] : 0u;
  }
}

template <int DW>
__device__ __forceinline__ void store_unit(uint8_t* p, const uint32_t (&d)[DW], int valid_dw) {
  if (valid_dw == DW) {
#pragma unroll
    for (int c = 0; c < DW / 4; c++)
      if (DW == 4) __builtin_nontemporal_store(u32x4{d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]}, (u32x4*)(p + 16 * c));
      else *(u32x4*)(p + 16 * c) = u32x4{d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]};
  } else {
#pragma unroll
    for (int t = 0; t < DW; t++)
      if (t < valid_dw) ((uint32_t*)p)[t] = d[t];
  }
}

// Store the metadata of one segment: lane L holds the FB-bit field of unit L
// (zero for units past the row's end); dword w of the segment covers bits
// [32w, 32w + 32), i.e. parts of at most ceil(32 / FB) + 1 consecutive fields.
// `ndw` dwords are written (the segment's 2 * FB, or up to the row's padded
// end for the row's last segment; dwords past 2 * FB are zero). ndw is
// uniform across the wave, so every lane runs the same cross-lane reads.
template <int FB>
__device__ __forceinline__ void store_seg_meta(uint8_t* dst, uint64_t f, int ndw, int lane) {
  constexpr int NL = (32 + FB - 1) / FB + 1;
  for (int w0 = 0; w0 < ndw; w0 += 64) {
    const int w = w0 + lane;
    const int L0 = (32 * w) / FB;
    uint32_t out = 0;
#pragma unroll
    for (int t = 0; t < NL; t++) {
      const int L = L0 + t;
      const int src = L < 64 ? L : 63;
      uint64_t g = (uint32_t)__shfl((int)(uint32_t)f, src);
      if (FB > 32) g |= (uint64_t)(uint32_t)__shfl((int)(uint32_t)(f >> 32), src) << 32;
      if (L < 64 && w < 2 * FB) {
        const int sh = L * FB - 32 * w;
        if (sh >= 0) out |= sh < 32 ? (uint32_t)(g << sh) : 0u;
        else out |= (uint32_t)(g >> (-sh));
      }
    }
    if (w < ndw) ((uint32_t*)dst)[w] = out;
  }
}

enum RowOp { R_PRUNE = 0, R_COMPRESS = 1, R_DECOMPRESS = 2 };

template <int DT, int ESZ, int N, int M, int OP>
__global__ void __launch_bounds__(256) row_kernel(RowArgs A) {
  using G = RowGeom<ESZ, N, M>;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t groups_row = A.k / M;

  uint32_t d[G::SPW][G::DW];       // dense unit (prune, compress) or its values (decompress)
  uint64_t fld[G::SPW];            // offsets (decompress input)
  // ---- loads for every segment first ----
#pragma unroll
  for (int s = 0; s < G::SPW; s++) {
    const int64_t seg = wave * G::SPW + s;
    const int64_t r = seg / A.segs;
    const int64_t u = (seg % A.segs) * 64 + lane;
    fld[s] = 0;
#pragma unroll
    for (int t = 0; t < G::DW; t++) d[s][t] = 0;
    if (r >= A.m || u >= A.units) continue;
    const int vg = (int)min((int64_t)G::GU, groups_row - u * G::GU);   // valid groups in this unit
    if (OP == R_DECOMPRESS) {
      const uint8_t* vp = A.vals + r * A.vld * ESZ + u * G::VB;
      if constexpr (G::VB == 16) {
        const u32x4 v = *(const u32x4*)vp;
        d[s][0] = v[0]; d[s][1] = v[1]; d[s][2] = v[2]; d[s][3] = v[3];
      } else if constexpr (G::VB == 8) {
        const u32x2 v = *(const u32x2*)vp;
        d[s][0] = v[0]; d[s][1] = v[1];
      } else {
        d[s][0] = *(const uint32_t*)vp;
      }
      const int64_t bit = u * G::FB;
      const uint32_t* mrow = (const uint32_t*)(A.meta + r * A.mld);
      const int64_t q = bit >> 5, nq = A.mld >> 2;
      const int sh = (int)(bit & 31);
      const uint32_t d0 = mrow[q];
      const uint32_t d1 = q + 1 < nq ? mrow[q + 1] : 0u;
      uint64_t f = ((uint64_t)d1 << 32 | d0) >> sh;
      if (G::FB > 32 && sh > 0) {
        const uint32_t d2 = q + 2 < nq ? mrow[q + 2] : 0u;
        f |= (uint64_t)d2 << (64 - sh);
      }
      fld[s] = f & ((1ull << G::FB) - 1ull);
    } else {
      load_unit<ESZ, G::DW>(d[s], A.a + (r * A.lda + u * G::EPU) * ESZ, vg * G::GD);
    }
  }

  // ---- per segment: compute and store ----
#pragma unroll
  for (int s = 0; s < G::SPW; s++) {
    const int64_t seg = wave * G::SPW + s;
    const int64_t r = seg / A.segs;
    const int64_t sr = seg % A.segs;
    const int64_t u = sr * 64 + lane;
    const bool row_ok = r < A.m;                      // uniform across the wave
    const bool live = row_ok && u < A.units;
    const int vg = live ? (int)min((int64_t)G::GU, groups_row - u * G::GU) : 0;
    if (OP == R_DECOMPRESS) {
      uint32_t o[G::DW];
#pragma unroll
      for (int t = 0; t < G::DW; t++) o[t] = 0;
#pragma unroll
      for (int g = 0; g < G::GU; g++) {
        if (g >= vg) break;
#pragma unroll
        for (int sl = 0; sl < N; sl++) {
          const int slot = g * N + sl;
          const int j = (int)((fld[s] >> (slot * G::B)) & (uint64_t)(M - 1));
          const uint32_t v = elem_of<ESZ>(d[s], slot);
          // later slots win when offsets repeat (non-canonical input)
#pragma unroll
          for (int e = 0; e < M; e++) {
            const int ge = g * M + e;
            const int sft = ESZ == 2 ? 16 * (ge & 1) : 8 * (ge & 3);
            const int wd = ESZ == 2 ? ge >> 1 : ge >> 2;
            const uint32_t msk = (ESZ == 2 ? 0xFFFFu : 0xFFu) << sft;
            if (j == e) o[wd] = (o[wd] & ~msk) | (v << sft);
          }
        }
      }
      if (live) store_unit<G::DW>(A.out + (r * A.lda + u * G::EPU) * ESZ, o, vg * G::GD);
      continue;
    }
    uint32_t keep[G::GU];
#pragma unroll
    for (int g = 0; g < G::GU; g++) {
      uint32_t mag[M];
#pragma unroll
      for (int j = 0; j < M; j++) mag[j] = magkey<DT>(elem_of<ESZ>(d[s], g * M + j));
      keep[g] = g < vg ? select_topn<M>(mag, N) : 0u;
    }
    if (OP == R_PRUNE) {
      if (!live) continue;
#pragma unroll
      for (int g = 0; g < G::GU; g++)
#pragma unroll
        for (int j = 0; j < M; j++) {
          const int ge = g * M + j;
          const int sft = ESZ == 2 ? 16 * (ge & 1) : 8 * (ge & 3);
          const int wd = ESZ == 2 ? ge >> 1 : ge >> 2;
          if (!((keep[g] >> j) & 1u)) d[s][wd] &= ~((ESZ == 2 ? 0xFFFFu : 0xFFu) << sft);
        }
      store_unit<G::DW>(A.out + (r * A.lda + u * G::EPU) * ESZ, d[s], vg * G::GD);
      if (A.mask) {
        uint32_t bits = 0;
#pragma unroll
        for (int g = 0; g < G::GU; g++) bits |= keep[g] << (g * M);
        uint8_t* mrow = (uint8_t*)(A.mask + r * A.mask_ld);
        const int64_t mb = u * (G::EPU / 8);
        if (G::EPU == 8) mrow[mb] = (uint8_t)bits;
        else if (G::EPU == 16) *(uint16_t*)(mrow + mb) = (uint16_t)bits;
        else *(uint32_t*)(mrow + mb) = bits;
        if (u == A.units - 1)   // rest of the row's last mask word(s)
          for (int64_t b = mb + G::EPU / 8; b < A.mask_ld * 4; b++) mrow[b] = 0;
      }
      continue;
    }
    // ---- compress ----
    uint32_t vo[G::VB / 4];
#pragma unroll
    for (int t = 0; t < G::VB / 4; t++) vo[t] = 0;
    uint64_t f = 0;
#pragma unroll
    for (int g = 0; g < G::GU; g++) {
      uint32_t kb = keep[g];
#pragma unroll
      for (int sl = 0; sl < N; sl++) {
        const int slot = g * N + sl;
        const int j = kb ? __builtin_ctz(kb) : 0;
        kb &= kb - 1u;
        const uint32_t v = g < vg ? pick_elem<ESZ, G::GD>(d[s] + g * G::GD, j) : 0u;
        const int sft = ESZ == 2 ? 16 * (slot & 1) : 8 * (slot & 3);
        vo[ESZ == 2 ? slot >> 1 : slot >> 2] |= v << sft;
        if (g < vg) f |= (uint64_t)j << (slot * G::B);
      }
    }
    if (live) {
      uint8_t* vrow = A.vals + r * A.vld * ESZ;
      uint8_t* vp = vrow + u * G::VB;
      if constexpr (G::VB == 16) *(u32x4*)vp = u32x4{vo[0], vo[1], vo[2], vo[3]};
      else if constexpr (G::VB == 8) *(u32x2*)vp = u32x2{vo[0], vo[1]};
      else *(uint32_t*)vp = vo[0];
      if (u == A.units - 1)   // zero padding of the values row
        for (int64_t b = (u + 1) * G::VB; b < A.vld * ESZ; b += 4) *(uint32_t*)(vrow + b) = 0u;
    }
    if (row_ok) {
      const int64_t mbyte0 = sr * 8 * G::FB;
      const int ndw = (int)((sr == A.segs - 1 ? A.mld - mbyte0 : 8 * (int64_t)G::FB) / 4);
      store_seg_meta<G::FB>(A.meta + r * A.mld + mbyte0, f, ndw, lane);
    }
  }
}

template <int DT, int ESZ, int N, int M, int OP>
static hipError_t launch_row(const nm_plan& pl, RowArgs A, hipStream_t s) {
  using G = RowGeom<ESZ, N, M>;
  A.units = ((pl.p.k / M) + G::GU - 1) / G::GU;
  A.segs = (A.units + 63) / 64;
  const int64_t waves = (pl.p.m * A.segs + G::SPW - 1) / G::SPW;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  NM_LAUNCH((row_kernel<DT, ESZ, N, M, OP>), dim3((unsigned)blocks), dim3(256), 0, s, A);
  return launch_status();
}

template <int DT, int ESZ, int OP>
static hipError_t dispatch_row_t(const nm_plan& pl, const RowArgs& A, hipStream_t s) {
  const int n = pl.p.nm_n, mm = pl.p.nm_m;
  if (n == 2 && mm == 4) return launch_row<DT, ESZ, 2, 4, OP>(pl, A, s);
  if (n == 4 && mm == 32) return launch_row<DT, ESZ, 4, 32, OP>(pl, A, s);
  return launch_row<DT, ESZ, 8, 32, OP>(pl, A, s);
}

template <int OP>
static hipError_t dispatch_row(const nm_plan& pl, const RowArgs& A, hipStream_t s) {
  switch (pl.p.type_ab) {
    case NM_F16: return dispatch_row_t<DT_F16, 2, OP>(pl, A, s);
    case NM_BF16: return dispatch_row_t<DT_BF16, 2, OP>(pl, A, s);
    default: return dispatch_row_t<DT_I8, 1, OP>(pl, A, s);
  }
}

bool row_path_ok(const nm_plan& pl) {
  if (pl.p.op_a != NM_OP_N) return false;
  if ((pl.p.lda * pl.esz_ab) % 16 != 0) return false;
  const int n = pl.p.nm_n, mm = pl.p.nm_m;
  return (n == 2 && mm == 4) || (n == 4 && mm == 32) || (n == 8 && mm == 32);
}

static RowArgs row_args(const nm_plan& pl) {
  RowArgs A{};
  A.m = pl.p.m; A.k = pl.p.k; A.lda = pl.p.lda;
  A.mask_ld = (pl.a_cols + 31) / 32;
  A.vld = pl.vld; A.mld = pl.mld;
  return A;
}

hipError_t launch_row_prune(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s) {
  RowArgs A = row_args(pl);
  A.a = (const uint8_t*)a; A.out = (uint8_t*)out; A.mask = mask;
  return dispatch_row<R_PRUNE>(pl, A, s);
}

hipError_t launch_row_compress(const nm_plan& pl, const void* a, void* vals, void* meta, hipStream_t s) {
  RowArgs A = row_args(pl);
  A.a = (const uint8_t*)a; A.vals = (uint8_t*)vals; A.meta = (uint8_t*)meta;
  return dispatch_row<R_COMPRESS>(pl, A, s);
}

hipError_t launch_row_decompress(const nm_plan& pl, const void* vals, const void* meta, void* out, hipStream_t s) {
  RowArgs A = row_args(pl);
  A.vals = (uint8_t*)vals; A.meta = (uint8_t*)meta; A.out = (uint8_t*)out;
  return dispatch_row<R_DECOMPRESS>(pl, A, s);
}

}  // namespace nm
